// HIP kernels for gfx950 (CDNA4): the level-1 bf16 -> fp32 reduce of TIDE's
// reduce-scatter, the all-gather placement step, the Slot-Reuse staging copy
// and the level-2 landing sum.
//
// All are HBM streams with no reuse, so the design is about bytes in flight
// and access width, not arithmetic:
//   * the placement and the staging give each thread kVec = 8 consecutive
//     elements of a parameter's flat index space, so a wave64 touches 1 KiB
//     of contiguous bf16 per instruction (16-byte accesses); the reduce lays
//     a wave's 512 elements out as two runs of 256, 4 elements per lane, so
//     its 8-byte bf16 loads and 16-byte fp32 stores are both contiguous
//     across the wave;
//   * the reduce keeps kRsUnroll steps x L contributors of loads in flight
//     before it adds, the placement kAgUnroll steps of gathers;
//   * the fp32 sum is a left fold over contributors in registers; LDS only
//     stages a reduce step whose destination starts mid-line, so that its
//     stores cover whole lines;
//   * the destination of the reduce and the source of the placement are
//     only guaranteed 4-byte (fp32) or 2-byte (bf16) aligned: dword-aligned
//     16-byte accesses are native on CDNA, and a bf16 run that starts
//     mid-dword is realigned in registers with a 16-bit funnel shift;
//   * vectors that straddle two ranks' pieces, and the ragged ends of
//     parameters and tiles, go element by element.
// The work list is a table of tiles (TileRec) built on the host; a kernel
// walks tiles [tile_lo, tile_hi) with a grid-stride loop, so the same kernel
// serves a full grid (one tile per workgroup) and a small fixed budget of
// workgroups.
#include "tide_internal.hpp"

namespace tide {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x2_a4 __attribute__((ext_vector_type(2), aligned(4)));
typedef uint32_t u32x3_a4 __attribute__((ext_vector_type(3), aligned(4)));
typedef float f32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));

// Pointers read from the per-call table are generic pointers to the compiler;
// naming their address space lets it emit global_ (not flat_) memory ops,
// which count only against vmcnt.
#define TIDE_GLOBAL __attribute__((address_space(1)))
template <class T>
__device__ __forceinline__ const TIDE_GLOBAL T* gbl(const void* p) {
    return (const TIDE_GLOBAL T*)(p);
}
template <class T>
__device__ __forceinline__ TIDE_GLOBAL T* gbl_mut(void* p) {
    return (TIDE_GLOBAL T*)(p);
}

// Streaming (non-temporal) loads and stores: every byte is touched once.
#ifndef TIDE_NT_LOAD
#define TIDE_NT_LOAD 1
#endif
#ifndef TIDE_NT_STORE
#define TIDE_NT_STORE 1
#endif
#if TIDE_NT_LOAD
#define TIDE_LD(p) __builtin_nontemporal_load(p)
#else
#define TIDE_LD(p) (*(p))
#endif
#if TIDE_NT_STORE
#define TIDE_ST(v, p) __builtin_nontemporal_store((v), (p))
#else
#define TIDE_ST(v, p) (*(p) = (v))
#endif

// Exact bf16 -> fp32 widening of the low / high half of a dword.
__device__ __forceinline__ float lo_bf16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float widen(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// A tile as the kernels use it: its first index, that index's rank and
// in-piece offset, and the index bounds [lo, hi) of the launch's rank range.
struct Span {
    int64_t idx0, j0, lo, hi;
    int64_t r0;
};

// Rank r and offset j inside rank r's piece of flat index f of tile t, for
// idx0 <= f < idx0 + tile. Since j0 < s, j < s + tile: one subtraction does
// when s >= tile, and a 32-bit division otherwise.
template <int64_t kTile>
__device__ __forceinline__ void locate(const Span& t, int64_t s, int64_t f, int64_t& r,
                                       int64_t& j) {
    j = t.j0 + (f - t.idx0);
    r = t.r0;
    if (j >= s) {
        if (s >= kTile) {
            j -= s;
            r += 1;
        } else {
            const uint32_t q = (uint32_t)j / (uint32_t)s;
            r += q;
            j -= (int64_t)q * s;
        }
    }
}

// Advance (r, j) by one element.
__device__ __forceinline__ void step(int64_t s, int64_t& r, int64_t& j) {
    if (++j == s) {
        j = 0;
        ++r;
    }
}

// Lane layout of a reduce step: a wave's 512 elements are two runs of 256,
// and lane l owns elements 4l..4l+3 of each run, so each wave-wide 16-byte
// store writes 1 KiB of fp32 with no gaps (whole cache lines) and each 8-byte
// load reads 512 contiguous bf16 bytes. (Eight consecutive elements per lane,
// with 16-byte loads and two gapped stores, measured 6% more write traffic.)
constexpr int kWave = 64;
constexpr int kHalf = kWave * 4;           // elements of one run

// Debug write counts (tide_launch.write_counts): in the kernels instantiated
// with CNT, every element written adds one to counts[idx .. idx + n). The
// normal kernels (CNT false) carry no trace of it.
template <bool CNT>
__device__ __forceinline__ void count_writes(uint32_t* counts, int64_t idx, int n) {
    if constexpr (CNT) {
        for (int e = 0; e < n; ++e) atomicAdd(counts + idx + e, 1u);
    } else {
        (void)counts;
        (void)idx;
        (void)n;
    }
}


// Write 4 fp32 results for flat indices f..f+3 (all inside the tile's range).
template <int64_t kTile, bool CNT>
__device__ __forceinline__ void store4(const Span& t, const ParamDev& pd, int64_t f,
                                       const float (&a)[4], float* __restrict__ out,
                                       int64_t stride, uint32_t* counts) {
    int64_t r, j;
    locate<kTile>(t, pd.s, f, r, j);
    if (j + 4 <= pd.s) {
        const f32x4_a4 x = {a[0], a[1], a[2], a[3]};
        TIDE_ST(x, reinterpret_cast<f32x4_a4*>(out + r * stride + pd.o + j));
        count_writes<CNT>(counts, r * stride + pd.o + j, 4);
    } else {
#pragma unroll 1
        for (int e = 0; e < 4; ++e) {
            out[r * stride + pd.o + j] = a[e];
            count_writes<CNT>(counts, r * stride + pd.o + j, 1);
            step(pd.s, r, j);
        }
    }
}

// XCD-aware tile order for the full grid. The dispatcher sends workgroup i
// to XCD i mod kXcds, and each XCD has its own L2. With a chunk C > 0,
// workgroup i takes tile (chunk * kXcds + xcd) * C + within, so every XCD
// walks runs of C consecutive tiles and a cache line shared by two
// neighbouring tiles goes through one L2 rather than two. The mapping is a
// bijection on the first multiple of kXcds * C tiles and the identity on the
// rest (C = 1 is the identity). The placement (whose bf16 source runs start
// at arbitrary 2-byte offsets) uses runs of 128: interleaved on MI355X
// against round robin, padding stress +1.3%, Llama +1.6%, Wan +1.4%, Qwen
// +0% (16: slower everywhere; 256: Qwen -1%). For the reduce the host picks
// C per call (reduce_xcd_log2 in plan.cpp).
#ifndef TIDE_XCD_CHUNK_AG
#define TIDE_XCD_CHUNK_AG 128
#endif
constexpr int64_t kXcds = 8;
template <int64_t C>
__device__ __forceinline__ int64_t xcd_tile(int64_t b, int64_t n) {
    if (C <= 0) return b;
    const int64_t full = n / (kXcds * C) * (kXcds * C);
    if (b >= full) return b;
    const int64_t xcd = b % kXcds, j = b / kXcds;
    return ((j / C) * kXcds + xcd) * C + j % C;
}
// The same with C = 2^lc chosen at run time.
__device__ __forceinline__ int64_t xcd_tile_rt(int64_t b, int64_t n, int lc) {
    const int64_t full = n >> (3 + lc) << (3 + lc);
    if (b >= full) return b;
    const int64_t xcd = b & (kXcds - 1), j = b >> 3;
    return ((((j >> lc) << 3) + xcd) << lc) + (j & ((int64_t(1) << lc) - 1));
}

// Write one wave's run of kHalf fp32 results: lane l holds a[0..3] for flat
// indices f_run + 4l .. f_run + 4l + 3. A run inside one rank's piece has a
// contiguous destination (one wave-wide 16-byte store, 1 KiB); a run that
// crosses into the next rank's piece goes lane by lane. Runs that start
// mid-line (prefix offsets that are not multiples of 4 elements) cost about
// 3.5% of bandwidth; neither realigning them across lanes nor plain
// write-back stores recovered it on MI355X.
template <int64_t kTile, bool CNT>
__device__ __forceinline__ void store_run(const Span& t, const ParamDev& pd, int64_t f_run,
                                          int lane, const float (&a)[4],
                                          float* __restrict__ out, int64_t stride,
                                          uint32_t* counts) {
    int64_t r, j;
    locate<kTile>(t, pd.s, f_run, r, j);
    if (j + kHalf > pd.s) {                   // the run crosses into the next rank's piece
        store4<kTile, CNT>(t, pd, f_run + 4 * lane, a, out, stride, counts);
        return;
    }
    const f32x4_a4 x = {a[0], a[1], a[2], a[3]};
    TIDE_ST(x, reinterpret_cast<f32x4_a4*>(out + r * stride + pd.o + j + 4 * lane));
    count_writes<CNT>(counts, r * stride + pd.o + j + 4 * lane, 4);
}

// Workgroup tracing (tide_launch.trace): the real-time counter at the start,
// and at the end, once every wave of the workgroup is done, one record with
// the hardware ids of the CU it ran on. `trace` is a kernel argument, so the
// branches are uniform and cost nothing when it is null.
constexpr int kHwregAll = 31 << 11;            // s_getreg: 32 bits from offset 0
constexpr int kHwregHwId = kHwregAll | 4;      // HW_ID
constexpr int kHwregXccId = kHwregAll | 20;    // XCC_ID
__device__ __forceinline__ uint64_t trace_begin(const tide_trace_rec* trace) {
    return trace ? __builtin_amdgcn_s_memrealtime() : 0;
}
__device__ __forceinline__ void trace_end(tide_trace_rec* trace, int64_t base, uint64_t t_begin) {
    if (!trace) return;
    __syncthreads();
    if (threadIdx.x == 0) {
        tide_trace_rec r;
        r.hw_id = __builtin_amdgcn_s_getreg(kHwregHwId);
        r.xcc_id = __builtin_amdgcn_s_getreg(kHwregXccId);
        r.t_begin = t_begin;
        r.t_end = __builtin_amdgcn_s_memrealtime();
        trace[base + blockIdx.x] = r;
    }
}

// The tile record of reduce tile t when no tile table exists (the
// allocation-free entry point): `hdr` = {P, cum[0..P]}, cum[p] the reduce
// tiles of the parameters before p over the launch's rank range, in
// parameter order. Tile t belongs to the last parameter p with cum[p] <= t
// and starts kTile * (t - cum[p]) past the vector-aligned start of that
// parameter's range: the records a tile table would hold, in parameter order.
template <int64_t kTile>
__device__ __forceinline__ TileRec derive_tile(const int64_t* __restrict__ hdr,
                                               const ParamDev* __restrict__ params, int32_t rb,
                                               int64_t t) {
    const int64_t* cum = hdr + 1;
    int64_t lo = 0, hi = hdr[0];
    while (hi - lo > 1) {
        const int64_t mid = (lo + hi) >> 1;
        if (cum[mid] <= t) lo = mid; else hi = mid;
    }
    const int64_t s = params[lo].s;
    const int64_t first = (int64_t)rb * s;
    TileRec r;
    r.idx0 = first - first % kVec + (t - cum[lo]) * kTile;
    r.p = (int32_t)lo;
    r.r0 = (int32_t)(r.idx0 / s);
    return r;
}

// Misaligned destinations through LDS (see the reduce's interior path).
#ifndef TIDE_RS_LDS_ALIGN
#define TIDE_RS_LDS_ALIGN 1
#endif

// Reduce: out[rank piece] = fold_c widen(g[c][f]) for f < valid, +0 past it.
// LT > 0: L known at compile time (fully unrolled); LT == 0: runtime L.
// A workgroup of NT threads is NT / kThreads independent quarters of kThreads
// threads; each quarter walks its own tiles (no barrier between quarters).
// SHIFTED: the variant that also reads gradients starting at 2 mod 4 bytes
// with vector loads (dword-aligned loads and a funnel shift). Its extra
// registers would cost the common, all-aligned case a resident wave per SIMD
// (81 instead of 80 VGPRs), so the host uses it only for calls that need it.
template <int LT, int NT, bool CNT, bool DERIVED, bool SHIFTED>
__global__ __launch_bounds__(NT) void reduce_kernel(
    const TileRec* __restrict__ tiles, int64_t tile_lo, int64_t tile_hi, int32_t rb, int32_t re,
    const ParamDev* __restrict__ params, const uint16_t* const* __restrict__ ptrs,
    const uint32_t* __restrict__ flags, int Lrt, float* __restrict__ out, int64_t out_stride,
    tide_trace_rec* __restrict__ trace, int64_t trace_base, uint32_t* __restrict__ counts,
    int32_t xcd_lc) {
    const uint64_t t_begin = trace_begin(trace);
    constexpr int kSubs = NT / kThreads;
    // Budgeted (fat) workgroups walk longer tiles with more loads in flight:
    // one workgroup per CU has no other workgroups to hide its latency.
    constexpr int64_t kTileR = NT == kFatThreads ? kRsTileFat : kRsTile;
    constexpr int kUR = NT == kFatThreads ? kRsUnrollFat : kRsUnroll;
    const int L = LT > 0 ? LT : Lrt;
    // Wave-uniform, and in the shifted variant also provably so to the
    // compiler (readfirstlane): the tile walk then runs in scalar registers
    // and each contributor's choice of loads is a scalar branch, so the loads
    // of all contributors are still issued before the first add waits (as
    // exec-masked regions, each contributor waited for its loads in turn:
    // 4.2 against 5.8 TB/s on MI355X for a group at 2 mod 4 bytes). The
    // aligned variant keeps the plain form, which measured 1-8% faster there,
    // and so do budgeted workgroups, where the scalar form runs out of SGPRs
    // and spills for some L.
    constexpr bool kUniform = SHIFTED && NT == kThreads;
    const int sub = kUniform ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / kThreads)
                             : (int)threadIdx.x / kThreads;
    const int tid = (int)threadIdx.x % kThreads;
#if TIDE_RS_LDS_ALIGN
    // Staging of one step for whole-line stores (full grid only; budgeted
    // workgroups keep their LDS reservation for the fence).
    __shared__ __attribute__((aligned(16))) float lds_stage[NT == kThreads ? kStep : 4];
    const int64_t out_e0 = (int64_t)(reinterpret_cast<uintptr_t>(out) >> 2);
#endif
    // One tile per workgroup (the full grid): XCD-aware order.
    const bool one_each = kSubs == 1 && (int64_t)gridDim.x == tile_hi - tile_lo;
    for (int64_t t = tile_lo + (int64_t)blockIdx.x * kSubs + sub; t < tile_hi;
         t += (int64_t)gridDim.x * kSubs) {
        const int64_t ti =
            one_each ? tile_lo + xcd_tile_rt(t - tile_lo, tile_hi - tile_lo, xcd_lc) : t;
        TileRec rec;
        if constexpr (DERIVED)
            rec = derive_tile<kTileR>(reinterpret_cast<const int64_t*>(tiles), params, rb, ti);
        else
            rec = tiles[ti];
        const ParamDev pd = params[rec.p];
        const uint16_t* const* g = ptrs + (int64_t)rec.p * L;
        const uint32_t fl = flags[rec.p];
        const bool vec = (fl & kFlagVector) != 0;
        const uint32_t odd = SHIFTED ? fl >> kOddShift : 0u;   // contributors at 2 mod 4 bytes
        const Span tr{rec.idx0, rec.idx0 - (int64_t)rec.r0 * pd.s, (int64_t)rb * pd.s,
                      (int64_t)re * pd.s, rec.r0};
        const int64_t end = min(tr.idx0 + kTileR, tr.hi);
        for (int64_t g0 = tr.idx0; g0 < end; g0 += kUR * kStep) {
            const int64_t g1 = g0 + kUR * kStep;
            const bool interior = vec && g0 >= tr.lo && g1 <= end;
            const int64_t f0 = g0 + (int64_t)tid * kVec;
            const int lane = tid % kWave;
            const int wv = kUniform ? __builtin_amdgcn_readfirstlane(tid / kWave) : tid / kWave;
            const int64_t fw = g0 + (int64_t)wv * (2 * kHalf);   // wave's first index
            const int64_t fh = fw + lane * 4;
            if (interior && g1 <= pd.valid) {
                // All loads are independent of the adds: they are all issued
                // before the first add waits.
                float a[kUR][2][4];
                constexpr int kCUnroll = LT > 0 ? LT : 1;
#pragma unroll kCUnroll
                for (int c = 0; c < L; ++c) {
                    u32x2 v[kUR][2];
                    if (odd & (1u << c)) {
                        // Contributor c starts at 2 mod 4 bytes: the lane's 4
                        // elements f..f+3 lie in the 3 dwords from element
                        // f - 1 (f is a multiple of 4, so f - 1 starts a
                        // dword); every dword read holds an element of the
                        // step's valid range, or the one before it, or the
                        // one after it in the same dword. Wave-uniform.
                        // (Measured on MI355X and not kept: 8-byte loads with
                        // the third dword from the next lane, over ds_bpermute
                        // or a DPP wavefront shift, both slower.)
                        const TIDE_GLOBAL u32x3_a4* gq = gbl<u32x3_a4>(g[c] + fh - 1);
#pragma unroll
                        for (int u = 0; u < kUR; ++u)
#pragma unroll
                            for (int h = 0; h < 2; ++h) {
                                const u32x3_a4 w = TIDE_LD(reinterpret_cast<const TIDE_GLOBAL u32x3_a4*>(
                                    reinterpret_cast<const TIDE_GLOBAL uint16_t*>(gq) + u * kStep + h * kHalf));
                                v[u][h][0] = __builtin_amdgcn_alignbit(w[1], w[0], 16);
                                v[u][h][1] = __builtin_amdgcn_alignbit(w[2], w[1], 16);
                            }
                    } else {
                        const TIDE_GLOBAL u32x2_a4* gc = gbl<u32x2_a4>(g[c] + fh);
#pragma unroll
                        for (int u = 0; u < kUR; ++u)
#pragma unroll
                            for (int h = 0; h < 2; ++h)
                                v[u][h] = TIDE_LD(gc + (u * kStep + h * kHalf) / 4);
                    }
#pragma unroll
                    for (int u = 0; u < kUR; ++u) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
#pragma unroll
                            for (int m = 0; m < 2; ++m) {
                                if (c == 0) {
                                    a[u][h][2 * m] = lo_bf16(v[u][h][m]);
                                    a[u][h][2 * m + 1] = hi_bf16(v[u][h][m]);
                                } else {
                                    a[u][h][2 * m] = a[u][h][2 * m] + lo_bf16(v[u][h][m]);
                                    a[u][h][2 * m + 1] = a[u][h][2 * m + 1] + hi_bf16(v[u][h][m]);
                                }
                            }
                        }
                    }
                }
                if constexpr (NT == kThreads && kUR == 1 && TIDE_RS_LDS_ALIGN) {
                    // A step inside one rank's piece whose destination starts
                    // mid-line (a prefix offset or shard stride not a multiple
                    // of 32 elements): its sums go through LDS, so that each
                    // wave-wide store covers whole 128-byte lines and only the
                    // two lines at the step's ends are partly written, element
                    // by element. Storing the runs in place leaves every run's
                    // two end lines partly written by different waves, and
                    // those partial lines cost 4-5% of the reduce's bandwidth
                    // on MI355X (the counters show them as extra writes); the
                    // LDS round trip costs nothing measurable.
                    int64_t r, j;
                    locate<kTileR>(tr, pd.s, g0, r, j);
                    const int64_t d0 = r * out_stride + pd.o + j;   // destination of g0
                    const int m = (int)((out_e0 + d0) & 31);
                    if (m != 0 && j + kStep <= pd.s) {
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            float* at = lds_stage + (fw - g0) + h * kHalf + 4 * lane;
                            *reinterpret_cast<float4*>(at) =
                                make_float4(a[0][h][0], a[0][h][1], a[0][h][2], a[0][h][3]);
                        }
                        __syncthreads();
                        const int a0 = 32 - m;                      // first element on a line start
                        float* dst = out + d0;
#pragma unroll
                        for (int k = 0; k < 2; ++k) {
                            const int q = tid + k * kThreads;       // quad of the whole lines
                            if (q < (kStep - 32) / 4) {
                                const int e = a0 + 4 * q;
                                const f32x4_a4 x = {lds_stage[e], lds_stage[e + 1], lds_stage[e + 2],
                                                    lds_stage[e + 3]};
                                TIDE_ST(x, reinterpret_cast<f32x4_a4*>(dst + e));
                                count_writes<CNT>(counts, d0 + e, 4);
                            }
                        }
                        if (tid < 32) {                             // the two partial lines
                            const int e = tid < a0 ? tid : kStep - 32 + tid;
                            dst[e] = lds_stage[e];
                            count_writes<CNT>(counts, d0 + e, 1);
                        }
                        __syncthreads();                            // lds_stage is reused by the next tile
                        continue;
                    }
                }
#pragma unroll
                for (int u = 0; u < kUR; ++u)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        store_run<kTileR, CNT>(tr, pd, fw + (int64_t)u * kStep + h * kHalf, lane, a[u][h],
                                  out, out_stride, counts);
            } else if (interior && g0 >= pd.valid) {
                const float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int u = 0; u < kUR; ++u)
#pragma unroll
                    for (int h = 0; h < 2; ++h)
                        store_run<kTileR, CNT>(tr, pd, fw + (int64_t)u * kStep + h * kHalf, lane, z, out,
                                  out_stride, counts);
            } else {
                // Ragged step: it crosses an end of the launch's range or of
                // the tile, or the valid end, or the parameter has pointers
                // that are not 4-byte aligned. A thread's group of 8
                // elements that lies wholly inside the step's bounds and on
                // one side of the valid end still goes as one vector; only
                // a group that straddles a bound goes element by element.
#pragma unroll 1
                for (int u = 0; u < kUR; ++u) {
                    const int64_t fu = f0 + (int64_t)u * kStep;
                    const bool whole = fu >= tr.lo && fu + kVec <= end;
                    if (whole && vec && odd == 0 && fu + kVec <= pd.valid) {
                        float a[2][4];
                        constexpr int kCUnroll = LT > 0 ? LT : 1;
#pragma unroll kCUnroll
                        for (int c = 0; c < L; ++c) {
                            const u32x4 v = TIDE_LD(gbl<u32x4_a4>(g[c] + fu));
#pragma unroll
                            for (int m = 0; m < 4; ++m) {
                                const float lo = lo_bf16(v[m]), hi = hi_bf16(v[m]);
                                float& x0 = a[m / 2][2 * (m % 2)];
                                float& x1 = a[m / 2][2 * (m % 2) + 1];
                                x0 = c == 0 ? lo : x0 + lo;
                                x1 = c == 0 ? hi : x1 + hi;
                            }
                        }
                        store4<kTileR, CNT>(tr, pd, fu, a[0], out, out_stride, counts);
                        store4<kTileR, CNT>(tr, pd, fu + 4, a[1], out, out_stride, counts);
                    } else if (whole && fu >= pd.valid) {
                        const float z[4] = {0.0f, 0.0f, 0.0f, 0.0f};
                        store4<kTileR, CNT>(tr, pd, fu, z, out, out_stride, counts);
                        store4<kTileR, CNT>(tr, pd, fu + 4, z, out, out_stride, counts);
                    } else {
                        int64_t r, j;
                        locate<kTileR>(tr, pd.s, fu, r, j);
#pragma unroll 1
                        for (int e = 0; e < kVec; ++e, step(pd.s, r, j)) {
                            const int64_t f = fu + e;
                            if (f < tr.lo || f >= end) continue;
                            float v = 0.0f;
                            if (f < pd.valid) {
                                if constexpr (LT > 0) {
                                    // All L loads issued before the first add.
                                    uint16_t h[LT > 0 ? LT : 1];
#pragma unroll
                                    for (int c = 0; c < LT; ++c) h[c] = gbl<uint16_t>(g[c])[f];
                                    v = widen(h[0]);
#pragma unroll
                                    for (int c = 1; c < LT; ++c) v = v + widen(h[c]);
                                } else {
                                    v = widen(gbl<uint16_t>(g[0])[f]);
#pragma unroll 1
                                    for (int c = 1; c < L; ++c) v = v + widen(gbl<uint16_t>(g[c])[f]);
                                }
                            }
                            out[r * out_stride + pd.o + j] = v;
                            count_writes<CNT>(counts, r * out_stride + pd.o + j, 1);
                        }
                    }
                }
            }
        }
    }
    trace_end(trace, trace_base, t_begin);
}

// Position of rank r's shard in a stage buffer that starts with rank first.
__device__ __forceinline__ int64_t stage_pos(int64_t r, int32_t first, int32_t n) {
    const int64_t q = r - first;
    return q < 0 ? q + n : q;
}

// 8 bf16 of the rank-major shards for flat parameter indices f..f+7.
template <int64_t kTile>
__device__ __forceinline__ u32x4 gather8(const Span& t, const ParamDev& pd, int64_t f,
                                         const uint16_t* __restrict__ shards, int64_t stride,
                                         int64_t shard_elems, int32_t first, int32_t n) {
    int64_t r, j;
    locate<kTile>(t, pd.s, f, r, j);
    if (j + kVec <= pd.s) {
        const int64_t e = stage_pos(r, first, n) * stride + pd.o + j;
        const uint16_t* src = shards + e;
        if ((reinterpret_cast<uintptr_t>(src) & 3) == 0)
            return TIDE_LD(reinterpret_cast<const u32x4_a4*>(src));
        if (e >= 1 && e + 9 <= shard_elems) {
            // src is 2 mod 4: load the 5 dwords covering elements e-1 .. e+8
            // (all inside the shard buffer) and shift them down 16 bits.
            const uint32_t* d = reinterpret_cast<const uint32_t*>(src - 1);
            const u32x4_a4 x = TIDE_LD(reinterpret_cast<const u32x4_a4*>(d));
            const uint32_t y = TIDE_LD(d + 4);
            u32x4 w;
            w[0] = __builtin_amdgcn_alignbit(x[1], x[0], 16);
            w[1] = __builtin_amdgcn_alignbit(x[2], x[1], 16);
            w[2] = __builtin_amdgcn_alignbit(x[3], x[2], 16);
            w[3] = __builtin_amdgcn_alignbit(y, x[3], 16);
            return w;
        }
    }
    // Straddles two ranks' pieces, or sits at the very ends of the buffer.
    uint32_t h[kVec];
#pragma unroll
    for (int e = 0; e < kVec; ++e) {
        h[e] = shards[stage_pos(r, first, n) * stride + pd.o + j];
        step(pd.s, r, j);
    }
    u32x4 w;
#pragma unroll
    for (int m = 0; m < 4; ++m) w[m] = h[2 * m] | (h[2 * m + 1] << 16);
    return w;
}

// gather8 for a step in which every lane of the wave takes part (the
// placement's interior steps). A source at 2 mod 4 needs the dword after its
// 16-byte load: when the next lane reads on in the same piece, that dword is
// the next lane's first one and comes over the lane crossbar instead of from
// a second load (measured on MI355X: the second load cost the placement 10%
// whenever half its sources sat at 2 mod 4).
#ifndef TIDE_AG_NEIGHBOUR
#define TIDE_AG_NEIGHBOUR 1
#endif
template <int64_t kTile, int U>
__device__ __forceinline__ void gather8_wave(const Span& t, const ParamDev& pd, int64_t f0, int lane,
                                             const uint16_t* __restrict__ shards, int64_t stride,
                                             int64_t shard_elems, int32_t first, int32_t n,
                                             u32x4 (&w)[U]) {
    int64_t r[U], j[U], e[U];
    bool direct[U], shift[U], from_next[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        locate<kTile>(t, pd.s, f0 + (int64_t)u * kStep, r[u], j[u]);
        e[u] = stage_pos(r[u], first, n) * stride + pd.o + j[u];
        const bool inside = j[u] + kVec <= pd.s;
        const bool odd = (reinterpret_cast<uintptr_t>(shards + e[u]) & 3) != 0;
        direct[u] = inside && !odd;
        shift[u] = inside && odd && e[u] >= 1 && e[u] + 9 <= shard_elems;
        // Lane l+1 then holds elements e+8.. of the same piece, at the same
        // alignment and inside the buffer: it takes the shifted load too, and
        // its first dword holds elements e+7, e+8.
        from_next[u] = shift[u] && lane != kWave - 1 && j[u] + 2 * kVec <= pd.s &&
                       e[u] + 17 <= shard_elems;
    }
    bool all_direct = true;
#pragma unroll
    for (int u = 0; u < U; ++u) all_direct = all_direct && direct[u];
    if (__builtin_amdgcn_ballot_w64(!all_direct) == 0) {   // wave-uniform: every source dword-aligned
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = TIDE_LD(reinterpret_cast<const u32x4_a4*>(shards + e[u]));
        return;
    }
    // All loads are issued before any result is used, the ninth pair of a
    // lane without a neighbour included.
    u32x4 x[U];
    uint32_t y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        x[u] = u32x4{0u, 0u, 0u, 0u};
        y[u] = 0u;
        if (direct[u])
            x[u] = TIDE_LD(reinterpret_cast<const u32x4_a4*>(shards + e[u]));
        else if (shift[u])
            x[u] = TIDE_LD(reinterpret_cast<const u32x4_a4*>(shards + e[u] - 1));
        if (shift[u] && !from_next[u]) y[u] = TIDE_LD(reinterpret_cast<const uint32_t*>(shards + e[u] - 1) + 4);
    }
    bool any_shift = false;
#pragma unroll
    for (int u = 0; u < U; ++u) any_shift = any_shift || shift[u];
    if (__builtin_amdgcn_ballot_w64(any_shift) != 0) {     // wave-uniform
#pragma unroll
        for (int u = 0; u < U; ++u) {
            // Every lane of the wave runs this: lane l receives lane l+1's first dword.
            const uint32_t next =
                (uint32_t)__builtin_amdgcn_ds_bpermute(((lane + 1) & (kWave - 1)) << 2, (int)x[u][0]);
            if (from_next[u]) y[u] = next;
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (direct[u]) {
            w[u] = x[u];
        } else if (shift[u]) {
            w[u][0] = __builtin_amdgcn_alignbit(x[u][1], x[u][0], 16);
            w[u][1] = __builtin_amdgcn_alignbit(x[u][2], x[u][1], 16);
            w[u][2] = __builtin_amdgcn_alignbit(x[u][3], x[u][2], 16);
            w[u][3] = __builtin_amdgcn_alignbit(y[u], x[u][3], 16);
        } else {
            // Straddles two ranks' pieces, or sits at the very ends of the buffer.
            int64_t rr = r[u], jj = j[u];
            uint32_t h[kVec];
#pragma unroll
            for (int k = 0; k < kVec; ++k) {
                h[k] = shards[stage_pos(rr, first, n) * stride + pd.o + jj];
                step(pd.s, rr, jj);
            }
#pragma unroll
            for (int m = 0; m < 4; ++m) w[u][m] = h[2 * m] | (h[2 * m + 1] << 16);
        }
    }
}

// Placement: param[f] = shards[rank(f) * stride + o_p + offset(f)] for true f.
template <int NT, bool CNT>
__global__ __launch_bounds__(NT) void place_kernel(
    const TileRec* __restrict__ tiles, int64_t tile_lo, int64_t tile_hi, int32_t rb, int32_t re,
    const ParamDev* __restrict__ params, uint16_t* const* __restrict__ ptrs,
    const uint32_t* __restrict__ flags, const uint16_t* __restrict__ shards, int64_t stride,
    int64_t shard_elems, int32_t first, int32_t nranks, tide_trace_rec* __restrict__ trace,
    int64_t trace_base, uint32_t* __restrict__ counts) {
    const uint64_t t_begin = trace_begin(trace);
    constexpr int kSubs = NT / kThreads;
    constexpr int64_t kTileA = NT == kFatThreads ? kAgTileFat : kAgTile;
    constexpr int kUA = NT == kFatThreads ? kAgUnrollFat : kAgUnroll;
    const int sub = (int)threadIdx.x / kThreads;
    const int tid = (int)threadIdx.x % kThreads;
    const bool one_each = kSubs == 1 && (int64_t)gridDim.x == tile_hi - tile_lo;
    for (int64_t t = tile_lo + (int64_t)blockIdx.x * kSubs + sub; t < tile_hi;
         t += (int64_t)gridDim.x * kSubs) {
        const TileRec rec =
            tiles[one_each ? tile_lo + xcd_tile<TIDE_XCD_CHUNK_AG>(t - tile_lo, tile_hi - tile_lo)
                           : t];
        const ParamDev pd = params[rec.p];
        uint16_t* dst = ptrs[rec.p];
        const bool vec = (flags[rec.p] & kFlagVector) != 0;
        const int64_t cbase = (int64_t)nranks * pd.o;   // write counts: N * o_p + f
        const Span tr{rec.idx0, rec.idx0 - (int64_t)rec.r0 * pd.s, (int64_t)rb * pd.s,
                      min((int64_t)re * pd.s, pd.valid), rec.r0};
        const int64_t end = min(tr.idx0 + kTileA, tr.hi);
        for (int64_t g0 = tr.idx0; g0 < end; g0 += kUA * kStep) {
            const int64_t g1 = g0 + kUA * kStep;
            const int64_t f0 = g0 + (int64_t)tid * kVec;
            if (vec && g0 >= tr.lo && g1 <= end) {
                u32x4 w[kUA];
#if TIDE_AG_NEIGHBOUR
                gather8_wave<kTileA, kUA>(tr, pd, f0, tid % kWave, shards, stride, shard_elems, first,
                                          nranks, w);
#else
#pragma unroll
                for (int u = 0; u < kUA; ++u)
                    w[u] = gather8<kTileA>(tr, pd, f0 + (int64_t)u * kStep, shards, stride, shard_elems,
                                   first, nranks);
#endif
                TIDE_GLOBAL u32x4* d4 = gbl_mut<u32x4>(dst + f0);
#pragma unroll
                for (int u = 0; u < kUA; ++u) {
                    TIDE_ST(w[u], d4 + u * (kStep / kVec));
                    count_writes<CNT>(counts, cbase + f0 + (int64_t)u * kStep, kVec);
                }
            } else {
                // Ragged step: a thread's group of 8 that lies wholly inside
                // the bounds still goes as one vector; only a group that
                // straddles a bound (or a parameter without 16-byte pointers)
                // goes element by element.
                TIDE_GLOBAL uint16_t* d = gbl_mut<uint16_t>(dst);
#pragma unroll 1
                for (int u = 0; u < kUA; ++u) {
                    const int64_t fu = f0 + (int64_t)u * kStep;
                    if (vec && fu >= tr.lo && fu + kVec <= end) {
                        const u32x4 w = gather8<kTileA>(tr, pd, fu, shards, stride, shard_elems, first, nranks);
                        TIDE_ST(w, gbl_mut<u32x4>(dst + fu));
                        count_writes<CNT>(counts, cbase + fu, kVec);
                        continue;
                    }
                    int64_t r, j;
                    locate<kTileA>(tr, pd.s, fu, r, j);
#pragma unroll 1
                    for (int e = 0; e < kVec; ++e, step(pd.s, r, j)) {
                        const int64_t f = fu + e;
                        if (f < tr.lo || f >= end) continue;
                        d[f] = shards[stage_pos(r, first, nranks) * stride + pd.o + j];
                        count_writes<CNT>(counts, cbase + f, 1);
                    }
                }
            }
        }
    }
    trace_end(trace, trace_base, t_begin);
}

// Slot-Reuse staging: dst[p][c][f] = src[p][c][f] for the launch's true
// indices f of each parameter (a plain copy; dst is the parameter's place in
// contributor c's slot). Work item t is tile t mod ntiles of the staging
// tiling, for contributor t / ntiles. With kFlagVector every pointer of the
// parameter is 4-byte aligned, so 16-byte accesses at 8-element steps are
// dword aligned.
template <int NT, bool CNT>
__global__ __launch_bounds__(NT) void stage_kernel(
    const TileRec* __restrict__ tiles, int64_t ntiles, int64_t tile_lo, int64_t tile_hi,
    int32_t rb, int32_t re, const ParamDev* __restrict__ params,
    const uint16_t* const* __restrict__ src, uint16_t* const* __restrict__ dst,
    const uint32_t* __restrict__ flags, int32_t L, tide_trace_rec* __restrict__ trace,
    int64_t trace_base, uint32_t* __restrict__ counts, int64_t slot_elems, int32_t nranks) {
    const uint64_t t_begin = trace_begin(trace);
    constexpr int kSubs = NT / kThreads;
    constexpr int64_t kTileS = NT == kFatThreads ? kStageTileFat : kStageTile;
    constexpr int kUS = NT == kFatThreads ? kStageUnrollFat : kStageUnroll;
    const int sub = (int)threadIdx.x / kThreads;
    const int tid = (int)threadIdx.x % kThreads;
    for (int64_t t = tile_lo + (int64_t)blockIdx.x * kSubs + sub; t < tile_hi;
         t += (int64_t)gridDim.x * kSubs) {
        const int64_t c = t / ntiles;
        const TileRec rec = tiles[t - c * ntiles];
        const ParamDev pd = params[rec.p];
        const uint16_t* s = src[(int64_t)rec.p * L + c];
        uint16_t* d = dst[(int64_t)rec.p * L + c];
        const bool vec = (flags[rec.p] & kFlagVector) != 0;
        const int64_t lo = (int64_t)rb * pd.s;
        const int64_t end = min(rec.idx0 + kTileS, min((int64_t)re * pd.s, pd.valid));
        const int64_t cbase = c * slot_elems + (int64_t)nranks * pd.o;   // write counts
        for (int64_t g0 = rec.idx0; g0 < end; g0 += kUS * kStep) {
            const int64_t f0 = g0 + (int64_t)tid * kVec;
            if (vec && g0 >= lo && g0 + kUS * kStep <= end) {
                u32x4_a4 w[kUS];
#pragma unroll
                for (int u = 0; u < kUS; ++u)
                    w[u] = TIDE_LD(gbl<u32x4_a4>(s + f0 + (int64_t)u * kStep));
#pragma unroll
                for (int u = 0; u < kUS; ++u) {
                    TIDE_ST(w[u], gbl_mut<u32x4_a4>(d + f0 + (int64_t)u * kStep));
                    count_writes<CNT>(counts, cbase + f0 + (int64_t)u * kStep, kVec);
                }
            } else {
                // Ragged step: whole groups of 8 inside the bounds as vectors,
                // a group that straddles a bound element by element.
                const TIDE_GLOBAL uint16_t* gs = gbl<uint16_t>(s);
                TIDE_GLOBAL uint16_t* gd = gbl_mut<uint16_t>(d);
#pragma unroll 1
                for (int u = 0; u < kUS; ++u) {
                    const int64_t fu = f0 + (int64_t)u * kStep;
                    if (vec && fu >= lo && fu + kVec <= end) {
                        const u32x4_a4 w = TIDE_LD(gbl<u32x4_a4>(s + fu));
                        TIDE_ST(w, gbl_mut<u32x4_a4>(d + fu));
                        count_writes<CNT>(counts, cbase + fu, kVec);
                        continue;
                    }
#pragma unroll 1
                    for (int e = 0; e < kVec; ++e) {
                        const int64_t f = fu + e;
                        if (f >= lo && f < end) {
                            gd[f] = gs[f];
                            count_writes<CNT>(counts, cbase + f, 1);
                        }
                    }
                }
            }
        }
    }
    trace_end(trace, trace_base, t_begin);
}

// Level-2 landing sum: shard_b[f] = fold_c inbox_{(s - c) mod L}[(s L + b) C + e]
// with s = f / C, e = f % C. All M inboxes are read at the same offset (the
// Latin-square seating puts a slice's copies at the same address on M
// GPUs), 16 bytes per lane, so each wave reads M contiguous 1 KiB runs.
template <int MT, int NT, bool CNT>
__global__ __launch_bounds__(NT) void landing_kernel(LandingPtrs ptrs, int32_t L, int32_t Mrt,
                                                     int64_t S, int64_t C, int64_t tiles_per_shard,
                                                     int64_t tile_lo, int64_t tile_hi,
                                                     int32_t accumulate, int32_t scalar,
                                                     tide_trace_rec* __restrict__ trace,
                                                     int64_t trace_base,
                                                     uint32_t* __restrict__ counts) {
    const uint64_t t_begin = trace_begin(trace);
    constexpr int kSubs = NT / kThreads;
    const int M = MT > 0 ? MT : Mrt;
    const int sub = (int)threadIdx.x / kThreads;
    const int tid = (int)threadIdx.x % kThreads;
    for (int64_t t = tile_lo + (int64_t)blockIdx.x * kSubs + sub; t < tile_hi;
         t += (int64_t)gridDim.x * kSubs) {
        const int64_t b = t / tiles_per_shard;
        const int64_t f0 = (t - b * tiles_per_shard) * kLandTile;
        const int64_t end = min(f0 + kLandTile, S);
        float* shard = ptrs.shard[b];
        for (int64_t fs = f0; fs < end; fs += (int64_t)kThreads * 4) {
            const int64_t f = fs + (int64_t)tid * 4;
            if (f >= end) continue;
            int64_t sl = f / C;
            int64_t e = f - sl * C;
            if (!scalar && f + 4 <= end && e + 4 <= C) {
                const int64_t at = (sl * L + b) * C + e;
                const int gs = (int)(sl % L);
                f32x4_a4 acc = TIDE_LD(gbl<f32x4_a4>(ptrs.inbox[gs] + at));
                constexpr int kMUnroll = MT > 0 ? MT : 1;
#pragma unroll kMUnroll
                for (int c = 1; c < M; ++c) {
                    const int g = gs - c < 0 ? gs - c + L : gs - c;
                    const f32x4_a4 v = TIDE_LD(gbl<f32x4_a4>(ptrs.inbox[g] + at));
                    acc = acc + v;
                }
                TIDE_GLOBAL f32x4_a4* dst = gbl_mut<f32x4_a4>(shard + f);
                if (accumulate) acc = *dst + acc;
                TIDE_ST(acc, dst);
                count_writes<CNT>(counts, b * S + f, 4);
            } else {
#pragma unroll 1
                for (int k = 0; k < 4 && f + k < end; ++k) {
                    const int64_t ff = f + k;
                    sl = ff / C;
                    e = ff - sl * C;
                    const int64_t at = (sl * L + b) * C + e;
                    const int gs = (int)(sl % L);
                    float acc = gbl<float>(ptrs.inbox[gs])[at];
#pragma unroll 1
                    for (int c = 1; c < M; ++c) {
                        const int g = gs - c < 0 ? gs - c + L : gs - c;
                        acc = acc + gbl<float>(ptrs.inbox[g])[at];
                    }
                    TIDE_GLOBAL float* dst = gbl_mut<float>(shard + ff);
                    *dst = accumulate ? *dst + acc : acc;
                    count_writes<CNT>(counts, b * S + ff, 1);
                }
            }
        }
    }
    trace_end(trace, trace_base, t_begin);
}

// Diagnostic occupant (tide_diag_occupy): holds its CU's resources (threads,
// the dynamic LDS of the launch) for spin_ticks of the real-time counter, then
// records where it ran. The wait is bounded by the counter, so it always ends.
__global__ __launch_bounds__(1024) void occupy_kernel(int64_t spin_ticks, tide_trace_rec* trace) {
    const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
    while ((int64_t)(__builtin_amdgcn_s_memrealtime() - t0) < spin_ticks) __builtin_amdgcn_s_sleep(2);
    trace_end(trace, 0, t0);
}

// Bandwidth ceilings (tide_diag_stream): the access patterns of the path with
// no layout logic. A unit is 128 threads x 16 bytes (kinds 0-2) or 1024
// elements of every source (kind 3); workgroups walk units grid-stride.
//   0: read 16 B per thread and unit (non-temporal), folded so the loads
//      stay live; kinds 0-2 keep up to kStreamDepth units per thread in flight;
//   1: write 16 B of zeros per thread;
//   2: copy 16 B per thread;
//   3: the reduce's pattern: each wave's 512 elements as two runs of 256,
//      8-byte bf16 loads from each of nsrc sources, the fp32 sum in source
//      order, one 16-byte store per run and lane.
constexpr int kStreamDepth = 4;
template <int KIND, int NT>
__global__ __launch_bounds__(NT) void stream_kernel(StreamSrcs srcs, int32_t nsrc,
                                                    void* __restrict__ dst, int64_t units) {
    // A workgroup of NT threads is NT / kThreads independent quarters, each
    // walking its own units (as the budgeted kernels do).
    constexpr int kSubs = NT / kThreads;
    const int tid = (int)threadIdx.x % kThreads;
    const int sub = (int)threadIdx.x / kThreads;
    uint32_t acc = 0;
    for (int64_t u = (int64_t)blockIdx.x * kSubs + sub; u < units; u += (int64_t)gridDim.x * kSubs) {
        if constexpr (KIND == 3) {
            const int lane = tid % kWave;
            const int64_t base = u * kStep + (int64_t)(tid / kWave) * (2 * kHalf) + 4 * lane;
            u32x2 v[kStreamMaxSrcs][2];
#pragma unroll
            for (int c = 0; c < kStreamMaxSrcs; ++c) {
                if (c >= nsrc) break;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    v[c][h] = TIDE_LD(gbl<u32x2_a4>(static_cast<const uint16_t*>(srcs.p[c]) + base + h * kHalf));
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                float a[4] = {lo_bf16(v[0][h][0]), hi_bf16(v[0][h][0]), lo_bf16(v[0][h][1]),
                              hi_bf16(v[0][h][1])};
#pragma unroll
                for (int c = 1; c < kStreamMaxSrcs; ++c) {
                    if (c >= nsrc) break;
                    a[0] = a[0] + lo_bf16(v[c][h][0]);
                    a[1] = a[1] + hi_bf16(v[c][h][0]);
                    a[2] = a[2] + lo_bf16(v[c][h][1]);
                    a[3] = a[3] + hi_bf16(v[c][h][1]);
                }
                const f32x4_a4 x = {a[0], a[1], a[2], a[3]};
                TIDE_ST(x, gbl_mut<f32x4_a4>(static_cast<float*>(dst) + base + h * kHalf));
            }
        } else {
            // Up to kStreamDepth units per thread in flight (a budgeted
            // workgroup walks many units; a full-grid one has a single unit).
            const int64_t us = (int64_t)gridDim.x * kSubs;
            u32x4 x[kStreamDepth];
#pragma unroll
            for (int k = 0; k < kStreamDepth; ++k) {
                const int64_t uk = u + k * us;
                if (KIND != 1 && uk < units) x[k] = TIDE_LD(gbl<u32x4>(srcs.p[0]) + uk * kThreads + tid);
            }
#pragma unroll
            for (int k = 0; k < kStreamDepth; ++k) {
                const int64_t uk = u + k * us;
                if (uk >= units) break;
                if constexpr (KIND == 0) {
                    acc ^= x[k][0] ^ x[k][3];
                } else if constexpr (KIND == 1) {
                    const u32x4 z = {0u, 0u, 0u, 0u};
                    TIDE_ST(z, gbl_mut<u32x4>(dst) + uk * kThreads + tid);
                } else {
                    TIDE_ST(x[k], gbl_mut<u32x4>(dst) + uk * kThreads + tid);
                }
            }
            u += (kStreamDepth - 1) * us;
        }
    }
    // Kind 0 writes only if the fold hits a value chosen never to occur in the
    // probe's data, which keeps every load live without a real write stream.
    if constexpr (KIND == 0)
        if (acc == 0x9E3779B9u && threadIdx.x == 0) static_cast<uint32_t*>(dst)[blockIdx.x] = acc;
}

template <int MT>
hipError_t launch_landing_t(int M, int grid, int threads, size_t lds, hipStream_t stream,
                            const LandingPtrs& ptrs, int32_t L, int64_t S, int64_t C,
                            int64_t tiles_per_shard, int64_t tile_lo, int64_t tile_hi,
                            int32_t accumulate, int32_t scalar, tide_trace_rec* trace,
                            int64_t trace_base, uint32_t* counts) {
    LandingPtrs p = ptrs;
    int32_t Mrt = M;
    void* args[] = {&p, &L, &Mrt, &S, &C, &tiles_per_shard, &tile_lo, &tile_hi, &accumulate,
                    &scalar, &trace, &trace_base, &counts};
    // Counted calls (debug) take the runtime-M kernel with counting compiled in.
    const void* fn =
        counts ? (threads == kFatThreads
                      ? reinterpret_cast<const void*>(&landing_kernel<0, kFatThreads, true>)
                      : reinterpret_cast<const void*>(&landing_kernel<0, kThreads, true>))
               : (threads == kFatThreads
                      ? reinterpret_cast<const void*>(&landing_kernel<MT, kFatThreads, false>)
                      : reinterpret_cast<const void*>(&landing_kernel<MT, kThreads, false>));
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, lds, stream);
}

template <int LT, bool DERIVED, bool SHIFTED>
const void* reduce_fn(int threads, bool counted) {
    // Counted calls (debug) take the runtime-L kernel with counting and the
    // shifted loads compiled in.
    if (counted)
        return threads == kFatThreads
                   ? reinterpret_cast<const void*>(&reduce_kernel<0, kFatThreads, true, DERIVED, true>)
                   : reinterpret_cast<const void*>(&reduce_kernel<0, kThreads, true, DERIVED, true>);
    return threads == kFatThreads
               ? reinterpret_cast<const void*>(&reduce_kernel<LT, kFatThreads, false, DERIVED, SHIFTED>)
               : reinterpret_cast<const void*>(&reduce_kernel<LT, kThreads, false, DERIVED, SHIFTED>);
}

template <int LT, bool DERIVED>
hipError_t launch_reduce_t(int L, int grid, int threads, size_t lds, hipStream_t stream,
                           const TileRec* tiles, int64_t tile_lo, int64_t tile_hi, int32_t rb,
                           int32_t re, const ParamDev* params, const uint16_t* const* ptrs,
                           const uint32_t* flags, float* out, int64_t out_stride,
                           tide_trace_rec* trace, int64_t trace_base, uint32_t* counts,
                           int32_t xcd_lc, bool shifted) {
    void* args[] = {&tiles, &tile_lo, &tile_hi, &rb, &re, &params, &ptrs, &flags, &L, &out,
                    &out_stride, &trace, &trace_base, &counts, &xcd_lc};
    const void* fn = shifted ? reduce_fn<LT, DERIVED, true>(threads, counts != nullptr)
                             : reduce_fn<LT, DERIVED, false>(threads, counts != nullptr);
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, lds, stream);
}

template <bool DERIVED>
hipError_t launch_reduce_l(int L, int grid, int threads, size_t lds, hipStream_t stream,
                           const TileRec* tiles, int64_t tile_lo, int64_t tile_hi, int32_t rb,
                           int32_t re, const ParamDev* params, const uint16_t* const* ptrs,
                           const uint32_t* flags, float* out, int64_t out_stride,
                           tide_trace_rec* trace, int64_t trace_base, uint32_t* counts,
                           int32_t xcd_lc, bool shifted) {
#define TIDE_REDUCE_CASE(n)                                                                   \
    case n:                                                                                   \
        return launch_reduce_t<n, DERIVED>(L, grid, threads, lds, stream, tiles, tile_lo,     \
                                           tile_hi, rb, re, params, ptrs, flags, out,         \
                                           out_stride, trace, trace_base, counts, xcd_lc,     \
                                           shifted);
    switch (L) {
        TIDE_REDUCE_CASE(1)
        TIDE_REDUCE_CASE(2)
        TIDE_REDUCE_CASE(3)
        TIDE_REDUCE_CASE(4)
        TIDE_REDUCE_CASE(5)
        TIDE_REDUCE_CASE(6)
        TIDE_REDUCE_CASE(7)
        TIDE_REDUCE_CASE(8)
        default:
            return launch_reduce_t<0, DERIVED>(L, grid, threads, lds, stream, tiles, tile_lo,
                                               tile_hi, rb, re, params, ptrs, flags, out,
                                               out_stride, trace, trace_base, counts, xcd_lc,
                                               shifted);
    }
#undef TIDE_REDUCE_CASE
}

}  // namespace

hipError_t launch_reduce(int L, int grid, int threads, size_t lds, hipStream_t stream,
                         const TileRec* tiles, int64_t tile_lo, int64_t tile_hi, int32_t rb,
                         int32_t re, const ParamDev* params, const uint16_t* const* ptrs,
                         const uint32_t* flags, float* out, int64_t out_stride,
                         tide_trace_rec* trace, int64_t trace_base, uint32_t* counts,
                         int32_t xcd_lc, bool shifted) {
    return launch_reduce_l<false>(L, grid, threads, lds, stream, tiles, tile_lo, tile_hi, rb, re,
                                  params, ptrs, flags, out, out_stride, trace, trace_base, counts,
                                  xcd_lc, shifted);
}

hipError_t launch_reduce_derived(int L, int grid, int threads, size_t lds, hipStream_t stream,
                                 const int64_t* tile_prefix, int64_t tile_lo, int64_t tile_hi,
                                 int32_t rb, int32_t re, const ParamDev* params,
                                 const uint16_t* const* ptrs, const uint32_t* flags, float* out,
                                 int64_t out_stride, tide_trace_rec* trace, int64_t trace_base,
                                 uint32_t* counts, int32_t xcd_lc, bool shifted) {
    return launch_reduce_l<true>(L, grid, threads, lds, stream,
                                 reinterpret_cast<const TileRec*>(tile_prefix), tile_lo, tile_hi,
                                 rb, re, params, ptrs, flags, out, out_stride, trace, trace_base,
                                 counts, xcd_lc, shifted);
}

hipError_t launch_place(int grid, int threads, size_t lds, hipStream_t stream,
                        const TileRec* tiles, int64_t tile_lo, int64_t tile_hi, int32_t rb,
                        int32_t re, const ParamDev* params, uint16_t* const* ptrs,
                        const uint32_t* flags, const uint16_t* shards, int64_t shard_stride,
                        int64_t shard_elems, int32_t first_rank, int32_t nranks,
                        tide_trace_rec* trace, int64_t trace_base, uint32_t* counts) {
    void* args[] = {&tiles, &tile_lo, &tile_hi, &rb, &re, &params, &ptrs, &flags, &shards,
                    &shard_stride, &shard_elems, &first_rank, &nranks, &trace, &trace_base,
                    &counts};
    const void* fn =
        counts ? (threads == kFatThreads
                      ? reinterpret_cast<const void*>(&place_kernel<kFatThreads, true>)
                      : reinterpret_cast<const void*>(&place_kernel<kThreads, true>))
               : (threads == kFatThreads
                      ? reinterpret_cast<const void*>(&place_kernel<kFatThreads, false>)
                      : reinterpret_cast<const void*>(&place_kernel<kThreads, false>));
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, lds, stream);
}

hipError_t launch_stage(int grid, int threads, size_t lds, hipStream_t stream,
                        const TileRec* tiles, int64_t ntiles, int64_t tile_lo, int64_t tile_hi,
                        int32_t rb, int32_t re, const ParamDev* params,
                        const uint16_t* const* src, uint16_t* const* dst, const uint32_t* flags,
                        int32_t L, tide_trace_rec* trace, int64_t trace_base, uint32_t* counts,
                        int64_t slot_elems, int32_t nranks) {
    void* args[] = {&tiles, &ntiles, &tile_lo, &tile_hi, &rb, &re, &params, &src, &dst, &flags,
                    &L, &trace, &trace_base, &counts, &slot_elems, &nranks};
    const void* fn =
        counts ? (threads == kFatThreads
                      ? reinterpret_cast<const void*>(&stage_kernel<kFatThreads, true>)
                      : reinterpret_cast<const void*>(&stage_kernel<kThreads, true>))
               : (threads == kFatThreads
                      ? reinterpret_cast<const void*>(&stage_kernel<kFatThreads, false>)
                      : reinterpret_cast<const void*>(&stage_kernel<kThreads, false>));
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, lds, stream);
}

hipError_t launch_landing(int M, int grid, int threads, size_t lds, hipStream_t stream,
                          const LandingPtrs& ptrs, int32_t L, int64_t S, int64_t C,
                          int64_t tiles_per_shard, int64_t tile_lo, int64_t tile_hi,
                          int32_t accumulate, int32_t scalar, tide_trace_rec* trace,
                          int64_t trace_base, uint32_t* counts) {
#define TIDE_LANDING_CASE(n)                                                                  \
    case n:                                                                                   \
        return launch_landing_t<n>(M, grid, threads, lds, stream, ptrs, L, S, C,             \
                                   tiles_per_shard, tile_lo, tile_hi, accumulate, scalar,     \
                                   trace, trace_base, counts);
    switch (M) {
        TIDE_LANDING_CASE(1)
        TIDE_LANDING_CASE(2)
        TIDE_LANDING_CASE(3)
        TIDE_LANDING_CASE(4)
        TIDE_LANDING_CASE(5)
        TIDE_LANDING_CASE(6)
        TIDE_LANDING_CASE(7)
        TIDE_LANDING_CASE(8)
        default:
            return launch_landing_t<0>(M, grid, threads, lds, stream, ptrs, L, S, C,
                                       tiles_per_shard, tile_lo, tile_hi, accumulate, scalar,
                                       trace, trace_base, counts);
    }
#undef TIDE_LANDING_CASE
}

template <int NT>
const void* stream_fn(int kind) {
    return kind == 0   ? reinterpret_cast<const void*>(&stream_kernel<0, NT>)
           : kind == 1 ? reinterpret_cast<const void*>(&stream_kernel<1, NT>)
           : kind == 2 ? reinterpret_cast<const void*>(&stream_kernel<2, NT>)
                       : reinterpret_cast<const void*>(&stream_kernel<3, NT>);
}

hipError_t launch_stream(int kind, int grid, int threads, hipStream_t stream,
                         const StreamSrcs& srcs, int32_t nsrc, void* dst, int64_t units) {
    StreamSrcs s = srcs;
    void* args[] = {&s, &nsrc, &dst, &units};
    const void* fn = threads == kFatThreads ? stream_fn<kFatThreads>(kind) : stream_fn<kThreads>(kind);
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, 0, stream);
}

hipError_t launch_occupy(int grid, int threads, size_t lds, hipStream_t stream, int64_t spin_ticks,
                         tide_trace_rec* trace) {
    const void* fn = reinterpret_cast<const void*>(&occupy_kernel);
    if (lds > 64 * 1024) {
        hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
    void* args[] = {&spin_ticks, &trace};
    return hipLaunchKernel(fn, dim3(grid), dim3(threads), args, lds, stream);
}

hipError_t allow_dynamic_lds_landing(int M, size_t lds) {
#define TIDE_LDS_LANDING_CASE(n)                                                              \
    case n: {                                                                                 \
        hipError_t e = hipFuncSetAttribute(                                                   \
            reinterpret_cast<const void*>(&landing_kernel<n, kFatThreads, false>),            \
            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);                            \
        if (e != hipSuccess) return e;                                                        \
        e = hipFuncSetAttribute(reinterpret_cast<const void*>(&landing_kernel<0, kFatThreads, true>), \
                                hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);        \
        if (e != hipSuccess) return e;                                                        \
        return hipFuncSetAttribute(reinterpret_cast<const void*>(&landing_kernel<n, kThreads, false>), \
                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);     \
    }
    switch (M) {
        TIDE_LDS_LANDING_CASE(1)
        TIDE_LDS_LANDING_CASE(2)
        TIDE_LDS_LANDING_CASE(3)
        TIDE_LDS_LANDING_CASE(4)
        TIDE_LDS_LANDING_CASE(5)
        TIDE_LDS_LANDING_CASE(6)
        TIDE_LDS_LANDING_CASE(7)
        TIDE_LDS_LANDING_CASE(8)
        TIDE_LDS_LANDING_CASE(0)
        default:
            return allow_dynamic_lds_landing(0, lds);
    }
#undef TIDE_LDS_LANDING_CASE
}

hipError_t allow_dynamic_lds(int L, size_t lds) {
    // Dynamic LDS beyond the default per-workgroup limit needs opting in per kernel.
    const void* fns[] = {reinterpret_cast<const void*>(&place_kernel<kFatThreads, false>),
                         reinterpret_cast<const void*>(&place_kernel<kFatThreads, true>),
                         reinterpret_cast<const void*>(&stage_kernel<kFatThreads, false>),
                         reinterpret_cast<const void*>(&stage_kernel<kFatThreads, true>),
                         reinterpret_cast<const void*>(&reduce_kernel<0, kFatThreads, true, false, true>),
                         reinterpret_cast<const void*>(&reduce_kernel<0, kFatThreads, true, true, true>)};
    for (const void* f : fns) {
        hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
    }
#define TIDE_LDS_CASE(n)                                                                      \
    case n: {                                                                                 \
        const void* fat[] = {                                                                 \
            reinterpret_cast<const void*>(&reduce_kernel<n, kFatThreads, false, false, false>), \
            reinterpret_cast<const void*>(&reduce_kernel<n, kFatThreads, false, false, true>), \
            reinterpret_cast<const void*>(&reduce_kernel<n, kFatThreads, false, true, false>), \
            reinterpret_cast<const void*>(&reduce_kernel<n, kFatThreads, false, true, true>)}; \
        for (const void* f : fat) {                                                           \
            hipError_t e = hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, \
                                               (int)lds);                                     \
            if (e != hipSuccess) return e;                                                    \
        }                                                                                     \
        return hipSuccess;                                                                    \
    }
    switch (L) {
        TIDE_LDS_CASE(1)
        TIDE_LDS_CASE(2)
        TIDE_LDS_CASE(3)
        TIDE_LDS_CASE(4)
        TIDE_LDS_CASE(5)
        TIDE_LDS_CASE(6)
        TIDE_LDS_CASE(7)
        TIDE_LDS_CASE(8)
        TIDE_LDS_CASE(0)
        default:
            return allow_dynamic_lds(0, lds);
    }
#undef TIDE_LDS_CASE
}

}  // namespace tide
