// Internal declarations shared by the host planner (plan.cpp) and the HIP
// kernels (kernels.hip). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tide.h"

namespace tide {

// Tuning knobs (overridable at build time for measurement sweeps). Defaults
// were picked by interleaved in-process timing on MI355X over the four large
// workloads: many small, short workgroups stream best (a workgroup covers
// 1024 elements of the reduce, 2048 of the placement).
#ifndef TIDE_THREADS
#define TIDE_THREADS 128
#endif
#ifndef TIDE_RS_UNROLL
#define TIDE_RS_UNROLL 1
#endif
#ifndef TIDE_AG_UNROLL
#define TIDE_AG_UNROLL 2
#endif
#ifndef TIDE_RS_TILE_STEPS
#define TIDE_RS_TILE_STEPS 1
#endif
#ifndef TIDE_AG_TILE_STEPS
#define TIDE_AG_TILE_STEPS 2
#endif

#ifndef TIDE_STAGE_UNROLL
#define TIDE_STAGE_UNROLL 2
#endif
// Budgeted (fat, 1024-thread) workgroups: one per CU, so each needs more
// loads in flight and fewer tile setups per byte (measured on MI355X: the
// reduce streams 45 instead of 35 GB/s per workgroup, the placement 54
// instead of 40).
#ifndef TIDE_RS_FAT_TILE_STEPS
#define TIDE_RS_FAT_TILE_STEPS 8
#endif
#ifndef TIDE_RS_FAT_UNROLL
#define TIDE_RS_FAT_UNROLL 2
#endif
#ifndef TIDE_AG_FAT_TILE_STEPS
#define TIDE_AG_FAT_TILE_STEPS 8
#endif
#ifndef TIDE_AG_FAT_UNROLL
#define TIDE_AG_FAT_UNROLL 4
#endif
#ifndef TIDE_STAGE_FAT_TILE_STEPS
#define TIDE_STAGE_FAT_TILE_STEPS 8
#endif
#ifndef TIDE_STAGE_FAT_UNROLL
#define TIDE_STAGE_FAT_UNROLL 4
#endif
#ifndef TIDE_STAGE_TILE_STEPS
#define TIDE_STAGE_TILE_STEPS 2
#endif

constexpr int kThreads = TIDE_THREADS;     // workgroup size of the full grid (wave64s x 64)
constexpr int kFatThreads = 1024;          // workgroup size of budgeted launches: 16 wave64s,
                                           // 4 independent quarters of kThreads
constexpr int kVec = 8;                    // elements a thread handles per step (16 B of bf16)
constexpr int kStep = kThreads * kVec;     // elements a workgroup handles per step
constexpr int kRsUnroll = TIDE_RS_UNROLL;  // steps whose loads a reduce thread keeps in flight
constexpr int kAgUnroll = TIDE_AG_UNROLL;  // same, placement
constexpr int64_t kRsTile = (int64_t)TIDE_RS_TILE_STEPS * kStep;   // elements per reduce tile
constexpr int64_t kAgTile = (int64_t)TIDE_AG_TILE_STEPS * kStep;   // elements per placement tile
constexpr int kStageUnroll = TIDE_STAGE_UNROLL;                          // same, staging copy
constexpr int64_t kStageTile = (int64_t)TIDE_STAGE_TILE_STEPS * kStep;   // elements per staging tile
static_assert(kStageTile % (kStageUnroll * kStep) == 0, "tile must hold whole groups");
constexpr int kRsUnrollFat = TIDE_RS_FAT_UNROLL;
constexpr int64_t kRsTileFat = (int64_t)TIDE_RS_FAT_TILE_STEPS * kStep;
constexpr int kAgUnrollFat = TIDE_AG_FAT_UNROLL;
constexpr int64_t kAgTileFat = (int64_t)TIDE_AG_FAT_TILE_STEPS * kStep;
constexpr int kStageUnrollFat = TIDE_STAGE_FAT_UNROLL;
constexpr int64_t kStageTileFat = (int64_t)TIDE_STAGE_FAT_TILE_STEPS * kStep;
static_assert(kRsTileFat % (kRsUnrollFat * kStep) == 0, "tile must hold whole groups");
static_assert(kAgTileFat % (kAgUnrollFat * kStep) == 0, "tile must hold whole groups");
static_assert(kStageTileFat % (kStageUnrollFat * kStep) == 0, "tile must hold whole groups");
static_assert(kRsTile % (kRsUnroll * kStep) == 0, "tile must hold whole groups");
static_assert(kAgTile % (kAgUnroll * kStep) == 0, "tile must hold whole groups");
static_assert(kFatThreads % kThreads == 0, "a fat workgroup is whole quarters");

// One unit of work: a run of up to one tile of flat element indices inside one
// parameter. For the reduce, the flat index runs over the parameter's padded
// storage [0, N * s_p) (index f is rank f / s_p, offset f % s_p of its piece);
// for the placement, over its true elements [0, T_p * K_p). A launch over
// ranks [rb, re) only touches indices in [rb * s_p, re * s_p) (placement: also
// below T_p * K_p); the kernel derives those bounds from the parameter.
struct TileRec {
    int64_t idx0;   // first index of the tile, a multiple of kVec
    int32_t p;      // parameter
    int32_t r0;     // rank that holds idx0 (idx0 / s_p)
};
static_assert(sizeof(TileRec) == 16, "TileRec layout");

struct ParamDev {
    int64_t s;      // s_p, elements per rank piece
    int64_t o;      // o_p, offset of the piece in a rank's shard
    int64_t valid;  // T_p * K_p, true elements
    int64_t pad;
};
static_assert(sizeof(ParamDev) == 32, "ParamDev layout");

// Per-parameter flag bits of the per-call table.
constexpr uint32_t kFlagVector = 1u;  // every pointer of this parameter allows 16-byte vector access
// Reduce only: bit kOddShift + c set when contributor c's gradient starts at
// 2 mod 4 bytes; the interior steps read it with dword-aligned loads and a
// 16-bit funnel shift (contributors 0 .. kMaxOddShift - 1; a parameter with a
// later contributor at 2 mod 4 goes element by element).
constexpr int kOddShift = 8;
constexpr int kMaxOddShift = 24;

// Launch wrappers (kernels.hip). threads is kThreads or kFatThreads; lds is
// dynamic LDS reserved per workgroup (unused by the kernels: it only keeps
// other kernels' workgroups off the CU). trace, when not null, receives one
// record per workgroup at trace[trace_base + blockIdx.x]; counts, when not
// null, gets one added per element written (reduce: at the output offset;
// placement: at N * o_p + f; staging: at c * N * S + N * o_p + f; landing: at
// b * S + f). Return the launch's hipError_t. The reduce's full grid hands
// tiles to the XCDs in runs of 2^xcd_lc (0: round robin, one tile each);
// `shifted` selects the variant that reads gradients at 2 mod 4 bytes with
// vector loads (needed when any flag word carries kOddShift bits).
hipError_t launch_reduce(int L, int grid, int threads, size_t lds, hipStream_t stream,
                         const TileRec* tiles, int64_t tile_lo, int64_t tile_hi, int32_t rb,
                         int32_t re, const ParamDev* params, const uint16_t* const* ptrs,
                         const uint32_t* flags, float* out, int64_t out_stride,
                         tide_trace_rec* trace, int64_t trace_base, uint32_t* counts,
                         int32_t xcd_lc, bool shifted);

// The same reduce with no tile table: tile_prefix points at {P, cum[0..P]},
// cum[p] = reduce tiles of the parameters before p over ranks [rb, re) (the
// kernel derives each tile's record from it, in parameter order).
hipError_t launch_reduce_derived(int L, int grid, int threads, size_t lds, hipStream_t stream,
                                 const int64_t* tile_prefix, int64_t tile_lo, int64_t tile_hi,
                                 int32_t rb, int32_t re, const ParamDev* params,
                                 const uint16_t* const* ptrs, const uint32_t* flags, float* out,
                                 int64_t out_stride, tide_trace_rec* trace, int64_t trace_base,
                                 uint32_t* counts, int32_t xcd_lc, bool shifted);

hipError_t launch_place(int grid, int threads, size_t lds, hipStream_t stream,
                        const TileRec* tiles, int64_t tile_lo, int64_t tile_hi, int32_t rb,
                        int32_t re, const ParamDev* params, uint16_t* const* ptrs,
                        const uint32_t* flags, const uint16_t* shards, int64_t shard_stride,
                        int64_t shard_elems, int32_t first_rank, int32_t nranks,
                        tide_trace_rec* trace, int64_t trace_base, uint32_t* counts);

// Slot-Reuse staging (kernels.hip): tiles [tile_lo, tile_hi) of L copies of
// the staging tiling (ntiles tiles of kStageTile elements over each
// parameter's true elements); src / dst hold P * L pointers, parameter-major
// (p * L + c).
hipError_t launch_stage(int grid, int threads, size_t lds, hipStream_t stream,
                        const TileRec* tiles, int64_t ntiles, int64_t tile_lo, int64_t tile_hi,
                        int32_t rb, int32_t re, const ParamDev* params,
                        const uint16_t* const* src, uint16_t* const* dst, const uint32_t* flags,
                        int32_t L, tide_trace_rec* trace, int64_t trace_base, uint32_t* counts,
                        int64_t slot_elems, int32_t nranks);

// Level-2 landing sum (kernels.hip). The node's inbox and shard pointers travel
// in the kernel arguments (at most kMaxLanding GPUs per node).
constexpr int kMaxLanding = 64;
constexpr int64_t kLandTile = 2 * kThreads * 4;   // elements per landing tile (4 per thread per step)
struct LandingPtrs {
    const float* inbox[kMaxLanding];
    float* shard[kMaxLanding];
};
hipError_t launch_landing(int M, int grid, int threads, size_t lds, hipStream_t stream,
                          const LandingPtrs& ptrs, int32_t L, int64_t S, int64_t C,
                          int64_t tiles_per_shard, int64_t tile_lo, int64_t tile_hi,
                          int32_t accumulate, int32_t scalar, tide_trace_rec* trace,
                          int64_t trace_base, uint32_t* counts);
// Bandwidth-ceiling kernels (tide_diag_stream): sources by value.
constexpr int kStreamMaxSrcs = 8;
struct StreamSrcs {
    const void* p[kStreamMaxSrcs];
};
hipError_t launch_stream(int kind, int grid, int threads, hipStream_t stream,
                         const StreamSrcs& srcs, int32_t nsrc, void* dst, int64_t units);
// Diagnostic occupant (tide_diag_occupy).
hipError_t launch_occupy(int grid, int threads, size_t lds, hipStream_t stream, int64_t spin_ticks,
                         tide_trace_rec* trace);
hipError_t allow_dynamic_lds_landing(int M, size_t lds);

// Bytes of the fixed device scratch the allocation-free reduce-scatter keeps
// its per-call tables in (noalloc.hip), and its device address on HIP
// device `dev` (looked up once per device, with that device current).
constexpr size_t kScratchBytes = (size_t)1 << 20;
hipError_t scratch_address(int dev, void** out);

// Allow `lds` bytes of dynamic LDS on every kernel variant for L contributors.
hipError_t allow_dynamic_lds(int L, size_t lds);

}  // namespace tide
