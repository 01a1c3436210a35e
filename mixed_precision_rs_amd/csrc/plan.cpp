// Host side of the C ABI declared in include/tide.h: the layout planner
// (page 3 Table 2 notation), argument validation, per-device tables, the
// per-call pointer-table ring, and the launch policies (full grid,
// CU-budgeted, runtime copies for the placement and the staging).
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <new>
#include <string>
#include <tuple>
#include <vector>

#include "tide.h"
#include "sdma.hpp"
#include "tide_internal.hpp"

using namespace tide;

namespace {

thread_local std::string g_detail;

tide_status fail(tide_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_detail = buf;
    return st;
}

tide_status hip_fail(hipError_t e, const char* what) {
    return fail(TIDE_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

#define TIDE_HIP_TRY(expr)                                      \
    do {                                                        \
        hipError_t e_ = (expr);                                 \
        if (e_ != hipSuccess) return hip_fail(e_, #expr);       \
    } while (0)

// Makes `dev` the current device for the guard's lifetime. Allocations,
// events and kernel attributes belong to the current device, and a caller's
// stream may sit on another one.
class DeviceGuard {
  public:
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev_) != hipSuccess) prev_ = -1;
        if (prev_ != dev) {
            status_ = hipSetDevice(dev);
            changed_ = status_ == hipSuccess && prev_ >= 0;
        }
    }
    ~DeviceGuard() {
        if (changed_) (void)hipSetDevice(prev_);
    }
    DeviceGuard(const DeviceGuard&) = delete;
    DeviceGuard& operator=(const DeviceGuard&) = delete;
    hipError_t status() const { return status_; }

  private:
    int prev_ = -1;
    bool changed_ = false;
    hipError_t status_ = hipSuccess;
};

// Defaults of the CU-budgeted mode: 16 summing + 4 landing blocks (page 1
// "Why does a communication kernel slow a matrix multiply by 69%?"; page 3
// Table 4 "TIDE, training 16+4"). The pages' blocks live 0.2-0.4 ms; here a
// budgeted workgroup lives about 50 us. On MI355X hipBLASLt runs the bf16
// GEMMs of M >= 512 (N = K = 8192) as 256 persistent workgroups, one per CU:
// a CU held by a collective workgroup delays that GEMM workgroup until the
// collective's ends, so the GEMM slows by about the collective workgroup's
// life over the GEMM's. Measured with a 0.4 ms M = 4096 GEMM beside the Wan
// block, three runs: 30-36% at 300 us, 8-10% at 100 us, 2.4-3.3% at 50 us
// (the pages' 256-row victim, 128 workgroups: 0.2-1.9% at any of the three).
// The collective alone takes 16% longer at 50 us (6x the launches).
constexpr int kDefaultReduceBlocks = 16;
constexpr int kDefaultPlaceBlocks = 4;
constexpr int kDefaultMaxLaunchUs = 50;
// Budgeted launches use fat workgroups (kFatThreads) that reserve most of
// their CU's LDS, so no other kernel's workgroup (a GEMM's, typically) shares
// the CU with them: the concurrent kernel's workgroups are placed on the many
// idle CUs instead of running beside a streaming workgroup.
#ifndef TIDE_BUDGET_LDS
#define TIDE_BUDGET_LDS (128 * 1024)
#endif
// Bytes one budgeted workgroup streams per microsecond with a CU to itself,
// per operation (measured on MI355X: per-workgroup streaming is latency
// bound); sizes the budgeted launches so a workgroup lives about
// max_launch_us.
#ifndef TIDE_WG_BYTES_PER_US_RS
#define TIDE_WG_BYTES_PER_US_RS 45000
#endif
#ifndef TIDE_WG_BYTES_PER_US_AG
#define TIDE_WG_BYTES_PER_US_AG 54000
#endif
#ifndef TIDE_WG_BYTES_PER_US_LANDING
#define TIDE_WG_BYTES_PER_US_LANDING 35000
#endif
constexpr int kBudgetThreads = kFatThreads;
constexpr size_t kBudgetLds = TIDE_BUDGET_LDS;
constexpr int64_t kWgBytesPerUsRs = TIDE_WG_BYTES_PER_US_RS;
constexpr int64_t kWgBytesPerUsAg = TIDE_WG_BYTES_PER_US_AG;       // placement and staging
constexpr int64_t kWgBytesPerUsLanding = TIDE_WG_BYTES_PER_US_LANDING;
// Full mode: at most this many workgroups per launch (they loop over tiles).
// A dispatch holds at most 2^32 - 1 work-items; 2^24 workgroups of 128
// threads stay well below that (a group of up to 16 G reduce elements still
// gets one workgroup per tile).
#ifndef TIDE_FULL_GRID_CAP
#define TIDE_FULL_GRID_CAP (1 << 24)
#endif
constexpr int kFullGridCap = TIDE_FULL_GRID_CAP;
static_assert((int64_t)kFullGridCap * kThreads < (int64_t(1) << 32), "dispatch size");
// Budgeted mode: at most this many workgroups per launch (of kFatThreads).
constexpr int32_t kMaxBudgetBlocks = 65536;
#ifndef TIDE_RS_GROUP_ELEMS
#define TIDE_RS_GROUP_ELEMS (1 << 20)
#endif
// Pieces under TIDE_RS_GROUP_SMALL elements (Qwen3-MoE's 384 experts, 24,576
// each) walk in much larger groups: interleaved on MI355X, groups of 16 M
// elements reduced that group 2.7% faster than groups of 1 M, while groups of
// medium pieces (Wan2.2's 409,600-element attention pieces) were 1.5-3% slower
// above 1 M and the other groups did not change.
#ifndef TIDE_RS_GROUP_SMALL
#define TIDE_RS_GROUP_SMALL (1 << 17)
#endif
#ifndef TIDE_RS_GROUP_SMALL_ELEMS
#define TIDE_RS_GROUP_SMALL_ELEMS (1 << 24)
#endif
constexpr int kRingSlots = 8;
constexpr int32_t kKnownFlags = TIDE_FLAG_SCALAR_PATH | TIDE_FLAG_NO_LDS_FENCE;

struct TileTable {
    TileRec* dev = nullptr;
    int64_t count = 0;
    uint64_t last_use = 0;   // DevState::use_clock at the last lookup
    int64_t pins = 0;        // prepared calls that launch from it (never evicted while > 0)
};

// Tile tables kept per device (one per operation, launch mode and rank
// range). Past this, the least recently used table no prepared call holds is
// freed, after the device has drained (its kernels may still be reading it).
constexpr size_t kMaxTileTables = 256;

// A call that read a slot: the last such call on `stream` is marked by `ev`
// (work on one stream completes in order, so one event per stream suffices).
struct Reader {
    hipStream_t stream;
    hipEvent_t ev;
};

struct Slot {
    void* dev = nullptr;
    void* host = nullptr;
    size_t used = 0;
    bool loaded = false;
    hipStream_t upload_stream = nullptr;
    hipEvent_t upload_done = nullptr;      // recorded after the upload copy
    std::vector<Reader> readers;           // per stream, recorded after its last call that read the slot
};

struct DevState {
    int device = -1;
    ParamDev* params = nullptr;
    std::map<std::tuple<int, int, int>, TileTable> tiles;   // (op + 4 * budgeted, rank_begin, rank_end)
    uint64_t use_clock = 0;
    size_t slot_cap = 0;
    char* ring_dev = nullptr;
    char* ring_host = nullptr;
    Slot slots[kRingSlots];
    int next_slot = 0;
    int last_slot = 0;
    std::vector<hipEvent_t> event_pool;
    bool lds_allowed[65] = {};             // allow_dynamic_lds done for this L

    ~DevState() {
        DeviceGuard guard(device);
        for (auto& kv : tiles) (void)hipFree(kv.second.dev);
        (void)hipFree(params);
        (void)hipFree(ring_dev);
        if (ring_host) (void)hipHostFree(ring_host);
        for (auto& s : slots) {
            for (const Reader& r : s.readers) {
                (void)hipEventSynchronize(r.ev);
                (void)hipEventDestroy(r.ev);
            }
            if (s.upload_done) (void)hipEventDestroy(s.upload_done);
        }
        for (hipEvent_t e : event_pool) (void)hipEventDestroy(e);
    }
};

struct ParamInfo {
    int64_t T, K, R, s, o, valid;
};

// Full-grid reduce tile order (the XCD runs of kernels.hip's xcd_tile_rt).
// Interleaved in one process on MI355X, against one tile per XCD in turn:
//  - groups whose destinations mostly start mid-line (the padding-stress
//    group: an odd S) reduce about 4% faster with runs of 128 tiles (64:
//    +2.3%; 256 to 1024: as 128); a step's two partly written end lines are
//    shared with the neighbouring steps, and in one run those neighbours go
//    through the same L2;
//  - groups of mostly small pieces (the Qwen MoE layer's 24,576-element
//    expert pieces) about 1% faster with runs of 16 (8 and 32: slower);
//  - groups of large, line-aligned pieces (Llama, Wan) 3% slower with either.
constexpr int kXcdRunMisaligned = 7;    // log2 of 128 tiles
constexpr int kXcdRunSmall = 4;         // log2 of 16 tiles
constexpr int64_t kSmallPiece = 1 << 17;

}  // namespace

struct tide_plan {
    int32_t P = 0, N = 0, L = 0;
    int64_t S = 0;
    bool mostly_small = false;   // more than half of every shard is in pieces under kSmallPiece
    std::vector<ParamInfo> prm;
    mutable std::mutex mu;
    mutable std::vector<std::unique_ptr<DevState>> devs;
};

namespace {

bool mul_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t* out) { return !__builtin_add_overflow(a, b, out); }

tide_status resolve_launch(const tide_plan* plan, const tide_launch* in, tide_launch* out) {
    tide_launch l{};
    if (in) l = *in;
    if (l.mode != TIDE_LAUNCH_FULL && l.mode != TIDE_LAUNCH_BUDGETED)
        return fail(TIDE_ERR_INVALID_ARG, "launch.mode %d is not FULL (0) or BUDGETED (1)", l.mode);
    if (l.reduce_blocks < 0 || l.place_blocks < 0 || l.max_launch_us < 0)
        return fail(TIDE_ERR_INVALID_ARG, "negative launch budget");
    if (l.reduce_blocks > kMaxBudgetBlocks || l.place_blocks > kMaxBudgetBlocks)
        return fail(TIDE_ERR_INVALID_ARG, "reduce_blocks %d / place_blocks %d above %d",
                    l.reduce_blocks, l.place_blocks, kMaxBudgetBlocks);
    if (l.reserved != 0 || (l.flags & ~kKnownFlags) != 0)
        return fail(TIDE_ERR_INVALID_ARG, "unknown launch flags 0x%x", l.flags);
    if (l.trace_capacity < 0) return fail(TIDE_ERR_INVALID_ARG, "negative trace_capacity");
    if (l.write_counts_elems < 0) return fail(TIDE_ERR_INVALID_ARG, "negative write_counts_elems");
    if (l.reduce_blocks == 0) l.reduce_blocks = kDefaultReduceBlocks;
    if (l.place_blocks == 0) l.place_blocks = kDefaultPlaceBlocks;
    if (l.max_launch_us == 0) l.max_launch_us = kDefaultMaxLaunchUs;
    if (l.rank_end == 0) l.rank_end = plan->N;
    if (l.rank_begin < 0 || l.rank_end > plan->N || l.rank_begin > l.rank_end)
        return fail(TIDE_ERR_INVALID_ARG, "rank range [%d, %d) outside [0, %d)", l.rank_begin,
                    l.rank_end, plan->N);
    *out = l;
    return TIDE_OK;
}

// Elements per tile of one op, for full-grid (fat = false) or budgeted launches.
int64_t tile_elems(int op, bool fat) {
    if (op == 0) return fat ? kRsTileFat : kRsTile;
    if (op == 1) return fat ? kAgTileFat : kAgTile;
    return fat ? kStageTileFat : kStageTile;
}

// Tiles of one op over ranks [rb, re). op 0: reduce over each parameter's
// padded index space restricted to [rb * s_p, re * s_p); op 1: placement over
// its true elements restricted the same way; op 2: staging, as op 1.
std::vector<TileRec> build_tiles(const tide_plan* plan, int op, int rb, int re, bool fat) {
    std::vector<TileRec> out;
    const int64_t tile = tile_elems(op, fat);
    for (int32_t p = 0; p < plan->P; ++p) {
        const ParamInfo& q = plan->prm[p];
        if (q.s == 0) continue;
        const int64_t lo = (int64_t)rb * q.s;
        int64_t hi = (int64_t)re * q.s;
        if (op != 0) hi = std::min(hi, q.valid);
        if (hi <= lo) continue;
        for (int64_t a = lo - lo % kVec; a < hi; a += tile) {
            TileRec t{};
            t.idx0 = a;
            t.p = p;
            t.r0 = (int32_t)(a / q.s);
            out.push_back(t);
        }
    }
#if TIDE_RS_GROUP_ELEMS > 0
    // Reduce: consecutive parameters are grouped, and each group is walked
    // rank by rank. Many small pieces of one rank are adjacent in its shard,
    // so this turns their short scattered writes into long runs; a large
    // parameter is a group of its own and keeps its order. A group closes
    // once its pieces hold TIDE_RS_GROUP_ELEMS elements, or, while every
    // piece in it is under TIDE_RS_GROUP_SMALL elements, TIDE_RS_GROUP_SMALL_ELEMS;
    // a piece at or above TIDE_RS_GROUP_SMALL does not join a group of small
    // pieces.
    if (op == 0 && plan->P > 1) {
        std::vector<int32_t> group(plan->P, 0);
        int32_t gid = 0;
        int64_t acc = 0;
        bool all_small = true;
        for (int32_t p = 0; p < plan->P; ++p) {
            const bool small = plan->prm[p].s < TIDE_RS_GROUP_SMALL;
            if (acc > 0 && all_small && !small) {
                ++gid;
                acc = 0;
            }
            if (acc == 0) all_small = true;
            group[p] = gid;
            acc += plan->prm[p].s;
            all_small = all_small && small;
            if (acc >= (all_small ? (int64_t)TIDE_RS_GROUP_SMALL_ELEMS : (int64_t)TIDE_RS_GROUP_ELEMS)) {
                ++gid;
                acc = 0;
            }
        }
        std::stable_sort(out.begin(), out.end(), [&](const TileRec& a, const TileRec& b) {
            if (group[a.p] != group[b.p]) return group[a.p] < group[b.p];
            return a.r0 != b.r0 ? a.r0 < b.r0 : a.p < b.p;
        });
    }
#endif
    return out;
}

// The number of tiles build_tiles makes, in O(P): what the host-only
// queries (launch and trace-record counts) need, without building the table.
int64_t count_tiles(const tide_plan* plan, int op, int rb, int re, bool fat) {
    const int64_t tile = tile_elems(op, fat);
    int64_t n = 0;
    for (int32_t p = 0; p < plan->P; ++p) {
        const ParamInfo& q = plan->prm[p];
        if (q.s == 0) continue;
        const int64_t lo = (int64_t)rb * q.s;
        int64_t hi = (int64_t)re * q.s;
        if (op != 0) hi = std::min(hi, q.valid);
        if (hi <= lo) continue;
        const int64_t a = lo - lo % kVec;
        n += (hi - a + tile - 1) / tile;
    }
    return n;
}

// Bytes a budgeted tile moves.
int64_t tile_bytes(const tide_plan* plan, int op) {
    return op == 0 ? tile_elems(0, true) * (2 * (int64_t)plan->L + 4) : tile_elems(op, true) * 4;
}

// Tiles one budgeted workgroup handles per launch.
int64_t budget_tiles_per_block(const tide_plan* plan, int op, const tide_launch& l) {
    const int64_t rate = op == 0 ? kWgBytesPerUsRs : kWgBytesPerUsAg;
    const int64_t per = ((int64_t)l.max_launch_us * rate) / tile_bytes(plan, op);
    return std::max<int64_t>(1, per);
}

int64_t count_launches(const tide_plan* plan, int op, const tide_launch& l, int64_t ntiles) {
    if (ntiles == 0) return 0;
    if (l.mode == TIDE_LAUNCH_FULL) return 1;
    const int64_t blocks = op == 0 ? l.reduce_blocks : l.place_blocks;
    const int64_t per_launch = blocks * budget_tiles_per_block(plan, op, l);
    return (ntiles + per_launch - 1) / per_launch;
}

tide_status stream_device(hipStream_t stream, int* dev) {
    if (stream) {
        hipError_t e = hipStreamGetDevice(stream, dev);
        if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
        return TIDE_OK;
    }
    hipError_t e = hipGetDevice(dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    return TIDE_OK;
}

// Device state of `plan` on `dev` (created on first use). Caller holds plan->mu.
tide_status get_dev_state(const tide_plan* plan, int dev, DevState** out) {
    for (auto& d : plan->devs) {
        if (d->device == dev) {
            *out = d.get();
            return TIDE_OK;
        }
    }
    std::unique_ptr<DevState> ds(new DevState());
    ds->device = dev;
    std::vector<ParamDev> pd(std::max<int32_t>(plan->P, 1));
    for (int32_t p = 0; p < plan->P; ++p) {
        pd[p].s = plan->prm[p].s;
        pd[p].o = plan->prm[p].o;
        pd[p].valid = plan->prm[p].valid;
        pd[p].pad = 0;
    }
    TIDE_HIP_TRY(hipMalloc(&ds->params, pd.size() * sizeof(ParamDev)));
    TIDE_HIP_TRY(hipMemcpy(ds->params, pd.data(), pd.size() * sizeof(ParamDev),
                           hipMemcpyHostToDevice));
    const size_t P = (size_t)std::max<int32_t>(plan->P, 1);
    // Largest per-call table: the staging's 2 * P * L pointers plus P flags.
    size_t cap = 2 * P * (size_t)plan->L * sizeof(void*) + P * sizeof(uint32_t);
    cap = (cap + 255) / 256 * 256;
    ds->slot_cap = cap;
    TIDE_HIP_TRY(hipMalloc(&ds->ring_dev, cap * kRingSlots));
    TIDE_HIP_TRY(hipHostMalloc(&ds->ring_host, cap * kRingSlots, hipHostMallocDefault));
    for (int i = 0; i < kRingSlots; ++i) {
        ds->slots[i].dev = ds->ring_dev + cap * i;
        ds->slots[i].host = ds->ring_host + cap * i;
        TIDE_HIP_TRY(hipEventCreateWithFlags(&ds->slots[i].upload_done, hipEventDisableTiming));
    }
    *out = ds.get();
    plan->devs.push_back(std::move(ds));
    return TIDE_OK;
}

tide_status get_tiles(const tide_plan* plan, DevState* ds, int op, int rb, int re, bool fat,
                      TileTable** out) {
    auto key = std::make_tuple(op + (fat ? 4 : 0), rb, re);
    auto it = ds->tiles.find(key);
    if (it != ds->tiles.end()) {
        it->second.last_use = ++ds->use_clock;
        *out = &it->second;
        return TIDE_OK;
    }
    if (ds->tiles.size() >= kMaxTileTables) {
        auto victim = ds->tiles.end();
        for (auto v = ds->tiles.begin(); v != ds->tiles.end(); ++v)
            if (v->second.pins == 0 && (victim == ds->tiles.end() ||
                                        v->second.last_use < victim->second.last_use))
                victim = v;
        if (victim != ds->tiles.end()) {
            TIDE_HIP_TRY(hipDeviceSynchronize());
            TIDE_HIP_TRY(hipFree(victim->second.dev));
            ds->tiles.erase(victim);
        }
    }
    std::vector<TileRec> t = build_tiles(plan, op, rb, re, fat);
    TileTable tt;
    tt.last_use = ++ds->use_clock;
    tt.count = (int64_t)t.size();
    if (!t.empty()) {
        TIDE_HIP_TRY(hipMalloc(&tt.dev, t.size() * sizeof(TileRec)));
        hipError_t e = hipMemcpy(tt.dev, t.data(), t.size() * sizeof(TileRec),
                                 hipMemcpyHostToDevice);
        if (e != hipSuccess) {
            (void)hipFree(tt.dev);
            return hip_fail(e, "hipMemcpy(tiles)");
        }
    }
    auto ins = ds->tiles.emplace(key, tt);
    *out = &ins.first->second;
    return TIDE_OK;
}

tide_status take_event(DevState* ds, hipEvent_t* ev) {
    if (!ds->event_pool.empty()) {
        *ev = ds->event_pool.back();
        ds->event_pool.pop_back();
        return TIDE_OK;
    }
    TIDE_HIP_TRY(hipEventCreateWithFlags(ev, hipEventDisableTiming));
    return TIDE_OK;
}

// Make the per-call table `bytes` visible on the device in stream order.
// Reuses the previous slot, with no copy, when the table is unchanged.
tide_status stage_table(DevState* ds, const void* bytes, size_t n, hipStream_t stream,
                        int* slot_out) {
    for (int i = 0; i < kRingSlots; ++i) {
        // Most recent first: callers typically alternate a few fixed tables.
        const int k = (ds->last_slot - i + 2 * kRingSlots) % kRingSlots;
        Slot& s = ds->slots[k];
        if (s.loaded && s.used == n && std::memcmp(s.host, bytes, n) == 0) {
            if (s.upload_stream != stream)
                TIDE_HIP_TRY(hipStreamWaitEvent(stream, s.upload_done, 0));
            ds->last_slot = k;
            *slot_out = k;
            return TIDE_OK;
        }
    }
    const int k = ds->next_slot;
    ds->next_slot = (k + 1) % kRingSlots;
    Slot& s = ds->slots[k];
    for (const Reader& r : s.readers) {       // earlier readers of this slot must be done
        TIDE_HIP_TRY(hipEventSynchronize(r.ev));
        ds->event_pool.push_back(r.ev);
    }
    s.readers.clear();
    // The slot's previous upload reads the pinned host copy when its stream
    // reaches it; every upload is followed by a reader event, but a call that
    // failed to record one must not let the copy be overwritten early.
    if (s.loaded) TIDE_HIP_TRY(hipEventSynchronize(s.upload_done));
    s.loaded = false;
    std::memcpy(s.host, bytes, n);
    TIDE_HIP_TRY(hipMemcpyAsync(s.dev, s.host, n, hipMemcpyHostToDevice, stream));
    TIDE_HIP_TRY(hipEventRecord(s.upload_done, stream));
    s.used = n;
    s.loaded = true;
    s.upload_stream = stream;
    ds->last_slot = k;
    *slot_out = k;
    return TIDE_OK;
}

// Mark the end of a call that read `slot` on `stream`. A stream that read the
// slot before re-records its event; readers on other streams whose events
// have completed are dropped, so the list stays as short as the number of
// streams with work still pending on the slot.
tide_status release_slot(DevState* ds, int slot, hipStream_t stream) {
    std::vector<Reader>& readers = ds->slots[slot].readers;
    for (const Reader& r : readers)
        if (r.stream == stream) {
            TIDE_HIP_TRY(hipEventRecord(r.ev, stream));
            return TIDE_OK;
        }
    for (size_t i = 0; i < readers.size();) {
        const hipError_t q = hipEventQuery(readers[i].ev);
        if (q == hipSuccess) {
            ds->event_pool.push_back(readers[i].ev);
            readers[i] = readers.back();
            readers.pop_back();
        } else if (q == hipErrorNotReady) {
            ++i;
        } else {
            return hip_fail(q, "hipEventQuery");
        }
    }
    hipEvent_t ev;
    tide_status st = take_event(ds, &ev);
    if (st != TIDE_OK) return st;
    hipError_t e = hipEventRecord(ev, stream);
    if (e != hipSuccess) {
        ds->event_pool.push_back(ev);
        return hip_fail(e, "hipEventRecord");
    }
    readers.push_back(Reader{stream, ev});
    return TIDE_OK;
}

// log2 of the full-grid reduce's XCD run length for output `out` with shard
// stride `stride` over ranks [rb, re): runs of 128 when more than half of the
// output elements are in pieces whose destination starts mid-line (128 B),
// of 16 when the group is mostly small pieces, else 0 (round robin). The
// residue of a piece's start modulo 32 elements repeats with a period that
// divides 32 ranks, so at most 32 ranks are looked at per parameter.
int reduce_xcd_log2(const tide_plan* plan, const float* out, int64_t stride, int32_t rb,
                    int32_t re) {
    const int64_t e0 = (int64_t)((reinterpret_cast<uintptr_t>(out) >> 2) & 31);
    const int64_t n = re - rb;
    if (n <= 0) return 0;
    int64_t mis = 0, tot = 0;
    for (const ParamInfo& q : plan->prm) {
        if (q.s == 0) continue;
        const int64_t period = std::min<int64_t>(32, n);
        int64_t mis_ranks = 0, in_period = 0;
        for (int64_t k = 0; k < period; ++k) {
            const int64_t r = rb + k;
            // ranks r, r + 32, r + 64, ... share the residue
            const int64_t count = (n - k + 31) / 32;
            if (((e0 + (r % 32) * (stride % 32) + q.o) & 31) != 0) mis_ranks += count;
            in_period += count;
        }
        mis += mis_ranks * q.s;
        tot += in_period * q.s;
    }
    if (2 * mis > tot) return kXcdRunMisaligned;
    if (plan->mostly_small) return kXcdRunSmall;
    return 0;
}

// Budgeted launches reserve dynamic LDS; opt the kernels in once per device.
tide_status prepare_budget(DevState* ds, int L, const tide_launch& l) {
    if (l.mode != TIDE_LAUNCH_BUDGETED || kBudgetLds == 0) return TIDE_OK;
    const int key = L <= 8 ? L : 0;
    if (ds->lds_allowed[key]) return TIDE_OK;
    TIDE_HIP_TRY(allow_dynamic_lds(key, kBudgetLds));
    ds->lds_allowed[key] = true;
    return TIDE_OK;
}

struct Range {
    uintptr_t lo, hi;
    int who;
};

// Devices on which the landing kernels were opted in to the budgeted LDS
// reservation (bit M, or bit 0 for the runtime-M kernel).
std::mutex g_landing_lds_mu;
uint64_t g_landing_lds_done[64] = {};

bool overlaps(const Range& a, const Range& b) { return a.lo < b.hi && b.lo < a.hi; }

// The run of tiles of each launch and the grid it uses.
template <typename F>
tide_status for_each_launch(const tide_plan* plan, int op, const tide_launch& l,
                            int64_t ntiles, F&& launch) {
    if (ntiles == 0) return TIDE_OK;
    int64_t per_launch;
    int grid_cap;
    if (l.mode == TIDE_LAUNCH_FULL) {
        per_launch = ntiles;                  // one launch; workgroups loop over tiles
        grid_cap = kFullGridCap;
    } else {
        const int blocks = op == 0 ? l.reduce_blocks : l.place_blocks;
        per_launch = (int64_t)blocks * budget_tiles_per_block(plan, op, l);
        grid_cap = blocks;
    }
    const int threads = l.mode == TIDE_LAUNCH_FULL ? kThreads : kBudgetThreads;
    const size_t lds =
        l.mode == TIDE_LAUNCH_FULL || (l.flags & TIDE_FLAG_NO_LDS_FENCE) ? 0 : kBudgetLds;
    int64_t trace_base = 0;
    for (int64_t lo = 0; lo < ntiles; lo += per_launch) {
        const int64_t hi = std::min(ntiles, lo + per_launch);
        const int grid = (int)std::min<int64_t>(grid_cap, hi - lo);
        hipError_t e = launch(grid, threads, lds, lo, hi, trace_base);
        trace_base += grid;
        if (e != hipSuccess)
            return hip_fail(e, op == 0 ? "reduce launch" : op == 1 ? "place launch" : "stage launch");
    }
    return TIDE_OK;
}

// Workgroups (trace records) of all launches for_each_launch makes.
int64_t launch_records(const tide_plan* plan, int op, const tide_launch& l, int64_t ntiles) {
    int64_t n = 0;
    (void)for_each_launch(plan, op, l, ntiles,
                          [&](int grid, int, size_t, int64_t, int64_t, int64_t) {
        n += grid;
        return hipSuccess;
    });
    return n;
}

// Calls that read a per-call pointer table from the ring cannot be captured
// into a graph: a replay would read whatever table the slot holds by then.
tide_status refuse_capture(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    TIDE_HIP_TRY(hipStreamIsCapturing(stream, &cs));
    if (cs != hipStreamCaptureStatusNone)
        return fail(TIDE_ERR_UNSUPPORTED,
                    "the stream is capturing a graph; this call reads a per-call pointer table "
                    "that a replay could not rely on (capture a prepared call, the runtime-copy "
                    "engine or the landing sum instead)");
    return TIDE_OK;
}

// The DMA-engine path waits on the host for the stream and for its copies, so
// it cannot be recorded into a graph.
tide_status refuse_capture_dma(hipStream_t stream) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    TIDE_HIP_TRY(hipStreamIsCapturing(stream, &cs));
    if (cs != hipStreamCaptureStatusNone)
        return fail(TIDE_ERR_UNSUPPORTED,
                    "the stream is capturing a graph; the DMA-engine path waits on the host and "
                    "cannot be captured (capture the kernel engine's prepared call instead)");
    return TIDE_OK;
}

// Run linear copies on the DMA engines of the stream's device (host-synchronous).
tide_status run_dma(hipStream_t stream, const std::vector<DmaCopy>& copies) {
    tide_status st = refuse_capture_dma(stream);
    if (st != TIDE_OK) return st;
    int dev;
    st = stream_device(stream, &dev);
    if (st != TIDE_OK) return st;
    std::string err;
    st = dma_copies(dev, stream, copies, nullptr, &err);
    if (st != TIDE_OK) return fail(st, "%s", err.c_str());
    return TIDE_OK;
}

// Append a copy, merging it into the previous one when both sides continue it.
void add_copy(std::vector<DmaCopy>& v, void* dst, const void* src, uint64_t bytes) {
    if (bytes == 0) return;
    if (!v.empty()) {
        DmaCopy& b = v.back();
        if (static_cast<char*>(b.dst) + b.bytes == dst &&
            static_cast<const char*>(b.src) + b.bytes == src) {
            b.bytes += bytes;
            return;
        }
    }
    v.push_back(DmaCopy{dst, src, bytes});
}

// A counted call needs `need` entries; checked before anything is enqueued.
tide_status check_counts(const tide_launch& l, int64_t need) {
    if (l.write_counts && l.write_counts_elems < need)
        return fail(TIDE_ERR_INVALID_ARG, "write_counts holds %lld entries, the call needs %lld",
                    (long long)l.write_counts_elems, (long long)need);
    return TIDE_OK;
}

// A traced call must have room for every record before anything is enqueued.
tide_status check_trace(const tide_launch& l, int64_t records) {
    if (l.trace && records > l.trace_capacity)
        return fail(TIDE_ERR_INVALID_ARG, "trace holds %lld records, the call needs %lld",
                    (long long)l.trace_capacity, (long long)records);
    return TIDE_OK;
}

}  // namespace

extern "C" {

tide_status tide_plan_create(const int64_t* rows, const int64_t* row_len, int32_t P, int32_t N,
                             int32_t L, tide_plan** out_plan) {
    try {
        if (!out_plan) return fail(TIDE_ERR_INVALID_ARG, "out_plan is NULL");
        *out_plan = nullptr;
        if (P < 0) return fail(TIDE_ERR_INVALID_ARG, "P = %d < 0", P);
        if (N < 1) return fail(TIDE_ERR_INVALID_ARG, "N = %d < 1", N);
        if (L < 1 || L > 64) return fail(TIDE_ERR_INVALID_ARG, "L = %d not in [1, 64]", L);
        if (P > 0 && (!rows || !row_len)) return fail(TIDE_ERR_INVALID_ARG, "rows/row_len NULL");
        std::unique_ptr<tide_plan> plan(new tide_plan());
        plan->P = P;
        plan->N = N;
        plan->L = L;
        plan->prm.resize(P);
        int64_t acc = 0;
        for (int32_t p = 0; p < P; ++p) {
            ParamInfo& q = plan->prm[p];
            q.T = rows[p];
            q.K = row_len[p];
            if (q.T < 0) return fail(TIDE_ERR_INVALID_ARG, "rows[%d] = %lld < 0", p, (long long)q.T);
            if (q.K < 1)
                return fail(TIDE_ERR_INVALID_ARG, "row_len[%d] = %lld < 1", p, (long long)q.K);
            q.R = q.T / N + (q.T % N != 0);                  // ceil(T_p / N)
            if (!mul_ok(q.R, q.K, &q.s) || !mul_ok(q.T, q.K, &q.valid))
                return fail(TIDE_ERR_OVERFLOW, "parameter %d size overflows int64", p);
            q.o = acc;
            if (!add_ok(acc, q.s, &acc)) return fail(TIDE_ERR_OVERFLOW, "S overflows int64");
        }
        plan->S = acc;
        int64_t small = 0;
        for (const ParamInfo& q : plan->prm)
            if (q.s < kSmallPiece) small += q.s;
        plan->mostly_small = 2 * small > plan->S;
        int64_t ns;
        if (!mul_ok(acc, N, &ns)) return fail(TIDE_ERR_OVERFLOW, "N * S overflows int64");
        // Byte offsets of the fp32 output must fit too.
        if (!mul_ok(ns, 4, &ns)) return fail(TIDE_ERR_OVERFLOW, "4 * N * S overflows int64");
        *out_plan = plan.release();
        return TIDE_OK;
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

void tide_plan_destroy(tide_plan* plan) {
    try {
        delete plan;
    } catch (...) {
    }
}

tide_status tide_plan_dims(const tide_plan* plan, int32_t* P, int32_t* N, int32_t* L, int64_t* S) {
    if (!plan) return fail(TIDE_ERR_INVALID_ARG, "plan is NULL");
    if (P) *P = plan->P;
    if (N) *N = plan->N;
    if (L) *L = plan->L;
    if (S) *S = plan->S;
    return TIDE_OK;
}

tide_status tide_plan_param(const tide_plan* plan, int32_t p, int64_t* rows, int64_t* row_len,
                            int64_t* R_p, int64_t* s_p, int64_t* o_p) {
    if (!plan) return fail(TIDE_ERR_INVALID_ARG, "plan is NULL");
    if (p < 0 || p >= plan->P) return fail(TIDE_ERR_INVALID_ARG, "p = %d out of range", p);
    const ParamInfo& q = plan->prm[p];
    if (rows) *rows = q.T;
    if (row_len) *row_len = q.K;
    if (R_p) *R_p = q.R;
    if (s_p) *s_p = q.s;
    if (o_p) *o_p = q.o;
    return TIDE_OK;
}

tide_status tide_plan_map(const tide_plan* plan, int32_t r, int32_t p, int64_t* rank_major,
                          int64_t* param_major, int64_t* valid) {
    if (!plan) return fail(TIDE_ERR_INVALID_ARG, "plan is NULL");
    if (p < 0 || p >= plan->P) return fail(TIDE_ERR_INVALID_ARG, "p = %d out of range", p);
    if (r < 0 || r >= plan->N) return fail(TIDE_ERR_INVALID_ARG, "r = %d out of range", r);
    const ParamInfo& q = plan->prm[p];
    if (rank_major) *rank_major = (int64_t)r * plan->S + q.o;
    if (param_major) *param_major = (int64_t)plan->N * q.o + (int64_t)r * q.s;
    if (valid) *valid = std::max<int64_t>(0, std::min(q.s, q.valid - (int64_t)r * q.s));
    return TIDE_OK;
}

tide_status tide_plan_launch_count(const tide_plan* plan, int32_t op, const tide_launch* launch,
                                   int64_t* launches) {
    try {
        if (!plan || !launches) return fail(TIDE_ERR_INVALID_ARG, "NULL argument");
        if (op < 0 || op > 2) return fail(TIDE_ERR_INVALID_ARG, "op %d not 0, 1 or 2", op);
        tide_launch l;
        tide_status st = resolve_launch(plan, launch, &l);
        if (st != TIDE_OK) return st;
        // The staging walks its tiling once per contributor.
        int64_t n = count_tiles(plan, op, l.rank_begin, l.rank_end, l.mode == TIDE_LAUNCH_BUDGETED);
        if (op == 2) n *= plan->L;
        *launches = count_launches(plan, op, l, n);
        return TIDE_OK;
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

}  // extern "C"

namespace {

// A validated call that reads a per-call pointer table (reduce-scatter, and
// placement and staging with the kernel engine): everything but the stream.
struct Prepared {
    int op = 0;                       // 0 reduce-scatter, 1 placement, 2 staging
    tide_launch l{};
    bool empty = false;               // nothing to launch
    std::vector<char> table;          // the per-call pointer table (and flag words)
    float* out = nullptr;             // op 0
    int64_t out_stride = 0;
    int32_t xcd_lc = 0;               // op 0: full-grid XCD run length (log2)
    bool shifted = false;             // op 0: some gradient starts at 2 mod 4 bytes
    const uint16_t* shards = nullptr; // op 1
    int64_t shard_stride = 0, shard_elems = 0;
    int32_t first_rank = 0;
    int64_t slot_elems = 0;           // op 2
};

tide_status prep_reduce(const tide_plan* plan, const uint16_t* const* grads, float* out,
                        int64_t out_stride, const tide_launch* launch, Prepared* pr) {
    if (!plan) return fail(TIDE_ERR_INVALID_ARG, "plan is NULL");
    pr->op = 0;
    tide_launch& l = pr->l;
    tide_status st = resolve_launch(plan, launch, &l);
    if (st != TIDE_OK) return st;
    const int32_t P = plan->P, L = plan->L;
    if (out_stride < plan->S)
        return fail(TIDE_ERR_INVALID_ARG, "out_stride %lld < S %lld", (long long)out_stride,
                    (long long)plan->S);
    int64_t total;
    if (!mul_ok(out_stride, plan->N, &total) || !mul_ok(total, 4, &total))
        return fail(TIDE_ERR_OVERFLOW, "N * out_stride * 4 overflows int64");
    st = check_counts(l, total / 4);
    if (st != TIDE_OK) return st;
    pr->out = out;
    pr->out_stride = out_stride;
    if (l.mode == TIDE_LAUNCH_FULL)
        pr->xcd_lc = reduce_xcd_log2(plan, out, out_stride, l.rank_begin, l.rank_end);
    if (plan->S == 0 || l.rank_end == l.rank_begin) {
        pr->empty = true;
        return TIDE_OK;
    }
    if (!out) return fail(TIDE_ERR_INVALID_ARG, "out is NULL");
    if (reinterpret_cast<uintptr_t>(out) & 3)
        return fail(TIDE_ERR_ALIGNMENT, "out is not 4-byte aligned");
    if (P > 0 && !grads) return fail(TIDE_ERR_INVALID_ARG, "grads is NULL");
    // Per-call table: P*L pointers (parameter-major) then P flag words.
    pr->table.assign((size_t)P * L * sizeof(void*) + (size_t)P * sizeof(uint32_t), 0);
    const uint16_t** tp = reinterpret_cast<const uint16_t**>(pr->table.data());
    uint32_t* fl = reinterpret_cast<uint32_t*>(pr->table.data() + (size_t)P * L * sizeof(void*));
    const Range w{reinterpret_cast<uintptr_t>(out) + (uintptr_t)l.rank_begin * out_stride * 4,
                  reinterpret_cast<uintptr_t>(out) + (uintptr_t)(l.rank_end - 1) * out_stride * 4 +
                      (uintptr_t)plan->S * 4,
                  -1};
    for (int32_t p = 0; p < P; ++p) {
        const ParamInfo& q = plan->prm[p];
        uint32_t f = (l.flags & TIDE_FLAG_SCALAR_PATH) ? 0u : kFlagVector;
        for (int32_t c = 0; c < L; ++c) {
            const uint16_t* g = grads[(size_t)c * P + p];
            tp[(size_t)p * L + c] = g;
            if (q.valid == 0) continue;
            if (!g) return fail(TIDE_ERR_INVALID_ARG, "grads[%d] (c=%d, p=%d) is NULL", c * P + p, c, p);
            const uintptr_t a = reinterpret_cast<uintptr_t>(g);
            if (a & 1) return fail(TIDE_ERR_ALIGNMENT, "grads[%d] is not 2-byte aligned", c * P + p);
            // Multi-dword loads need dword alignment only; a gradient at 2 mod 4
            // bytes is read with dword-aligned loads and a funnel shift.
            if (a & 3) {
                if (c < kMaxOddShift) f |= 1u << (kOddShift + c);
                else f &= ~kFlagVector;
            }
            if ((f & kFlagVector) && (f >> kOddShift)) pr->shifted = true;
            const Range in{a, a + (uintptr_t)q.valid * 2, c * P + p};
            if (overlaps(in, w))
                return fail(TIDE_ERR_INVALID_ARG, "grads[%d] overlaps the output", c * P + p);
        }
        fl[p] = f;
    }
    return TIDE_OK;
}

tide_status prep_place(const tide_plan* plan, const uint16_t* shards, int64_t shard_stride,
                       int32_t first_rank, uint16_t* const* params, int32_t engine,
                       const tide_launch* launch, Prepared* pr) {
    if (!plan) return fail(TIDE_ERR_INVALID_ARG, "plan is NULL");
    pr->op = 1;
    if (first_rank < 0 || first_rank >= plan->N)
        return fail(TIDE_ERR_INVALID_ARG, "first_rank %d outside [0, %d)", first_rank, plan->N);
    tide_launch& l = pr->l;
    tide_status st = resolve_launch(plan, launch, &l);
    if (st != TIDE_OK) return st;
    if (engine != TIDE_ENGINE_KERNEL && engine != TIDE_ENGINE_RUNTIME &&
        engine != TIDE_ENGINE_SDMA)
        return fail(TIDE_ERR_INVALID_ARG, "engine %d is not KERNEL (0), RUNTIME (1) or SDMA (2)",
                    engine);
    if (l.write_counts && engine != TIDE_ENGINE_KERNEL)
        return fail(TIDE_ERR_INVALID_ARG, "write counts need the kernel engine");
    st = check_counts(l, (int64_t)plan->N * plan->S);
    if (st != TIDE_OK) return st;
    const int32_t P = plan->P;
    if (shard_stride < plan->S)
        return fail(TIDE_ERR_INVALID_ARG, "shard_stride %lld < S %lld",
                    (long long)shard_stride, (long long)plan->S);
    int64_t shard_elems;
    if (!mul_ok(shard_stride, plan->N, &shard_elems) || !mul_ok(shard_elems, 2, &shard_elems))
        return fail(TIDE_ERR_OVERFLOW, "N * shard_stride * 2 overflows int64");
    pr->shards = shards;
    pr->shard_stride = shard_stride;
    // The extent the caller guarantees: the last shard ends at S, not at the
    // stride. The kernel's realigning loads stay inside it.
    pr->shard_elems = (int64_t)(plan->N - 1) * shard_stride + plan->S;
    pr->first_rank = first_rank;
    if (plan->S == 0 || l.rank_end == l.rank_begin) {
        pr->empty = true;
        return TIDE_OK;
    }
    if (!shards) return fail(TIDE_ERR_INVALID_ARG, "shards is NULL");
    if (reinterpret_cast<uintptr_t>(shards) & 1)
        return fail(TIDE_ERR_ALIGNMENT, "shards is not 2-byte aligned");
    if (P > 0 && !params) return fail(TIDE_ERR_INVALID_ARG, "params is NULL");
    pr->table.assign((size_t)P * sizeof(void*) + (size_t)P * sizeof(uint32_t), 0);
    uint16_t** tp = reinterpret_cast<uint16_t**>(pr->table.data());
    uint32_t* fl = reinterpret_cast<uint32_t*>(pr->table.data() + (size_t)P * sizeof(void*));
    const uintptr_t sb = reinterpret_cast<uintptr_t>(shards);
    // Shards read: ranks [rank_begin, rank_end) in place, or the whole
    // stage buffer when it is rotated.
    const Range rd = first_rank == 0
        ? Range{sb + (uintptr_t)l.rank_begin * shard_stride * 2,
                sb + (uintptr_t)(l.rank_end - 1) * shard_stride * 2 + (uintptr_t)plan->S * 2, -1}
        : Range{sb, sb + (uintptr_t)(plan->N - 1) * shard_stride * 2 + (uintptr_t)plan->S * 2, -1};
    std::vector<Range> wr;
    for (int32_t p = 0; p < P; ++p) {
        const ParamInfo& q = plan->prm[p];
        uint16_t* d = params[p];
        tp[p] = d;
        fl[p] = (l.flags & TIDE_FLAG_SCALAR_PATH) ? 0u : kFlagVector;
        if (q.valid == 0) continue;
        if (!d) return fail(TIDE_ERR_INVALID_ARG, "params[%d] is NULL", p);
        const uintptr_t a = reinterpret_cast<uintptr_t>(d);
        if (a & 1) return fail(TIDE_ERR_ALIGNMENT, "params[%d] is not 2-byte aligned", p);
        if (a & 15) fl[p] = 0;
        const Range r{a, a + (uintptr_t)q.valid * 2, p};
        if (overlaps(r, rd)) return fail(TIDE_ERR_INVALID_ARG, "params[%d] overlaps the shards", p);
        wr.push_back(r);
    }
    std::sort(wr.begin(), wr.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
    for (size_t i = 1; i < wr.size(); ++i)
        if (wr[i].lo < wr[i - 1].hi)
            return fail(TIDE_ERR_INVALID_ARG, "params[%d] and params[%d] overlap", wr[i - 1].who,
                        wr[i].who);
    return TIDE_OK;
}

tide_status prep_stage(const tide_plan* plan, const uint16_t* const* grads, uint16_t* const* slots,
                       int32_t engine, const tide_launch* launch, Prepared* pr) {
    if (!plan) return fail(TIDE_ERR_INVALID_ARG, "plan is NULL");
    pr->op = 2;
    tide_launch& l = pr->l;
    tide_status st = resolve_launch(plan, launch, &l);
    if (st != TIDE_OK) return st;
    if (engine != TIDE_ENGINE_KERNEL && engine != TIDE_ENGINE_RUNTIME &&
        engine != TIDE_ENGINE_SDMA)
        return fail(TIDE_ERR_INVALID_ARG, "engine %d is not KERNEL (0), RUNTIME (1) or SDMA (2)",
                    engine);
    const int32_t P = plan->P, L = plan->L;
    const int64_t slot_elems = (int64_t)plan->N * plan->S;   // fits: checked at plan creation
    pr->slot_elems = slot_elems;
    if (l.write_counts && engine != TIDE_ENGINE_KERNEL)
        return fail(TIDE_ERR_INVALID_ARG, "write counts need the kernel engine");
    int64_t counts_need;
    if (!mul_ok(slot_elems, L, &counts_need))
        return fail(TIDE_ERR_OVERFLOW, "L * N * S overflows int64");
    st = check_counts(l, counts_need);
    if (st != TIDE_OK) return st;
    if (plan->S == 0 || l.rank_end == l.rank_begin) {
        pr->empty = true;
        return TIDE_OK;
    }
    if (!slots) return fail(TIDE_ERR_INVALID_ARG, "slots is NULL");
    if (P > 0 && !grads) return fail(TIDE_ERR_INVALID_ARG, "grads is NULL");
    std::vector<Range> sr;
    for (int32_t c = 0; c < L; ++c) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(slots[c]);
        if (!a) return fail(TIDE_ERR_INVALID_ARG, "slots[%d] is NULL", c);
        if (a & 1) return fail(TIDE_ERR_ALIGNMENT, "slots[%d] is not 2-byte aligned", c);
        sr.push_back(Range{a, a + (uintptr_t)slot_elems * 2, c});
    }
    {
        std::vector<Range> sorted = sr;
        std::sort(sorted.begin(), sorted.end(),
                  [](const Range& a, const Range& b) { return a.lo < b.lo; });
        for (size_t i = 1; i < sorted.size(); ++i)
            if (sorted[i].lo < sorted[i - 1].hi)
                return fail(TIDE_ERR_INVALID_ARG, "slots[%d] and slots[%d] overlap",
                            sorted[i - 1].who, sorted[i].who);
    }
    // Per-call table: P*L sources, P*L destinations (both parameter-major,
    // p * L + c), then P flag words.
    const size_t np = (size_t)P * L;
    pr->table.assign(2 * np * sizeof(void*) + (size_t)P * sizeof(uint32_t), 0);
    const uint16_t** ts = reinterpret_cast<const uint16_t**>(pr->table.data());
    uint16_t** td = reinterpret_cast<uint16_t**>(pr->table.data() + np * sizeof(void*));
    uint32_t* fl = reinterpret_cast<uint32_t*>(pr->table.data() + 2 * np * sizeof(void*));
    for (int32_t p = 0; p < P; ++p) {
        const ParamInfo& q = plan->prm[p];
        uint32_t f = (l.flags & TIDE_FLAG_SCALAR_PATH) ? 0u : kFlagVector;
        for (int32_t c = 0; c < L; ++c) {
            const uint16_t* g = grads[(size_t)c * P + p];
            uint16_t* d = slots[c] + (int64_t)plan->N * q.o;
            ts[(size_t)p * L + c] = g;
            td[(size_t)p * L + c] = d;
            if (q.valid == 0) continue;
            if (!g) return fail(TIDE_ERR_INVALID_ARG, "grads[%d] (c=%d, p=%d) is NULL", c * P + p, c, p);
            const uintptr_t a = reinterpret_cast<uintptr_t>(g);
            if (a & 1) return fail(TIDE_ERR_ALIGNMENT, "grads[%d] is not 2-byte aligned", c * P + p);
            if ((a | reinterpret_cast<uintptr_t>(d)) & 3) f = 0;
            const Range in{a, a + (uintptr_t)q.valid * 2, c * P + p};
            for (const Range& r : sr)
                if (overlaps(in, r))
                    return fail(TIDE_ERR_INVALID_ARG, "grads[%d] overlaps slots[%d]", c * P + p, r.who);
        }
        fl[p] = f;
    }
    return TIDE_OK;
}

// Device state and tile table of a prepared call on `dev`, with its trace and
// LDS checks done. Caller holds plan->mu.
tide_status device_side(const tide_plan* plan, const Prepared& pr, int dev, DevState** ds,
                        TileTable** tt) {
    const tide_launch& l = pr.l;
    tide_status st = get_dev_state(plan, dev, ds);
    if (st != TIDE_OK) return st;
    st = get_tiles(plan, *ds, pr.op, l.rank_begin, l.rank_end, l.mode == TIDE_LAUNCH_BUDGETED, tt);
    if (st != TIDE_OK) return st;
    // The host-only counts must describe the table the kernels walk.
    if ((*tt)->count != count_tiles(plan, pr.op, l.rank_begin, l.rank_end,
                                    l.mode == TIDE_LAUNCH_BUDGETED))
        return fail(TIDE_ERR_INVALID_ARG, "internal: tile table and tile count disagree");
    const int64_t items = pr.op == 2 ? (*tt)->count * plan->L : (*tt)->count;
    st = check_trace(l, launch_records(plan, pr.op, l, items));
    if (st != TIDE_OK) return st;
    return prepare_budget(*ds, plan->L, l);
}

// Enqueue the kernels of a prepared call, its pointer table at `dtab`.
tide_status launch_prepared(const tide_plan* plan, const Prepared& pr, const DevState* ds,
                            const TileTable* tt, const char* dtab, hipStream_t stream) {
    const tide_launch& l = pr.l;
    const int32_t P = plan->P, L = plan->L;
    if (tt->count == 0) return TIDE_OK;
    if (pr.op == 0) {
        const uint16_t* const* dptrs = reinterpret_cast<const uint16_t* const*>(dtab);
        const uint32_t* dflags = reinterpret_cast<const uint32_t*>(dtab + (size_t)P * L * sizeof(void*));
        return for_each_launch(plan, 0, l, tt->count,
                               [&](int grid, int threads, size_t lds, int64_t lo, int64_t hi,
                                   int64_t tb) {
            return launch_reduce(L, grid, threads, lds, stream, tt->dev, lo, hi, l.rank_begin,
                                 l.rank_end, ds->params, dptrs, dflags, pr.out, pr.out_stride,
                                 l.trace, tb, l.write_counts, pr.xcd_lc, pr.shifted);
        });
    }
    if (pr.op == 1) {
        uint16_t* const* dptrs = reinterpret_cast<uint16_t* const*>(const_cast<char*>(dtab));
        const uint32_t* dflags = reinterpret_cast<const uint32_t*>(dtab + (size_t)P * sizeof(void*));
        return for_each_launch(plan, 1, l, tt->count,
                               [&](int grid, int threads, size_t lds, int64_t lo, int64_t hi,
                                   int64_t tb) {
            return launch_place(grid, threads, lds, stream, tt->dev, lo, hi, l.rank_begin,
                                l.rank_end, ds->params, dptrs, dflags, pr.shards, pr.shard_stride,
                                pr.shard_elems, pr.first_rank, plan->N, l.trace, tb,
                                l.write_counts);
        });
    }
    const size_t np = (size_t)P * L;
    const uint16_t* const* dsrc = reinterpret_cast<const uint16_t* const*>(dtab);
    uint16_t* const* ddst =
        reinterpret_cast<uint16_t* const*>(const_cast<char*>(dtab) + np * sizeof(void*));
    const uint32_t* dflags = reinterpret_cast<const uint32_t*>(dtab + 2 * np * sizeof(void*));
    const int64_t ntiles = tt->count;
    return for_each_launch(plan, 2, l, ntiles * L,
                           [&](int grid, int threads, size_t lds, int64_t lo, int64_t hi,
                               int64_t tb) {
        return launch_stage(grid, threads, lds, stream, tt->dev, ntiles, lo, hi, l.rank_begin,
                            l.rank_end, ds->params, dsrc, ddst, dflags, L, l.trace, tb,
                            l.write_counts, pr.slot_elems, plan->N);
    });
}

// An eager call: its table goes through the plan's ring.
tide_status run_eager(const tide_plan* plan, const Prepared& pr, hipStream_t stream) {
    if (pr.empty) return TIDE_OK;
    tide_status st = refuse_capture(stream);
    if (st != TIDE_OK) return st;
    std::lock_guard<std::mutex> lock(plan->mu);
    int dev;
    st = stream_device(stream, &dev);
    if (st != TIDE_OK) return st;
    DeviceGuard guard(dev);
    if (guard.status() != hipSuccess) return hip_fail(guard.status(), "hipSetDevice");
    DevState* ds;
    TileTable* tt;
    st = device_side(plan, pr, dev, &ds, &tt);
    if (st != TIDE_OK) return st;
    if (tt->count == 0) return TIDE_OK;
    int slot;
    st = stage_table(ds, pr.table.data(), pr.table.size(), stream, &slot);
    if (st != TIDE_OK) return st;
    st = launch_prepared(plan, pr, ds, tt, static_cast<const char*>(ds->slots[slot].dev), stream);
    tide_status st2 = release_slot(ds, slot, stream);
    return st != TIDE_OK ? st : st2;
}

}  // namespace

// A prepared call: fixed buffers, its own device copy of the pointer table.
struct tide_call {
    const tide_plan* plan = nullptr;
    Prepared pr;
    int device = -1;
    const DevState* ds = nullptr;
    TileTable* tt = nullptr;          // pinned in the plan's cache while the call lives
    void* dtab = nullptr;
};

namespace {

tide_status make_call(const tide_plan* plan, Prepared&& pr, tide_call** out) {
    std::unique_ptr<tide_call> call(new tide_call());
    call->plan = plan;
    call->pr = std::move(pr);
    TIDE_HIP_TRY(hipGetDevice(&call->device));
    if (!call->pr.empty) {
        std::lock_guard<std::mutex> lock(plan->mu);
        DevState* ds;
        TileTable* tt;
        tide_status st = device_side(plan, call->pr, call->device, &ds, &tt);
        if (st != TIDE_OK) return st;
        call->ds = ds;
        call->tt = tt;
        ++tt->pins;
        if (tt->count > 0) {
            TIDE_HIP_TRY(hipMalloc(&call->dtab, call->pr.table.size()));
            hipError_t e = hipMemcpy(call->dtab, call->pr.table.data(), call->pr.table.size(),
                                     hipMemcpyHostToDevice);
            if (e != hipSuccess) {
                (void)hipFree(call->dtab);
                return hip_fail(e, "hipMemcpy(call table)");
            }
        }
    }
    *out = call.release();
    return TIDE_OK;
}

}  // namespace

extern "C" {

tide_status tide_reduce_scatter_bf16_fp32(const tide_plan* plan, const uint16_t* const* grads,
                                          float* out, int64_t out_stride, void* stream_v,
                                          const tide_launch* launch) {
    try {
        Prepared pr;
        tide_status st = prep_reduce(plan, grads, out, out_stride, launch, &pr);
        if (st != TIDE_OK) return st;
        return run_eager(plan, pr, reinterpret_cast<hipStream_t>(stream_v));
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

}  // extern "C"

namespace {

// What the allocation-free reduce-scatter last wrote into each device's
// scratch, so that an unchanged table is not uploaded again (the upload is
// from pageable memory, which the runtime performs synchronously).
std::mutex g_noalloc_mu;
std::map<int, std::vector<char>> g_noalloc_image;
bool g_noalloc_lds[64][65] = {};

size_t align_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

}  // namespace

extern "C" {

tide_status tide_reduce_scatter_bf16_fp32_noalloc(const tide_plan* plan,
                                                  const uint16_t* const* grads, float* out,
                                                  int64_t out_stride, void* stream_v,
                                                  const tide_launch* launch) {
    try {
        Prepared pr;
        tide_status st = prep_reduce(plan, grads, out, out_stride, launch, &pr);
        if (st != TIDE_OK || pr.empty) return st;
        const tide_launch& l = pr.l;
        const int32_t P = plan->P, L = plan->L;
        const bool fat = l.mode == TIDE_LAUNCH_BUDGETED;
        // Scratch image: ParamDev[P] | {P, cum[0..P]} | pointers[P * L] | flags[P].
        const size_t off_hdr = align_up((size_t)P * sizeof(ParamDev), 16);
        const size_t off_ptrs = align_up(off_hdr + ((size_t)P + 2) * sizeof(int64_t), 16);
        const size_t off_flags = off_ptrs + (size_t)P * L * sizeof(void*);
        const size_t total = off_flags + (size_t)P * sizeof(uint32_t);
        if (total > kScratchBytes)
            return fail(TIDE_ERR_INVALID_ARG,
                        "the group's tables need %zu bytes, more than the %zu-byte fixed scratch of "
                        "the allocation-free reduce-scatter (about P * (44 + 8 L) bytes are needed)",
                        total, kScratchBytes);
        std::vector<char> img(total, 0);
        ParamDev* pd = reinterpret_cast<ParamDev*>(img.data());
        int64_t* hdr = reinterpret_cast<int64_t*>(img.data() + off_hdr);
        hdr[0] = P;
        int64_t* cum = hdr + 1;
        cum[0] = 0;
        const int64_t tile = tile_elems(0, fat);
        for (int32_t p = 0; p < P; ++p) {
            const ParamInfo& q = plan->prm[p];
            pd[p].s = q.s;
            pd[p].o = q.o;
            pd[p].valid = q.valid;
            pd[p].pad = 0;
            int64_t n = 0;
            if (q.s > 0) {   // the tiles build_tiles makes for this parameter
                const int64_t lo = (int64_t)l.rank_begin * q.s, hi = (int64_t)l.rank_end * q.s;
                if (hi > lo) n = (hi - (lo - lo % kVec) + tile - 1) / tile;
            }
            cum[p + 1] = cum[p] + n;
        }
        std::memcpy(img.data() + off_ptrs, pr.table.data(), pr.table.size());
        const int64_t ntiles = cum[P];
        st = check_trace(l, launch_records(plan, 0, l, ntiles));
        if (st != TIDE_OK) return st;
        if (ntiles == 0) return TIDE_OK;
        hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
        st = refuse_capture(stream);
        if (st != TIDE_OK) return st;
        int dev;
        st = stream_device(stream, &dev);
        if (st != TIDE_OK) return st;
        if (dev < 0 || dev >= 64) return fail(TIDE_ERR_UNSUPPORTED, "device %d beyond 63", dev);
        DeviceGuard guard(dev);
        if (guard.status() != hipSuccess) return hip_fail(guard.status(), "hipSetDevice");
        void* base = nullptr;
        TIDE_HIP_TRY(scratch_address(dev, &base));
        {
            std::lock_guard<std::mutex> lock(g_noalloc_mu);
            if (fat) {
                const int key = L <= 8 ? L : 0;
                if (!g_noalloc_lds[dev][key]) {
                    TIDE_HIP_TRY(allow_dynamic_lds(key, kBudgetLds));
                    g_noalloc_lds[dev][key] = true;
                }
            }
            std::vector<char>& last = g_noalloc_image[dev];
            if (last != img) {
                TIDE_HIP_TRY(hipMemcpyAsync(base, img.data(), total, hipMemcpyHostToDevice, stream));
                last.swap(img);
            }
        }
        const char* b = static_cast<const char*>(base);
        const ParamDev* dparams = reinterpret_cast<const ParamDev*>(b);
        const int64_t* dhdr = reinterpret_cast<const int64_t*>(b + off_hdr);
        const uint16_t* const* dptrs = reinterpret_cast<const uint16_t* const*>(b + off_ptrs);
        const uint32_t* dflags = reinterpret_cast<const uint32_t*>(b + off_flags);
        return for_each_launch(plan, 0, l, ntiles,
                               [&](int grid, int threads, size_t lds, int64_t lo, int64_t hi,
                                   int64_t tb) {
            return launch_reduce_derived(L, grid, threads, lds, stream, dhdr, lo, hi, l.rank_begin,
                                         l.rank_end, dparams, dptrs, dflags, out, out_stride,
                                         l.trace, tb, l.write_counts, pr.xcd_lc, pr.shifted);
        });
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

tide_status tide_allgather_place(const tide_plan* plan, const uint16_t* shards,
                                 int64_t shard_stride, uint16_t* const* params, void* stream_v,
                                 int32_t engine, const tide_launch* launch) {
    return tide_allgather_place_stage(plan, shards, shard_stride, 0, params, stream_v, engine,
                                      launch);
}

tide_status tide_allgather_place_stage(const tide_plan* plan, const uint16_t* shards,
                                       int64_t shard_stride, int32_t first_rank,
                                       uint16_t* const* params, void* stream_v, int32_t engine,
                                       const tide_launch* launch) {
    try {
        Prepared pr;
        tide_status st = prep_place(plan, shards, shard_stride, first_rank, params, engine, launch,
                                    &pr);
        if (st != TIDE_OK || pr.empty) return st;
        hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
        if (engine == TIDE_ENGINE_RUNTIME) {
            // One 2-D copy per parameter for its full pieces (rows of s_p
            // elements, source pitch = shard stride, destination contiguous),
            // split in two where a rotated stage wraps, plus one 1-D copy for
            // a partial last piece.
            const tide_launch& l = pr.l;
            const int64_t N = plan->N;
            auto pos = [&](int64_t r) { return (r - first_rank + N) % N; };
            for (int32_t p = 0; p < plan->P; ++p) {
                const ParamInfo& q = plan->prm[p];
                if (q.valid == 0) continue;
                const int64_t full = q.valid / q.s;                   // ranks with a whole piece
                const int64_t fb = std::min<int64_t>(l.rank_begin, full);
                const int64_t fe = std::min<int64_t>(l.rank_end, full);
                const uint16_t* src0 = shards + q.o;
                const int64_t cut = std::min(std::max<int64_t>(first_rank, fb), fe);
                const int64_t seg[2][2] = {{fb, cut}, {cut, fe}};
                for (const auto& sg : seg) {
                    if (sg[1] <= sg[0]) continue;
                    TIDE_HIP_TRY(hipMemcpy2DAsync(params[p] + sg[0] * q.s, (size_t)q.s * 2,
                                                  src0 + pos(sg[0]) * shard_stride,
                                                  (size_t)shard_stride * 2, (size_t)q.s * 2,
                                                  (size_t)(sg[1] - sg[0]), hipMemcpyDeviceToDevice,
                                                  stream));
                }
                const int64_t rem = q.valid - full * q.s;
                if (rem > 0 && full >= l.rank_begin && full < l.rank_end)
                    TIDE_HIP_TRY(hipMemcpyAsync(params[p] + full * q.s,
                                                src0 + pos(full) * shard_stride, (size_t)rem * 2,
                                                hipMemcpyDeviceToDevice, stream));
            }
            return TIDE_OK;
        }
        if (engine == TIDE_ENGINE_SDMA) {
            // One linear copy per (parameter, rank) piece: the piece's true
            // rows, from its place in the (rotated) rank-major buffer to rows
            // r * R_p.. of the parameter.
            const tide_launch& l = pr.l;
            const int64_t N = plan->N;
            std::vector<DmaCopy> cp;
            for (int32_t p = 0; p < plan->P; ++p) {
                const ParamInfo& q = plan->prm[p];
                if (q.valid == 0) continue;
                for (int64_t r = l.rank_begin; r < l.rank_end; ++r) {
                    const int64_t v = std::min(q.s, q.valid - r * q.s);
                    if (v <= 0) break;
                    add_copy(cp, params[p] + r * q.s,
                             shards + ((r - first_rank + N) % N) * shard_stride + q.o,
                             (uint64_t)v * 2);
                }
            }
            return run_dma(stream, cp);
        }
        return run_eager(plan, pr, stream);
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

tide_status tide_stage_grads_bf16(const tide_plan* plan, const uint16_t* const* grads,
                                  uint16_t* const* slots, void* stream_v, int32_t engine,
                                  const tide_launch* launch) {
    try {
        Prepared pr;
        tide_status st = prep_stage(plan, grads, slots, engine, launch, &pr);
        if (st != TIDE_OK || pr.empty) return st;
        hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
        if (engine != TIDE_ENGINE_KERNEL) {
            // One contiguous copy per (contributor, parameter): the rows of
            // ranks [rank_begin, rank_end) are one run on both sides.
            const int32_t P = plan->P, L = plan->L;
            const size_t np = (size_t)P * L;
            const uint16_t* const* ts = reinterpret_cast<const uint16_t* const*>(pr.table.data());
            uint16_t* const* td =
                reinterpret_cast<uint16_t* const*>(pr.table.data() + np * sizeof(void*));
            std::vector<DmaCopy> cp;
            for (int32_t p = 0; p < P; ++p) {
                const ParamInfo& q = plan->prm[p];
                const int64_t lo = (int64_t)pr.l.rank_begin * q.s;
                const int64_t hi = std::min((int64_t)pr.l.rank_end * q.s, q.valid);
                if (hi <= lo) continue;
                for (int32_t c = 0; c < L; ++c) {
                    if (engine == TIDE_ENGINE_SDMA)
                        add_copy(cp, td[(size_t)p * L + c] + lo, ts[(size_t)p * L + c] + lo,
                                 (uint64_t)(hi - lo) * 2);
                    else
                        TIDE_HIP_TRY(hipMemcpyAsync(td[(size_t)p * L + c] + lo,
                                                    ts[(size_t)p * L + c] + lo,
                                                    (size_t)(hi - lo) * 2,
                                                    hipMemcpyDeviceToDevice, stream));
                }
            }
            if (engine == TIDE_ENGINE_SDMA) return run_dma(stream, cp);
            return TIDE_OK;
        }
        return run_eager(plan, pr, stream);
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

tide_status tide_prepare_reduce_scatter_bf16_fp32(const tide_plan* plan,
                                                  const uint16_t* const* grads, float* out,
                                                  int64_t out_stride, const tide_launch* launch,
                                                  tide_call** call) {
    try {
        if (!call) return fail(TIDE_ERR_INVALID_ARG, "call is NULL");
        *call = nullptr;
        Prepared pr;
        tide_status st = prep_reduce(plan, grads, out, out_stride, launch, &pr);
        if (st != TIDE_OK) return st;
        return make_call(plan, std::move(pr), call);
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

tide_status tide_prepare_allgather_place_stage(const tide_plan* plan, const uint16_t* shards,
                                               int64_t shard_stride, int32_t first_rank,
                                               uint16_t* const* params, const tide_launch* launch,
                                               tide_call** call) {
    try {
        if (!call) return fail(TIDE_ERR_INVALID_ARG, "call is NULL");
        *call = nullptr;
        Prepared pr;
        tide_status st = prep_place(plan, shards, shard_stride, first_rank, params,
                                    TIDE_ENGINE_KERNEL, launch, &pr);
        if (st != TIDE_OK) return st;
        return make_call(plan, std::move(pr), call);
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

tide_status tide_prepare_stage_grads_bf16(const tide_plan* plan, const uint16_t* const* grads,
                                          uint16_t* const* slots, const tide_launch* launch,
                                          tide_call** call) {
    try {
        if (!call) return fail(TIDE_ERR_INVALID_ARG, "call is NULL");
        *call = nullptr;
        Prepared pr;
        tide_status st = prep_stage(plan, grads, slots, TIDE_ENGINE_KERNEL, launch, &pr);
        if (st != TIDE_OK) return st;
        return make_call(plan, std::move(pr), call);
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

tide_status tide_call_enqueue(const tide_call* call, void* stream_v) {
    if (!call) return fail(TIDE_ERR_INVALID_ARG, "call is NULL");
    if (call->pr.empty || !call->tt || call->tt->count == 0) return TIDE_OK;
    hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
    int dev;
    tide_status st = stream_device(stream, &dev);
    if (st != TIDE_OK) return st;
    if (dev != call->device)
        return fail(TIDE_ERR_INVALID_ARG, "stream is on device %d, the call was prepared on %d", dev,
                    call->device);
    return launch_prepared(call->plan, call->pr, call->ds, call->tt,
                           static_cast<const char*>(call->dtab), stream);
}

void tide_call_destroy(tide_call* call) {
    if (!call) return;
    if (call->tt) {
        std::lock_guard<std::mutex> lock(call->plan->mu);
        --call->tt->pins;
    }
    if (call->dtab) {
        DeviceGuard guard(call->device);
        (void)hipFree(call->dtab);
    }
    delete call;
}

tide_status tide_latin_square(int32_t M, int32_t L, int32_t dst_node, int32_t src_node, int32_t* c,
                              int32_t* slice_of_src_gpu, int32_t* dst_gpu_of_slice) {
    if (M < 1 || L < 1) return fail(TIDE_ERR_INVALID_ARG, "M = %d, L = %d must be >= 1", M, L);
    if (dst_node < 0 || dst_node >= M || src_node < 0 || src_node >= M)
        return fail(TIDE_ERR_INVALID_ARG, "nodes %d, %d outside [0, %d)", dst_node, src_node, M);
    const int32_t cc = ((dst_node - src_node) % M + M) % M;   // relative index; destination is 0
    if (c) *c = cc;
    for (int32_t j = 0; j < L; ++j) {
        if (slice_of_src_gpu) slice_of_src_gpu[j] = (j + cc) % L;
        if (dst_gpu_of_slice) dst_gpu_of_slice[j] = ((j - cc) % L + L) % L;
    }
    return TIDE_OK;
}

}  // extern "C"

namespace {

// The landing sum's launches: each is (grid, threads, lds, tile_lo, tile_hi).
template <typename F>
hipError_t for_each_landing_launch(int32_t L, int32_t M, int64_t S, int32_t accumulate,
                                   const tide_launch& l, F&& launch) {
    const int64_t tiles_per_shard = (S + kLandTile - 1) / kLandTile;
    const int64_t ntiles = tiles_per_shard * L;
    if (ntiles == 0) return hipSuccess;
    if (l.mode == TIDE_LAUNCH_FULL)
        return launch((int)std::min<int64_t>(ntiles, kFullGridCap), kThreads, (size_t)0,
                      (int64_t)0, ntiles, (int64_t)0);
    const size_t lds = (l.flags & TIDE_FLAG_NO_LDS_FENCE) ? 0 : kBudgetLds;
    const int64_t tile_b = kLandTile * (4 * (int64_t)M + 4 + 4 * accumulate);
    const int64_t per_block =
        std::max<int64_t>(1, (int64_t)l.max_launch_us * kWgBytesPerUsLanding / tile_b);
    const int64_t per_launch = (int64_t)l.place_blocks * per_block;
    int64_t base = 0;
    for (int64_t lo = 0; lo < ntiles; lo += per_launch) {
        const int64_t hi = std::min(ntiles, lo + per_launch);
        const int grid = (int)std::min<int64_t>(l.place_blocks, hi - lo);
        hipError_t e = launch(grid, kBudgetThreads, lds, lo, hi, base);
        if (e != hipSuccess) return e;
        base += grid;
    }
    return hipSuccess;
}

// Validates and completes the landing sum's launch options.
tide_status landing_launch(int32_t L, int32_t M, int64_t S, int32_t accumulate,
                           const tide_launch* launch, tide_launch* out) {
    if (L < 1 || L > kMaxLanding)
        return fail(TIDE_ERR_INVALID_ARG, "L = %d not in [1, %d]", L, kMaxLanding);
    if (M < 1 || M > L) return fail(TIDE_ERR_INVALID_ARG, "M = %d not in [1, L = %d]", M, L);
    if (S < 0) return fail(TIDE_ERR_INVALID_ARG, "S = %lld < 0", (long long)S);
    if (accumulate != 0 && accumulate != 1)
        return fail(TIDE_ERR_INVALID_ARG, "accumulate must be 0 or 1");
    tide_launch l{};
    if (launch) l = *launch;
    if (l.rank_begin != 0 || l.rank_end != 0)
        return fail(TIDE_ERR_INVALID_ARG, "rank_begin / rank_end do not apply to the landing sum");
    if (l.mode != TIDE_LAUNCH_FULL && l.mode != TIDE_LAUNCH_BUDGETED)
        return fail(TIDE_ERR_INVALID_ARG, "launch.mode %d is not FULL (0) or BUDGETED (1)", l.mode);
    if (l.reduce_blocks < 0 || l.place_blocks < 0 || l.max_launch_us < 0)
        return fail(TIDE_ERR_INVALID_ARG, "negative launch budget");
    if (l.reduce_blocks > kMaxBudgetBlocks || l.place_blocks > kMaxBudgetBlocks)
        return fail(TIDE_ERR_INVALID_ARG, "reduce_blocks %d / place_blocks %d above %d",
                    l.reduce_blocks, l.place_blocks, kMaxBudgetBlocks);
    if (l.reserved != 0 || (l.flags & ~kKnownFlags) != 0)
        return fail(TIDE_ERR_INVALID_ARG, "unknown launch flags 0x%x", l.flags);
    if (l.trace_capacity < 0) return fail(TIDE_ERR_INVALID_ARG, "negative trace_capacity");
    if (l.write_counts_elems < 0) return fail(TIDE_ERR_INVALID_ARG, "negative write_counts_elems");
    if (l.place_blocks == 0) l.place_blocks = kDefaultPlaceBlocks;
    if (l.max_launch_us == 0) l.max_launch_us = kDefaultMaxLaunchUs;
    *out = l;
    return TIDE_OK;
}

}  // namespace

extern "C" {

tide_status tide_landing_trace_records(int32_t L, int32_t M, int64_t S, int32_t accumulate,
                                       const tide_launch* launch, int64_t* records) {
    if (!records) return fail(TIDE_ERR_INVALID_ARG, "records is NULL");
    tide_launch l;
    tide_status st = landing_launch(L, M, S, accumulate, launch, &l);
    if (st != TIDE_OK) return st;
    int64_t n = 0;
    (void)for_each_landing_launch(L, M, S, accumulate, l,
                                  [&](int grid, int, size_t, int64_t, int64_t, int64_t) {
        n += grid;
        return hipSuccess;
    });
    *records = n;
    return TIDE_OK;
}

tide_status tide_landing_sum_fp32(int32_t L, int32_t M, int64_t S, const float* const* inboxes,
                                  float* const* shards, int32_t accumulate, void* stream_v,
                                  const tide_launch* launch) {
    try {
        tide_launch l;
        tide_status st = landing_launch(L, M, S, accumulate, launch, &l);
        if (st != TIDE_OK) return st;
        if (S == 0) return TIDE_OK;
        if (!inboxes || !shards) return fail(TIDE_ERR_INVALID_ARG, "inboxes / shards is NULL");
        const int64_t C = S / L + (S % L != 0);
        int64_t inbox_elems, bytes;
        if (!mul_ok((int64_t)L * L, C, &inbox_elems) || !mul_ok(inbox_elems, 4, &bytes))
            return fail(TIDE_ERR_OVERFLOW, "inbox size overflows int64");
        LandingPtrs ptrs{};
        std::vector<Range> rd, wr;
        for (int32_t g = 0; g < L; ++g) {
            const uintptr_t a = reinterpret_cast<uintptr_t>(inboxes[g]);
            const uintptr_t w = reinterpret_cast<uintptr_t>(shards[g]);
            if (!a || !w) return fail(TIDE_ERR_INVALID_ARG, "inboxes[%d] or shards[%d] is NULL", g, g);
            if ((a & 3) || (w & 3)) return fail(TIDE_ERR_ALIGNMENT, "GPU %d: pointer not 4-byte aligned", g);
            ptrs.inbox[g] = inboxes[g];
            ptrs.shard[g] = shards[g];
            rd.push_back(Range{a, a + (uintptr_t)bytes, g});
            wr.push_back(Range{w, w + (uintptr_t)S * 4, g});
        }
        std::sort(wr.begin(), wr.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
        for (size_t i = 1; i < wr.size(); ++i)
            if (wr[i].lo < wr[i - 1].hi)
                return fail(TIDE_ERR_INVALID_ARG, "shards[%d] and shards[%d] overlap", wr[i - 1].who, wr[i].who);
        for (const Range& w : wr)
            for (const Range& r : rd)
                if (overlaps(w, r))
                    return fail(TIDE_ERR_INVALID_ARG, "shards[%d] overlaps inboxes[%d]", w.who, r.who);
        int64_t records = 0;
        (void)for_each_landing_launch(L, M, S, accumulate, l,
                                      [&](int grid, int, size_t, int64_t, int64_t, int64_t) {
            records += grid;
            return hipSuccess;
        });
        st = check_trace(l, records);
        if (st != TIDE_OK) return st;
        st = check_counts(l, (int64_t)L * S);
        if (st != TIDE_OK) return st;
        hipStream_t stream = reinterpret_cast<hipStream_t>(stream_v);
        const int64_t tiles_per_shard = (S + kLandTile - 1) / kLandTile;
        const int32_t scalar = (l.flags & TIDE_FLAG_SCALAR_PATH) ? 1 : 0;
        if (l.mode == TIDE_LAUNCH_BUDGETED && kBudgetLds > 0 && !(l.flags & TIDE_FLAG_NO_LDS_FENCE)) {
            std::lock_guard<std::mutex> lock(g_landing_lds_mu);
            int dev = 0;
            st = stream_device(stream, &dev);
            if (st != TIDE_OK) return st;
            DeviceGuard guard(dev);
            if (guard.status() != hipSuccess) return hip_fail(guard.status(), "hipSetDevice");
            const int key = M <= 8 ? M : 0;
            const uint64_t bit = (uint64_t)1 << key;
            if (dev < 64 && !(g_landing_lds_done[dev] & bit)) {
                TIDE_HIP_TRY(allow_dynamic_lds_landing(key, kBudgetLds));
                g_landing_lds_done[dev] |= bit;
            }
        }
        TIDE_HIP_TRY(for_each_landing_launch(L, M, S, accumulate, l,
                     [&](int grid, int threads, size_t lds, int64_t lo, int64_t hi, int64_t tb) {
            return launch_landing(M, grid, threads, lds, stream, ptrs, L, S, C, tiles_per_shard,
                                  lo, hi, accumulate, scalar, l.trace, tb, l.write_counts);
        }));
        return TIDE_OK;
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

tide_status tide_rd_schedule(int32_t M, int32_t node, int64_t piece_bytes, int64_t head_bytes,
                             tide_rd_step* steps, int32_t capacity, int32_t* nsteps) {
    if (M < 1) return fail(TIDE_ERR_INVALID_ARG, "M = %d < 1", M);
    if (node < 0 || node >= M) return fail(TIDE_ERR_INVALID_ARG, "node %d outside [0, %d)", node, M);
    if (piece_bytes < 0 || head_bytes < 0) return fail(TIDE_ERR_INVALID_ARG, "negative byte count");
    if (!nsteps) return fail(TIDE_ERR_INVALID_ARG, "nsteps is NULL");
    if (head_bytes == 0) head_bytes = (int64_t)8 << 20;   // 8 MiB of heads (page 1)
    int32_t rounds = 0;
    while (((int64_t)1 << rounds) < M) ++rounds;          // ceil(log2 M)
    if (rounds > 0 && (!steps || capacity < rounds))
        return fail(TIDE_ERR_INVALID_ARG, "capacity %d < %d rounds", capacity, rounds);
    int32_t held = 1;                                      // slots filled: own piece at slot 0
    for (int32_t d = 0; d < rounds; ++d) {
        const int32_t step = 1 << d;
        const int32_t count = std::min(step, M - step);
        int64_t bytes;
        if (!mul_ok(count, piece_bytes, &bytes)) return fail(TIDE_ERR_OVERFLOW, "round bytes overflow");
        tide_rd_step& t = steps[d];
        t.round = d;
        t.send_to = (int32_t)(((int64_t)node - step % M + M) % M);
        t.recv_from = (int32_t)(((int64_t)node + step) % M);
        t.count = count;
        t.send_slot = 0;
        t.recv_slot = held;
        t.head_bytes = std::min(bytes, head_bytes);
        t.tail_bytes = bytes - t.head_bytes;
        held += count;
    }
    *nsteps = rounds;
    return TIDE_OK;
}

const char* tide_status_string(tide_status s) {
    switch (s) {
        case TIDE_OK: return "TIDE_OK";
        case TIDE_ERR_INVALID_ARG: return "TIDE_ERR_INVALID_ARG";
        case TIDE_ERR_ALIGNMENT: return "TIDE_ERR_ALIGNMENT";
        case TIDE_ERR_OVERFLOW: return "TIDE_ERR_OVERFLOW";
        case TIDE_ERR_UNSUPPORTED: return "TIDE_ERR_UNSUPPORTED";
        case TIDE_ERR_NO_MEMORY: return "TIDE_ERR_NO_MEMORY";
        case TIDE_ERR_HIP: return "TIDE_ERR_HIP";
    }
    return "TIDE_ERR_UNKNOWN";
}

const char* tide_last_error_detail(void) { return g_detail.c_str(); }

int32_t tide_version(void) { return (1 << 16) | 0; }

tide_status tide_plan_slot_grads(const tide_plan* plan, uint16_t* const* slots,
                                 const uint16_t** grads) {
    if (!plan || !grads) return fail(TIDE_ERR_INVALID_ARG, "NULL argument");
    if (plan->P > 0 && !slots) return fail(TIDE_ERR_INVALID_ARG, "slots is NULL");
    for (int32_t c = 0; c < plan->L && plan->P > 0; ++c) {
        if (!slots[c]) return fail(TIDE_ERR_INVALID_ARG, "slots[%d] is NULL", c);
        for (int32_t p = 0; p < plan->P; ++p)
            grads[(size_t)c * plan->P + p] = slots[c] + (int64_t)plan->N * plan->prm[p].o;
    }
    return TIDE_OK;
}

tide_status tide_dma_engine_count(int32_t device, int32_t* engines) {
    if (!engines) return fail(TIDE_ERR_INVALID_ARG, "engines is NULL");
    int n = 0;
    if (hipGetDeviceCount(&n) != hipSuccess || device < 0 || device >= n)
        return fail(TIDE_ERR_INVALID_ARG, "device %d is not a HIP device", device);
    std::string err;
    int e = 0;
    tide_status st = dma_engine_count(device, &e, &err);
    if (st != TIDE_OK) return fail(st, "%s", err.c_str());
    *engines = e;
    return TIDE_OK;
}

tide_status tide_plan_event_count(const tide_plan* plan, int64_t* events) {
    if (!plan || !events) return fail(TIDE_ERR_INVALID_ARG, "NULL argument");
    std::lock_guard<std::mutex> lock(plan->mu);
    int64_t n = 0;
    for (const auto& d : plan->devs) {
        n += (int64_t)d->event_pool.size();
        for (const Slot& sl : d->slots) n += (int64_t)sl.readers.size() + (sl.upload_done ? 1 : 0);
    }
    *events = n;
    return TIDE_OK;
}

tide_status tide_plan_trace_records(const tide_plan* plan, int32_t op, const tide_launch* launch,
                                    int64_t* records) {
    try {
        if (!plan || !records) return fail(TIDE_ERR_INVALID_ARG, "NULL argument");
        if (op < 0 || op > 2) return fail(TIDE_ERR_INVALID_ARG, "op %d not 0, 1 or 2", op);
        tide_launch l;
        tide_status st = resolve_launch(plan, launch, &l);
        if (st != TIDE_OK) return st;
        int64_t n = count_tiles(plan, op, l.rank_begin, l.rank_end, l.mode == TIDE_LAUNCH_BUDGETED);
        if (op == 2) n *= plan->L;
        *records = launch_records(plan, op, l, n);
        return TIDE_OK;
    } catch (const std::bad_alloc&) {
        return fail(TIDE_ERR_NO_MEMORY, "host allocation failed");
    } catch (...) {
        return fail(TIDE_ERR_INVALID_ARG, "unexpected exception");
    }
}

tide_status tide_diag_stream(int32_t kind, const void* const* srcs, int32_t nsrc, void* dst,
                             int64_t n, int32_t workgroups, void* stream_v) {
    if (kind < 0 || kind > 3) return fail(TIDE_ERR_INVALID_ARG, "kind %d not in 0..3", kind);
    if (workgroups < 0 || workgroups > kMaxBudgetBlocks)
        return fail(TIDE_ERR_INVALID_ARG, "workgroups = %d not in [0, %d]", workgroups,
                    kMaxBudgetBlocks);
    const int64_t unit = kind == 3 ? (int64_t)kStep : (int64_t)kThreads * 16;
    if (n < 0 || n % unit) return fail(TIDE_ERR_INVALID_ARG, "n = %lld is not a multiple of %lld",
                                       (long long)n, (long long)unit);
    const int need = kind == 1 ? 0 : kind == 3 ? nsrc : 1;
    if (kind == 3 && (nsrc < 1 || nsrc > kStreamMaxSrcs))
        return fail(TIDE_ERR_INVALID_ARG, "nsrc = %d not in [1, %d]", nsrc, kStreamMaxSrcs);
    if (need > 0 && !srcs) return fail(TIDE_ERR_INVALID_ARG, "srcs is NULL");
    StreamSrcs sp{};
    for (int i = 0; i < need; ++i) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(srcs[i]);
        if (!a) return fail(TIDE_ERR_INVALID_ARG, "srcs[%d] is NULL", i);
        if (a & (kind == 3 ? 3 : 15)) return fail(TIDE_ERR_ALIGNMENT, "srcs[%d] misaligned", i);
        sp.p[i] = srcs[i];
    }
    if (!dst) return fail(TIDE_ERR_INVALID_ARG, "dst is NULL");
    if (reinterpret_cast<uintptr_t>(dst) & 15) return fail(TIDE_ERR_ALIGNMENT, "dst is not 16-byte aligned");
    const int64_t units = n / unit;
    if (units == 0) return TIDE_OK;
    const int grid = workgroups > 0 ? workgroups : (int)std::min<int64_t>(units, kFullGridCap);
    TIDE_HIP_TRY(launch_stream(kind, grid, workgroups > 0 ? kFatThreads : kThreads,
                               reinterpret_cast<hipStream_t>(stream_v), sp, kind == 3 ? nsrc : 1,
                               dst, units));
    return TIDE_OK;
}

tide_status tide_diag_occupy(int32_t workgroups, int32_t threads, int32_t lds_bytes,
                             int64_t spin_ticks, tide_trace_rec* trace, void* stream_v) {
    if (workgroups < 1) return fail(TIDE_ERR_INVALID_ARG, "workgroups = %d < 1", workgroups);
    if (threads < 64 || threads > 1024 || threads % 64)
        return fail(TIDE_ERR_INVALID_ARG, "threads = %d is not a multiple of 64 in [64, 1024]", threads);
    if (lds_bytes < 0 || lds_bytes > 160 * 1024)
        return fail(TIDE_ERR_INVALID_ARG, "lds_bytes = %d not in [0, 160 KiB]", lds_bytes);
    if (spin_ticks < 0 || spin_ticks > 100000000)
        return fail(TIDE_ERR_INVALID_ARG, "spin_ticks = %lld not in [0, 1e8]", (long long)spin_ticks);
    if (!trace) return fail(TIDE_ERR_INVALID_ARG, "trace is NULL");
    TIDE_HIP_TRY(launch_occupy(workgroups, threads, (size_t)lds_bytes,
                               reinterpret_cast<hipStream_t>(stream_v), spin_ticks, trace));
    return TIDE_OK;
}

}  // extern "C"
