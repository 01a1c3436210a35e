/*
 * tide.h -- C ABI of a one-GPU (MI355X, gfx950) implementation of two steps of
 * TIDE's layout-aware FSDP2 collectives:
 *
 *   1. the level-1 (node-local) mixed-precision reduce-scatter: L contributor
 *      sets of per-parameter bf16 gradients, read where they lie, summed in
 *      fp32 into zero-padded rank-major fp32 shards
 *      (page 1 "Reduce-scatter: two levels of addition"; page 2 "What shipped";
 *      page 3 abstract and Figure 6(a));
 *   2. the all-gather placement step: rank-major bf16 shards written straight
 *      to their final parameter-major addresses
 *      (page 1 "All-gather: parameters land at their final address";
 *      page 3 Figure 5(b), one strided copy per parameter).
 *
 * Notation (page 3 "Table 2. Notation"): a parameter group of P tensors,
 * N ranks, L contributors. Parameter p has T_p true rows along dim 0 and row
 * length K_p (the product of its remaining dims; 1 for a 1-D tensor). Dim-0
 * sharding gives every rank R_p = ceil(T_p / N) rows, zero-padded past T_p,
 * so rank r's piece of p has s_p = R_p * K_p elements; o_p is the prefix sum
 * of s_q over q < p in the order the parameters were given, and the per-rank
 * shard has S = sum of s_p elements. Rank r's piece of p sits at element
 * r * stride + o_p of a rank-major buffer (the order of page 1's worked
 * example), and holds true rows r * R_p .. min(T_p, (r+1) * R_p) - 1.
 *
 * All sizes and offsets are in ELEMENTS (bf16 or fp32 as stated), 64-bit.
 *
 * Conventions shared by every call:
 *   - Every function returns a tide_status; nothing aborts and no C++
 *     exception crosses this boundary. On a non-OK status,
 *     tide_last_error_detail() gives a thread-local description.
 *   - All argument checks happen on the host before anything is enqueued: a
 *     call that fails has enqueued nothing.
 *   - Device buffers are owned by the caller and must stay alive until the
 *     stream has executed the call. The library owns the plan and the small
 *     device tables it creates for it (freed by tide_plan_destroy).
 *   - Pointer arrays (grads, params) are host arrays, read during the call
 *     only. The pointers in them are device pointers.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream). The
 *     device used is the stream's device. The compute calls only enqueue,
 *     except that the first call of a plan on a device, and the first for
 *     each (operation, launch mode, rank range), builds the plan's small
 *     device tables there with a synchronous allocation and upload (kept up
 *     to 256 per device; past that, the least recently used one that no
 *     prepared call holds is freed after the device has drained). The
 *     TIDE_ENGINE_SDMA path is host-synchronous (see tide_engine).
 *   - A plan may be used from several threads and streams at once; it is
 *     immutable after creation except for internally locked caches.
 */
#ifndef TIDE_H
#define TIDE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct tide_plan tide_plan;

typedef enum tide_status {
    TIDE_OK = 0,
    TIDE_ERR_INVALID_ARG = 1,   /* null/negative/out-of-range argument, overlapping buffers */
    TIDE_ERR_ALIGNMENT = 2,     /* bf16 pointer not 2-byte aligned, fp32 pointer not 4-byte aligned */
    TIDE_ERR_OVERFLOW = 3,      /* a size or offset does not fit int64 */
    TIDE_ERR_UNSUPPORTED = 4,   /* valid request this library does not serve; caller falls back */
    TIDE_ERR_NO_MEMORY = 5,     /* host or device allocation failed */
    TIDE_ERR_HIP = 6            /* a HIP runtime call failed (no GPU, bad stream, launch error) */
} tide_status;

/* Data-movement engine of the placement and the Slot-Reuse staging (page 1:
 * the all-gather's data movement runs on copy engines and uses no compute
 * units; page 3 Table 1, all-gather SM budget 0; page 3 Figure 2(b) step 4,
 * copy-engine staging of bf16 slices). */
typedef enum tide_engine {
    TIDE_ENGINE_KERNEL = 0,     /* this library's HIP kernels */
    TIDE_ENGINE_RUNTIME = 1,    /* HIP runtime device-to-device copies (placement: one
                                   hipMemcpy2DAsync per parameter, +1 for a partial rank;
                                   staging: one hipMemcpyAsync per contributor and
                                   parameter). The runtime runs these as its own blit
                                   kernels, so they occupy compute units too. */
    TIDE_ENGINE_SDMA = 2        /* the GPU's DMA (SDMA) engines through the HSA runtime,
                                   no compute units: one linear copy per piece (placement:
                                   per parameter and rank; staging: per contributor and
                                   parameter), spread over every engine the device offers
                                   for copies inside its memory (14 on MI355X, about
                                   60 GB/s each). Host-synchronous: the call waits for the
                                   work already enqueued on `stream`, runs the copies and
                                   returns once all have completed; it fails with
                                   TIDE_ERR_HIP if they have not completed within
                                   10 s + 1 s per GB copied, and with TIDE_ERR_UNSUPPORTED
                                   on a capturing stream or a device without such engines.
                                   Only launch.rank_begin / rank_end apply. */
} tide_engine;

typedef enum tide_launch_mode {
    TIDE_LAUNCH_FULL = 0,       /* enough workgroups to fill the GPU */
    TIDE_LAUNCH_BUDGETED = 1    /* few, short-lived workgroups (page 1 "Why does a communication
                                   kernel slow a matrix multiply by 69%?": 16 summing + 4 landing
                                   blocks, single blocks, each living 0.2-0.4 ms) */
} tide_launch_mode;

/* One workgroup of a traced launch (the analog of the pages' SM-id probe,
 * page 3 Figure 3 and Table 5): where it ran and for how long. */
typedef struct tide_trace_rec {
    uint32_t hw_id;          /* HW_ID hardware register of the workgroup's first wave
                                (bits 8-11 CU, 12 shader array, 13-15 shader engine) */
    uint32_t xcc_id;         /* XCC_ID hardware register (bits 0-3: the accelerator die) */
    uint64_t t_begin;        /* constant-rate real-time counter when the workgroup started */
    uint64_t t_end;          /* same, once all of its waves had finished their work */
} tide_trace_rec;

/* Graph capture. The eager reduce-scatter, and the eager placement and
 * staging with the kernel engine, read a per-call pointer table from a small
 * ring the library reuses; a captured graph would replay against whatever the
 * ring holds by then. On a capturing stream these calls return
 * TIDE_ERR_UNSUPPORTED before enqueuing anything. Prepared calls
 * (tide_call_enqueue), the runtime-copy engine, the landing sum and the
 * diagnostic occupant keep everything they read fixed and may be captured. */

/* Launch options. A zero-filled struct (or a NULL pointer) means: full grid,
 * all ranks. Fields equal to 0 take their defaults. */
typedef struct tide_launch {
    int32_t mode;            /* tide_launch_mode */
    int32_t reduce_blocks;   /* BUDGETED: workgroups of each reduce launch (0 -> 16; at most 65536) */
    int32_t place_blocks;    /* BUDGETED: workgroups of each placement or landing launch (0 -> 4;
                                at most 65536) */
    int32_t max_launch_us;   /* BUDGETED: work per launch sized so a workgroup lives about
                                this long (0 -> 50). Each launch is a separate kernel; no
                                workgroup ever waits on another. A GEMM that fills the GPU
                                with one workgroup per CU slows by about this life over its
                                own duration (each CU a collective workgroup holds delays
                                one of its workgroups until then). */
    int32_t rank_begin;      /* first rank whose shard is processed (default 0) */
    int32_t rank_end;        /* one past the last rank; 0 -> N */
    int32_t flags;           /* TIDE_FLAG_* */
    int32_t reserved;        /* must be 0 */
    tide_trace_rec* trace;   /* optional device array: when set, every workgroup of every launch
                                of the call writes one record, launches in order, workgroups in
                                blockIdx order (tide_plan_trace_records gives the count) */
    int64_t trace_capacity;  /* records `trace` holds; a call that needs more fails with
                                INVALID_ARG before enqueuing anything */
    uint32_t* write_counts;  /* optional device array (debug): every element the call writes adds
                                one (atomically) at its index, so a test can check that each
                                output element lands exactly once. Indices: reduce-scatter
                                r * out_stride + o_p + j (N * out_stride entries); placement
                                N * o_p + f, f the element of parameter p (N * S entries);
                                staging c * N * S + N * o_p + f (L * N * S entries); landing
                                b * S + f (L * S entries). Kernel engine only. */
    int64_t write_counts_elems; /* entries `write_counts` holds; fewer than the call needs is
                                INVALID_ARG */
} tide_launch;

/* Force the element-at-a-time path everywhere (for testing the slow path). */
#define TIDE_FLAG_SCALAR_PATH 0x1
/* BUDGETED: launch without the LDS reservation that keeps other kernels'
 * workgroups off the CUs a budgeted workgroup holds (for measuring its effect). */
#define TIDE_FLAG_NO_LDS_FENCE 0x2

/*
 * Build the layout of one parameter group (page 3 Table 2 notation).
 *   rows[p]    = T_p >= 0 true dim-0 rows of parameter p (P entries)
 *   row_len[p] = K_p >= 1 (P entries)
 *   P >= 0 parameters (no upper cap: groups of several hundred tensors are served),
 *   N >= 1 ranks, L >= 1 contributors (L <= 64).
 * Host-only: allocates nothing on the GPU (device tables are made on first use
 * on each device). *out_plan receives a plan to free with tide_plan_destroy.
 * Errors: INVALID_ARG (bad counts, null arrays when P > 0), OVERFLOW (N*S or a
 * per-parameter size beyond int64), NO_MEMORY.
 */
tide_status tide_plan_create(const int64_t* rows, const int64_t* row_len, int32_t P,
                             int32_t N, int32_t L, tide_plan** out_plan);

/* Free a plan and its device tables. NULL-safe. No call using it may be in flight. */
void tide_plan_destroy(tide_plan* plan);

/* Group dimensions: P, N, L and S (per-rank shard elements). Any out pointer may be NULL. */
tide_status tide_plan_dims(const tide_plan* plan, int32_t* P, int32_t* N, int32_t* L, int64_t* S);

/* Per-parameter layout (page 3 Table 2): T_p, K_p, R_p, s_p, o_p in elements.
 * Any out pointer may be NULL. INVALID_ARG if p is out of range. */
tide_status tide_plan_param(const tide_plan* plan, int32_t p, int64_t* rows, int64_t* row_len,
                            int64_t* R_p, int64_t* s_p, int64_t* o_p);

/* The two addressings of rank r's piece of parameter p (page 1 worked example):
 *   rank_major  = r * S + o_p            start in a packed rank-major buffer
 *   param_major = N * o_p + r * s_p      start in the group's parameters laid end to
 *                                        end, each padded to N * R_p rows
 *   valid       = true elements in the piece (s_p minus its zero padding)
 * Any out pointer may be NULL. */
tide_status tide_plan_map(const tide_plan* plan, int32_t r, int32_t p, int64_t* rank_major,
                          int64_t* param_major, int64_t* valid);

/*
 * Level-1 reduce-scatter, bf16 in, fp32 out.
 *   grads[c * P + p]: device pointer to contributor c's bf16 gradient of parameter
 *       p, T_p x K_p contiguous, 2-byte aligned (may be NULL when T_p * K_p == 0).
 *       Read only; gradients are read in place, with no packed copy. Speed:
 *       gradients are read with vector loads; one that starts at 2 mod 4 bytes
 *       (a view at an odd element offset) with dword-aligned loads and a
 *       16-bit funnel shift, which also read, and discard, the 2 bytes before
 *       its first element and after its last that share their aligned dwords.
 *       A parameter with such a gradient from contributor 24 or later is
 *       summed element by element. Every path gives the same result.
 *   out: device pointer to N fp32 shards; shard r starts at out + r * out_stride
 *       (out_stride >= S), 4-byte aligned; the buffer must span
 *       (N - 1) * out_stride + S elements.
 * For every rank r in [rank_begin, rank_end), every element of out[r][0..S) is
 * written exactly once: the fp32 sum over c = 0..L-1, in that order (a left
 * fold, binary32 round-to-nearest-even, subnormals kept), of the widened bf16
 * values of the element's true row, or +0.0f for a padded row. Elements
 * out[r][S..out_stride) and shards outside the range are not touched.
 * The inputs must not overlap the written output (INVALID_ARG).
 * Uses one small per-call table uploaded with an async host-to-device copy on
 * `stream` (skipped when the pointers equal the previous call's).
 */
tide_status tide_reduce_scatter_bf16_fp32(const tide_plan* plan, const uint16_t* const* grads,
                                          float* out, int64_t out_stride, void* stream,
                                          const tide_launch* launch);

/*
 * The level-1 reduce-scatter of tide_reduce_scatter_bf16_fp32, for callers
 * that cannot allocate device memory (code under graph capture, tight serving
 * loops, harnesses that forbid allocation): it calls no hipMalloc, hipFree or
 * other allocating routine, on any call. Same arguments, checks and result,
 * bit for bit, as tide_reduce_scatter_bf16_fp32 (sharing its kernel).
 *   - Its per-call tables (per-parameter layout, the tile prefix, the L * P
 *     gradient pointers and flags) live in a fixed 1 MiB device array of the
 *     library, one per GPU, held until the process ends. A group whose tables
 *     need more (about P * (44 + 8 L) bytes) is refused with
 *     TIDE_ERR_INVALID_ARG before anything is enqueued.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's tables: calls that overlap on one GPU (different streams, or
 *     different host threads with no ordering between them) race. Calls
 *     ordered on one stream do not.
 *   - The tables are uploaded with a host-to-device copy on `stream` from
 *     pageable memory, which the runtime performs synchronously; the upload
 *     is skipped when they equal what the array already holds.
 *   - Tiles are walked in parameter order (the eager call groups small pieces
 *     rank by rank), so small-piece groups may run a little slower.
 *   - A capturing stream is refused (TIDE_ERR_UNSUPPORTED).
 */
tide_status tide_reduce_scatter_bf16_fp32_noalloc(const tide_plan* plan,
                                                  const uint16_t* const* grads, float* out,
                                                  int64_t out_stride, void* stream,
                                                  const tide_launch* launch);

/*
 * All-gather placement, bf16.
 *   shards: device pointer to N rank-major bf16 shards, shard r at
 *       shards + r * shard_stride (shard_stride >= S), 2-byte aligned. Read only;
 *       the buffer must span (N - 1) * shard_stride + S elements. The kernel
 *       engine's realigning loads of a piece at 2 mod 4 bytes may also read,
 *       and discard, the one element before and the one after the piece, always
 *       inside that span; nothing else outside the pieces is read.
 *   params[p]: device pointer to parameter p's storage, T_p x K_p contiguous,
 *       2-byte aligned (may be NULL when T_p * K_p == 0). Speed: a parameter
 *       is written with 16-byte stores only when params[p] is 16-byte aligned;
 *       otherwise element by element, with the same bytes.
 * For every rank r in [rank_begin, rank_end), the true rows of rank r's piece
 * of every parameter are copied bit for bit to rows r * R_p.. of params[p];
 * padded rows are not written, and nothing else in params is touched.
 * engine: TIDE_ENGINE_KERNEL (this library's kernel; asynchronous on `stream`),
 * TIDE_ENGINE_RUNTIME (one hipMemcpy2DAsync per parameter; asynchronous) or
 * TIDE_ENGINE_SDMA (one DMA-engine copy per piece, no compute units;
 * host-synchronous, see tide_engine). All three write the same bytes. The
 * parameters must not overlap each other or the shards read.
 */
tide_status tide_allgather_place(const tide_plan* plan, const uint16_t* shards,
                                 int64_t shard_stride, uint16_t* const* params, void* stream,
                                 int32_t engine, const tide_launch* launch);

/*
 * All-gather placement from a stage buffer in arrival order. After the
 * recursive-doubling exchange (page 1 "All-gather: parameters land at their
 * final address"; page 3 Figure 5), node n holds the shards of nodes n,
 * n+1, ... (mod M) in its stage slots 0, 1, ...; with L ranks per node the
 * shard of rank r sits at stage position (r - first_rank) mod N with
 * first_rank = n * L. Same contract as tide_allgather_place, whose call is this
 * one with first_rank = 0 (first_rank must lie in [0, N)).
 */
tide_status tide_allgather_place_stage(const tide_plan* plan, const uint16_t* stage,
                                       int64_t shard_stride, int32_t first_rank,
                                       uint16_t* const* params, void* stream, int32_t engine,
                                       const tide_launch* launch);

/*
 * Slot-Reuse staging (page 1 "When gradients can be freed also needs
 * planning"; page 2 "What shipped"; page 3 abstract and Figure 7): copy each
 * contributor's bf16 gradients into an all-gather slot whose last use is over,
 * so that the gradient storage can be released as soon as the copy has run;
 * the level-1 reduce then reads the slot instead of the gradients.
 *
 *   grads:  L * P bf16 pointers, grads[c * P + p], as for
 *           tide_reduce_scatter_bf16_fp32 (T_p x K_p row-major, 2-byte aligned).
 *   slots:  L device pointers (2-byte aligned); slots[c] is contributor c's slot
 *           of N * S bf16 elements, the size of the group's gathered
 *           parameters. Parameter p goes to slots[c] + N * o_p, its place in the
 *           group's parameter-major padded layout (tide_plan_map's param_major
 *           at rank 0), rows in order; the padding rows after it are not
 *           written. The reduce then reads the table tide_plan_slot_grads
 *           builds (grads'[c * P + p] = slots[c] + N * o_p).
 *   engine: TIDE_ENGINE_KERNEL: one copy kernel for all (c, p), 16-byte
 *           accesses when every pointer of a parameter is 4-byte aligned;
 *           TIDE_ENGINE_RUNTIME: one hipMemcpyAsync per (c, p);
 *           TIDE_ENGINE_SDMA: the same copies on the DMA engines, spread over
 *           all of them, leaving the compute units free; host-synchronous
 *           (see tide_engine).
 *   launch: rank_begin / rank_end restrict the copy to those ranks' rows (rank r
 *           holds rows [r R_p, (r + 1) R_p)), so staging and the reduce can be
 *           pipelined by rank range; FULL, or BUDGETED with place_blocks
 *           workgroups per launch.
 * Ordering: asynchronous on `stream`. The gradients may be released once work
 * ordered after this call on `stream` may run (an event recorded after it, or
 * a stream-ordered allocator's release on `stream`). The slot must not be
 * refilled by the next all-gather before the reduce that reads it has run.
 * The slots, and the gradient bytes read, are owned by the caller.
 * Errors: INVALID_ARG (NULL pointer with work to do, slots overlapping one
 * another or any gradient, unknown engine); ALIGNMENT (odd address);
 * HIP (a launch or copy failed).
 */
tide_status tide_stage_grads_bf16(const tide_plan* plan, const uint16_t* const* grads,
                                  uint16_t* const* slots, void* stream, int32_t engine,
                                  const tide_launch* launch);

/*
 * The reduce-scatter's gradient table for gradients staged into slots by
 * tide_stage_grads_bf16: grads[c * P + p] = slots[c] + N * o_p (L * P entries,
 * a caller array). slots: L device pointers. Host-only; no pointer is
 * dereferenced. Errors: INVALID_ARG (NULL arrays or slot pointers).
 */
tide_status tide_plan_slot_grads(const tide_plan* plan, uint16_t* const* slots,
                                 const uint16_t** grads);

/*
 * DMA engines TIDE_ENGINE_SDMA spreads its copies over on HIP device `device`
 * (queried from the HSA runtime on first use, then cached). Host-only.
 * Errors: INVALID_ARG (not a device), UNSUPPORTED (no such engines, or the HSA
 * agent of the device cannot be identified).
 */
tide_status tide_dma_engine_count(int32_t device, int32_t* engines);

/*
 * Prepared calls. A training step issues the same collectives on the same
 * buffers every time; a prepared call validates those buffers once, copies
 * its pointer table to a device allocation of its own, and is then enqueued
 * with no host-side table work at all. Because its table never changes,
 * tide_call_enqueue may be captured into a HIP graph and replayed.
 *   - The tide_prepare_* calls take the same arguments as the eager calls
 *     (kernel engine only), validate them the same way, and build the call on
 *     the current HIP device. They allocate (device table, the plan's
 *     per-device tables on first use) and copy synchronously.
 *   - tide_call_enqueue(call, stream): stream must be on the call's device.
 *     Launches the call's kernels, nothing else; allocates nothing; may be
 *     captured. The buffers given at preparation must still be valid, and
 *     their contents are read or written at the time the work runs.
 *   - tide_call_destroy: frees the device table (NULL-safe). Destroy a call
 *     after the work it enqueued has completed, and before its plan.
 */
typedef struct tide_call tide_call;

tide_status tide_prepare_reduce_scatter_bf16_fp32(const tide_plan* plan,
                                                  const uint16_t* const* grads, float* out,
                                                  int64_t out_stride, const tide_launch* launch,
                                                  tide_call** call);
tide_status tide_prepare_allgather_place_stage(const tide_plan* plan, const uint16_t* shards,
                                               int64_t shard_stride, int32_t first_rank,
                                               uint16_t* const* params, const tide_launch* launch,
                                               tide_call** call);
tide_status tide_prepare_stage_grads_bf16(const tide_plan* plan, const uint16_t* const* grads,
                                          uint16_t* const* slots, const tide_launch* launch,
                                          tide_call** call);
tide_status tide_call_enqueue(const tide_call* call, void* stream);
void tide_call_destroy(tide_call* call);

/* One round of node n's recursive-doubling all-gather schedule. */
typedef struct tide_rd_step {
    int32_t round;        /* d = 0, 1, ... */
    int32_t send_to;      /* node (n - 2^d) mod M */
    int32_t recv_from;    /* node (n + 2^d) mod M */
    int32_t count;        /* pieces sent and received: min(2^d, M - 2^d) */
    int32_t send_slot;    /* first stage slot sent (slots send_slot .. send_slot + count - 1) */
    int32_t recv_slot;    /* first stage slot the received pieces fill */
    int64_t head_bytes;   /* head of this round's send: min(count * piece_bytes, head limit) */
    int64_t tail_bytes;   /* the rest of the send */
} tide_rd_step;

/*
 * Node `node`'s recursive-doubling all-gather schedule over M nodes (page 1
 * "All-gather: parameters land at their final address"; page 3 Figure 5(a)).
 * In round d the node sends the first min(2^d, M - 2^d) pieces it holds to
 * node n - 2^d and receives as many from node n + 2^d (mod M); there are
 * ceil(log2 M) rounds, and no piece arrives twice. Stage slot k ends up
 * holding node (n + k) mod M's piece. Each round's send is split into a head
 * of at most head_bytes (0 -> 8 MiB) and a tail, for pacing.
 *   steps: caller array of `capacity` entries (capacity >= ceil(log2 M));
 *   *nsteps receives the round count. Host-only.
 * Errors: INVALID_ARG (M < 1, node outside [0, M), piece_bytes < 0,
 * head_bytes < 0, capacity too small, NULL pointers).
 */
tide_status tide_rd_schedule(int32_t M, int32_t node, int64_t piece_bytes, int64_t head_bytes,
                             tide_rd_step* steps, int32_t capacity, int32_t* nsteps);

/*
 * Level 2 of the reduce-scatter on one destination node: the landing sum
 * (page 1 "Reduce-scatter: two levels of addition, the last one done by
 * NVSwitch"; page 3 Figure 6(b)). Plan-free; one call covers the node's L GPUs.
 *
 * Every GPU b of the node finally holds an fp32 shard of S elements. A source
 * node's fp32 partial of the node's part is cut into L slices: slice s is the
 * s-th chunk of C = ceil(S / L) elements of every local shard, one block per
 * GPU b. A source with relative index c = (destination - source) mod M sends
 * slice s to GPU (s - c) mod L (the Latin-square seating, tide_latin_square),
 * so the M copies of a slice sit on M different GPUs at the same offset.
 *   inboxes[g] (g < L): device pointer to GPU g's inbox, L slots x L blocks x C
 *       fp32; slot s, block b starts at element (s * L + b) * C. 4-byte aligned.
 *       Only slots that a source with c < M filled are read. Read only.
 *   shards[b] (b < L): device pointer to GPU b's fp32 shard (S elements), 4-byte
 *       aligned; must not overlap any inbox or another shard.
 *   1 <= M <= L <= 64 sources (batches of at most L sources: call once per
 *   batch with accumulate = 1 after the first).
 * shards[b][s * C + e] = fold_{c = 0..M-1} inboxes[(s - c) mod L][(s * L + b) * C + e]
 * as a left fold in source order (binary32 round-to-nearest-even); with
 * accumulate = 1 the fold is then added to the shard's current value.
 * launch: FULL or BUDGETED (place_blocks workgroups: the pages' 4 landing
 * blocks); rank_begin / rank_end must be 0. Async on `stream`; allocates nothing.
 */
tide_status tide_landing_sum_fp32(int32_t L, int32_t M, int64_t S, const float* const* inboxes,
                                  float* const* shards, int32_t accumulate, void* stream,
                                  const tide_launch* launch);

/*
 * The Latin-square seating for one (destination, source) node pair (page 1,
 * the 4-GPU hand calculation; page 3 Figure 6(b)): *c = (dst - src) mod M;
 * slice_of_src_gpu[j] = (j + c) mod L, the slice source GPU j handles and sends
 * over rail j; dst_gpu_of_slice[s] = (s - c) mod L, the destination GPU slice s
 * lands on. Arrays of L entries (may be NULL). Host-only.
 */
tide_status tide_latin_square(int32_t M, int32_t L, int32_t dst_node, int32_t src_node, int32_t* c,
                              int32_t* slice_of_src_gpu, int32_t* dst_gpu_of_slice);

/* Kernel launches a call with these options makes (op 0 = reduce-scatter,
 * 1 = placement with the kernel engine, 2 = Slot-Reuse staging with the
 * kernel engine). Host-only. */
tide_status tide_plan_launch_count(const tide_plan* plan, int32_t op, const tide_launch* launch,
                                   int64_t* launches);

/* Trace records (workgroups) a call with these options launches, for op 0
 * (reduce-scatter), 1 (placement, kernel engine) or 2 (staging, kernel engine).
 * Host-only. */
tide_status tide_plan_trace_records(const tide_plan* plan, int32_t op, const tide_launch* launch,
                                    int64_t* records);

/* Trace records (workgroups) tide_landing_sum_fp32 launches with these
 * arguments. Host-only. */
tide_status tide_landing_trace_records(int32_t L, int32_t M, int64_t S, int32_t accumulate,
                                       const tide_launch* launch, int64_t* records);

/*
 * Diagnostic occupant: `workgroups` workgroups of `threads` threads, each
 * reserving `lds_bytes` of LDS, each waiting `spin_ticks` ticks of the
 * real-time counter (a bounded wait: it ends when the counter has advanced
 * that far) and writing one tide_trace_rec to trace[blockIdx]. Launched beside
 * a budgeted collective, its records show whether a workgroup shaped like a
 * GEMM's (page 3 Figure 3: one wave of 256x8192x8192) lands on a CU that a
 * collective workgroup holds. threads: a multiple of 64 in [64, 1024];
 * lds_bytes <= 160 KiB; spin_ticks in [0, 10^8]; trace: device array of at
 * least `workgroups` records. Async on `stream`.
 * Errors: INVALID_ARG (out-of-range argument, NULL trace); HIP.
 */
tide_status tide_diag_occupy(int32_t workgroups, int32_t threads, int32_t lds_bytes,
                             int64_t spin_ticks, tide_trace_rec* trace, void* stream);

/*
 * Diagnostic bandwidth ceilings: the access patterns of the path with no
 * layout logic, in this library's own kernels (128-thread workgroups,
 * non-temporal accesses), for timing against the real kernels.
 *   kind 0: read n bytes from srcs[0] (16-byte aligned; dst receives nothing
 *           in practice but must be a valid 16-byte-aligned device pointer);
 *   kind 1: write n bytes of zeros to dst;
 *   kind 2: copy n bytes from srcs[0] to dst;
 *   kind 3: the reduce's pattern: dst[i] = sum over c < nsrc, in order, of the
 *           widened bf16 srcs[c][i], for i < n (n elements; srcs 4-byte
 *           aligned, nsrc in [1, 8]; dst holds n fp32).
 * n is a multiple of 2048 (kinds 0-2, bytes) or 1024 (kind 3, elements).
 * workgroups = 0: a full grid of 128-thread workgroups (the full-grid
 * kernels' shape); > 0: that many 1024-thread workgroups, the budgeted
 * kernels' shape (with fewer workgroups than CUs the dispatcher spreads them
 * one to a CU, so the rate per workgroup is the per-CU ceiling).
 * Async on `stream`. Errors: INVALID_ARG, ALIGNMENT, HIP.
 */
tide_status tide_diag_stream(int32_t kind, const void* const* srcs, int32_t nsrc, void* dst,
                             int64_t n, int32_t workgroups, void* stream);

/* HIP events the plan holds across its devices: per-call table uploads, the
 * readers of each table slot (one per stream with pending work), and the pool
 * of spare events. Bounded by the ring size and the number of streams in use,
 * not by the number of calls. Host-only (diagnostic). */
tide_status tide_plan_event_count(const tide_plan* plan, int64_t* events);

/* Static text for a status code. */
const char* tide_status_string(tide_status status);

/* Thread-local description of the last non-OK status returned on this thread. */
const char* tide_last_error_detail(void);

/* Library ABI version, (major << 16) | minor. */
int32_t tide_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TIDE_H */
