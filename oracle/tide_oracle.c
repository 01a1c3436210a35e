/*
 * tide_oracle.c -- plain, slow, CPU reference of the layout-aware
 * mixed-precision reduce-scatter (node-local level) and of the all-gather
 * placement step of TIDE, written from the pages that describe it.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path links, loads or calls
 * this file: only the tests, the package's smoke check and the benchmark's
 * CPU-baseline leg do. It shares no code, header, table or helper with the HIP
 * library; it derives the layout again from the parameter list on every call.
 *
 * What it computes (all sizes in elements, all offsets 64-bit):
 *
 *   Notation, page 3 "Table 2. Notation": N ranks, P parameters, parameter p
 *   has padded per-rank rows R_p of row length K_p, per-rank shard size s_p
 *   and prefix offset o_p; S is the per-rank packed shard size.
 *
 *   Layout. Parameter p has T_p true dim-0 rows. FSDP2 slices every
 *   parameter along dim 0 and zero-pads it (page 1, "What problem is it
 *   actually solving?"); dim-0 chunking gives every rank R_p = ceil(T_p / N)
 *   rows, so s_p = R_p * K_p, o_p = sum of s_q over q < p in list order (no
 *   alignment padding: the worked example on page 1 uses the plain prefix
 *   sum), and S = sum of s_p. Rank r's shard is the concatenation of rank r's
 *   pieces of every parameter, and the shards follow one another in rank
 *   order (page 1 "What problem is it actually solving?": the collective
 *   library's flat buffers are ordered by rank). Local row i of rank r holds true row t = r * R_p + i.
 *
 *   Reduce-scatter, level 1. Every contributor c = 0..L-1 holds a bf16
 *   gradient of every parameter (T_p x K_p, contiguous). The output element
 *   of (r, p, i, k) is the fp32 sum of the L contributors' bf16 values of
 *   row t, column k, when t < T_p, and +0.0f when t >= T_p (a padded row).
 *   The pages have each owner sum its L staged bf16 copies into one fp32 copy
 *   (page 1 "Reduce-scatter: two levels of addition"; page 2 "What shipped";
 *   page 3 abstract); the order of that sum is not stated, and this oracle
 *   takes a left fold in contributor order: acc = f32(g_0), then
 *   acc = acc + f32(g_c) for c = 1..L-1, each add binary32 round-to-nearest-
 *   even, subnormals kept. bf16 -> fp32 is the exact widening (bits << 16).
 *   At L = 1 this is the stock path's result: each rank's rows sliced out,
 *   zero-padded, widened to fp32 and packed (page 1).
 *
 *   All-gather placement. Rank r's piece of parameter p, read from the
 *   rank-major buffer at r * stride + o_p, lands at the parameter's own
 *   storage at row r * R_p (page 1 "All-gather: parameters land at their final
 *   address"; page 3 Figure 5(b), one strided copy per parameter). Padded rows
 *   (t >= T_p) are not written; it is a 16-bit copy.
 *
 * Build: cc -O2 -ffp-contract=off -std=c11 -fPIC -shared (no -ffast-math, so
 * no flush-to-zero and no reassociation).
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* Exact bf16 -> fp32 widening: a bf16 value is the top half of a binary32. */
static float widen_bf16(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/*
 * Layout of one parameter group (Table 2 notation). Returns 0 on success,
 * -1 on invalid input (N < 1, P < 0, T_p < 0, K_p < 1) or int64 overflow.
 * R, s, o receive P entries each; *S the per-rank packed size.
 */
int oracle_layout(int32_t P, const int64_t *rows, const int64_t *row_len, int32_t N,
                  int64_t *R, int64_t *s, int64_t *o, int64_t *S)
{
    int64_t acc = 0;
    if (P < 0 || N < 1)
        return -1;
    for (int32_t p = 0; p < P; ++p) {
        int64_t Rp, sp;
        if (rows[p] < 0 || row_len[p] < 1)
            return -1;
        Rp = rows[p] / N + (rows[p] % N != 0);      /* ceil(T_p / N) */
        if (__builtin_mul_overflow(Rp, row_len[p], &sp))
            return -1;
        R[p] = Rp;
        s[p] = sp;
        o[p] = acc;
        if (__builtin_add_overflow(acc, sp, &acc))
            return -1;
    }
    *S = acc;
    return 0;
}

/* Scratch copy of the layout, so each entry point stands alone. */
struct layout {
    int64_t *R, *s, *o;
    int64_t S;
};

static int layout_alloc(struct layout *lay, int32_t P, const int64_t *rows,
                        const int64_t *row_len, int32_t N)
{
    size_t n = (size_t)(P > 0 ? P : 1);
    lay->R = (int64_t *)calloc(n, sizeof(int64_t));
    lay->s = (int64_t *)calloc(n, sizeof(int64_t));
    lay->o = (int64_t *)calloc(n, sizeof(int64_t));
    if (!lay->R || !lay->s || !lay->o)
        return -1;
    return oracle_layout(P, rows, row_len, N, lay->R, lay->s, lay->o, &lay->S);
}

static void layout_free(struct layout *lay)
{
    free(lay->R);
    free(lay->s);
    free(lay->o);
}

/*
 * Starts of rank r's piece of parameter p in the three addressings the pages
 * contrast (page 1 worked example; page 3 Figure 1):
 *   rank_major        = r * S + o_p          (offset in the flat rank-major buffer)
 *   param_major       = r * s_p              (offset inside parameter p's padded storage)
 *   param_major_group = N * o_p + r * s_p    (offset in the group's parameters
 *                                             laid end to end, each padded to N * R_p rows)
 */
int oracle_piece_start(int32_t P, const int64_t *rows, const int64_t *row_len, int32_t N,
                       int32_t r, int32_t p, int64_t *rank_major, int64_t *param_major,
                       int64_t *param_major_group)
{
    struct layout lay;
    int rc = layout_alloc(&lay, P, rows, row_len, N);
    if (rc == 0 && (r < 0 || r >= N || p < 0 || p >= P))
        rc = -1;
    if (rc == 0) {
        *rank_major = (int64_t)r * lay.S + lay.o[p];
        *param_major = (int64_t)r * lay.s[p];
        *param_major_group = (int64_t)N * lay.o[p] + (int64_t)r * lay.s[p];
    }
    layout_free(&lay);
    return rc;
}

/*
 * Level-1 reduce-scatter of L contributors into N rank-major fp32 shards.
 *   grads[c * P + p]  contributor c's bf16 gradient of parameter p (T_p x K_p)
 *   out               fp32, shard r starts at out + r * out_stride
 * Only shards rank_begin <= r < rank_end are written. If write_count is not
 * NULL, write_count[d] is incremented for every output element d written.
 */
int oracle_reduce_scatter(int32_t P, const int64_t *rows, const int64_t *row_len,
                          int32_t N, int32_t L, const uint16_t *const *grads,
                          float *out, int64_t out_stride, int32_t rank_begin,
                          int32_t rank_end, uint32_t *write_count)
{
    struct layout lay;
    int rc = layout_alloc(&lay, P, rows, row_len, N);
    if (rc == 0 && (L < 1 || out_stride < lay.S || rank_begin < 0 ||
                    rank_end > N || rank_begin > rank_end))
        rc = -1;
    if (rc != 0) {
        layout_free(&lay);
        return rc;
    }
    for (int32_t r = rank_begin; r < rank_end; ++r) {
        for (int32_t p = 0; p < P; ++p) {
            const int64_t T = rows[p], K = row_len[p], Rp = lay.R[p];
            for (int64_t i = 0; i < Rp; ++i) {
                const int64_t t = (int64_t)r * Rp + i;     /* true row at local row i */
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t d = (int64_t)r * out_stride + lay.o[p] + i * K + k;
                    float v;
                    if (t < T) {
                        v = widen_bf16(grads[0 * (int64_t)P + p][t * K + k]);
                        for (int32_t c = 1; c < L; ++c)
                            v = v + widen_bf16(grads[(int64_t)c * P + p][t * K + k]);
                    } else {
                        v = 0.0f;                             /* zero-padded row */
                    }
                    out[d] = v;
                    if (write_count)
                        write_count[d] += 1;
                }
            }
        }
    }
    layout_free(&lay);
    return 0;
}

/*
 * First true row and number of true rows of rank r's piece of parameter p
 * (rows r * R_p .. r * R_p + nrows - 1; nrows may be 0 for an all-padding piece).
 */
int oracle_piece_rows(int32_t P, const int64_t *rows, const int64_t *row_len, int32_t N,
                      int32_t r, int32_t p, int64_t *first_row, int64_t *nrows)
{
    struct layout lay;
    int rc = layout_alloc(&lay, P, rows, row_len, N);
    if (rc == 0 && (r < 0 || r >= N || p < 0 || p >= P))
        rc = -1;
    if (rc == 0) {
        int64_t first = (int64_t)r * lay.R[p];
        int64_t n = rows[p] - first;
        if (n < 0)
            n = 0;
        if (n > lay.R[p])
            n = lay.R[p];
        *first_row = first;
        *nrows = n;
    }
    layout_free(&lay);
    return rc;
}

/*
 * One piece of the reduce-scatter, from inputs that hold only that piece's
 * true rows: rank_rows[c] points at contributor c's row r * R_p of parameter p.
 * dst receives the s_p fp32 elements of the piece (true rows summed, padded
 * rows +0.0f). Used to check samples of very large groups one piece at a time.
 */
int oracle_reduce_piece(int32_t P, const int64_t *rows, const int64_t *row_len, int32_t N,
                        int32_t L, int32_t r, int32_t p, const uint16_t *const *rank_rows,
                        float *dst)
{
    int64_t first = 0, n = 0;
    struct layout lay;
    int rc = oracle_piece_rows(P, rows, row_len, N, r, p, &first, &n);
    if (rc != 0 || L < 1)
        return -1;
    if (layout_alloc(&lay, P, rows, row_len, N) != 0) {
        layout_free(&lay);
        return -1;
    }
    {
        const int64_t K = row_len[p];
        const int64_t Rp = lay.R[p];                       /* the layout's rows per rank */
        for (int64_t i = 0; i < Rp; ++i) {
            for (int64_t k = 0; k < K; ++k) {
                float v;
                if (i < n) {
                    v = widen_bf16(rank_rows[0][i * K + k]);
                    for (int32_t c = 1; c < L; ++c)
                        v = v + widen_bf16(rank_rows[c][i * K + k]);
                } else {
                    v = 0.0f;
                }
                dst[i * K + k] = v;
            }
        }
    }
    layout_free(&lay);
    return 0;
}

/*
 * All-gather placement: params[p] (T_p x K_p bf16) receives, for every rank
 * rank_begin <= r < rank_end, the true rows of rank r's piece, read from
 * shards + r * shard_stride + o_p. If write_count is not NULL,
 * write_count[p][e] is incremented for each element e of parameter p written.
 */
int oracle_allgather_place(int32_t P, const int64_t *rows, const int64_t *row_len,
                           int32_t N, const uint16_t *shards, int64_t shard_stride,
                           uint16_t *const *params, int32_t rank_begin, int32_t rank_end,
                           uint32_t *const *write_count)
{
    struct layout lay;
    int rc = layout_alloc(&lay, P, rows, row_len, N);
    if (rc == 0 && (shard_stride < lay.S || rank_begin < 0 || rank_end > N ||
                    rank_begin > rank_end))
        rc = -1;
    if (rc != 0) {
        layout_free(&lay);
        return rc;
    }
    for (int32_t r = rank_begin; r < rank_end; ++r) {
        for (int32_t p = 0; p < P; ++p) {
            const int64_t T = rows[p], K = row_len[p], Rp = lay.R[p];
            for (int64_t i = 0; i < Rp; ++i) {
                const int64_t t = (int64_t)r * Rp + i;
                if (t >= T)
                    break;                                 /* padded rows stay behind */
                for (int64_t k = 0; k < K; ++k) {
                    const int64_t src = (int64_t)r * shard_stride + lay.o[p] + i * K + k;
                    params[p][t * K + k] = shards[src];
                    if (write_count)
                        write_count[p][t * K + k] += 1;
                }
            }
        }
    }
    layout_free(&lay);
    return 0;
}

/*
 * All-gather placement from a stage buffer in arrival order. After the
 * recursive-doubling exchange on page 1 ("All-gather: parameters land at
 * their final address"), node n holds the pieces of nodes n, n+1, ... (mod M)
 * in its stage slots 0, 1, ...; with L ranks per node, rank r's shard sits at
 * stage position (r - first_rank) mod N, first_rank = n * L. This is the
 * placement above with shard r read from stage + ((r - first_rank) mod N) *
 * shard_stride.
 */
int oracle_allgather_place_stage(int32_t P, const int64_t *rows, const int64_t *row_len,
                                 int32_t N, const uint16_t *stage, int64_t shard_stride,
                                 int32_t first_rank, uint16_t *const *params,
                                 int32_t rank_begin, int32_t rank_end)
{
    struct layout lay;
    int rc = layout_alloc(&lay, P, rows, row_len, N);
    if (rc == 0 && (shard_stride < lay.S || rank_begin < 0 || rank_end > N ||
                    rank_begin > rank_end || first_rank < 0 || first_rank >= N))
        rc = -1;
    if (rc != 0) {
        layout_free(&lay);
        return rc;
    }
    for (int32_t r = rank_begin; r < rank_end; ++r) {
        const int64_t slot = ((int64_t)r - first_rank + N) % N;   /* stage position of rank r */
        for (int32_t p = 0; p < P; ++p) {
            const int64_t T = rows[p], K = row_len[p], Rp = lay.R[p];
            for (int64_t i = 0; i < Rp; ++i) {
                const int64_t t = (int64_t)r * Rp + i;
                if (t >= T)
                    break;
                for (int64_t k = 0; k < K; ++k)
                    params[p][t * K + k] = stage[slot * shard_stride + lay.o[p] + i * K + k];
            }
        }
    }
    layout_free(&lay);
    return 0;
}

/*
 * Level 2 of the reduce-scatter on one destination node: the landing sum
 * (page 1 "Reduce-scatter: two levels of addition, the last one done by
 * NVSwitch"; page 3 Figure 6(b)).
 *
 * The node's L GPUs finally hold one fp32 shard of S elements each. Every
 * source node's fp32 partial of this node's part is cut into L slices; slice
 * s is the s-th chunk of C = ceil(S / L) elements of every local shard, one
 * block per destination GPU b (block b of slice s = elements s*C .. of GPU b's
 * shard; the last chunk may be shorter or empty). A source with relative
 * index c = (destination - source) mod M (the destination itself is 0) sends
 * slice s to destination GPU (s - c) mod L: the Latin-square seating, so that
 * the M copies of a slice sit on M different GPUs at the same address. Each
 * destination GPU g has an inbox of L slots of L blocks of C elements; slot s,
 * block b is at inbox_g[(s * L + b) * C]. M <= L sources fill the slots.
 *
 * GPU b's shard element s * C + e is the fp32 sum over c = 0..M-1 of
 * inbox_{(s - c) mod L}[(s * L + b) * C + e], taken here as a left fold in
 * the order c = 0, 1, ... (the switch's own order is not stated); with
 * accumulate != 0 the sum is added to the shard's current value.
 *   inboxes[g]  destination GPU g's inbox (L * L * C floats)
 *   shards[b]   destination GPU b's shard (S floats)
 */
int oracle_landing_sum(int32_t L, int32_t M, int64_t S, const float *const *inboxes,
                       float *const *shards, int32_t accumulate)
{
    if (L < 1 || M < 1 || M > L || S < 0)
        return -1;
    {
        const int64_t C = S / L + (S % L != 0);            /* ceil(S / L) */
        for (int32_t b = 0; b < L; ++b) {
            for (int64_t f = 0; f < S; ++f) {
                const int64_t s = f / C, e = f % C;
                const int64_t at = (s * L + b) * C + e;        /* same offset in every inbox */
                float v = inboxes[(int32_t)(s % L)][at];       /* c = 0: GPU s mod L */
                for (int32_t c = 1; c < M; ++c) {
                    const int32_t g = (int32_t)(((s - c) % L + L) % L);
                    v = v + inboxes[g][at];
                }
                shards[b][f] = accumulate ? shards[b][f] + v : v;
            }
        }
    }
    return 0;
}

/*
 * The Latin-square seating for one (destination, source) node pair: the
 * source's relative index c = (dst - src) mod M; the source's GPU j sends
 * slice (j + c) mod L; slice s from that source lands on destination GPU
 * (s - c) mod L (page 1, the worked 4-GPU example; page 3 Figure 6(b)).
 */
int oracle_latin_square(int32_t M, int32_t L, int32_t dst, int32_t src, int32_t *c,
                        int32_t *slice_of_src_gpu, int32_t *dst_gpu_of_slice)
{
    if (M < 1 || L < 1 || dst < 0 || dst >= M || src < 0 || src >= M)
        return -1;
    *c = ((dst - src) % M + M) % M;
    for (int32_t j = 0; j < L; ++j)
        slice_of_src_gpu[j] = (j + *c) % L;
    for (int32_t s = 0; s < L; ++s)
        dst_gpu_of_slice[s] = ((s - *c) % L + L) % L;
    return 0;
}

/*
 * Slot-Reuse staging (page 1 "When gradients can be freed also needs
 * planning"; page 2 "What shipped"; page 3 abstract and Figure 7): each
 * contributor's bf16 gradients are copied into a vacated all-gather slot so
 * that the gradient storage can be freed; the reduce then reads the slot.
 * Inside slot c, parameter p's T_p x K_p gradient is placed at element
 * N * o_p, the group's parameter-major layout (each parameter padded to
 * N * R_p rows; the page-1 worked example's "9 MB" address). Only the rows
 * of ranks [rank_begin, rank_end) are copied (rank r holds rows
 * r * R_p .. r * R_p + R_p - 1); padding rows are never written.
 * slots[c] holds N * S elements.
 */
int oracle_stage_grads(int32_t P, const int64_t *rows, const int64_t *row_len, int32_t N,
                       int32_t L, int32_t rank_begin, int32_t rank_end,
                       const uint16_t *const *grads, uint16_t *const *slots)
{
    struct layout lay;
    int rc = layout_alloc(&lay, P, rows, row_len, N);
    if (rc != 0 || L < 1 || rank_begin < 0 || rank_end > N || rank_begin > rank_end) {
        layout_free(&lay);
        return -1;
    }
    for (int32_t c = 0; c < L; ++c)
        for (int32_t p = 0; p < P; ++p)
            for (int32_t r = rank_begin; r < rank_end; ++r) {
                /* rank r holds rows [r R_p, r R_p + R_p), clipped to the true rows */
                const int64_t t0 = (int64_t)r * lay.R[p];
                const int64_t t1 = t0 + lay.R[p] < rows[p] ? t0 + lay.R[p] : rows[p];
                for (int64_t t = t0; t < t1; ++t)
                    for (int64_t k = 0; k < row_len[p]; ++k)
                        slots[c][(int64_t)N * lay.o[p] + t * row_len[p] + k] =
                            grads[(int64_t)c * P + p][t * row_len[p] + k];
            }
    layout_free(&lay);
    return 0;
}
