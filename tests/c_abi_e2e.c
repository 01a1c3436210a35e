/*
 * End-to-end use of the C ABI (include/tide.h) from plain C11: no Python and
 * no torch. Device buffers come from the HIP runtime; reduce-scatters and
 * placements go through libtide and are compared bit for bit with the CPU
 * oracle (test infrastructure, linked into this test program only).
 *
 * Cases: a ragged group (T_p < N for one parameter, odd row lengths) with a
 * shard stride above S and the output one float past an aligned address,
 * full grid and CU-budgeted, a rank subset, and a refused call that must
 * leave the output untouched. Prints "c-abi: ok" and exits 0 on success.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tide.h"

/* The oracle's entry points (oracle/tide_oracle.c). */
int oracle_reduce_scatter(int32_t P, const int64_t *rows, const int64_t *row_len, int32_t N,
                          int32_t L, const uint16_t *const *grads, float *out, int64_t out_stride,
                          int32_t rank_begin, int32_t rank_end, uint32_t *write_count);
int oracle_allgather_place(int32_t P, const int64_t *rows, const int64_t *row_len, int32_t N,
                           const uint16_t *shards, int64_t shard_stride, uint16_t *const *params,
                           int32_t rank_begin, int32_t rank_end, uint32_t *const *write_count);

#define P 4
#define N 4
#define L 3
static const int64_t ROWS[P] = {37, 5, 16, 2};
static const int64_t ROW_LEN[P] = {24, 3, 9, 61};

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint16_t random_bf16(void)
{
    /* xorshift64*; exponent 0xFF (Inf/NaN) excluded so every sum is finite */
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    uint16_t h = (uint16_t)((rng_state * 0x2545F4914F6CDD1Dull) >> 48);
    if (((h >> 7) & 0xFF) == 0xFF) h &= 0xBFFF;
    return h;
}

#define HIP_OK(x)                                                                  \
    do {                                                                           \
        hipError_t e_ = (x);                                                       \
        if (e_ != hipSuccess) {                                                    \
            printf("c-abi: %s failed: %s\n", #x, hipGetErrorString(e_));          \
            return 1;                                                              \
        }                                                                          \
    } while (0)
#define TIDE_OK_(x)                                                                \
    do {                                                                           \
        tide_status s_ = (x);                                                      \
        if (s_ != TIDE_OK) {                                                       \
            printf("c-abi: %s failed: %s: %s\n", #x, tide_status_string(s_),       \
                   tide_last_error_detail());                                      \
            return 1;                                                              \
        }                                                                          \
    } while (0)

int main(void)
{
    tide_plan *plan = NULL;
    TIDE_OK_(tide_plan_create(ROWS, ROW_LEN, P, N, L, &plan));
    int64_t S = 0;
    TIDE_OK_(tide_plan_dims(plan, NULL, NULL, NULL, &S));
    const int64_t stride = S + 3;
    const int64_t out_elems = N * stride;

    /* gradients: L x P host and device buffers, contributor-major */
    uint16_t *h_grads[L * P];
    uint16_t *d_grads[L * P];
    for (int c = 0; c < L; ++c)
        for (int p = 0; p < P; ++p) {
            const int64_t n = ROWS[p] * ROW_LEN[p];
            uint16_t *h = malloc((size_t)n * 2);
            if (!h) return 1;
            for (int64_t i = 0; i < n; ++i) h[i] = random_bf16();
            h_grads[c * P + p] = h;
            HIP_OK(hipMalloc((void **)&d_grads[c * P + p], (size_t)n * 2));
            HIP_OK(hipMemcpy(d_grads[c * P + p], h, (size_t)n * 2, hipMemcpyHostToDevice));
        }

    /* output one float past an aligned address, NaN-filled around it */
    float *d_buf;
    HIP_OK(hipMalloc((void **)&d_buf, (size_t)(out_elems + 2) * 4));
    float *d_out = d_buf + 1;
    float *want = malloc((size_t)out_elems * 4), *got = malloc((size_t)out_elems * 4);
    if (!want || !got) return 1;

    struct { int mode, rb, re; } cases[] = {{TIDE_LAUNCH_FULL, 0, 0}, {TIDE_LAUNCH_BUDGETED, 0, 0},
                                            {TIDE_LAUNCH_FULL, 1, 3}};
    for (int k = 0; k < 3; ++k) {
        tide_launch lc;
        memset(&lc, 0, sizeof lc);
        lc.mode = cases[k].mode;
        lc.rank_begin = cases[k].rb;
        lc.rank_end = cases[k].re;
        HIP_OK(hipMemset(d_buf, 0xFF, (size_t)(out_elems + 2) * 4));
        TIDE_OK_(tide_reduce_scatter_bf16_fp32(plan, (const uint16_t *const *)d_grads, d_out, stride,
                                               NULL, &lc));
        HIP_OK(hipDeviceSynchronize());
        HIP_OK(hipMemcpy(got, d_out, (size_t)out_elems * 4, hipMemcpyDeviceToHost));
        memset(want, 0xFF, (size_t)out_elems * 4);
        if (oracle_reduce_scatter(P, ROWS, ROW_LEN, N, L, (const uint16_t *const *)h_grads, want,
                                  stride, cases[k].rb, cases[k].re ? cases[k].re : N, NULL) != 0) {
            printf("c-abi: oracle_reduce_scatter failed\n");
            return 1;
        }
        if (memcmp(want, got, (size_t)out_elems * 4) != 0) {
            printf("c-abi: reduce-scatter case %d differs from the oracle\n", k);
            return 1;
        }
    }

    /* a refused call enqueues nothing: the output keeps the last case's bits */
    if (tide_reduce_scatter_bf16_fp32(plan, (const uint16_t *const *)d_grads, d_out, S - 1, NULL,
                                      NULL) != TIDE_ERR_INVALID_ARG) {
        printf("c-abi: out_stride < S was not refused\n");
        return 1;
    }
    HIP_OK(hipDeviceSynchronize());
    HIP_OK(hipMemcpy(want, d_out, (size_t)out_elems * 4, hipMemcpyDeviceToHost));
    if (memcmp(want, got, (size_t)out_elems * 4) != 0) {
        printf("c-abi: a refused call changed the output\n");
        return 1;
    }

    /* placement from rank-major bf16 shards (stride above S) */
    uint16_t *h_sh = malloc((size_t)out_elems * 2);
    if (!h_sh) return 1;
    for (int64_t i = 0; i < out_elems; ++i) h_sh[i] = random_bf16();
    uint16_t *d_sh;
    HIP_OK(hipMalloc((void **)&d_sh, (size_t)out_elems * 2));
    HIP_OK(hipMemcpy(d_sh, h_sh, (size_t)out_elems * 2, hipMemcpyHostToDevice));
    uint16_t *d_par[P], *h_want[P], *h_got[P];
    for (int p = 0; p < P; ++p) {
        const int64_t n = ROWS[p] * ROW_LEN[p];
        HIP_OK(hipMalloc((void **)&d_par[p], (size_t)n * 2));
        HIP_OK(hipMemset(d_par[p], 0xFF, (size_t)n * 2));
        h_want[p] = malloc((size_t)n * 2);
        h_got[p] = malloc((size_t)n * 2);
        if (!h_want[p] || !h_got[p]) return 1;
        memset(h_want[p], 0xFF, (size_t)n * 2);
    }
    for (int engine = TIDE_ENGINE_KERNEL; engine <= TIDE_ENGINE_RUNTIME; ++engine) {
        TIDE_OK_(tide_allgather_place(plan, d_sh, stride, d_par, NULL, engine, NULL));
        HIP_OK(hipDeviceSynchronize());
    }
    if (oracle_allgather_place(P, ROWS, ROW_LEN, N, h_sh, stride, h_want, 0, N, NULL) != 0) {
        printf("c-abi: oracle_allgather_place failed\n");
        return 1;
    }
    for (int p = 0; p < P; ++p) {
        const int64_t n = ROWS[p] * ROW_LEN[p];
        HIP_OK(hipMemcpy(h_got[p], d_par[p], (size_t)n * 2, hipMemcpyDeviceToHost));
        if (memcmp(h_want[p], h_got[p], (size_t)n * 2) != 0) {
            printf("c-abi: placement of parameter %d differs from the oracle\n", p);
            return 1;
        }
    }

    for (int i = 0; i < L * P; ++i) {
        HIP_OK(hipFree(d_grads[i]));
        free(h_grads[i]);
    }
    for (int p = 0; p < P; ++p) {
        HIP_OK(hipFree(d_par[p]));
        free(h_want[p]);
        free(h_got[p]);
    }
    HIP_OK(hipFree(d_buf));
    HIP_OK(hipFree(d_sh));
    free(want);
    free(got);
    free(h_sh);
    tide_plan_destroy(plan);
    printf("c-abi: ok (3 reduce-scatter cases, 1 refused call, 2 placement engines)\n");
    return 0;
}
