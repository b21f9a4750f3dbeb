/*
 * c_abi_check.c -- drives the library through its C ABI from plain C (no
 * C++, no Python): per-token cast, fused SwiGLU cast, per-block cast,
 * RMSNorm + cast and dequantization on device buffers, each compared byte
 * for byte with the CPU oracle (test infrastructure, linked for checking
 * only), plus the error path of an invalid argument.
 * Exit status 0 when every check passes.
 */
#define __HIP_PLATFORM_AMD__ 1
#include <hip/hip_runtime_api.h>

#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "tk_quant.h"

/* the oracle's entry points (oracle/tk_oracle.c) */
int oracle_per_token_cast(const uint16_t *x, int64_t rows, int64_t cols, int64_t x_ld, uint8_t *q, int64_t q_ld,
                          void *scales, int64_t s_ld, int32_t group, int32_t qdtype, int32_t round_pow2,
                          int32_t scale_fmt, float *work);
int oracle_swiglu_per_token_cast(const uint16_t *gate_up, int64_t rows, int64_t cols, int64_t x_ld, uint8_t *q,
                                 int64_t q_ld, void *scales, int64_t s_ld, int32_t group, int32_t qdtype,
                                 int32_t round_pow2, int32_t scale_fmt, float *work);
int oracle_per_block_cast(const uint16_t *x, int64_t rows, int64_t cols, int64_t x_ld, uint8_t *q, int64_t q_ld,
                          void *scales, int64_t s_ld, int64_t block_rows, int64_t block_cols, int32_t qdtype,
                          int32_t round_pow2, int32_t scale_fmt);
int oracle_rmsnorm_cast(const uint16_t *x, int64_t rows, int64_t cols, int64_t x_ld, const uint16_t *w, float eps,
                        uint8_t *q, int64_t q_ld, void *scales, int64_t s_ld, int32_t group, int32_t qdtype,
                        int32_t round_pow2, int32_t scale_fmt, float *work);
int oracle_per_token_dequant(const uint8_t *q, int64_t rows, int64_t cols, int64_t q_ld, const void *scales,
                             int64_t s_ld, int32_t group, int32_t qdtype, int32_t scale_fmt, void *y, int64_t y_ld,
                             int32_t y_dtype);

static int failures = 0;

#define HIP_OK(call)                                                                   \
    do {                                                                               \
        hipError_t e_ = (call);                                                        \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "HIP error %d at %s:%d\n", (int)e_, __FILE__, __LINE__); \
            exit(2);                                                                   \
        }                                                                              \
    } while (0)

static void check(const char *what, int ok)
{
    printf("%-44s %s\n", what, ok ? "ok" : "MISMATCH");
    if (!ok) ++failures;
}

static void check_status(const char *what, tk_status st, tk_status want)
{
    printf("%-44s %s (%s)\n", what, st == want ? "ok" : "WRONG STATUS", tk_status_string(st));
    if (st != want) ++failures;
}

/* deterministic bf16 test values: sign, exponent in [-12, 6], 7-bit significand */
static uint32_t lcg_state = 12345u;
static uint32_t lcg(void)
{
    lcg_state = lcg_state * 1664525u + 1013904223u;
    return lcg_state >> 8;
}
static uint16_t rand_bf16(void)
{
    uint32_t r = lcg();
    uint32_t sign = r & 1u, mant = (r >> 1) & 0x7Fu, e = 127u - 12u + ((r >> 8) % 19u);
    return (uint16_t)((sign << 15) | (e << 7) | mant);
}

static void *dev_copy(const void *h, size_t n)
{
    void *d = NULL;
    HIP_OK(hipMalloc(&d, n ? n : 16));
    if (n && h) HIP_OK(hipMemcpy(d, h, n, hipMemcpyHostToDevice));   /* h == NULL: allocate only */
    return d;
}

static void *host_back(const void *d, size_t n)
{
    void *h = malloc(n ? n : 16);
    if (n) HIP_OK(hipMemcpy(h, d, n, hipMemcpyDeviceToHost));
    return h;
}

int main(void)
{
    const int64_t rows = 37, cols = 2048, group = 32;
    const size_t nx = (size_t)(rows * cols);
    uint16_t *x = malloc(nx * 2), *gu = malloc(nx * 4), *w = malloc((size_t)cols * 2);
    for (size_t i = 0; i < nx; ++i) x[i] = rand_bf16();
    for (size_t i = 0; i < 2 * nx; ++i) gu[i] = rand_bf16();
    for (int64_t i = 0; i < cols; ++i) w[i] = rand_bf16();
    float *work = malloc((size_t)cols * 4);
    void *dx = dev_copy(x, nx * 2), *dgu = dev_copy(gu, nx * 4), *dw = dev_copy(w, (size_t)cols * 2);

    printf("tk_abi_version %d\n", tk_abi_version());
    check("abi version", tk_abi_version() == TK_ABI_VERSION);

    /* per-token cast, E2M1, G32, power-of-two UE8M0 scales */
    {
        const size_t qn = nx / 2, sn = (size_t)(rows * cols / group / 4) * 4;
        void *dq = dev_copy(NULL, qn), *ds = dev_copy(NULL, sn);
        check_status("tk_per_token_cast", tk_per_token_cast(dx, rows, cols, cols, dq, cols / 2, ds, cols / group / 4,
                                                           (int32_t)group, TK_QDTYPE_E2M1, 1, TK_SCALE_UE8M0_X4, NULL),
                     TK_SUCCESS);
        HIP_OK(hipDeviceSynchronize());
        uint8_t *q = host_back(dq, qn), *wq = calloc(qn, 1);
        uint32_t *s = host_back(ds, sn), *ws = calloc(sn, 1);
        oracle_per_token_cast(x, rows, cols, cols, wq, cols / 2, ws, cols / group / 4, (int32_t)group, 1, 1, 1, work);
        check("  codes", memcmp(q, wq, qn) == 0);
        check("  scales", memcmp(s, ws, sn) == 0);

        /* dequantization of those codes back to fp32 */
        void *dy = dev_copy(NULL, nx * 4);
        check_status("tk_per_token_dequant", tk_per_token_dequant(dq, rows, cols, cols / 2, ds, cols / group / 4,
                                                                 (int32_t)group, TK_QDTYPE_E2M1, TK_SCALE_UE8M0_X4, dy,
                                                                 cols, TK_OUT_F32, NULL),
                     TK_SUCCESS);
        HIP_OK(hipDeviceSynchronize());
        float *y = host_back(dy, nx * 4), *wy = malloc(nx * 4);
        oracle_per_token_dequant(wq, rows, cols, cols / 2, ws, cols / group / 4, (int32_t)group, 1, 1, wy, cols, 1);
        check("  dequantized values", memcmp(y, wy, nx * 4) == 0);
        free(q); free(wq); free(s); free(ws); free(y); free(wy);
        HIP_OK(hipFree(dq)); HIP_OK(hipFree(ds)); HIP_OK(hipFree(dy));
    }

    /* fused SwiGLU cast, E4M3, G128, fp32 power-of-two scales */
    {
        const size_t qn = nx, sn = (size_t)(rows * cols / 128) * 4;
        void *dq = dev_copy(NULL, qn), *ds = dev_copy(NULL, sn);
        check_status("tk_swiglu_per_token_cast",
                     tk_swiglu_per_token_cast(dgu, rows, cols, 2 * cols, dq, cols, ds, cols / 128, 128, TK_QDTYPE_E4M3,
                                              1, TK_SCALE_F32, NULL),
                     TK_SUCCESS);
        HIP_OK(hipDeviceSynchronize());
        uint8_t *q = host_back(dq, qn), *wq = calloc(qn, 1);
        float *s = host_back(ds, sn), *ws = calloc(sn, 1);
        oracle_swiglu_per_token_cast(gu, rows, cols, 2 * cols, wq, cols, ws, cols / 128, 128, 0, 1, 0, work);
        check("  codes", memcmp(q, wq, qn) == 0);
        check("  scales", memcmp(s, ws, sn) == 0);
        free(q); free(wq); free(s); free(ws);
        HIP_OK(hipFree(dq)); HIP_OK(hipFree(ds));
    }

    /* per-block cast, 16 x 64 blocks, E4M3, fp32 scales (partial last block row) */
    {
        const int64_t br = 16, bc = 64, nbr = (rows + br - 1) / br, nbc = cols / bc;
        const size_t qn = nx, sn = (size_t)(nbr * nbc) * 4;
        void *dq = dev_copy(NULL, qn), *ds = dev_copy(NULL, sn);
        check_status("tk_per_block_cast", tk_per_block_cast(dx, rows, cols, cols, dq, cols, ds, nbc, br, bc,
                                                           TK_QDTYPE_E4M3, 0, TK_SCALE_F32, NULL),
                     TK_SUCCESS);
        HIP_OK(hipDeviceSynchronize());
        uint8_t *q = host_back(dq, qn), *wq = calloc(qn, 1);
        float *s = host_back(ds, sn), *ws = calloc(sn, 1);
        oracle_per_block_cast(x, rows, cols, cols, wq, cols, ws, nbc, br, bc, 0, 0, 0);
        check("  codes", memcmp(q, wq, qn) == 0);
        check("  scales", memcmp(s, ws, sn) == 0);
        free(q); free(wq); free(s); free(ws);
        HIP_OK(hipFree(dq)); HIP_OK(hipFree(ds));
    }

    /* RMSNorm + cast, E4M3, G128, power-of-two UE8M0 scales */
    {
        const size_t qn = nx, sn = (size_t)(rows * cols / 128 / 4) * 4;
        void *dq = dev_copy(NULL, qn), *ds = dev_copy(NULL, sn);
        check_status("tk_rmsnorm_cast", tk_rmsnorm_cast(dx, rows, cols, cols, dw, 1e-6f, dq, cols, ds, cols / 128 / 4,
                                                       128, TK_QDTYPE_E4M3, 1, TK_SCALE_UE8M0_X4, NULL),
                     TK_SUCCESS);
        HIP_OK(hipDeviceSynchronize());
        uint8_t *q = host_back(dq, qn), *wq = calloc(qn, 1);
        uint32_t *s = host_back(ds, sn), *ws = calloc(sn, 1);
        oracle_rmsnorm_cast(x, rows, cols, cols, w, 1e-6f, wq, cols, ws, cols / 128 / 4, 128, 0, 1, 1, work);
        check("  codes", memcmp(q, wq, qn) == 0);
        check("  scales", memcmp(s, ws, sn) == 0);
        free(q); free(wq); free(s); free(ws);
        HIP_OK(hipFree(dq)); HIP_OK(hipFree(ds));
    }

    /* errors are return codes; nothing is launched */
    check_status("invalid group", tk_per_token_cast(dx, rows, cols, cols, dx, cols, dx, cols, 48, TK_QDTYPE_E4M3, 0,
                                                    TK_SCALE_F32, NULL),
                 TK_ERROR_INVALID_VALUE);
    check_status("misaligned input", tk_per_token_cast((const char *)dx + 2, rows, cols, cols, dx, cols, dx, cols, 32,
                                                       TK_QDTYPE_E4M3, 0, TK_SCALE_F32, NULL),
                 TK_ERROR_MISALIGNED);

    HIP_OK(hipFree(dx)); HIP_OK(hipFree(dgu)); HIP_OK(hipFree(dw));
    free(x); free(gu); free(w); free(work);
    printf("%s\n", failures ? "FAILED" : "ALL PASSED");
    return failures ? 1 : 0;
}
