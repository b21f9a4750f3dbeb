/*
 * tk_oracle.c -- plain, slow CPU oracle for the per-token / per-group
 * activation cast and for its fused SwiGLU form.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this file's library; the product
 * path (the HIP library and its Python binding) never does, and the two
 * share no code, header, table or constant.
 *
 * What is computed, and where it comes from:
 *   - "Tile Kernels" (PyPI project page, v2.0.0), Features: activations are
 *     cast per token to FP8 or FP4, and SwiGLU has a form fused with the cast.
 *   - "TileKernels" (aiwiki.ai), section Quantization: each scale covers G
 *     channels of a row, G one of 16, 32, 64, 128; scales may be rounded up
 *     to powers of two and stored packed as UE8M0 bytes; the input is BF16.
 *   - "TileKernels, TileLang kernels for MoE routing and low-precision
 *     quantization" (hysenlabs.com), section "Seven kernel families": the
 *     fused form computes SwiGLU and the cast in a single kernel.
 * The pages print no formula.  The one this oracle follows is the method's
 * fixed definition, step by step, for every row r and every group j of G
 * consecutive channels (columns jG .. jG+G-1):
 *   1. a = max |x_i| over the group, x_i widened exactly from bf16 to fp32;
 *   2. a = max(a, 1e-4f);
 *   3. s = a / D in fp32 (IEEE division), D = 448 for e4m3, 6 for e2m1;
 *   4. optionally s = 2^ceil(log2 s), read exactly from s's exponent and
 *      mantissa bits;
 *   5. the scale is stored as fp32 s, or as the UE8M0 byte (biased exponent
 *      of s) packed four to a little-endian int32 (group 4k+b in byte b);
 *   6. v_i = x_i / s in fp32 (IEEE division), clamped to [-D, D], then
 *      rounded to the nearest e4m3 / e2m1 value with ties to the even
 *      code, keeping the sign (also of zero);
 *   7. SwiGLU form: x_i is replaced by h_i = fl32(silu32(g_i) * u_i), where
 *      silu32(g) is the fp32 value nearest to g / (1 + e^-g).
 * Dequantization ("Tile Kernels" (PyPI, v2.0.0), Features: the inverse of
 * the cast) maps a code back to y = fl32(value(code) * s), returned as
 * fp32 or rounded to bf16 (nearest, ties to even); the
 * cast-and-cast-back ("TileKernels" (aiwiki.ai), Version 2.0.0) is the
 * per-token cast above followed by that dequantization, bf16 out.  The per-block and
 * per-channel casts ("Tile Kernels" (PyPI, v2.0.0), Features) take step 1
 * over a block of rows x channels or over a whole column.  RMSNorm forward
 * with the optional fused cast ("TileKernels" (aiwiki.ai), Version 2.0.0) is
 * defined where it is implemented below.
 * Every float operation below is one IEEE binary32 operation rounded to
 * nearest-even; build with -O2 -ffp-contract=off and without fast-math.
 * Results for NaN or Inf inputs are outside the contract.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

enum { ORACLE_E4M3 = 0, ORACLE_E2M1 = 1 };
enum { ORACLE_SCALE_F32 = 0, ORACLE_SCALE_UE8M0_X4 = 1 };

static float f32_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_from_f32(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 is the top half of an fp32 bit pattern: widening is exact. */
static float bf16_to_f32(uint16_t b) { return f32_from_bits((uint32_t)b << 16); }

/* ---- the two target formats, decoded from their definitions ---------- */

/* OCP FP8 E4M3FN: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent
 * field 0 is subnormal (m * 2^-9); S.1111.111 is NaN, so the largest finite
 * magnitude is code 0x7E = 1.75 * 2^8 = 448.  Positive codes 0..126 are
 * strictly increasing in value. */
#define E4M3_NCODES 127
static double e4m3_value(int code)
{
    int e = (code >> 3) & 15, m = code & 7;
    if (e == 0) return ldexp((double)m, -9);
    return ldexp(1.0 + m / 8.0, e - 7);
}

/* FP4 E2M1: 1 sign, 2 exponent (bias 1), 1 mantissa bit, no Inf/NaN.
 * Magnitudes of codes 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
#define E2M1_NCODES 8
static double e2m1_value(int code)
{
    int e = (code >> 1) & 3, m = code & 1;
    if (e == 0) return 0.5 * m;
    return ldexp(1.0 + m / 2.0, e - 1);
}

static double g_e4m3[E4M3_NCODES], g_e2m1[E2M1_NCODES];

/* Filled once when the library is loaded, before any caller thread runs. */
__attribute__((constructor)) static void init_tables(void)
{
    for (int c = 0; c < E4M3_NCODES; ++c) g_e4m3[c] = e4m3_value(c);
    for (int c = 0; c < E2M1_NCODES; ++c) g_e2m1[c] = e2m1_value(c);
}

/* Nearest code to a (0 <= a <= largest grid value), ties to the even code.
 * The grid is ascending and a code's low bit is its mantissa's low bit, so
 * "even code" is "even mantissa".  a is an fp32 value and every grid value
 * and midpoint is a short dyadic rational, so all comparisons in double are
 * exact. */
static int nearest_code(double a, const double *grid, int n)
{
    int lo = 0, hi = n - 1;
    while (lo < hi) {                       /* smallest k with grid[k] >= a */
        int mid = (lo + hi) / 2;
        if (grid[mid] >= a) hi = mid; else lo = mid + 1;
    }
    int k = lo;
    if (k == 0 || grid[k] == a) return k;
    double midpoint = 0.5 * (grid[k - 1] + grid[k]);
    if (a < midpoint) return k - 1;
    if (a > midpoint) return k;
    return (k % 2 == 0) ? k : k - 1;
}

/* Step 6 after the division: saturate to [-M, M], round to nearest even,
 * keep the sign bit of v (so -0.0 and negative values that round to zero
 * give the negative-zero code). */
uint8_t oracle_encode_e4m3(float v)
{
    const float M = 448.0f;
    int neg = signbit(v) != 0;
    float a = fabsf(v);
    if (a > M) a = M;
    int code = nearest_code((double)a, g_e4m3, E4M3_NCODES);
    return (uint8_t)(code | (neg ? 0x80 : 0));
}

/* Returns one e2m1 nibble (0..15) in the low bits. */
uint8_t oracle_encode_e2m1(float v)
{
    const float M = 6.0f;
    int neg = signbit(v) != 0;
    float a = fabsf(v);
    if (a > M) a = M;
    int code = nearest_code((double)a, g_e2m1, E2M1_NCODES);
    return (uint8_t)(code | (neg ? 0x8 : 0));
}

/* Steps 2-4: the group scale from the group amax.  On return *e8 holds the
 * biased exponent byte of the result (its UE8M0 encoding when the result
 * is a power of two). */
float oracle_group_scale(float amax, int32_t qdtype, int32_t round_pow2, uint8_t *e8)
{
    const float D = (qdtype == ORACLE_E4M3) ? 448.0f : 6.0f;
    const float floor_value = 1e-4f;
    float a = amax;
    if (a < floor_value) a = floor_value;
    float s = a / D;
    uint32_t b = bits_from_f32(s);
    uint32_t E = (b >> 23) & 0xFF, m = b & 0x7FFFFF;
    if (round_pow2) {
        /* s = 2^(E-127) * (1 + m/2^23) is normal here (s >= 1e-4f / 448),
         * so ceil(log2 s) = E-127 when m == 0 and E-126 otherwise. */
        if (m != 0) E += 1;
        s = f32_from_bits(E << 23);
    }
    if (e8) *e8 = (uint8_t)E;
    return s;
}

/* Step 7: fp32 nearest to g / (1 + e^-g).  The quotient is formed in the
 * x87 80-bit format (64-bit significand) and rounded once to fp32.  The
 * tests check the result for every bf16 g against a 60-digit evaluation. */
float oracle_silu32(float g)
{
    long double x = (long double)g;
    long double r = x / (1.0L + expl(-x));
    return (float)r;
}

/* ---- whole-tensor cast ------------------------------------------------ */

static int valid_common(int64_t rows, int64_t cols, int32_t group, int32_t qdtype,
                        int32_t round_pow2, int32_t scale_fmt)
{
    if (rows < 0 || cols <= 0) return 0;
    if (group != 16 && group != 32 && group != 64 && group != 128) return 0;
    if (cols % group != 0) return 0;
    if (qdtype != ORACLE_E4M3 && qdtype != ORACLE_E2M1) return 0;
    if (scale_fmt != ORACLE_SCALE_F32 && scale_fmt != ORACLE_SCALE_UE8M0_X4) return 0;
    if (scale_fmt == ORACLE_SCALE_UE8M0_X4 && (!round_pow2 || (cols / group) % 4 != 0)) return 0;
    return 1;
}

/* Cast one row of fp32 values v[0..cols) (already widened from bf16, or the
 * SwiGLU products) into codes qrow and scales srow. */
static void cast_row(const float *v, int64_t cols, uint8_t *qrow, void *srow, int32_t group,
                     int32_t qdtype, int32_t round_pow2, int32_t scale_fmt)
{
    int64_t ngroups = cols / group;
    if (qdtype == ORACLE_E2M1) memset(qrow, 0, (size_t)(cols / 2));
    if (scale_fmt == ORACLE_SCALE_UE8M0_X4) memset(srow, 0, (size_t)(ngroups / 4) * 4);
    for (int64_t j = 0; j < ngroups; ++j) {
        const float *x = v + j * group;
        float amax = 0.0f;                                   /* step 1 */
        for (int i = 0; i < group; ++i) {
            float a = fabsf(x[i]);
            if (a > amax) amax = a;
        }
        uint8_t e8 = 0;
        float s = oracle_group_scale(amax, qdtype, round_pow2, &e8);   /* steps 2-4 */
        if (scale_fmt == ORACLE_SCALE_F32) {                 /* step 5 */
            ((float *)srow)[j] = s;
        } else {
            uint32_t *dw = (uint32_t *)srow + j / 4;
            *dw |= (uint32_t)e8 << (8 * (j % 4));
        }
        for (int i = 0; i < group; ++i) {                    /* step 6 */
            float q = x[i] / s;
            int64_t c = j * group + i;
            if (qdtype == ORACLE_E4M3) {
                qrow[c] = oracle_encode_e4m3(q);
            } else {
                uint8_t nib = oracle_encode_e2m1(q);
                qrow[c / 2] |= (uint8_t)((c % 2 == 0) ? nib : (nib << 4));
            }
        }
    }
}

/* x: bf16 bits [rows, cols], row stride x_ld elements.
 * q: [rows, cols] bytes (e4m3) or [rows, cols/2] bytes (e2m1), row stride
 *    q_ld bytes.
 * scales: fp32 [rows, cols/group] or int32 [rows, cols/group/4], row stride
 *    s_ld elements of that type.
 * Returns 0, or -1 when the arguments describe no valid cast. */
int oracle_per_token_cast(const uint16_t *x, int64_t rows, int64_t cols, int64_t x_ld,
                          uint8_t *q, int64_t q_ld, void *scales, int64_t s_ld,
                          int32_t group, int32_t qdtype, int32_t round_pow2, int32_t scale_fmt,
                          float *work /* cols floats */)
{
    if (!valid_common(rows, cols, group, qdtype, round_pow2, scale_fmt)) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) work[c] = bf16_to_f32(x[r * x_ld + c]);
        void *srow = (scale_fmt == ORACLE_SCALE_F32) ? (void *)((float *)scales + r * s_ld)
                                                     : (void *)((uint32_t *)scales + r * s_ld);
        cast_row(work, cols, q + r * q_ld, srow, group, qdtype, round_pow2, scale_fmt);
    }
    return 0;
}

/* The same cast of fp32 activations ("TileKernels" (aiwiki.ai),
 * Quantization: casts of BF16 or FP32 activations): x fp32 [rows, cols], row
 * stride x_ld elements; step 1 uses the values as they are. */
int oracle_per_token_cast_f32(const float *x, int64_t rows, int64_t cols, int64_t x_ld,
                              uint8_t *q, int64_t q_ld, void *scales, int64_t s_ld,
                              int32_t group, int32_t qdtype, int32_t round_pow2, int32_t scale_fmt,
                              float *work /* cols floats */)
{
    if (!valid_common(rows, cols, group, qdtype, round_pow2, scale_fmt)) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) work[c] = x[r * x_ld + c];
        void *srow = (scale_fmt == ORACLE_SCALE_F32) ? (void *)((float *)scales + r * s_ld)
                                                     : (void *)((uint32_t *)scales + r * s_ld);
        cast_row(work, cols, q + r * q_ld, srow, group, qdtype, round_pow2, scale_fmt);
    }
    return 0;
}

/* gate_up: bf16 bits [rows, 2*cols]; gate = columns [0, cols), up =
 * columns [cols, 2*cols).  Outputs as in oracle_per_token_cast with cols. */
int oracle_swiglu_per_token_cast(const uint16_t *gate_up, int64_t rows, int64_t cols, int64_t x_ld,
                                 uint8_t *q, int64_t q_ld, void *scales, int64_t s_ld,
                                 int32_t group, int32_t qdtype, int32_t round_pow2,
                                 int32_t scale_fmt, float *work /* cols floats */)
{
    if (!valid_common(rows, cols, group, qdtype, round_pow2, scale_fmt)) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *row = gate_up + r * x_ld;
        for (int64_t c = 0; c < cols; ++c) {
            float g = bf16_to_f32(row[c]);
            float u = bf16_to_f32(row[cols + c]);
            float sg = oracle_silu32(g);
            work[c] = sg * u;
        }
        void *srow = (scale_fmt == ORACLE_SCALE_F32) ? (void *)((float *)scales + r * s_ld)
                                                     : (void *)((uint32_t *)scales + r * s_ld);
        cast_row(work, cols, q + r * q_ld, srow, group, qdtype, round_pow2, scale_fmt);
    }
    return 0;
}

/* ---- per-block and per-channel casts ---------------------------------- */

/* "Tile Kernels" (PyPI, v2.0.0), Features: the cast also comes with one
 * scale per block of rows x channels, or one per column.  The same steps 1-6 with the amax taken over a block of
 * block_rows x block_cols elements: rows [bi*Br, min(rows, (bi+1)*Br)) and
 * columns [bj*Bc, (bj+1)*Bc).  The last block row may be partial; cols must be
 * a multiple of Bc.  scales: fp32 [ceil(rows/Br), cols/Bc], or UE8M0 bytes of
 * 4 consecutive column blocks per little-endian int32 [ceil(rows/Br),
 * cols/Bc/4]; row stride s_ld elements.  Per-channel = Br = rows, Bc = 1.
 * x: bf16 bits; q as for the per-token cast. */
int oracle_per_block_cast(const uint16_t *x, int64_t rows, int64_t cols, int64_t x_ld,
                          uint8_t *q, int64_t q_ld, void *scales, int64_t s_ld,
                          int64_t block_rows, int64_t block_cols, int32_t qdtype,
                          int32_t round_pow2, int32_t scale_fmt)
{
    if (rows < 0 || cols <= 0 || block_rows <= 0 || block_cols <= 0 || cols % block_cols != 0) return -1;
    if (qdtype != ORACLE_E4M3 && qdtype != ORACLE_E2M1) return -1;
    if (qdtype == ORACLE_E2M1 && cols % 2 != 0) return -1;
    int64_t nbc = cols / block_cols;
    if (scale_fmt == ORACLE_SCALE_UE8M0_X4 && (!round_pow2 || nbc % 4 != 0)) return -1;
    if (scale_fmt != ORACLE_SCALE_F32 && scale_fmt != ORACLE_SCALE_UE8M0_X4) return -1;
    int64_t nbr = (rows + block_rows - 1) / block_rows;
    for (int64_t r = 0; r < rows; ++r)
        if (qdtype == ORACLE_E2M1) memset(q + r * q_ld, 0, (size_t)(cols / 2));
    for (int64_t bi = 0; bi < nbr; ++bi) {
        int64_t r0 = bi * block_rows, r1 = r0 + block_rows < rows ? r0 + block_rows : rows;
        if (scale_fmt == ORACLE_SCALE_UE8M0_X4) memset((uint32_t *)scales + bi * s_ld, 0, (size_t)(nbc / 4) * 4);
        for (int64_t bj = 0; bj < nbc; ++bj) {
            int64_t c0 = bj * block_cols;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c0 + block_cols; ++c) {
                    float a = fabsf(bf16_to_f32(x[r * x_ld + c]));
                    if (a > amax) amax = a;
                }
            uint8_t e8 = 0;
            float s = oracle_group_scale(amax, qdtype, round_pow2, &e8);
            if (scale_fmt == ORACLE_SCALE_F32) {
                ((float *)scales)[bi * s_ld + bj] = s;
            } else {
                uint32_t *dw = (uint32_t *)scales + bi * s_ld + bj / 4;
                *dw |= (uint32_t)e8 << (8 * (bj % 4));
            }
            for (int64_t r = r0; r < r1; ++r)
                for (int64_t c = c0; c < c0 + block_cols; ++c) {
                    float v = bf16_to_f32(x[r * x_ld + c]) / s;
                    if (qdtype == ORACLE_E4M3) {
                        q[r * q_ld + c] = oracle_encode_e4m3(v);
                    } else {
                        uint8_t nib = oracle_encode_e2m1(v);
                        q[r * q_ld + c / 2] |= (uint8_t)((c % 2 == 0) ? nib : (nib << 4));
                    }
                }
        }
    }
    return 0;
}

/* ---- dequantization and cast-back ------------------------------------ */

/* fp32 -> bf16 bit pattern, round to nearest, ties to even (finite inputs
 * and infinities; NaN is outside the contract). */
static uint16_t f32_to_bf16_rne(float f)
{
    uint32_t b = bits_from_f32(f);
    uint32_t lsb = (b >> 16) & 1u;
    return (uint16_t)((b + 0x7FFFu + lsb) >> 16);
}

/* Value of a code: E4M3 byte, or E2M1 nibble (low 4 bits). */
static float code_value(int32_t qdtype, uint8_t code)
{
    if (qdtype == ORACLE_E4M3) {
        double m = g_e4m3[code & 0x7F];       /* 0x7F (NaN) is never produced */
        return (float)((code & 0x80) ? -m : m);
    }
    double m = g_e2m1[code & 0x7];
    return (float)((code & 0x8) ? -m : m);
}

/* q: codes [rows, cols] (E4M3) or [rows, cols/2] (E2M1), row stride q_ld
 * bytes; scales as produced by the cast (fp32 or UE8M0 x4 int32, row stride
 * s_ld elements); y: fp32 (y_f32 != 0) or bf16 bits [rows, cols], row stride
 * y_ld elements.  y = fl32(value(code) * s), then bf16 RNE when asked. */
int oracle_per_token_dequant(const uint8_t *q, int64_t rows, int64_t cols, int64_t q_ld,
                             const void *scales, int64_t s_ld, int32_t group, int32_t qdtype,
                             int32_t scale_fmt, void *y, int64_t y_ld, int32_t y_f32)
{
    if (!valid_common(rows, cols, group, qdtype, scale_fmt == ORACLE_SCALE_UE8M0_X4, scale_fmt)) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            int64_t j = c / group;
            float s;
            if (scale_fmt == ORACLE_SCALE_F32) {
                s = ((const float *)scales)[r * s_ld + j];
            } else {
                uint32_t dw = ((const uint32_t *)scales)[r * s_ld + j / 4];
                uint32_t e = (dw >> (8 * (j % 4))) & 0xFF;
                s = f32_from_bits(e << 23);    /* 2^(e - 127); e in [1, 254] */
            }
            uint8_t code;
            if (qdtype == ORACLE_E4M3) {
                code = q[r * q_ld + c];
            } else {
                uint8_t byte = q[r * q_ld + c / 2];
                code = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            }
            float v = code_value(qdtype, code) * s;
            if (y_f32) ((float *)y)[r * y_ld + c] = v;
            else ((uint16_t *)y)[r * y_ld + c] = f32_to_bf16_rne(v);
        }
    }
    return 0;
}

/* Cast then dequantize, bf16 out: y [rows, cols] bf16 bits, row stride y_ld. */
int oracle_per_token_cast_back(const uint16_t *x, int64_t rows, int64_t cols, int64_t x_ld,
                               uint16_t *y, int64_t y_ld, int32_t group, int32_t qdtype,
                               int32_t round_pow2, float *work /* cols floats */,
                               uint8_t *qwork /* cols bytes */, float *swork /* cols/group floats */)
{
    if (!valid_common(rows, cols, group, qdtype, round_pow2, ORACLE_SCALE_F32)) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) work[c] = bf16_to_f32(x[r * x_ld + c]);
        cast_row(work, cols, qwork, swork, group, qdtype, round_pow2, ORACLE_SCALE_F32);
        if (oracle_per_token_dequant(qwork, 1, cols, cols, swork, cols / group, group, qdtype,
                                     ORACLE_SCALE_F32, y + r * y_ld, y_ld, 0) != 0)
            return -1;
    }
    return 0;
}

/* ---- RMSNorm forward, alone and followed by the per-token cast -------- */

/* "TileKernels" (aiwiki.ai), Version 2.0.0: RMSNorm forward, which can be
 * followed by an FP8 cast in the same kernel.  The pages name the operation only; this is the
 * textbook root-mean-square normalisation of a row of C values with a
 * per-channel weight w (bf16, or none = all ones) and eps > 0:
 *   ss  = sum_j x_j^2, the exact sum rounded once to fp32 (nearest-even);
 *   t   = fl32(ss / C);  t = fl32(t + eps);
 *   r   = fl32(1 / fl32(sqrt(t)));
 *   y_j = fl32(x_j * r), then y_j = fl32(y_j * w_j) with a weight.
 * The fused form casts y per token exactly as the cast above casts fp32
 * activations. */

/* A little-endian multiword integer of 32-bit words holding sum_j x_j^2 *
 * 2^266: a nonzero bf16 value is M * 2^k (M < 2^8, k >= -133), so x^2 =
 * M^2 * 2^(2k) with 2k + 266 >= 0; the largest, 2k + 266 <= 506 plus 16 bits
 * of M^2, leaves room for 2^40 terms below 18 * 32 bits. */
#define SQ_WORDS 18
#define SQ_SHIFT 266

static void sq_add(uint32_t *acc, uint16_t b)
{
    uint32_t e = (b >> 7) & 0xFFu, m = b & 0x7Fu;
    if (e == 0 && m == 0) return;
    int k = (e == 0) ? -133 : (int)e - 134;          /* value = M * 2^k */
    uint32_t M = (e == 0) ? m : (m | 0x80u);
    int p = 2 * k + SQ_SHIFT;                        /* bit position of M^2 */
    uint64_t v = (uint64_t)(M * M) << (p % 32);
    int w = p / 32;
    uint64_t carry = 0;
    for (int i = w; i < SQ_WORDS; ++i) {
        uint64_t add = (i == w) ? (v & 0xFFFFFFFFu) : (i == w + 1) ? (v >> 32) : 0;
        uint64_t t = (uint64_t)acc[i] + add + carry;
        acc[i] = (uint32_t)t;
        carry = t >> 32;
        if (carry == 0 && i > w) break;
    }
}

static int sq_bit(const uint32_t *acc, int i)
{
    return (int)((acc[i / 32] >> (i % 32)) & 1u);
}

/* The multiword value * 2^-266 rounded to fp32, nearest with ties to even
 * (subnormal results rounded at 2^-149; overflow gives +Inf). */
static float sq_round_f32(const uint32_t *acc)
{
    int top = -1;
    for (int i = SQ_WORDS * 32 - 1; i >= 0; --i)
        if (sq_bit(acc, i)) { top = i; break; }
    if (top < 0) return 0.0f;
    int lsb = top - 23;
    if (lsb < SQ_SHIFT - 149) lsb = SQ_SHIFT - 149;
    uint64_t mant = 0;
    for (int i = top; i >= lsb; --i) mant = (mant << 1) | (uint64_t)sq_bit(acc, i);
    int round = (lsb >= 1) ? sq_bit(acc, lsb - 1) : 0;
    int sticky = 0;
    for (int i = lsb - 2; i >= 0 && !sticky; --i) sticky = sq_bit(acc, i);
    if (round && (sticky || (mant & 1u))) mant += 1;
    double v = ldexp((double)mant, lsb - SQ_SHIFT);   /* exact: mant <= 2^24 */
    if (v > (double)FLT_MAX) return INFINITY;
    return (float)v;
}

float oracle_sum_squares_f32(const uint16_t *x, int64_t n)
{
    uint32_t acc[SQ_WORDS];
    memset(acc, 0, sizeof(acc));
    for (int64_t j = 0; j < n; ++j) sq_add(acc, x[j]);
    return sq_round_f32(acc);
}

static void rmsnorm_row(const uint16_t *x, int64_t cols, const uint16_t *w, float eps, float *y)
{
    float ss = oracle_sum_squares_f32(x, cols);
    float t = ss / (float)cols;
    t = t + eps;
    float rs = sqrtf(t);
    float r = 1.0f / rs;
    for (int64_t j = 0; j < cols; ++j) {
        float v = bf16_to_f32(x[j]) * r;
        y[j] = w ? v * bf16_to_f32(w[j]) : v;
    }
}

static int valid_rmsnorm(int64_t rows, int64_t cols, float eps)
{
    return rows >= 0 && cols > 0 && cols < (1 << 24) && eps > 0.0f && isfinite(eps);
}

/* x: bf16 bits [rows, cols] (row stride x_ld); w: bf16 bits [cols] or NULL;
 * y: [rows, cols] with row stride y_ld, bf16 bits (y_dtype 0, nearest-even
 * from the fp32 y) or fp32 (y_dtype 1).  Returns 0 or -1 (bad arguments). */
int oracle_rmsnorm(const uint16_t *x, int64_t rows, int64_t cols, int64_t x_ld, const uint16_t *w, float eps,
                   void *y, int64_t y_ld, int32_t y_dtype, float *work /* cols floats */)
{
    if (!valid_rmsnorm(rows, cols, eps) || (y_dtype != 0 && y_dtype != 1)) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        rmsnorm_row(x + r * x_ld, cols, w, eps, work);
        for (int64_t c = 0; c < cols; ++c) {
            if (y_dtype == 1) ((float *)y)[r * y_ld + c] = work[c];
            else ((uint16_t *)y)[r * y_ld + c] = f32_to_bf16_rne(work[c]);
        }
    }
    return 0;
}

/* RMSNorm followed by the per-token cast of the fp32 y; outputs as in
 * oracle_per_token_cast. */
int oracle_rmsnorm_cast(const uint16_t *x, int64_t rows, int64_t cols, int64_t x_ld, const uint16_t *w, float eps,
                        uint8_t *q, int64_t q_ld, void *scales, int64_t s_ld, int32_t group, int32_t qdtype,
                        int32_t round_pow2, int32_t scale_fmt, float *work /* cols floats */)
{
    if (!valid_rmsnorm(rows, cols, eps)) return -1;
    if (!valid_common(rows, cols, group, qdtype, round_pow2, scale_fmt)) return -1;
    for (int64_t r = 0; r < rows; ++r) {
        rmsnorm_row(x + r * x_ld, cols, w, eps, work);
        void *srow = (scale_fmt == ORACLE_SCALE_F32) ? (void *)((float *)scales + r * s_ld)
                                                     : (void *)((uint32_t *)scales + r * s_ld);
        cast_row(work, cols, q + r * q_ld, srow, group, qdtype, round_pow2, scale_fmt);
    }
    return 0;
}

void oracle_sum_squares_rows(const uint16_t *x, int64_t rows, int64_t cols, int64_t x_ld, float *out)
{
    for (int64_t r = 0; r < rows; ++r) out[r] = oracle_sum_squares_f32(x + r * x_ld, cols);
}

/* ---- array forms of the single steps, for the pin tests -------------- */

void oracle_encode_e4m3_n(const float *v, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_encode_e4m3(v[i]);
}

void oracle_encode_e2m1_n(const float *v, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_encode_e2m1(v[i]);
}

void oracle_silu32_n(const float *g, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_silu32(g[i]);
}

void oracle_group_scale_n(const float *amax, float *s, uint8_t *e8, int64_t n, int32_t qdtype,
                          int32_t round_pow2)
{
    for (int64_t i = 0; i < n; ++i) s[i] = oracle_group_scale(amax[i], qdtype, round_pow2, &e8[i]);
}

void oracle_code_value_n(const uint8_t *codes, float *out, int64_t n, int32_t qdtype)
{
    for (int64_t i = 0; i < n; ++i) out[i] = code_value(qdtype, codes[i]);
}

void oracle_f32_to_bf16_n(const float *v, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = f32_to_bf16_rne(v[i]);
}

/* Step 6's division, elementwise: out[i] = x[i] / s[i]. */
void oracle_div_n(const float *x, const float *s, float *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = x[i] / s[i];
}
