// tk_quant.hip -- gfx950 kernels and C ABI for the per-token / per-group
// activation cast and its fused SwiGLU form.
//
// What is computed: "Tile Kernels" (PyPI, v2.0.0), Features (per-token FP8/FP4
// casting, fused SwiGLU + quantization); "TileKernels" (aiwiki.ai), section
// Quantization (groups of 16/32/64/128 channels, power-of-two scale rounding,
// packed UE8M0 scales); "TileKernels, TileLang kernels for MoE routing and
// low-precision quantization" (hysenlabs.com), Seven kernel families (the
// activation and the narrowing in one pass).  The arithmetic contract is
// written out in include/tk_quant.h.
//
// Design (CDNA4, wave64): the cast is a pure stream, so there is no MFMA and
// no LDS staging of data.  A wave owns a run of U "segments" of one row; a
// segment is 512 columns, one 16-byte load (8 bf16) per lane, so each load
// instruction reads 1 KiB contiguously.  Every group size divides 512, and a
// group of G columns is G/8 consecutive lanes of one DPP row (16 lanes), so
// the group amax is a 1..4-step DPP butterfly with no LDS and no barrier.
// All U segments are loaded before any is converted, to keep U KiB per wave
// in flight.  Codes are written with one 8-byte (E4M3) or 4-byte (E2M1)
// store per lane, i.e. 512 or 256 contiguous bytes per wave instruction.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "tk_quant.h"

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;
constexpr int kBlock = kWave * kWavesPerBlock;
constexpr int kSegCols = kWave * 8;   // columns per wave per segment

constexpr int kE4M3 = TK_QDTYPE_E4M3;
constexpr int kE2M1 = TK_QDTYPE_E2M1;
constexpr int kScaleF32 = TK_SCALE_F32;
constexpr int kScaleUE8M0 = TK_SCALE_UE8M0_X4;

struct CastParams {
    const uint16_t *x;   // bf16 bits
    int64_t rows, cols, x_ld;
    uint8_t *q;
    int64_t q_ld;
    void *s;
    int64_t s_ld;
};

// ---------------------------------------------------------------------------
// silu32 table.  silu32(g) = fp32 nearest to g / (1 + e^-g) is needed exactly
// (correctly rounded) for every bf16 gate.  Outside |g| in [2^-26, 128] it has
// closed forms:
//   |g| < 2^-26: silu(g) = (g/2)(1 + g/2 + O(g^3)); the relative offset from
//                g/2 is below 2^-27, under half an fp32 ulp, and g/2 is an
//                fp32 value, so silu32(g) = g * 0.5f.
//   g > 128:     g - silu(g) = g e^-g / (1 + e^-g) < g 2^-184: rounds to g.
//   g < -128:    |silu(g)| < |g| e^g < 2^-150 for all such g: rounds to -0.
// Inside, the value comes from a table indexed by the bf16 magnitude and sign,
// built once per device by silu_table_kernel in fp64 and rounded once to fp32.
constexpr uint32_t kSiluLo = 0x3280;   // bf16 magnitude bits of 2^-26
constexpr uint32_t kSiluHi = 0x4300;   // bf16 magnitude bits of 128
constexpr int kSiluEntries = 2 * int(kSiluHi - kSiluLo + 1);   // sign interleaved

__device__ float g_silu_table[kSiluEntries];

// Round main + tail (|tail| small against |main|) to the nearest fp32, ties
// to even, as one rounding of the exact sum.  TwoSum (Knuth) gives s + e ==
// main + tail exactly; s alone decides unless it sits exactly on a midpoint
// between two fp32 values, where the sign of e decides.  main is never 0 here.
__device__ float round_sum_to_f32(double main, double tail)
{
    const double s = main + tail;
    const double bb = s - main;
    const double e = (main - (s - bb)) + (tail - bb);
    const float f = float(s);
    if (e == 0.0) return f;
    const uint32_t fb = __float_as_uint(f);
    const float away = __uint_as_float(fb + 1u);     // next fp32 away from zero
    const float toward = __uint_as_float(fb - 1u);   // next fp32 toward zero
    const bool e_outward = (e > 0.0) == (f > 0.0f);
    if (s == 0.5 * (double(f) + double(away))) return e_outward ? away : f;
    if (s == 0.5 * (double(f) + double(toward))) return e_outward ? f : toward;
    return f;
}

// One table entry per thread.
//   |g| < 2^-6: silu(g) = g/2 + g^2/4 - g^4/48 + g^6/480 - 17 g^8/80640 + ...
//     g/2 + g^2/4 is exact in fp64 (g has 8 significant bits); the tail is
//     added by round_sum_to_f32.  Here g/2 + g^2/4 can fall exactly on an fp32
//     midpoint (e.g. g = -1.125 * 2^-17), where only the tail's sign decides.
//   |g| >= 2^-6: every exact table value lies at least 4e-5 fp32 ulp away
//     from a midpoint between two fp32 values (checked at 50 digits, subnormal
//     results included), while the fp64 evaluation errs by well under 2^-26
//     fp32 ulp, so one fp64 -> fp32 rounding gives the correctly rounded value.
__global__ void silu_table_kernel()
{
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= kSiluEntries) return;
    const uint32_t mag = kSiluLo + uint32_t(i >> 1);
    const uint32_t bits = (uint32_t(i & 1) << 15) | mag;
    const double g = double(__uint_as_float(bits << 16));
    float r;
    if (fabs(g) < 0x1p-6) {
        const double g2 = g * g;
        const double head = g * 0.5 + g2 * 0.25;
        const double tail = g2 * g2 * (-1.0 / 48.0 + g2 * (1.0 / 480.0 - g2 * (17.0 / 80640.0)));
        r = round_sum_to_f32(head, tail);
    } else if (g >= 0.0) {
        r = float(g / (1.0 + exp(-g)));
    } else {
        const double e = exp(g);
        r = float((g * e) / (1.0 + e));
    }
    g_silu_table[i] = r;
}

// ---------------------------------------------------------------------------
// Cross-lane helpers.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v)
{
    // Every DPP pattern used here reads a lane inside the same 16-lane row, so
    // all lanes are written (row and bank masks full).
    return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), CTRL, 0xF, 0xF, false));
}

// Max over the G/8 consecutive lanes that hold one group; every lane of the
// group receives the result.  Values are fp32 bit patterns of |x|, for which
// unsigned order equals numeric order.
template <int G>
__device__ __forceinline__ uint32_t group_max(uint32_t v)
{
    if constexpr (G >= 16) v = max(v, dpp_mov<0xB1>(v));    // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (G >= 32) v = max(v, dpp_mov<0x4E>(v));    // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (G >= 64) v = max(v, dpp_mov<0x141>(v));   // row_half_mirror: 8-lane halves
    if constexpr (G >= 128) v = max(v, dpp_mov<0x140>(v));  // row_mirror: 16-lane row
    return v;
}

__device__ __forceinline__ uint32_t shfl_u32(uint32_t v, int src_lane)
{
    return uint32_t(__builtin_amdgcn_ds_bpermute((src_lane & 63) << 2, int(v)));
}

// ---------------------------------------------------------------------------
// The per-segment cast: 8 fp32 values per lane (columns col .. col+7 of one
// row), their |max| bits, the row's output pointers.

template <int G, int QD, bool POW2, int SF>
__device__ __forceinline__ void cast_segment(const float (&x)[8], uint32_t amax_bits, bool valid,
                                             int lane, int64_t col, uint8_t *qrow, void *srow)
{
    constexpr float D = (QD == kE4M3) ? 448.0f : 6.0f;
    amax_bits = group_max<G>(amax_bits);
    const float a = fmaxf(__uint_as_float(amax_bits), 1e-4f);
    float s = a / D;                       // IEEE fp32 division
    float inv = 0.0f;
    uint32_t e8 = 0;
    if constexpr (POW2) {
        // s is normal (>= 1e-4f / 448): 2^ceil(log2 s) from the exponent and
        // mantissa fields; E lies in [105, 253], so 2^(127-E) is normal too.
        const uint32_t b = __float_as_uint(s);
        const uint32_t E = (b >> 23) + ((b & 0x7FFFFFu) != 0u);
        e8 = E;
        s = __uint_as_float(E << 23);
        inv = __uint_as_float((254u - E) << 23);
    }
    float v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        // x * 2^-e is the exact quotient x / 2^e rounded once, as x / s is.
        v[i] = POW2 ? x[i] * inv : x[i] / s;
        v[i] = __builtin_amdgcn_fmed3f(v[i], D, -D);
    }
    if (valid) {
        if constexpr (QD == kE4M3) {
            uint32_t lo = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], 0, false));
            lo = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], int(lo), true));
            uint32_t hi = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], 0, false));
            hi = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], int(hi), true));
            *reinterpret_cast<uint2 *>(qrow + col) = make_uint2(lo, hi);
        } else {
            uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0], v[1], 1.0f, 0);
            r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], 1.0f, 1);
            r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], 1.0f, 2);
            r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], 1.0f, 3);
            *reinterpret_cast<uint32_t *>(qrow + col / 2) = r;
        }
    }
    constexpr int kLanesPerGroup = G / 8;
    if constexpr (SF == kScaleF32) {
        if (valid && (lane % kLanesPerGroup) == 0)
            static_cast<float *>(srow)[col / G] = s;
    } else {
        // Four consecutive groups' exponent bytes -> one little-endian int32,
        // written by the first lane of the first group.
        const uint32_t b1 = shfl_u32(e8, lane + kLanesPerGroup);
        const uint32_t b2 = shfl_u32(e8, lane + 2 * kLanesPerGroup);
        const uint32_t b3 = shfl_u32(e8, lane + 3 * kLanesPerGroup);
        if (valid && (lane % (4 * kLanesPerGroup)) == 0)
            static_cast<uint32_t *>(srow)[col / (4 * G)] = e8 | (b1 << 8) | (b2 << 16) | (b3 << 24);
    }
}

__device__ __forceinline__ void widen8(const uint4 &w, float (&x)[8])
{
    const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(ws[k] << 16);
        x[2 * k + 1] = __uint_as_float(ws[k] & 0xFFFF0000u);
    }
}

// |x| max of 8 bf16 as fp32 bits: bf16 magnitudes compare as unsigned 16-bit
// integers, two per packed max.
__device__ __forceinline__ uint32_t amax_bits_bf16x8(const uint4 &w)
{
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    const uint32_t m = 0x7FFF7FFFu;
    const uint32_t a = w.x & m, b = w.y & m, c = w.z & m, d = w.w & m;
    u16x2 va = __builtin_bit_cast(u16x2, a), vb = __builtin_bit_cast(u16x2, b);
    u16x2 vc = __builtin_bit_cast(u16x2, c), vd = __builtin_bit_cast(u16x2, d);
    u16x2 t = __builtin_elementwise_max(__builtin_elementwise_max(va, vb),
                                        __builtin_elementwise_max(vc, vd));
    const uint32_t lo = t.x, hi = t.y;
    return max(lo, hi) << 16;
}

// ---------------------------------------------------------------------------
// Kernels.  Work unit = (row, run of U segments); a wave takes units in a
// grid-stride loop (the unit index is wave-uniform, so DPP and bpermute always
// run with every lane active; lanes past the row end only skip their stores).

template <int G, int QD, bool POW2, int SF, int U>
__global__ __launch_bounds__(kBlock) void cast_kernel(CastParams p)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    const int64_t nwaves = int64_t(gridDim.x) * kWavesPerBlock;
    const int64_t nseg = (p.cols + kSegCols - 1) / kSegCols;
    const int64_t runs = (nseg + U - 1) / U;
    const int64_t units = p.rows * runs;
    for (int64_t unit = wave; unit < units; unit += nwaves) {
        const int64_t row = unit / runs;
        const int64_t col0 = (unit - row * runs) * U * kSegCols + lane * 8;
        const uint16_t *xrow = p.x + row * p.x_ld;
        uint4 w[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t col = col0 + k * kSegCols;
            w[k] = (col < p.cols) ? *reinterpret_cast<const uint4 *>(xrow + col) : make_uint4(0, 0, 0, 0);
        }
        uint8_t *qrow = p.q + row * p.q_ld;
        void *srow = (SF == kScaleF32) ? static_cast<void *>(static_cast<float *>(p.s) + row * p.s_ld)
                                       : static_cast<void *>(static_cast<uint32_t *>(p.s) + row * p.s_ld);
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t col = col0 + k * kSegCols;
            float x[8];
            widen8(w[k], x);
            cast_segment<G, QD, POW2, SF>(x, amax_bits_bf16x8(w[k]), col < p.cols, lane, col, qrow, srow);
        }
    }
}

__device__ __forceinline__ float silu32_lookup(uint32_t gbits, float g, const float *tab)
{
    const uint32_t mag = gbits & 0x7FFFu;
    const uint32_t neg = (gbits >> 15) & 1u;
    const uint32_t m = min(max(mag, kSiluLo), kSiluHi);
    const float t = tab[2 * (m - kSiluLo) + neg];
    float r = (mag < kSiluLo) ? g * 0.5f : t;
    r = (mag > kSiluHi) ? (neg ? -0.0f : g) : r;
    return r;
}

__global__ __launch_bounds__(kBlock) void silu32_kernel(const uint16_t *g, float *out, int64_t n)
{
    const int64_t i = int64_t(blockIdx.x) * kBlock + threadIdx.x;
    if (i >= n) return;
    const uint32_t b = g[i];
    out[i] = silu32_lookup(b, __uint_as_float(b << 16), g_silu_table);
}

template <int G, int QD, bool POW2, int SF, int U>
__global__ __launch_bounds__(kBlock) void swiglu_cast_kernel(CastParams p)
{
    __shared__ float tab[kSiluEntries];
    for (int i = threadIdx.x; i < kSiluEntries; i += kBlock) tab[i] = g_silu_table[i];
    __syncthreads();

    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = int64_t(blockIdx.x) * kWavesPerBlock + (threadIdx.x >> 6);
    const int64_t nwaves = int64_t(gridDim.x) * kWavesPerBlock;
    const int64_t nseg = (p.cols + kSegCols - 1) / kSegCols;
    const int64_t runs = (nseg + U - 1) / U;
    const int64_t units = p.rows * runs;
    for (int64_t unit = wave; unit < units; unit += nwaves) {
        const int64_t row = unit / runs;
        const int64_t col0 = (unit - row * runs) * U * kSegCols + lane * 8;
        const uint16_t *grow = p.x + row * p.x_ld;
        const uint16_t *urow = grow + p.cols;
        uint4 wg[U], wu[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t col = col0 + k * kSegCols;
            const bool ok = col < p.cols;
            wg[k] = ok ? *reinterpret_cast<const uint4 *>(grow + col) : make_uint4(0, 0, 0, 0);
            wu[k] = ok ? *reinterpret_cast<const uint4 *>(urow + col) : make_uint4(0, 0, 0, 0);
        }
        uint8_t *qrow = p.q + row * p.q_ld;
        void *srow = (SF == kScaleF32) ? static_cast<void *>(static_cast<float *>(p.s) + row * p.s_ld)
                                       : static_cast<void *>(static_cast<uint32_t *>(p.s) + row * p.s_ld);
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t col = col0 + k * kSegCols;
            float g[8], u[8], h[8];
            widen8(wg[k], g);
            widen8(wu[k], u);
            const uint32_t gw[4] = {wg[k].x, wg[k].y, wg[k].z, wg[k].w};
            uint32_t amax = 0;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const uint32_t gb = (i & 1) ? (gw[i / 2] >> 16) : (gw[i / 2] & 0xFFFFu);
                h[i] = silu32_lookup(gb, g[i], tab) * u[i];
                amax = max(amax, __float_as_uint(h[i]) & 0x7FFFFFFFu);
            }
            cast_segment<G, QD, POW2, SF>(h, amax, col < p.cols, lane, col, qrow, srow);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    std::once_flag once;
    tk_status status = TK_ERROR_DEVICE;
    int cus = 0;
    std::once_flag table_once;
    tk_status table_status = TK_ERROR_DEVICE;
};
DeviceInfo g_devices[kMaxDevices];

tk_status device_info(int *dev_out, DeviceInfo **info_out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return TK_ERROR_DEVICE;
    DeviceInfo &d = g_devices[dev];
    std::call_once(d.once, [&] {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
        if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return;
        d.cus = prop.multiProcessorCount;
        d.status = TK_SUCCESS;
    });
    *dev_out = dev;
    *info_out = &d;
    return d.status;
}

tk_status prepare_tables(DeviceInfo &d, hipStream_t stream)
{
    std::call_once(d.table_once, [&] {
        const int threads = 256;
        hipLaunchKernelGGL(silu_table_kernel, dim3((kSiluEntries + threads - 1) / threads), dim3(threads),
                           0, stream);
        if (hipGetLastError() != hipSuccess) { d.table_status = TK_ERROR_LAUNCH; return; }
        if (hipStreamSynchronize(stream) != hipSuccess) { d.table_status = TK_ERROR_DEVICE; return; }
        d.table_status = TK_SUCCESS;
    });
    return d.table_status;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

tk_status validate(const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *q, int64_t q_ld,
                   void *scales, int64_t s_ld, int32_t group, int32_t out_dtype, int32_t round_pow2,
                   int32_t scale_fmt, bool swiglu)
{
    if (group != 16 && group != 32 && group != 64 && group != 128) return TK_ERROR_INVALID_VALUE;
    if (out_dtype != kE4M3 && out_dtype != kE2M1) return TK_ERROR_INVALID_VALUE;
    if (scale_fmt != kScaleF32 && scale_fmt != kScaleUE8M0) return TK_ERROR_INVALID_VALUE;
    if (rows < 0 || cols <= 0 || cols % group != 0) return TK_ERROR_INVALID_VALUE;
    const int64_t ngroups = cols / group;
    if (scale_fmt == kScaleUE8M0 && (!round_pow2 || ngroups % 4 != 0)) return TK_ERROR_INVALID_VALUE;
    const int64_t in_cols = swiglu ? 2 * cols : cols;
    const int64_t q_cols = (out_dtype == kE4M3) ? cols : cols / 2;
    const int64_t s_cols = (scale_fmt == kScaleF32) ? ngroups : ngroups / 4;
    if (x_ld < in_cols || q_ld < q_cols || s_ld < s_cols) return TK_ERROR_INVALID_VALUE;
    if (rows == 0) return TK_SUCCESS;
    if (!x || !q || !scales) return TK_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || (x_ld * 2) % 16 != 0) return TK_ERROR_MISALIGNED;
    const int64_t qa = (out_dtype == kE4M3) ? 8 : 4;
    if (!aligned(q, uintptr_t(qa)) || q_ld % qa != 0) return TK_ERROR_MISALIGNED;
    if (!aligned(scales, 4)) return TK_ERROR_MISALIGNED;
    return TK_SUCCESS;
}

using KernelFn = void (*)(CastParams);

// Kernel pointers by [group index][out dtype][variant]; variant 0 = plain
// fp32 scale, 1 = power-of-two fp32 scale, 2 = power-of-two UE8M0 x4.
struct KernelTable {
    KernelFn fn[4][2][3];
};

template <bool SWIGLU, int G, int QD, bool POW2, int SF, int U>
constexpr KernelFn pick()
{
    if constexpr (SWIGLU) return swiglu_cast_kernel<G, QD, POW2, SF, U>;
    else return cast_kernel<G, QD, POW2, SF, U>;
}

template <bool SWIGLU, int G, int QD, int U>
void fill_variants(KernelFn (&t)[3])
{
    t[0] = pick<SWIGLU, G, QD, false, kScaleF32, U>();
    t[1] = pick<SWIGLU, G, QD, true, kScaleF32, U>();
    t[2] = pick<SWIGLU, G, QD, true, kScaleUE8M0, U>();
}

template <bool SWIGLU, int U>
KernelTable make_table()
{
    KernelTable t;
    fill_variants<SWIGLU, 16, kE4M3, U>(t.fn[0][0]);
    fill_variants<SWIGLU, 16, kE2M1, U>(t.fn[0][1]);
    fill_variants<SWIGLU, 32, kE4M3, U>(t.fn[1][0]);
    fill_variants<SWIGLU, 32, kE2M1, U>(t.fn[1][1]);
    fill_variants<SWIGLU, 64, kE4M3, U>(t.fn[2][0]);
    fill_variants<SWIGLU, 64, kE2M1, U>(t.fn[2][1]);
    fill_variants<SWIGLU, 128, kE4M3, U>(t.fn[3][0]);
    fill_variants<SWIGLU, 128, kE2M1, U>(t.fn[3][1]);
    return t;
}

int group_index(int32_t g) { return g == 16 ? 0 : g == 32 ? 1 : g == 64 ? 2 : 3; }

tk_status launch(bool swiglu, const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *q,
                 int64_t q_ld, void *scales, int64_t s_ld, int32_t group, int32_t out_dtype,
                 int32_t round_pow2, int32_t scale_fmt, void *stream)
{
    tk_status st = validate(x, rows, cols, x_ld, q, q_ld, scales, s_ld, group, out_dtype, round_pow2,
                            scale_fmt, swiglu);
    if (st != TK_SUCCESS || rows == 0) return st;
    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (swiglu) {
        st = prepare_tables(*info, s);
        if (st != TK_SUCCESS) return st;
    }

    const int variant = !round_pow2 ? 0 : (scale_fmt == kScaleF32 ? 1 : 2);
    const int gi = group_index(group);
    const int64_t nseg = (cols + kSegCols - 1) / kSegCols;
    KernelFn fn;
    int U;
    if (!swiglu) {
        static const KernelTable t1 = make_table<false, 1>();
        static const KernelTable t4 = make_table<false, 4>();
        static const KernelTable t7 = make_table<false, 7>();
        if (nseg % 7 == 0) { fn = t7.fn[gi][out_dtype][variant]; U = 7; }
        else if (nseg >= 4) { fn = t4.fn[gi][out_dtype][variant]; U = 4; }
        else { fn = t1.fn[gi][out_dtype][variant]; U = 1; }
    } else {
        static const KernelTable t1 = make_table<true, 1>();
        static const KernelTable t4 = make_table<true, 4>();
        if (nseg >= 4) { fn = t4.fn[gi][out_dtype][variant]; U = 4; }
        else { fn = t1.fn[gi][out_dtype][variant]; U = 1; }
    }
    const int64_t units = rows * ((nseg + U - 1) / U);
    int64_t blocks = (units + kWavesPerBlock - 1) / kWavesPerBlock;
    // SwiGLU blocks first copy the silu32 table into LDS: keep the grid near
    // two resident blocks per CU so that copy is amortised over many rows.
    const int64_t cap = swiglu ? int64_t(info->cus) * 2 : int64_t(1) << 30;
    if (blocks > cap) blocks = cap;
    CastParams p{static_cast<const uint16_t *>(x), rows, cols, x_ld, static_cast<uint8_t *>(q), q_ld,
                 scales, s_ld};
    void *args[] = {&p};
    if (hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(uint32_t(blocks)), dim3(kBlock), args, 0, s)
        != hipSuccess)
        return TK_ERROR_LAUNCH;
    return TK_SUCCESS;
}

}  // namespace

extern "C" {

tk_status tk_per_token_cast(const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *q,
                            int64_t q_ld, void *scales, int64_t s_ld, int32_t group, int32_t out_dtype,
                            int32_t round_pow2, int32_t scale_fmt, void *stream)
{
    return launch(false, x, rows, cols, x_ld, q, q_ld, scales, s_ld, group, out_dtype, round_pow2,
                  scale_fmt, stream);
}

tk_status tk_swiglu_per_token_cast(const void *gate_up, int64_t rows, int64_t cols, int64_t x_ld,
                                   void *q, int64_t q_ld, void *scales, int64_t s_ld, int32_t group,
                                   int32_t out_dtype, int32_t round_pow2, int32_t scale_fmt,
                                   void *stream)
{
    return launch(true, gate_up, rows, cols, x_ld, q, q_ld, scales, s_ld, group, out_dtype, round_pow2,
                  scale_fmt, stream);
}

tk_status tk_silu32_bf16(const void *g, void *out, int64_t n, void *stream)
{
    if (n < 0) return TK_ERROR_INVALID_VALUE;
    if (n == 0) return TK_SUCCESS;
    if (!g || !out) return TK_ERROR_INVALID_VALUE;
    if (!aligned(g, 2) || !aligned(out, 4)) return TK_ERROR_MISALIGNED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    tk_status st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    st = prepare_tables(*info, s);
    if (st != TK_SUCCESS) return st;
    const uint16_t *gp = static_cast<const uint16_t *>(g);
    float *op = static_cast<float *>(out);
    void *args[] = {&gp, &op, &n};
    const int64_t blocks = (n + kBlock - 1) / kBlock;
    if (blocks > int64_t(0x7FFFFFFF)) return TK_ERROR_INVALID_VALUE;
    if (hipLaunchKernel(reinterpret_cast<const void *>(silu32_kernel), dim3(uint32_t(blocks)), dim3(kBlock),
                        args, 0, s) != hipSuccess)
        return TK_ERROR_LAUNCH;
    return TK_SUCCESS;
}

tk_status tk_prepare_device(void)
{
    int dev = 0;
    DeviceInfo *info = nullptr;
    tk_status st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    return prepare_tables(*info, nullptr);
}

const char *tk_status_string(int32_t status)
{
    switch (status) {
    case TK_SUCCESS: return "TK_SUCCESS";
    case TK_ERROR_INVALID_VALUE: return "TK_ERROR_INVALID_VALUE: invalid size, group, format or null pointer";
    case TK_ERROR_UNSUPPORTED: return "TK_ERROR_UNSUPPORTED: request not provided by this build";
    case TK_ERROR_MISALIGNED: return "TK_ERROR_MISALIGNED: pointer or row stride breaks the alignment rule";
    case TK_ERROR_LAUNCH: return "TK_ERROR_LAUNCH: the HIP runtime refused the kernel launch";
    case TK_ERROR_DEVICE: return "TK_ERROR_DEVICE: no usable gfx950 device";
    default: return "TK_ERROR_UNKNOWN";
    }
}

int32_t tk_abi_version(void) { return TK_ABI_VERSION; }

}  // extern "C"
