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
// All U segments are loaded before any is converted.  Codes are written with
// one 8-byte (E4M3) or 4-byte (E2M1) store per lane, i.e. 512 or 256
// contiguous bytes per wave instruction.  Rows are addressed through buffer
// resource descriptors whose size is the row's length, so loads past the row
// end return zero and stores past it are dropped by the hardware: ragged
// tails need no predication.  Inputs and codes stream non-temporally; the
// short scale rows use write-back stores so that L2 merges their pieces.
// The plain cast runs the row form (cast_rows_kernel: one workgroup per row,
// the row's scale words gathered in LDS and stored once); the unit form
// (cast_kernel) serves rows whose scale words exceed the LDS staging size.

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "tk_device.h"
#include "tk_host.h"

namespace {

struct CastParams {
    const uint16_t *x;   // bf16 bits
    int64_t rows, cols, x_ld;
    uint8_t *q;
    int64_t q_ld;
    void *s;
    int64_t s_ld;
    int32_t xcd_log2;    // xcd_order run length over the workgroups (-1: none)
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
// Inside, the value comes from a table indexed by (bf16 magnitude, sign),
// built once per device by silu_table_kernel in fp64 and rounded once to
// fp32.  Entry 0 and the last entry hold a NaN: the fast lookup clamps the
// index onto them for gates outside the table, and the NaN then flags the
// group for the exact (closed-form) path.
constexpr uint32_t kSiluLo = 0x3280;   // bf16 magnitude bits of 2^-26
constexpr uint32_t kSiluHi = 0x4300;   // bf16 magnitude bits of 128
constexpr int kSiluValues = 2 * int(kSiluHi - kSiluLo + 1);
constexpr int kSiluEntries = kSiluValues + 2;
constexpr uint32_t kSentinel = 0x7FC00000u;   // quiet NaN

__device__ __align__(16) float g_silu_table[kSiluEntries];
static_assert(kSiluEntries % 4 == 0, "the table is copied in 16-byte pieces");

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
    if (i == 0 || i == kSiluEntries - 1) {
        g_silu_table[i] = __uint_as_float(kSentinel);
        return;
    }
    const int j = i - 1;
    const uint32_t mag = kSiluLo + uint32_t(j >> 1);
    const uint32_t bits = (uint32_t(j & 1) << 15) | mag;
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

// Byte offsets into the table for the two bf16 gates packed in w, with packed
// 16-bit integer ops: index = clamp((mag << 1 | sign) - (2 Lo - 1), 0, last).
// Gates below the table land on entry 0, gates above it on the last entry.
__device__ __forceinline__ u16x2 silu_offsets(uint32_t w)
{
    const u16x2 h = __builtin_bit_cast(u16x2, w);
    const u16x2 key = (h << (unsigned short)1) | (h >> (unsigned short)15);
    const u16x2 idx = __builtin_elementwise_min(
        __builtin_elementwise_sub_sat(key, u16x2((unsigned short)(2 * kSiluLo - 1))),
        u16x2((unsigned short)(kSiluEntries - 1)));
    return idx << (unsigned short)2;
}

__device__ __forceinline__ float table_at(const float *tab, unsigned short byte_off)
{
    return *reinterpret_cast<const float *>(reinterpret_cast<const char *>(tab) + byte_off);
}

// The closed forms outside the table, for the rare exact path.
__device__ float silu32_exact(uint32_t b, const float *tab)
{
    const uint32_t mag = b & 0x7FFFu, neg = (b >> 15) & 1u;
    const float g = __uint_as_float(b << 16);
    if (mag < kSiluLo) return g * 0.5f;
    if (mag > kSiluHi) return neg ? -0.0f : g;
    return tab[1 + 2 * (mag - kSiluLo) + neg];
}

// Codes and scales of one segment to the row's buffers.
template <int G, int QD, int SF>
__device__ __forceinline__ void store_segment(const Quantized &qz, int lane, uint32_t col,
                                              __amdgpu_buffer_rsrc_t qrow, __amdgpu_buffer_rsrc_t srow)
{
    if constexpr (QD == kE4M3) store8(qrow, col, qz.codes);
    else store4(qrow, col / 2, qz.codes.x);
    constexpr int kLanesPerGroup = G / 8;
    if constexpr (SF == kScaleF32) {
        if ((lane % kLanesPerGroup) == 0) store_scale(srow, (col / G) * 4, __float_as_uint(qz.s));
    } else {
        // Four consecutive groups' exponent bytes -> one little-endian int32,
        // written by the first lane of the first group.
        const uint32_t word = pack_e8_word<G>(qz.e8, lane);
        if ((lane % (4 * kLanesPerGroup)) == 0) store_scale(srow, (col / (4 * G)) * 4, word);
    }
}

// The scale words of a whole work unit (U segments) in one store: lane j
// fetches word j of the unit from the lane that computed it, then the first
// U * words-per-segment lanes write them contiguously (64 words per pass).
template <int G, int SF, int U>
__device__ __forceinline__ void store_unit_scales(const Quantized (&qz)[U], int lane, uint32_t unit_col0,
                                                  __amdgpu_buffer_rsrc_t srow)
{
    constexpr int kLanesPerGroup = G / 8;
    constexpr int kWordsPerSeg = SF == kScaleF32 ? kSegCols / G : kSegCols / G / 4;
    constexpr int kLanesPerWord = SF == kScaleF32 ? kLanesPerGroup : 4 * kLanesPerGroup;
    constexpr int kUnitWords = U * kWordsPerSeg;
    uint32_t word[U];
#pragma unroll
    for (int k = 0; k < U; ++k) {
        if constexpr (SF == kScaleF32) {
            word[k] = __float_as_uint(qz[k].s);
        } else {
            word[k] = pack_e8_word<G>(qz[k].e8, lane);
        }
    }
    const uint32_t first_word = SF == kScaleF32 ? unit_col0 / G : unit_col0 / (4 * G);
#pragma unroll
    for (int base = 0; base < kUnitWords; base += kWave) {
        const int j = base + lane;
        const int seg = j / kWordsPerSeg;
        const int src = (j % kWordsPerSeg) * kLanesPerWord;
        uint32_t v = 0;
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t t = shfl_u32(word[k], src);
            v = (seg == k) ? t : v;
        }
        if (j < kUnitWords) store_scale(srow, (first_word + uint32_t(j)) * 4u, v);
    }
}

template <int G, int QD, bool POW2, int SF>
__device__ __forceinline__ void cast_segment(const float (&x)[8], uint32_t amax_bits, int lane, uint32_t col,
                                             __amdgpu_buffer_rsrc_t qrow, __amdgpu_buffer_rsrc_t srow)
{
    store_segment<G, QD, SF>(quantize_segment<G, QD, POW2, kApplyClamp>(x, amax_bits), lane, col, qrow, srow);
}

// ---------------------------------------------------------------------------
// Work decomposition.  A row has nseg = ceil(cols / 512) segments, grouped in
// runs of U; a work unit is one (row, run).  Units are numbered row-major and
// handed out in order, so the waves resident at any moment cover one compact
// address window (the DRAM pages of a few consecutive rows), which measured
// faster than giving each workgroup its own distant stretch of rows.

struct Unit {
    int64_t row;
    uint32_t col0;   // first column of this lane in the run
};

template <int U>
__device__ __forceinline__ Unit decode_unit(int64_t unit, int64_t runs, int lane)
{
    int64_t row, run;
    if (unit <= int64_t(0xFFFFFFFF) && runs <= int64_t(0xFFFFFFFF)) {   // 32-bit division
        const uint32_t u32 = uint32_t(unit), r32 = uint32_t(runs);
        row = u32 / r32;
        run = u32 - uint32_t(row) * r32;
    } else {
        row = unit / runs;
        run = unit - row * runs;
    }
    return Unit{row, uint32_t(run) * uint32_t(U * kSegCols) + uint32_t(lane) * 8u};
}

// Descriptors of one row's codes and scales, sized to exactly that row.
template <int G, int QD, int SF>
__device__ __forceinline__ void output_rows(const CastParams &p, int64_t row, __amdgpu_buffer_rsrc_t &qrow,
                                            __amdgpu_buffer_rsrc_t &srow)
{
    const uint32_t cols = uint32_t(p.cols);
    qrow = row_buffer(p.q + row * p.q_ld, QD == kE4M3 ? cols : cols / 2);
    if constexpr (SF == kScaleF32)
        srow = row_buffer(static_cast<float *>(p.s) + row * p.s_ld, (cols / G) * 4u);
    else
        srow = row_buffer(static_cast<uint32_t *>(p.s) + row * p.s_ld, cols / G);
}

// ---------------------------------------------------------------------------
// Kernels.  A wave takes units in a grid-stride loop (one unit per wave when
// the grid covers all units).  The unit index is wave-uniform, so DPP and
// bpermute always run with every lane active.

template <int G, int QD, bool POW2, int SF, int U, int WPB>
__global__ __launch_bounds__(kWave * WPB) void cast_kernel(CastParams p)
{
    const int lane = threadIdx.x & (kWave - 1);
    // threadIdx.x >> 6 is the same on every lane of a wave; readfirstlane tells
    // the compiler so, which keeps the row descriptors in scalar registers.
    const int64_t wave = int64_t(blockIdx.x) * WPB + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = int64_t(gridDim.x) * WPB;
    const int64_t nseg = (p.cols + kSegCols - 1) / kSegCols;
    const int64_t runs = (nseg + U - 1) / U;
    const int64_t units = p.rows * runs;
    for (int64_t unit = wave; unit < units; unit += nwaves) {
        const Unit un = decode_unit<U>(unit, runs, lane);
        const __amdgpu_buffer_rsrc_t xrow = row_buffer(p.x + un.row * p.x_ld, uint32_t(p.cols) * 2u);
        u32x4 w[U];
#pragma unroll
        for (int k = 0; k < U; ++k) w[k] = load16(xrow, (un.col0 + k * kSegCols) * 2u);
        __amdgpu_buffer_rsrc_t qrow, srow;
        output_rows<G, QD, SF>(p, un.row, qrow, srow);
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float x[8];
            widen8(w[k], x);
            cast_segment<G, QD, POW2, SF>(x, amax_bits_bf16x8(w[k]), lane, un.col0 + k * kSegCols, qrow, srow);
        }
    }
}

// Row-per-workgroup form of the cast.  The scale stores of the unit form are
// many small partial-line writes (one per 512-column segment); here every
// wave of the workgroup puts its scales into LDS and the row's scales leave in
// one coalesced store per 256 bytes after a barrier.  Workgroups take rows in
// order (grid-stride), so the resident rows still form one compact window.
// Wave w of the W in the workgroup converts runs w, w + W, ... of the row.
template <int G, int QD, bool POW2, int SF, int U>
__global__ __launch_bounds__(1024) void cast_rows_kernel(CastParams p)
{
    extern __shared__ uint32_t row_scales[];     // the row's scale words
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = int(blockDim.x) >> 6;
    const uint32_t cols = uint32_t(p.cols);
    const int runs = int((cols + U * kSegCols - 1) / (U * kSegCols));
    const uint32_t s_words = SF == kScaleF32 ? cols / G : cols / G / 4;
    constexpr int kLanesPerGroup = G / 8;
    for (int64_t row = xcd_order(blockIdx.x, p.rows, p.xcd_log2); row < p.rows; row += gridDim.x) {
        const __amdgpu_buffer_rsrc_t xrow = row_buffer(p.x + row * p.x_ld, cols * 2u);
        __amdgpu_buffer_rsrc_t qrow, srow;
        output_rows<G, QD, SF>(p, row, qrow, srow);
        for (int run = wave; run < runs; run += nw) {
            const uint32_t col0 = uint32_t(run) * uint32_t(U * kSegCols) + uint32_t(lane) * 8u;
            u32x4 w[U];
#pragma unroll
            for (int k = 0; k < U; ++k) w[k] = load16(xrow, (col0 + k * kSegCols) * 2u);
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const uint32_t col = col0 + k * kSegCols;
                float x[8];
                widen8(w[k], x);
                const uint32_t amax = amax_bits_bf16x8(w[k]);
                const Quantized qz = quantize_segment<G, QD, POW2, kApplyClamp>(x, amax);
                if constexpr (QD == kE4M3) store8(qrow, col, qz.codes);
                else store4(qrow, col / 2, qz.codes.x);
                if constexpr (SF == kScaleF32) {
                    if ((lane % kLanesPerGroup) == 0 && col < cols) row_scales[col / G] = __float_as_uint(qz.s);
                } else {
                    // four groups' bytes packed with DPP moves, one word per 4 groups
                    // (a byte per group straight into LDS, fewer VALU instructions,
                    // measured 1 % slower on this memory-bound kernel)
                    const uint32_t word = pack_e8_word<G>(qz.e8, lane);
                    if ((lane % (4 * kLanesPerGroup)) == 0 && col < cols) row_scales[col / (4 * G)] = word;
                }
            }
        }
        __syncthreads();
        for (uint32_t t = threadIdx.x; t < s_words; t += blockDim.x) store_scale(srow, t * 4u, row_scales[t]);
        __syncthreads();                         // the next row reuses row_scales
    }
}

// Row form of the cast of fp32 activations.  A lane's 16-byte load holds 4
// consecutive values, so each load instruction covers 1 KiB of the row
// contiguously (reading 8 consecutive values per lane as two 16-byte loads
// 32 bytes apart measured 8-10 % slower as a plain read stream): a piece of
// 256 columns per instruction, P pieces per wave and run.  A group spans G/4
// lanes of a piece; its scale is staged in LDS by the group's first lane
// (UE8M0: one byte per group, four groups to the word).  P = 4 for up to
// 4096 rows and 2 above (measured at 7168 columns: P = 4 is 6 % faster at
// 4096 rows, P = 2 3-5 % faster at 16384 and 32768).
constexpr int kF32Cols = 256;              // columns per piece (one 1 KiB load per wave)
constexpr int64_t kF32FewRows = 4096;
constexpr int64_t kF32HalvesBytes = int64_t(512) << 20;

// Max over the G/4 consecutive lanes that hold one group of a piece.
template <int G>
__device__ __forceinline__ uint32_t piece_group_max(uint32_t v, int lane)
{
    if constexpr (G <= 64) return group_max<2 * G>(v);
    else {
        v = group_max<128>(v);                   // 16 lanes
        return max(v, shfl_u32(v, lane ^ 16));   // 32 lanes
    }
}

// 4 clamped values -> codes: E4M3 in 4 bytes, E2M1 in 4 nibbles of the low
// 16 bits (value 2i in the low nibble of byte i; the high 16 bits are not
// defined, and only the low half is stored).  As in encode8, the first
// converter is given its own first input's bits as the word to write into.
template <int QD>
__device__ __forceinline__ uint32_t encode4(const float (&v)[4])
{
    if constexpr (QD == kE4M3) {
        const uint32_t lo = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], __float_as_int(v[0]), false));
        return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], int(lo), true));
    } else {
        const uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(v[0]), v[0], v[1], 1.0f, 0);
        return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], 1.0f, 1);
    }
}

template <int G, int QD, bool POW2, int SF, int P, int PARTS = 1>
__global__ __launch_bounds__(1024) void cast_rows_f32_kernel(CastParams p)
{
    extern __shared__ uint32_t row_scales[];     // the part's scale words
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = int(blockDim.x) >> 6;
    const uint32_t cols = uint32_t(p.cols);
    const uint32_t part_cols = cols / PARTS;     // whole runs and scale words (host-checked)
    constexpr uint32_t kRunCols = P * kF32Cols;
    const int runs = int((part_cols + kRunCols - 1) / kRunCols);
    const uint32_t s_words = SF == kScaleF32 ? part_cols / G : part_cols / G / 4;
    constexpr int kLanesPerGroup = G / 4;
    const float *xf = reinterpret_cast<const float *>(p.x);
    const int64_t items = p.rows * PARTS;
    for (int64_t item = xcd_order(blockIdx.x, items, p.xcd_log2); item < items; item += gridDim.x) {
        const int64_t row = item / PARTS;
        const uint32_t c0 = uint32_t(item % PARTS) * part_cols;
        const __amdgpu_buffer_rsrc_t xrow = row_buffer(xf + row * p.x_ld, cols * 4u);
        __amdgpu_buffer_rsrc_t qrow, srow;
        output_rows<G, QD, SF>(p, row, qrow, srow);
        for (int run = wave; run < runs; run += nw) {
            const uint32_t col0 = c0 + uint32_t(run) * kRunCols + uint32_t(lane) * 4u;
            u32x4 w[P];
#pragma unroll
            for (int k = 0; k < P; ++k) w[k] = load16(xrow, (col0 + k * kF32Cols) * 4u);
#pragma unroll
            for (int k = 0; k < P; ++k) {
                const uint32_t col = col0 + k * kF32Cols;
                uint32_t amax = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) amax = max(amax, w[k][i] & 0x7FFFFFFFu);
                const Scale<QD, POW2> sc = group_scale<QD, POW2>(piece_group_max<G>(amax, lane));
                float v[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) v[i] = scaled<QD, POW2, kApplyClamp>(__uint_as_float(w[k][i]), sc.s, sc.inv);
                const uint32_t codes = encode4<QD>(v);
                if constexpr (QD == kE4M3) store4(qrow, col, codes);
                else __builtin_amdgcn_raw_buffer_store_b16(uint16_t(codes), qrow, int(col / 2), 0, kNonTemporal);
                if ((lane % kLanesPerGroup) == 0 && col < cols) {
                    if constexpr (SF == kScaleF32) row_scales[(col - c0) / G] = __float_as_uint(sc.s);
                    else reinterpret_cast<uint8_t *>(row_scales)[(col - c0) / G] = uint8_t(sc.e8);
                }
            }
        }
        __syncthreads();
        const uint32_t w0 = SF == kScaleF32 ? c0 / G : c0 / G / 4;   // the part's first scale word
        for (uint32_t t = threadIdx.x; t < s_words; t += blockDim.x) store_scale(srow, (w0 + t) * 4u, row_scales[t]);
        __syncthreads();                         // the next row reuses row_scales
    }
}

// Fused cast-and-cast-back: the cast's codes and scales stay in registers and
// are decoded straight back to bf16.
struct BackParams {
    const uint16_t *x;
    int64_t rows, cols, x_ld;
    uint16_t *y;         // bf16 bits
    int64_t y_ld;
    int32_t xcd_log2;    // xcd_order run length over the workgroups (-1: none)
};

template <int G, int QD, bool POW2, int U, int WPB>
__global__ __launch_bounds__(kWave * WPB) void cast_back_kernel(BackParams p)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = xcd_order(blockIdx.x, gridDim.x, p.xcd_log2) * WPB +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = int64_t(gridDim.x) * WPB;
    const int64_t nseg = (p.cols + kSegCols - 1) / kSegCols;
    const int64_t runs = (nseg + U - 1) / U;
    const int64_t units = p.rows * runs;
    const uint32_t row_bytes = uint32_t(p.cols) * 2u;
    for (int64_t unit = wave; unit < units; unit += nwaves) {
        const Unit un = decode_unit<U>(unit, runs, lane);
        const __amdgpu_buffer_rsrc_t xrow = row_buffer(p.x + un.row * p.x_ld, row_bytes);
        const __amdgpu_buffer_rsrc_t yrow = row_buffer(p.y + un.row * p.y_ld, row_bytes);
        u32x4 w[U];
#pragma unroll
        for (int k = 0; k < U; ++k) w[k] = load16(xrow, (un.col0 + k * kSegCols) * 2u);
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float x[8], y[8];
            widen8(w[k], x);
            const Quantized qz = quantize_segment<G, QD, POW2, kApplyClamp>(x, amax_bits_bf16x8(w[k]));
            dequant_codes<QD>(qz.codes, qz.s, y);
            store16(yrow, (un.col0 + k * kSegCols) * 2u, pack_bf16x8(y));
        }
    }
}

// Dequantization: codes + scales -> y = fl32(value * s), bf16 or fp32.
struct DequantParams {
    const uint8_t *q;
    int64_t rows, cols, q_ld;
    const void *s;
    int64_t s_ld;
    void *y;
    int64_t y_ld;        // elements of y's type
};

template <int G, int QD, int SF, bool OUT_F32, int U, int WPB>
__global__ __launch_bounds__(kWave * WPB) void dequant_kernel(DequantParams p)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = int64_t(blockIdx.x) * WPB + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = int64_t(gridDim.x) * WPB;
    const int64_t nseg = (p.cols + kSegCols - 1) / kSegCols;
    const int64_t runs = (nseg + U - 1) / U;
    const int64_t units = p.rows * runs;
    const uint32_t cols = uint32_t(p.cols);
    for (int64_t unit = wave; unit < units; unit += nwaves) {
        const Unit un = decode_unit<U>(unit, runs, lane);
        const __amdgpu_buffer_rsrc_t qrow = row_buffer(p.q + un.row * p.q_ld, QD == kE4M3 ? cols : cols / 2);
        const __amdgpu_buffer_rsrc_t srow =
            SF == kScaleF32 ? row_buffer(static_cast<const float *>(p.s) + un.row * p.s_ld, (cols / G) * 4u)
                            : row_buffer(static_cast<const uint32_t *>(p.s) + un.row * p.s_ld, cols / G);
        const __amdgpu_buffer_rsrc_t yrow =
            OUT_F32 ? row_buffer(static_cast<float *>(p.y) + un.row * p.y_ld, cols * 4u)
                    : row_buffer(static_cast<uint16_t *>(p.y) + un.row * p.y_ld, cols * 2u);
        u32x2 codes[U];
        uint32_t sw[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t col = un.col0 + k * kSegCols;
            if constexpr (QD == kE4M3)
                codes[k] = __builtin_amdgcn_raw_buffer_load_b64(qrow, int(col), 0, kNonTemporal);
            else
                codes[k] = u32x2{__builtin_amdgcn_raw_buffer_load_b32(qrow, int(col / 2), 0, kNonTemporal), 0u};
            sw[k] = SF == kScaleF32 ? __builtin_amdgcn_raw_buffer_load_b32(srow, int((col / G) * 4), 0, 0)
                                    : __builtin_amdgcn_raw_buffer_load_b32(srow, int((col / (4 * G)) * 4), 0, 0);
        }
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const uint32_t col = un.col0 + k * kSegCols;
            float sc;
            if constexpr (SF == kScaleF32) sc = __uint_as_float(sw[k]);
            else sc = __uint_as_float(((sw[k] >> (8 * ((col / G) % 4))) & 0xFFu) << 23);   // 2^(byte-127)
            float y[8];
            dequant_codes<QD>(codes[k], sc, y);
            if constexpr (OUT_F32) {
                store16(yrow, col * 4u, u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                                               __float_as_uint(y[3])});
                store16(yrow, col * 4u + 16u, u32x4{__float_as_uint(y[4]), __float_as_uint(y[5]),
                                                     __float_as_uint(y[6]), __float_as_uint(y[7])});
            } else {
                store16(yrow, col * 2u, pack_bf16x8(y));
            }
        }
    }
}

constexpr int kSiluBlock = 256;

// Diagnostic: silu32 of n bf16 gates (two per thread) through the same fast
// lookup + exact path as the fused kernel.
__global__ __launch_bounds__(kSiluBlock) void silu32_kernel(const uint16_t *g, float *out, int64_t n)
{
    const int64_t i = 2 * (int64_t(blockIdx.x) * kSiluBlock + threadIdx.x);
    if (i >= n) return;
    const uint32_t b0 = g[i], b1 = (i + 1 < n) ? g[i + 1] : 0u;
    const u16x2 off = silu_offsets(b0 | (b1 << 16));
    float r0 = table_at(g_silu_table, off.x), r1 = table_at(g_silu_table, off.y);
    if (__float_as_uint(r0) == kSentinel) r0 = silu32_exact(b0, g_silu_table);
    if (__float_as_uint(r1) == kSentinel) r1 = silu32_exact(b1, g_silu_table);
    out[i] = r0;
    if (i + 1 < n) out[i + 1] = r1;
}

template <int G, int QD, bool POW2, int SF, int U, int WPB>
__global__ __launch_bounds__(kWave * WPB) void swiglu_cast_kernel(CastParams p)
{
    __shared__ __align__(16) float tab[kSiluEntries];
    const int lane = threadIdx.x & (kWave - 1);
    // threadIdx.x >> 6 is the same on every lane of a wave; readfirstlane tells
    // the compiler so, which keeps the row descriptors in scalar registers.
    const int64_t wave = xcd_order(blockIdx.x, gridDim.x, p.xcd_log2) * WPB +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t nwaves = int64_t(gridDim.x) * WPB;
    const int64_t nseg = (p.cols + kSegCols - 1) / kSegCols;
    const int64_t runs = (nseg + U - 1) / U;
    const int64_t units = p.rows * runs;
    const uint32_t half_bytes = uint32_t(p.cols) * 2u;
    u32x4 wg[U], wu[U];
    auto load_unit = [&](const Unit &un) {
        const uint16_t *grow = p.x + un.row * p.x_ld;
        const __amdgpu_buffer_rsrc_t gate = row_buffer(grow, half_bytes);
        const __amdgpu_buffer_rsrc_t up = row_buffer(grow + p.cols, half_bytes);
#pragma unroll
        for (int k = 0; k < U; ++k) {
            wg[k] = load16(gate, (un.col0 + k * kSegCols) * 2u);
            wu[k] = load16(up, (un.col0 + k * kSegCols) * 2u);
        }
    };

    // The wave's first unit is requested before the table is copied; the
    // copy reads 16-byte pieces, all of a thread's in flight at once.
    int64_t unit = wave;
    Unit un{};
    if (unit < units) {
        un = decode_unit<U>(unit, runs, lane);
        load_unit(un);
    }
    {
        constexpr int kPieces = kSiluEntries / 4;
        constexpr int kPerThread = (kPieces + kWave * WPB - 1) / (kWave * WPB);
        const u32x4 *src = reinterpret_cast<const u32x4 *>(g_silu_table);
        u32x4 t[kPerThread];
#pragma unroll
        for (int c = 0; c < kPerThread; ++c) {
            const int i = int(threadIdx.x) + c * kWave * WPB;
            if (i < kPieces) t[c] = src[i];
        }
#pragma unroll
        for (int c = 0; c < kPerThread; ++c) {
            const int i = int(threadIdx.x) + c * kWave * WPB;
            if (i < kPieces) reinterpret_cast<u32x4 *>(tab)[i] = t[c];
        }
    }
    __syncthreads();

    for (; unit < units; ) {
        __amdgpu_buffer_rsrc_t qrow, srow;
        output_rows<G, QD, SF>(p, un.row, qrow, srow);
        Quantized qz[U];
#pragma unroll
        for (int k = 0; k < U; ++k) {
            float u[8], h[8];
            widen8(wu[k], u);
            uint32_t amax = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const u16x2 off = silu_offsets(wg[k][j]);
                h[2 * j] = table_at(tab, off.x) * u[2 * j];
                h[2 * j + 1] = table_at(tab, off.y) * u[2 * j + 1];
                amax = max(amax, max(__float_as_uint(h[2 * j]) & 0x7FFFFFFFu,
                                     __float_as_uint(h[2 * j + 1]) & 0x7FFFFFFFu));
            }
            // A NaN from a sentinel entry (a gate outside the table) makes the
            // bits exceed every finite magnitude; such segments, rare and
            // wave-uniform, take the exact path.
            if (__builtin_amdgcn_ballot_w64(amax > 0x7F7FFFFFu) != 0) {
                amax = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t gb = (i & 1) ? (wg[k][i / 2] >> 16) : (wg[k][i / 2] & 0xFFFFu);
                    h[i] = silu32_exact(gb, tab) * u[i];
                    amax = max(amax, __float_as_uint(h[i]) & 0x7FFFFFFFu);
                }
            }
            qz[k] = quantize_segment<G, QD, POW2, kApplyMul>(h, amax);
            if constexpr (QD == kE4M3) store8(qrow, un.col0 + k * kSegCols, qz[k].codes);
            else store4(qrow, (un.col0 + k * kSegCols) / 2, qz[k].codes.x);
        }
        store_unit_scales<G, SF, U>(qz, lane, un.col0 - uint32_t(lane) * 8u, srow);
        unit += nwaves;
        if (unit < units) {
            un = decode_unit<U>(unit, runs, lane);
            load_unit(un);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.

// Builds the current device's silu32 table once: a kernel on `stream`, then a
// wait for it.  The launch's own return code is checked (not hipGetLastError,
// which may hold an error left by an unrelated earlier call).  Inside a graph
// capture the kernel would only be recorded, so the build is refused there.
tk_status prepare_tables(DeviceInfo &d, hipStream_t stream)
{
    if (d.table_ready.load(std::memory_order_acquire)) return TK_SUCCESS;
    std::lock_guard<std::mutex> lock(d.table_mutex);
    if (d.table_ready.load(std::memory_order_relaxed)) return TK_SUCCESS;
    hipStreamCaptureStatus capture = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &capture) != hipSuccess) return TK_ERROR_LAUNCH;
    if (capture != hipStreamCaptureStatusNone) return TK_ERROR_UNSUPPORTED;
    const int threads = 256;
    if (hipLaunchKernel(reinterpret_cast<const void *>(silu_table_kernel),
                        dim3((kSiluEntries + threads - 1) / threads), dim3(threads), nullptr, 0, stream) != hipSuccess)
        return TK_ERROR_LAUNCH;
    if (hipStreamSynchronize(stream) != hipSuccess) return TK_ERROR_DEVICE;
    d.table_ready.store(true, std::memory_order_release);
    return TK_SUCCESS;
}

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
    if (in_cols >= (int64_t(1) << 29)) return TK_ERROR_UNSUPPORTED;   // row byte offsets are 32-bit
    if (!span_ok(rows, x_ld, in_cols, 2) || !span_ok(rows, q_ld, q_cols, 1) || !span_ok(rows, s_ld, s_cols, 4))
        return TK_ERROR_INVALID_VALUE;
    if (rows == 0) return TK_SUCCESS;
    if (!x || !q || !scales) return TK_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || (x_ld * 2) % 16 != 0) return TK_ERROR_MISALIGNED;
    const int64_t qa = (out_dtype == kE4M3) ? 8 : 4;
    if (!aligned(q, uintptr_t(qa)) || q_ld % qa != 0) return TK_ERROR_MISALIGNED;
    if (!aligned(scales, 4)) return TK_ERROR_MISALIGNED;
    return TK_SUCCESS;
}

using KernelFn = void (*)(CastParams);

// Launch shape of each kernel family (measured on MI355X over the cast's
// workloads): U segments (U KiB of bf16 per wave per unit) and WPB waves per
// workgroup.  The plain cast runs one unit per wave; the SwiGLU form keeps a
// bounded grid so that each workgroup's copy of the silu32 table into LDS
// serves many units.
#ifndef TK_CAST_U
#define TK_CAST_U 2
#endif
#ifndef TK_CAST_WPB
#define TK_CAST_WPB 2
#endif
#ifndef TK_SWIGLU_U
#define TK_SWIGLU_U 2
#endif
#ifndef TK_SWIGLU_WPB
#define TK_SWIGLU_WPB 16
#endif
#ifndef TK_SWIGLU_BLOCKS_PER_CU
#define TK_SWIGLU_BLOCKS_PER_CU 2
#endif
constexpr int kCastU = TK_CAST_U, kCastWPB = TK_CAST_WPB;
constexpr int kSwigluU = TK_SWIGLU_U, kSwigluWPB = TK_SWIGLU_WPB;
constexpr int kSwigluBlocksPerCU = TK_SWIGLU_BLOCKS_PER_CU;
constexpr int64_t kSwigluShortUnits = 1;
constexpr int kSwigluXcdRunLog2 = 4;

#ifndef TK_CAST_ROWS
#define TK_CAST_ROWS 1
#endif
constexpr bool kCastRows = TK_CAST_ROWS != 0;
constexpr int64_t kRowScaleLdsBytes = 32768;   // rows with more scale bytes use the unit form
constexpr int kCastFewU = 4;
constexpr int64_t kCastFewElems = int64_t(4096) * 7168;
constexpr int kRowMaxWaves = 16;

using CastFn = void (*)(CastParams);
struct RowTable {
    CastFn fn[4][2][3];
};

template <int P, int G, int QD, int U, int PARTS = 1>
void fill_rows(CastFn (&t)[3])
{
    if constexpr (P > 0) {                       // fp32 input, P pieces per wave, PARTS workgroups per row
        t[0] = cast_rows_f32_kernel<G, QD, false, kScaleF32, P, PARTS>;
        t[1] = cast_rows_f32_kernel<G, QD, true, kScaleF32, P, PARTS>;
        t[2] = cast_rows_f32_kernel<G, QD, true, kScaleUE8M0, P, PARTS>;
    } else {
        t[0] = cast_rows_kernel<G, QD, false, kScaleF32, U>;
        t[1] = cast_rows_kernel<G, QD, true, kScaleF32, U>;
        t[2] = cast_rows_kernel<G, QD, true, kScaleUE8M0, U>;
    }
}

// P = 0: the bf16 row kernel with runs of U segments; P > 0: the fp32 row
// kernel with P pieces per wave.
template <int P, int U = kCastU, int PARTS = 1>
RowTable make_row_table()
{
    RowTable t;
    fill_rows<P, 16, kE4M3, U, PARTS>(t.fn[0][0]);  fill_rows<P, 16, kE2M1, U, PARTS>(t.fn[0][1]);
    fill_rows<P, 32, kE4M3, U, PARTS>(t.fn[1][0]);  fill_rows<P, 32, kE2M1, U, PARTS>(t.fn[1][1]);
    fill_rows<P, 64, kE4M3, U, PARTS>(t.fn[2][0]);  fill_rows<P, 64, kE2M1, U, PARTS>(t.fn[2][1]);
    fill_rows<P, 128, kE4M3, U, PARTS>(t.fn[3][0]); fill_rows<P, 128, kE2M1, U, PARTS>(t.fn[3][1]);
    return t;
}

// Kernel pointers by [group index][out dtype][variant]; variant 0 = plain
// fp32 scale, 1 = power-of-two fp32 scale, 2 = power-of-two UE8M0 x4.
struct KernelTable {
    KernelFn fn[4][2][3];
};

template <bool SWIGLU, int G, int QD, bool POW2, int SF, int SU>
constexpr KernelFn pick()
{
    if constexpr (SWIGLU) return swiglu_cast_kernel<G, QD, POW2, SF, SU, kSwigluWPB>;
    else return cast_kernel<G, QD, POW2, SF, kCastU, kCastWPB>;
}

template <bool SWIGLU, int G, int QD, int SU>
void fill_variants(KernelFn (&t)[3])
{
    t[0] = pick<SWIGLU, G, QD, false, kScaleF32, SU>();
    t[1] = pick<SWIGLU, G, QD, true, kScaleF32, SU>();
    t[2] = pick<SWIGLU, G, QD, true, kScaleUE8M0, SU>();
}

// SU: segments per SwiGLU unit (the plain cast's unit form always takes kCastU).
template <bool SWIGLU, int SU = kSwigluU>
KernelTable make_table()
{
    KernelTable t;
    fill_variants<SWIGLU, 16, kE4M3, SU>(t.fn[0][0]);
    fill_variants<SWIGLU, 16, kE2M1, SU>(t.fn[0][1]);
    fill_variants<SWIGLU, 32, kE4M3, SU>(t.fn[1][0]);
    fill_variants<SWIGLU, 32, kE2M1, SU>(t.fn[1][1]);
    fill_variants<SWIGLU, 64, kE4M3, SU>(t.fn[2][0]);
    fill_variants<SWIGLU, 64, kE2M1, SU>(t.fn[2][1]);
    fill_variants<SWIGLU, 128, kE4M3, SU>(t.fn[3][0]);
    fill_variants<SWIGLU, 128, kE2M1, SU>(t.fn[3][1]);
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

    static const KernelTable cast_table = make_table<false>();
    static const KernelTable swiglu_table = make_table<true>();
    static const KernelTable swiglu_short_table = make_table<true, 1>();
    const int variant = !round_pow2 ? 0 : (scale_fmt == kScaleF32 ? 1 : 2);
    const int64_t s_words = scale_fmt == kScaleF32 ? cols / group : cols / group / 4;
    if (!swiglu && kCastRows && s_words * 4 <= kRowScaleLdsBytes) {
        // Runs of kCastFewU segments (fewer, longer-lived waves) for inputs of
        // up to kCastFewElems values whose grid still fills every wave slot of
        // the chip (32 per CU) at least once, kCastU otherwise.  Measured on
        // MI355X at 7168 columns: 4-segment runs 3.7 % faster at 4096 rows,
        // 1 % slower at 16384 and 9 % at 32768, 7 % slower at 128 rows.
        static const RowTable row_table = make_row_table<0>();
        static const RowTable row_table_few = make_row_table<0, kCastFewU>();
        const int64_t few_runs = (cols + kCastFewU * kSegCols - 1) / (kCastFewU * kSegCols);
        const bool few = rows * cols <= kCastFewElems && rows * few_runs >= int64_t(info->cus) * 32;
        const int U = few ? kCastFewU : kCastU;
        const int64_t runs = (cols + U * kSegCols - 1) / (U * kSegCols);
        const int waves = int(runs < kRowMaxWaves ? runs : kRowMaxWaves);
        int64_t blocks = rows < int64_t(0x7FFFFFFF) ? rows : int64_t(0x7FFFFFFF);
        CastParams p{static_cast<const uint16_t *>(x), rows, cols, x_ld, static_cast<uint8_t *>(q), q_ld,
                     scales, s_ld, xcd_run_log2(rows, blocks, cols * 2)};
        void *args[] = {&p};
        const CastFn fn = (few ? row_table_few : row_table).fn[group_index(group)][out_dtype][variant];
        if (hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(uint32_t(blocks)), dim3(kWave * waves), args,
                            size_t(s_words * 4), s) != hipSuccess)
            return TK_ERROR_LAUNCH;
        return TK_SUCCESS;
    }
    // SwiGLU: one-segment units while the persistent grid has a wave for each
    // of them, kSwigluU segments per unit above.  Measured on MI355X at 2048
    // columns: one-segment units 11 % faster at 2048 rows (one unit per
    // wave); two-segment units 2.8 % faster at 8192 rows on the workload's
    // gate N(0, std 2) and up N(0, 1) (four units per wave) and 4 % at 32768.
    const int64_t nseg = (cols + kSegCols - 1) / kSegCols;
    const bool short_units =
        swiglu && rows * nseg <= int64_t(info->cus) * kSwigluBlocksPerCU * kSwigluWPB * kSwigluShortUnits;
    const KernelTable &table = !swiglu ? cast_table : short_units ? swiglu_short_table : swiglu_table;
    const KernelFn fn = table.fn[group_index(group)][out_dtype][variant];
    const int U = !swiglu ? kCastU : short_units ? 1 : kSwigluU;
    const int wpb = swiglu ? kSwigluWPB : kCastWPB;
    const int64_t units = rows * ((nseg + U - 1) / U);
    int64_t blocks = (units + wpb - 1) / wpb;
    const int64_t cap = swiglu ? int64_t(info->cus) * kSwigluBlocksPerCU : int64_t(0x7FFFFFFF);
    if (blocks > cap) blocks = cap;     // the kernels loop over the remaining units
    // The SwiGLU grid's workgroups in XCD runs of 16 (measured on MI355X at
    // 8192 x 2 * 2048: 2.5 % faster than round-robin order; runs of 32: 1 %,
    // 64: slower; at 32768 rows 0.7 %).
    const int xcd = swiglu ? kSwigluXcdRunLog2 : -1;
    CastParams p{static_cast<const uint16_t *>(x), rows, cols, x_ld, static_cast<uint8_t *>(q), q_ld,
                 scales, s_ld, xcd};
    void *args[] = {&p};
    if (hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(uint32_t(blocks)), dim3(kWave * wpb), args,
                        0, s) != hipSuccess)
        return TK_ERROR_LAUNCH;
    return TK_SUCCESS;
}

// Cast-and-cast-back and dequantization run the plain cast's launch shape.
using BackFn = void (*)(BackParams);
using DequantFn = void (*)(DequantParams);

struct BackTable {
    BackFn fn[4][2][2];          // [group][code format][pow2]
};
struct DequantTable {
    DequantFn fn[4][2][2][2];    // [group][code format][scale format][fp32 out]
};

template <int G, int QD>
void fill_back(BackFn (&t)[2])
{
    t[0] = cast_back_kernel<G, QD, false, kCastU, kCastWPB>;
    t[1] = cast_back_kernel<G, QD, true, kCastU, kCastWPB>;
}

template <int G, int QD>
void fill_dequant(DequantFn (&t)[2][2])
{
    t[0][0] = dequant_kernel<G, QD, kScaleF32, false, kCastU, kCastWPB>;
    t[0][1] = dequant_kernel<G, QD, kScaleF32, true, kCastU, kCastWPB>;
    t[1][0] = dequant_kernel<G, QD, kScaleUE8M0, false, kCastU, kCastWPB>;
    t[1][1] = dequant_kernel<G, QD, kScaleUE8M0, true, kCastU, kCastWPB>;
}

BackTable make_back_table()
{
    BackTable t;
    fill_back<16, kE4M3>(t.fn[0][0]);  fill_back<16, kE2M1>(t.fn[0][1]);
    fill_back<32, kE4M3>(t.fn[1][0]);  fill_back<32, kE2M1>(t.fn[1][1]);
    fill_back<64, kE4M3>(t.fn[2][0]);  fill_back<64, kE2M1>(t.fn[2][1]);
    fill_back<128, kE4M3>(t.fn[3][0]); fill_back<128, kE2M1>(t.fn[3][1]);
    return t;
}

DequantTable make_dequant_table()
{
    DequantTable t;
    fill_dequant<16, kE4M3>(t.fn[0][0]);  fill_dequant<16, kE2M1>(t.fn[0][1]);
    fill_dequant<32, kE4M3>(t.fn[1][0]);  fill_dequant<32, kE2M1>(t.fn[1][1]);
    fill_dequant<64, kE4M3>(t.fn[2][0]);  fill_dequant<64, kE2M1>(t.fn[2][1]);
    fill_dequant<128, kE4M3>(t.fn[3][0]); fill_dequant<128, kE2M1>(t.fn[3][1]);
    return t;
}

bool valid_group(int32_t g) { return g == 16 || g == 32 || g == 64 || g == 128; }

// params points to the kernel's parameter struct; xcd_log2, if given, to its
// run-length field, set for workgroups that read wg_bytes of input each.
// Measured on MI355X at 32768 x 7168: the cast-and-cast-back 1.2 % faster in
// XCD order, dequantization 0.8 % slower (it keeps its order).
tk_status launch_unit_grid(const void *fn, int64_t rows, int64_t cols, void *params, int32_t *xcd_log2,
                           int64_t wg_bytes, hipStream_t s)
{
    const int64_t nseg = (cols + kSegCols - 1) / kSegCols;
    const int64_t units = rows * ((nseg + kCastU - 1) / kCastU);
    const int64_t need = (units + kCastWPB - 1) / kCastWPB;
    const int64_t blocks = need > int64_t(0x7FFFFFFF) ? int64_t(0x7FFFFFFF) : need;   // the kernels loop
    if (xcd_log2) *xcd_log2 = xcd_run_log2(need, blocks, wg_bytes);
    void *args[] = {params};
    if (hipLaunchKernel(fn, dim3(uint32_t(blocks)), dim3(kWave * kCastWPB), args, 0, s) != hipSuccess)
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

tk_status tk_per_token_cast_f32(const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *q,
                                int64_t q_ld, void *scales, int64_t s_ld, int32_t group, int32_t out_dtype,
                                int32_t round_pow2, int32_t scale_fmt, void *stream)
{
    // The bf16 checks apply to everything but the input's element size.
    tk_status st = validate(x, rows, cols, x_ld, q, q_ld, scales, s_ld, group, out_dtype, round_pow2,
                            scale_fmt, false);
    if (st == TK_ERROR_MISALIGNED && aligned(x, 16) && (x_ld * 4) % 16 == 0) {
        // recheck the outputs' alignment alone
        const int64_t qa = (out_dtype == kE4M3) ? 8 : 4;
        st = (!aligned(q, uintptr_t(qa)) || q_ld % qa != 0 || !aligned(scales, 4)) ? TK_ERROR_MISALIGNED
                                                                                   : TK_SUCCESS;
    }
    if (st != TK_SUCCESS || rows == 0) return st;
    if (!span_ok(rows, x_ld, cols, 4)) return TK_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || (x_ld * 4) % 16 != 0) return TK_ERROR_MISALIGNED;
    const int64_t s_words = scale_fmt == kScaleF32 ? cols / group : cols / group / 4;
    if (s_words * 4 > kRowScaleLdsBytes) return TK_ERROR_UNSUPPORTED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    static const RowTable table4 = make_row_table<4>();
    static const RowTable table2 = make_row_table<2>();
    static const RowTable table2h = make_row_table<2, kCastU, 2>();
    const bool few = rows <= kF32FewRows;
    const int variant = !round_pow2 ? 0 : (scale_fmt == kScaleF32 ? 1 : 2);
    const int64_t run_cols = (few ? 4 : 2) * kF32Cols;
    // Two workgroups per row (7 waves each at 7168 columns, in XCD order over the
    // halves) above kF32HalvesBytes of input, when each half is whole runs and
    // whole scale words.  Measured on MI355X at 7168 columns against one
    // 14-wave workgroup per row: -2.3 % at 32768 rows (940 MB), +0.7 % at
    // 16384, -0.9 % at 8192, equal at 4097.
    const int64_t word_cols = scale_fmt == kScaleF32 ? group : 4 * group;
    const int parts = (rows * cols * 4 > kF32HalvesBytes && cols % (2 * run_cols) == 0 && (cols / 2) % word_cols == 0)
                          ? 2 : 1;
    const RowTable &table = few ? table4 : parts == 2 ? table2h : table2;
    const int64_t runs = (cols / parts + run_cols - 1) / run_cols;
    const int waves = int(runs < kRowMaxWaves ? runs : kRowMaxWaves);
    const int64_t items = rows * parts;
    const int64_t blocks = items < int64_t(0x7FFFFFFF) ? items : int64_t(0x7FFFFFFF);
    CastParams p{static_cast<const uint16_t *>(x), rows, cols, x_ld, static_cast<uint8_t *>(q), q_ld, scales,
                 s_ld, xcd_run_log2(items, blocks, cols * 4 / parts)};
    void *args[] = {&p};
    const CastFn fn = table.fn[group_index(group)][out_dtype][variant];
    if (hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(uint32_t(blocks)), dim3(kWave * waves), args,
                        size_t(s_words * 4), static_cast<hipStream_t>(stream)) != hipSuccess)
        return TK_ERROR_LAUNCH;
    return TK_SUCCESS;
}

tk_status tk_per_token_cast_back(const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *y, int64_t y_ld,
                                 int32_t group, int32_t out_dtype, int32_t round_pow2, void *stream)
{
    if (!valid_group(group) || (out_dtype != kE4M3 && out_dtype != kE2M1)) return TK_ERROR_INVALID_VALUE;
    if (rows < 0 || cols <= 0 || cols % group != 0) return TK_ERROR_INVALID_VALUE;
    if (x_ld < cols || y_ld < cols) return TK_ERROR_INVALID_VALUE;
    if (cols >= (int64_t(1) << 29)) return TK_ERROR_UNSUPPORTED;
    if (!span_ok(rows, x_ld, cols, 2) || !span_ok(rows, y_ld, cols, 2)) return TK_ERROR_INVALID_VALUE;
    if (rows == 0) return TK_SUCCESS;
    if (!x || !y) return TK_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || (x_ld * 2) % 16 != 0 || !aligned(y, 16) || (y_ld * 2) % 16 != 0)
        return TK_ERROR_MISALIGNED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    tk_status st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    static const BackTable table = make_back_table();
    BackParams p{static_cast<const uint16_t *>(x), rows, cols, x_ld, static_cast<uint16_t *>(y), y_ld, -1};
    return launch_unit_grid(reinterpret_cast<const void *>(table.fn[group_index(group)][out_dtype][round_pow2 ? 1 : 0]),
                            rows, cols, &p, &p.xcd_log2, int64_t(kCastWPB) * kCastU * kSegCols * 2,
                            static_cast<hipStream_t>(stream));
}

tk_status tk_per_token_dequant(const void *q, int64_t rows, int64_t cols, int64_t q_ld, const void *scales,
                               int64_t s_ld, int32_t group, int32_t in_dtype, int32_t scale_fmt, void *y,
                               int64_t y_ld, int32_t y_dtype, void *stream)
{
    if (!valid_group(group) || (in_dtype != kE4M3 && in_dtype != kE2M1)) return TK_ERROR_INVALID_VALUE;
    if ((scale_fmt != kScaleF32 && scale_fmt != kScaleUE8M0) || (y_dtype != TK_OUT_BF16 && y_dtype != TK_OUT_F32))
        return TK_ERROR_INVALID_VALUE;
    if (rows < 0 || cols <= 0 || cols % group != 0) return TK_ERROR_INVALID_VALUE;
    const int64_t ngroups = cols / group;
    if (scale_fmt == kScaleUE8M0 && ngroups % 4 != 0) return TK_ERROR_INVALID_VALUE;
    const int64_t q_cols = (in_dtype == kE4M3) ? cols : cols / 2;
    const int64_t s_cols = (scale_fmt == kScaleF32) ? ngroups : ngroups / 4;
    if (q_ld < q_cols || s_ld < s_cols || y_ld < cols) return TK_ERROR_INVALID_VALUE;
    if (cols >= (int64_t(1) << 29)) return TK_ERROR_UNSUPPORTED;
    const int64_t ysize = (y_dtype == TK_OUT_F32) ? 4 : 2;
    if (!span_ok(rows, q_ld, q_cols, 1) || !span_ok(rows, s_ld, s_cols, 4) || !span_ok(rows, y_ld, cols, ysize))
        return TK_ERROR_INVALID_VALUE;
    if (rows == 0) return TK_SUCCESS;
    if (!q || !scales || !y) return TK_ERROR_INVALID_VALUE;
    const int64_t qa = (in_dtype == kE4M3) ? 8 : 4;
    if (!aligned(q, uintptr_t(qa)) || q_ld % qa != 0 || !aligned(scales, 4) || !aligned(y, 16) ||
        (y_ld * ysize) % 16 != 0)
        return TK_ERROR_MISALIGNED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    tk_status st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    static const DequantTable table = make_dequant_table();
    DequantParams p{static_cast<const uint8_t *>(q), rows, cols, q_ld, scales, s_ld, y, y_ld};
    const DequantFn fn = table.fn[group_index(group)][in_dtype][scale_fmt][y_dtype == TK_OUT_F32 ? 1 : 0];
    return launch_unit_grid(reinterpret_cast<const void *>(fn), rows, cols, &p, nullptr, 0,
                            static_cast<hipStream_t>(stream));
}

tk_status tk_silu32_bf16(const void *g, void *out, int64_t n, void *stream)
{
    if (n < 0 || n > kMaxSpanBytes / 4) return TK_ERROR_INVALID_VALUE;
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
    const int64_t blocks = ((n + 1) / 2 + kSiluBlock - 1) / kSiluBlock;
    if (blocks > int64_t(0x7FFFFFFF)) return TK_ERROR_INVALID_VALUE;
    if (hipLaunchKernel(reinterpret_cast<const void *>(silu32_kernel), dim3(uint32_t(blocks)), dim3(kSiluBlock),
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
    case TK_ERROR_UNSUPPORTED: return "TK_ERROR_UNSUPPORTED: request not provided by this library";
    case TK_ERROR_MISALIGNED: return "TK_ERROR_MISALIGNED: pointer or row stride breaks the alignment rule";
    case TK_ERROR_LAUNCH: return "TK_ERROR_LAUNCH: the HIP runtime refused the kernel launch";
    case TK_ERROR_DEVICE: return "TK_ERROR_DEVICE: no usable gfx950 device";
    default: return "TK_ERROR_UNKNOWN";
    }
}

int32_t tk_abi_version(void) { return TK_ABI_VERSION; }

}  // extern "C"
