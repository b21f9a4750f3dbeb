// tk_norm.hip -- gfx950 kernels and C ABI for RMSNorm forward, alone and
// with the per-token cast fused after it ("TileKernels" (aiwiki.ai), Version
// 2.0.0: RMSNorm forward, which can be followed by an FP8 cast in the same
// kernel).  The arithmetic
// contract is written out in include/tk_quant.h.
//
// Design.  Rows of up to 7168 channels run one row per wave
// (rmsnorm_wave_kernel below), for the fused cast and the plain forward
// alike.  Wider rows: a workgroup owns one row at a
// time (a persistent grid strides over the rows, each workgroup prefetching
// its next row) and holds the whole row in registers: W = ceil(cols / 1024)
// waves, each lane 2 segments of 8 bf16 (16-byte loads, 1 KiB per wave
// instruction), so rows of up to 16384 channels are read from memory exactly
// once.  The weight row is loaded once per workgroup.
//
// The sum of squares is defined as the exact sum rounded once to fp32.  Each
// lane sums its squares in fp64 (a bf16 square is exact in fp64), the lanes
// and waves reduce in a fixed order, and the fp64 result D is certified: the
// exact sum S differs from D by at most n roundings of 2^-53 relative, n = the
// additions on any path (workgroup kernel: 16 per lane, 6 shuffle levels, up
// to 15 wave sums; wave kernel: up to 112 per lane and 6 levels), which is at
// most n units in the last place of D's binade.  fl32(D) is accepted unless
// the 29 low mantissa bits that fl32 drops lie within 256 units of the
// halfway pattern (certified()).  Otherwise (about one row in 2^20 for random
// data; also every row whose exact sum sits on a midpoint, and sums outside
// the fp32 normal range) the row is summed again exactly with an integer
// accumulator in LDS and rounded by hand.  In the workgroup kernel wave 0
// alone turns the wave sums into r and hands it to the other waves.

#include <hip/hip_runtime.h>

#include <float.h>
#include <stdint.h>

#include "tk_device.h"
#include "tk_host.h"

namespace {

constexpr int kNormU = 2;                         // segments per lane
constexpr int kNormMaxWaves = 16;
constexpr int64_t kNormMaxCols = int64_t(kNormMaxWaves) * kNormU * kSegCols;   // 16384
constexpr int kExactDigits = 18;                  // 32-bit digits of the exact accumulator
constexpr int kExactShift = 266;                  // x^2 * 2^266 is an integer for every bf16 x

enum { kOutCast = 0, kOutBF16 = 1, kOutF32 = 2 };

struct NormParams {
    const uint16_t *x;
    int64_t rows, cols, x_ld;
    const uint16_t *w;    // bf16 [cols] or null
    float eps;
    void *out;            // codes, or y
    int64_t out_ld;       // bytes (codes) or elements (y)
    void *s;
    int64_t s_ld;
};

__device__ __forceinline__ double shfl_xor_f64(double v, int mask, int lane)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = shfl_u32(uint32_t(b), lane ^ mask), hi = shfl_u32(uint32_t(b >> 32), lane ^ mask);
    return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

// True when fl32(D) is certainly the exact sum S rounded to fp32, given
// |S - D| below 256 units in the last place of D's binade (S, D >= 0).  The
// fp32 rounding midpoints in that binade are exactly the values whose 29 low
// mantissa bits (the ones fl32 drops) read 2^28, so fl32(D) is safe unless
// those bits lie within 256 of 2^28; D outside the fp32 normal range (below
// 2^-126, or from 2^127 up, where fl32 may overflow) is left to the exact
// path too.
__device__ __forceinline__ bool certified(double d)
{
    if (d == 0.0) return true;                    // all squares zero: exact
    const uint64_t b = __builtin_bit_cast(uint64_t, d);
    const uint32_t e = uint32_t(b >> 52);         // biased exponent, d > 0
    if (e < 1023u - 126u || e >= 1023u + 127u) return false;
    const uint32_t dropped = uint32_t(b) & 0x1FFFFFFFu;
    const uint32_t half = 0x10000000u;
    const uint32_t dist = dropped > half ? dropped - half : half - dropped;
    return dist > 256u;
}

// Every square of the lane's N segments of 8 bf16 into the digit array:
// |x| = M 2^k with an 8-bit integer M, so x^2 2^266 = M^2 2^(2k + 266) is an
// integer of at most 16 bits at a non-negative bit position; its two 32-bit
// pieces go to the digits they fall in with 64-bit LDS atomic adds.
template <int N>
__device__ __forceinline__ void add_squares_exact(const u32x4 (&w)[N], unsigned long long *acc)
{
#pragma unroll
    for (int k = 0; k < N; ++k) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t b = (w[k][i / 2] >> (16 * (i % 2))) & 0x7FFFu;
            const uint32_t e = b >> 7, m = b & 0x7Fu;
            if (b != 0u) {
                const int kexp = e ? int(e) - 134 : -133;      // |x| = M * 2^kexp
                const uint32_t M = e ? (m | 0x80u) : m;
                const int pos = 2 * kexp + kExactShift;         // >= 0
                const uint64_t v = uint64_t(M * M) << (pos & 31);
                atomicAdd(&acc[pos >> 5], (unsigned long long)(v & 0xFFFFFFFFull));
                atomicAdd(&acc[(pos >> 5) + 1], (unsigned long long)(v >> 32));
            }
        }
    }
}

// The exact sum held in the digit array (digit i weighs 2^(32 i - 266);
// carries not yet propagated), rounded to fp32 by hand: to nearest, ties to
// even, subnormal spacing below 2^-126, infinity above the largest finite
// value.  Called by one thread.
__device__ float round_exact_digits(const unsigned long long *acc)
{
    uint32_t dig[kExactDigits];
    uint64_t carry = 0;
    for (int i = 0; i < kExactDigits; ++i) {
        const uint64_t t = acc[i] + carry;
        dig[i] = uint32_t(t);
        carry = t >> 32;
    }
    int top = -1;
    for (int i = kExactDigits - 1; i >= 0 && top < 0; --i)
        if (dig[i]) top = i * 32 + 31 - __builtin_clz(dig[i]);
    float r = 0.0f;
    if (top >= 0) {
        int lsb = top - 23;
        if (lsb < kExactShift - 149) lsb = kExactShift - 149;     // fp32 subnormal spacing
        auto bit = [&](int i) -> uint32_t { return (dig[i >> 5] >> (i & 31)) & 1u; };
        uint64_t mant = 0;
        for (int i = top; i >= lsb; --i) mant = (mant << 1) | bit(i);
        const uint32_t round = lsb >= 1 ? bit(lsb - 1) : 0u;
        uint32_t sticky = 0;
        for (int i = lsb - 2; i >= 0 && !sticky; --i) sticky = bit(i);
        if (round && (sticky || (mant & 1u))) mant += 1;
        const double v = __builtin_ldexp(double(mant), lsb - kExactShift);   // exact
        r = v > double(FLT_MAX) ? __builtin_inff() : float(v);
    }
    return r;
}

// Exact sum of squares of the row, rounded to fp32 by hand: integer digits
// in LDS (64-bit atomic adds of 32-bit pieces, carries resolved at the end by
// one thread).  Called by every thread of the workgroup.
__device__ float exact_sum_squares(const u32x4 (&w)[kNormU], unsigned long long *acc, float *result)
{
    if (threadIdx.x < kExactDigits) acc[threadIdx.x] = 0ull;
    __syncthreads();
    add_squares_exact<kNormU>(w, acc);
    __syncthreads();
    if (threadIdx.x == 0) *result = round_exact_digits(acc);
    __syncthreads();
    return *result;
}

// r = fl32(1 / fl32(sqrt(fl32(fl32(ss / C) + eps)))): IEEE fp32 division
// and square root (HIP's defaults: correctly rounded), one rounding per step.
__device__ __forceinline__ float inv_rms(float ss, float cols_f, float eps)
{
    const float t = ss / cols_f + eps;
    return 1.0f / __builtin_sqrtf(t);
}

// Sum over the wave of an fp64 value, every lane receiving the same result:
// four DPP steps within each 16-lane row (lane ^ 1, lane ^ 2, then the
// half-row and row mirrors), then two cross-row shuffles.  Each step adds two
// partners' identical-order sums, so all lanes stay bit-identical.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v)
{
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = dpp_mov<CTRL>(uint32_t(b)), hi = dpp_mov<CTRL>(uint32_t(b >> 32));
    return __builtin_bit_cast(double, (uint64_t(hi) << 32) | lo);
}

__device__ __forceinline__ double wave_sum_f64(double v, int lane)
{
    v += dpp_f64<0xB1>(v);
    v += dpp_f64<0x4E>(v);
    v += dpp_f64<0x141>(v);
    v += dpp_f64<0x140>(v);
    v += shfl_xor_f64(v, 16, lane);
    v += shfl_xor_f64(v, 32, lane);
    return v;
}

// Persistent form: a workgroup takes rows blockIdx.x, blockIdx.x + gridDim.x,
// ... and loads its next row before it reduces the current one, so a row's
// load latency overlaps the previous row's reduction, barrier and stores.
template <int G, int QD, bool POW2, int SF, int OUT>
__global__ __launch_bounds__(kWave * kNormMaxWaves) void rmsnorm_kernel(NormParams p)
{
    extern __shared__ uint32_t row_scales[];      // the row's scale words (cast form)
    __shared__ double wave_sum[kNormMaxWaves];
    __shared__ unsigned long long exact_acc[kExactDigits];
    __shared__ float exact_result;
    __shared__ float row_r;
    __shared__ int row_exact;
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = int(blockDim.x) >> 6;
    const uint32_t cols = uint32_t(p.cols);
    const uint32_t col0 = uint32_t(wave) * uint32_t(kNormU * kSegCols) + uint32_t(lane) * 8u;
    const float cols_f = float(p.cols);           // exact: cols < 2^24

    // weight row in the x layout, kept as packed bf16 (zeros past the row
    // end); without a weight every factor is 1.0, and x * r * 1 = x * r.
    u32x4 wt[kNormU];
#pragma unroll
    for (int k = 0; k < kNormU; ++k) wt[k] = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
    if (p.w) {
        const __amdgpu_buffer_rsrc_t wrow = row_buffer(p.w, cols * 2u);
#pragma unroll
        for (int k = 0; k < kNormU; ++k)
            wt[k] = __builtin_amdgcn_raw_buffer_load_b128(wrow, int((col0 + k * kSegCols) * 2u), 0, 0);
    }

    auto load_row = [&](int64_t row, u32x4 (&w)[kNormU]) {
        const __amdgpu_buffer_rsrc_t xrow = row_buffer(p.x + row * p.x_ld, cols * 2u);
#pragma unroll
        for (int k = 0; k < kNormU; ++k) w[k] = load16(xrow, (col0 + k * kSegCols) * 2u);
    };

    int64_t row = blockIdx.x;
    u32x4 w[kNormU];
    if (row < p.rows) load_row(row, w);
    for (; row < p.rows; row += gridDim.x) {
        u32x4 wn[kNormU];
        const int64_t next = row + gridDim.x;
#pragma unroll
        for (int k = 0; k < kNormU; ++k) wn[k] = u32x4{0u, 0u, 0u, 0u};
        if (next < p.rows) load_row(next, wn);

        // fp64 sum of squares: per lane, across the wave, across the waves
        double acc = 0.0;
#pragma unroll
        for (int k = 0; k < kNormU; ++k) {
            float x[8];
            widen8(w[k], x);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc = __builtin_fma(double(x[i]), double(x[i]), acc);
        }
        acc = wave_sum_f64(acc, lane);
        if (lane == 0) wave_sum[wave] = acc;
        __syncthreads();
        if (wave == 0) {
            double d = 0.0;
            for (int v = 0; v < nw; ++v) d += wave_sum[v];
            const bool ok = certified(d);
            const float r0 = ok ? inv_rms(float(d), cols_f, p.eps) : 0.0f;
            if (lane == 0) {
                row_r = r0;
                row_exact = ok ? 0 : 1;
            }
        }
        __syncthreads();
        float r;
        if (row_exact) r = inv_rms(exact_sum_squares(w, exact_acc, &exact_result), cols_f, p.eps);   // uniform
        else r = row_r;

        if constexpr (OUT == kOutCast) {
            constexpr int kLanesPerGroup = G / 8;
            const uint32_t s_words = SF == kScaleF32 ? cols / G : cols / G / 4;
            const __amdgpu_buffer_rsrc_t qrow =
                row_buffer(static_cast<uint8_t *>(p.out) + row * p.out_ld, QD == kE4M3 ? cols : cols / 2);
#pragma unroll
            for (int k = 0; k < kNormU; ++k) {
                const uint32_t col = col0 + k * kSegCols;
                float x[8], wf[8], y[8];
                widen8(w[k], x);
                widen8(wt[k], wf);
                uint32_t amax = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    y[i] = (x[i] * r) * wf[i];
                    amax = max(amax, __float_as_uint(y[i]) & 0x7FFFFFFFu);
                }
                const Quantized qz = quantize_segment<G, QD, POW2, kApplyScaledCvt>(y, amax);
                if constexpr (QD == kE4M3) store8(qrow, col, qz.codes);
                else store4(qrow, col / 2, qz.codes.x);
                if constexpr (SF == kScaleF32) {
                    if ((lane % kLanesPerGroup) == 0 && col < cols) row_scales[col / G] = __float_as_uint(qz.s);
                } else {
                    const uint32_t word = pack_e8_word<G>(qz.e8, lane);
                    if ((lane % (4 * kLanesPerGroup)) == 0 && col < cols) row_scales[col / (4 * G)] = word;
                }
            }
            __syncthreads();
            __amdgpu_buffer_rsrc_t srow;
            if constexpr (SF == kScaleF32) srow = row_buffer(static_cast<float *>(p.s) + row * p.s_ld, s_words * 4u);
            else srow = row_buffer(static_cast<uint32_t *>(p.s) + row * p.s_ld, s_words * 4u);
            for (uint32_t t2 = threadIdx.x; t2 < s_words; t2 += blockDim.x) store_scale(srow, t2 * 4u, row_scales[t2]);
        } else {
#pragma unroll
            for (int k = 0; k < kNormU; ++k) {
                const uint32_t col = col0 + k * kSegCols;
                float x[8], wf[8], y[8];
                widen8(w[k], x);
                widen8(wt[k], wf);
#pragma unroll
                for (int i = 0; i < 8; ++i) y[i] = (x[i] * r) * wf[i];
                if constexpr (OUT == kOutBF16) {
                    const __amdgpu_buffer_rsrc_t yrow =
                        row_buffer(static_cast<uint16_t *>(p.out) + row * p.out_ld, cols * 2u);
                    store16(yrow, col * 2u, pack_bf16x8(y));
                } else {
                    const __amdgpu_buffer_rsrc_t yrow =
                        row_buffer(static_cast<float *>(p.out) + row * p.out_ld, cols * 4u);
                    u32x4 a, b;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        a[i] = __float_as_uint(y[i]);
                        b[i] = __float_as_uint(y[4 + i]);
                    }
                    store16(yrow, col * 4u, a);
                    store16(yrow, col * 4u + 16u, b);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kNormU; ++k) w[k] = wn[k];
    }
}

// ---------------------------------------------------------------------------
// One wave per row, for rows of up to 7168 channels.  Each wave of a workgroup
// of WPB waves (4, or 8 for the row counts chosen at launch) converts its own
// rows (rows wave_id, wave_id + total waves, ...):
// the row's NS 512-column segments stay in registers, the sum of squares needs
// only the in-wave reduction, the per-row scalar work (certification,
// division, square root, reciprocal) is spread over 8 NS values per lane, and
// no workgroup barrier is taken after the weight row is staged.  The weight row is staged
// once per workgroup in LDS as fp32 (zeros past the row end); each wave
// gathers its row's scale words in its own LDS slice and writes them with one
// coalesced store per 256 bytes.  Segments past the row end load zeros and
// store nothing (buffer bounds), so NS only has to cover the row.  A lane sums
// up to 8 NS = 112 squares in sequence: with the 6 shuffle levels that is at
// most 118 roundings, within the 256-unit margin of certified().

constexpr int kNormWaveWavesPerSIMD = 4;          // at most 128 VGPRs, so 16 waves fit on a CU
constexpr int kNormWaveSlotsPerCU = 4 * kNormWaveWavesPerSIMD;

// Exact sum of squares of one wave's row (its lanes' NS segments), rounded
// to fp32; the arithmetic of exact_sum_squares, with the digits in this
// wave's own LDS slice and no workgroup barrier (a wave's LDS operations take
// effect in program order).
template <int NS>
__device__ float exact_sum_squares_wave(const u32x4 (&xs)[NS], unsigned long long *acc, int lane)
{
    if (lane < kExactDigits) acc[lane] = 0ull;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    add_squares_exact<NS>(xs, acc);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    uint32_t result = 0;
    if (lane == 0) result = __float_as_uint(round_exact_digits(acc));
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    return __uint_as_float(__builtin_amdgcn_readfirstlane(result));
}

// The weight row in LDS, fp32, split per 512-column segment into two halves:
// weights col .. col+3 of the 8 that lane l of a segment holds (col = 512 k
// + 8 l) sit at 512 k + 4 l, weights col+4 .. col+7 at 512 k + 256 + 4 l.
// Each 16-byte read of a wave then covers 1 KiB of consecutive LDS; in
// column order the lanes' reads lie 32 bytes apart and collide pairwise on
// the banks (16.5 M conflict cycles per call at 32768 x 7168).
__device__ __forceinline__ uint32_t weight_slot(uint32_t col)   // col a multiple of 8
{
    return (col & ~511u) + ((col & 511u) >> 1);
}

// 8 consecutive fp32 weights from LDS (col a multiple of 8: two 16-byte reads)
__device__ __forceinline__ void weight8(const float *w, uint32_t col, float (&wf)[8])
{
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const uint32_t at = weight_slot(col);
    const f32x4 a = *reinterpret_cast<const f32x4 *>(w + at), b = *reinterpret_cast<const f32x4 *>(w + at + 256);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        wf[i] = a[i];
        wf[4 + i] = b[i];
    }
}

// r of one wave's row: the lanes' fp64 sums of squares, the wave sum, its
// certification (else the exact sum) and the fp32 steps of inv_rms.
template <int NS>
__device__ __forceinline__ float row_inv_rms(u32x4 (&xs)[NS], unsigned long long *exact_acc, int lane,
                                             float cols_f, float eps)
{
    double acc = 0.0;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        float x[8];
        widen8(xs[k], x);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = __builtin_fma(double(x[i]), double(x[i]), acc);
    }
    // the widened values are recomputed by the cast rather than kept alive
    // across the reduction (8 registers per segment instead of 4)
#pragma unroll
    for (int k = 0; k < NS; ++k) asm volatile("" : "+v"(xs[k]) :);
    const double d = wave_sum_f64(acc, lane);
    const float ss = certified(d) ? float(d) : exact_sum_squares_wave<NS>(xs, exact_acc, lane);
    return inv_rms(ss, cols_f, eps);
}

// Segment of a row at column col: y = (x * r) * w, its groups' scales and
// codes.  The group maximum is taken over |y| as fp32 (y is finite:
// |x * r| <= sqrt(C)), which orders like the magnitude bits.
template <int G, int QD, bool POW2>
__device__ __forceinline__ Quantized norm_segment(const u32x4 &xk, float r, const float *lds_weight, uint32_t col)
{
    float x[8], y[8], wf[8];
    widen8(xk, x);
    weight8(lds_weight, col, wf);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        y[i] = (x[i] * r) * wf[i];
        amax = __builtin_fmaxf(amax, __builtin_fabsf(y[i]));
    }
    return quantize_segment<G, QD, POW2, kApplyScaledCvt>(y, __float_as_uint(amax));
}

// The segment's group scales into the wave's LDS slice of scale words.
// UE8M0 bytes: groups of up to 32 columns pack their words with DPP moves
// inside a 16-lane row; wider groups write their byte straight into the word
// (byte g % 4 of word g / 4, little-endian), which needs no cross-lane
// addresses held in registers.
template <int G, int SF>
__device__ __forceinline__ void stage_scales(const Quantized &qz, uint32_t col, uint32_t cols, int lane,
                                             uint32_t *stage)
{
    constexpr int kLanesPerGroup = G / 8;
    if constexpr (SF == kScaleF32) {
        if ((lane % kLanesPerGroup) == 0 && col < cols) stage[col / G] = __float_as_uint(qz.s);
    } else {
        // the group's byte straight into its word: packing four groups' bytes
        // with DPP moves first cost ten VALU instructions per segment (this
        // kernel's hot loop: 10.95 -> 9.70 VALU instructions per element)
        if ((lane % kLanesPerGroup) == 0 && col < cols) reinterpret_cast<uint8_t *>(stage)[col / G] = uint8_t(qz.e8);
    }
}

template <int QD>
__device__ __forceinline__ void store_codes(__amdgpu_buffer_rsrc_t qrow, int lane, int k, u32x2 codes)
{
    if constexpr (QD == kE4M3)
        __builtin_amdgcn_raw_buffer_store_b64(codes, qrow, int(lane * 8), k * kSegCols, kNonTemporal);
    else
        __builtin_amdgcn_raw_buffer_store_b32(codes.x, qrow, int(lane * 4), k * kSegCols / 2, kNonTemporal);
}

// The row's scale words, gathered in the wave's LDS slice, in coalesced stores.
template <int G, int SF>
__device__ __forceinline__ void store_row_scales(const NormParams &p, int64_t row, uint32_t cols, int lane,
                                                 const uint32_t *stage)
{
    const uint32_t s_words = SF == kScaleF32 ? cols / G : cols / G / 4;
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __amdgpu_buffer_rsrc_t srow;
    if constexpr (SF == kScaleF32) srow = row_buffer(static_cast<float *>(p.s) + row * p.s_ld, s_words * 4u);
    else srow = row_buffer(static_cast<uint32_t *>(p.s) + row * p.s_ld, s_words * 4u);
    for (uint32_t t = uint32_t(lane); t < s_words; t += kWave) store_scale(srow, t * 4u, stage[t]);
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Segment k of a row of the plain forward: y = (x * r) * w stored as bf16 or
// fp32 with 16-byte stores whose offset lies wholly in the vector offset
// (the scalar offset is zero): for a 16-byte buffer store with a register in
// the scalar-offset field the compiler inserts no wait state before a VALU
// write of the stored registers, and on gfx950 such a write right after the
// store was seen to change the stored data.
template <int OUT>
__device__ __forceinline__ void norm_segment_out(const NormParams &p, int64_t row, uint32_t cols, const u32x4 &xk,
                                                 float r, const float *lds_weight, int lane, int k)
{
    const uint32_t col = uint32_t(k) * kSegCols + uint32_t(lane) * 8u;
    float x[8], y[8], wf[8];
    widen8(xk, x);
    weight8(lds_weight, col, wf);
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (x[i] * r) * wf[i];
    if constexpr (OUT == kOutBF16) {
        const __amdgpu_buffer_rsrc_t yrow = row_buffer(static_cast<uint16_t *>(p.out) + row * p.out_ld, cols * 2u);
        store16(yrow, col * 2u, pack_bf16x8(y));
    } else {
        const __amdgpu_buffer_rsrc_t yrow = row_buffer(static_cast<float *>(p.out) + row * p.out_ld, cols * 4u);
        store16(yrow, col * 4u, u32x4{__float_as_uint(y[0]), __float_as_uint(y[1]), __float_as_uint(y[2]),
                                      __float_as_uint(y[3])});
        store16(yrow, col * 4u + 16u, u32x4{__float_as_uint(y[4]), __float_as_uint(y[5]), __float_as_uint(y[6]),
                                            __float_as_uint(y[7])});
    }
}

// The same value on every lane: keeps row indices and descriptors in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v)
{
    return int64_t(uint64_t(uint32_t(__builtin_amdgcn_readfirstlane(int(v >> 32)))) << 32 |
                   uint32_t(__builtin_amdgcn_readfirstlane(int(v))));
}

// The grid has a wave for every row (up to 2^31 - 1 workgroups of 4; taller
// inputs loop, wave w taking rows w, w + total waves, ...), workgroups
// dispatched in row order, so the rows in flight form one compact window as
// in the row-form cast.  A wave keeps its row's codes in registers and stores
// them together after the row is converted.  Measured against a persistent
// grid of 16 waves per CU whose waves load their next row into the registers
// the cast frees: 7 % faster at 32768 x 7168, 2 % at 16384; storing each
// segment's codes as it is converted: 9 % slower at 4096 x 7168.
template <int G, int QD, bool POW2, int SF, int OUT, int NS, int WPB>
__global__ __launch_bounds__(kWave * WPB, kNormWaveWavesPerSIMD) void rmsnorm_wave_kernel(NormParams p)
{
    constexpr int kCols = NS * kSegCols;
    extern __shared__ float lds_weight[];                                 // fp32 [NS * 512]
    __shared__ uint32_t stage[WPB][kCols / 16];
    __shared__ unsigned long long exact_acc[WPB][kExactDigits];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t cols = uint32_t(p.cols);
    const float cols_f = float(p.cols);

    // Segment k of a lane is byte lane * 16 + k * 1024 of the row, the
    // segment offset in the instruction's scalar offset.  The first row's
    // loads go out together with the weight pieces that this thread stages:
    // in 4-wave workgroups after them, so that the barrier below waits for the
    // weight pieces alone and each wave starts on its row as soon as the row
    // is in; in 8-wave workgroups (the one-round band chosen at launch) before
    // them, so that the barrier waits for the workgroup's rows too.  Measured
    // on MI355X against rows first for both: weight pieces first 2-6 % faster
    // at 4096 to 32768 rows of 7168 channels, 11-19 % at 256 to 2560 rows,
    // 6-14 % at 4096 channels; 1.7 % slower at exactly 3072 x 7168 and 3 % at
    // 6144 x 2048 (grids of exactly one round), and 1-4 % slower in the 8-wave
    // band.
    const int64_t nwaves = int64_t(gridDim.x) * WPB;
    int64_t row = uniform64(int64_t(blockIdx.x) * WPB + wave);
    const uint32_t q_bytes = QD == kE4M3 ? cols : cols / 2;
    u32x4 xs[NS];
    auto load_row = [&](int64_t r) {
        const __amdgpu_buffer_rsrc_t xrow = row_buffer(p.x + r * p.x_ld, cols * 2u);
#pragma unroll
        for (int k = 0; k < NS; ++k)
            xs[k] = __builtin_amdgcn_raw_buffer_load_b128(xrow, int(lane * 16), k * kSegCols * 2, kNonTemporal);
    };
    constexpr bool kWeightFirst = WPB == 4;
    if constexpr (!kWeightFirst) {
        if (row < p.rows) load_row(row);
    }

    // Weight row into LDS as fp32 (w_j, or 1.0 without a weight; 0 past the
    // row end) in the layout of weight_slot, read from memory in 16-byte
    // pieces that are all in flight at once.
    {
        constexpr int kPieces = kCols / 8;                                  // 8 weights each
        constexpr int kPerThread = (kPieces + kWave * WPB - 1) / (kWave * WPB);
        u32x4 wraw[kPerThread];
        const __amdgpu_buffer_rsrc_t wrow = row_buffer(p.w, p.w ? cols * 2u : 0u);
#pragma unroll
        for (int c = 0; c < kPerThread; ++c)
            wraw[c] = __builtin_amdgcn_raw_buffer_load_b128(wrow, int((threadIdx.x + c * kWave * WPB) * 16u),
                                                            0, 0);
        if constexpr (kWeightFirst) {
            // Issued after the weight pieces whatever the compiler's schedule,
            // and without a branch (a wave without a row reads nothing through
            // an empty descriptor), so that the wait for the weight pieces
            // leaves the row's loads in flight.
            __builtin_amdgcn_sched_barrier(0);
            const bool valid = row < p.rows;
            const __amdgpu_buffer_rsrc_t xrow =
                row_buffer(p.x + (valid ? row : 0) * p.x_ld, valid ? cols * 2u : 0u);
#pragma unroll
            for (int k = 0; k < NS; ++k)
                xs[k] = __builtin_amdgcn_raw_buffer_load_b128(xrow, int(lane * 16), k * kSegCols * 2, kNonTemporal);
            __builtin_amdgcn_sched_barrier(0);
        }
        typedef float f32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
        for (int c = 0; c < kPerThread; ++c) {
            const uint32_t piece = threadIdx.x + c * kWave * WPB;
            if (kPieces % (kWave * WPB) == 0 || piece < uint32_t(kPieces)) {
                float f[8];
                widen8(wraw[c], f);
                if (!p.w) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) f[i] = piece * 8u + i < cols ? 1.0f : 0.0f;
                }
                const uint32_t at = weight_slot(piece * 8u);
                *reinterpret_cast<f32x4 *>(lds_weight + at) = f32x4{f[0], f[1], f[2], f[3]};
                *reinterpret_cast<f32x4 *>(lds_weight + at + 256u) = f32x4{f[4], f[5], f[6], f[7]};
            }
        }
    }
    __syncthreads();                              // the only workgroup barrier

    for (bool first = true; row < p.rows; row = uniform64(row + nwaves), first = false) {
        if (!first) load_row(row);
        const float r = row_inv_rms<NS>(xs, exact_acc[wave], lane, cols_f, p.eps);
        if constexpr (OUT != kOutCast) {          // plain forward: each segment's y leaves at once
#pragma unroll
            for (int k = 0; k < NS; ++k) norm_segment_out<OUT>(p, row, cols, xs[k], r, lds_weight, lane, k);
            continue;
        }
        const __amdgpu_buffer_rsrc_t qrow = row_buffer(static_cast<uint8_t *>(p.out) + row * p.out_ld, q_bytes);
        u32x2 codes[NS];
#pragma unroll
        for (int k = 0; k < NS; ++k) {
            const uint32_t col = uint32_t(k) * kSegCols + uint32_t(lane) * 8u;
            const Quantized qz = norm_segment<G, QD, POW2>(xs[k], r, lds_weight, col);
            codes[k] = qz.codes;
            // converted now, not at the store (E2M1 codes are one word)
            if constexpr (QD == kE4M3) asm volatile("" : "+v"(codes[k].x), "+v"(codes[k].y));
            else asm volatile("" : "+v"(codes[k].x));
            stage_scales<G, SF>(qz, col, cols, lane, stage[wave]);
        }
#pragma unroll
        for (int k = 0; k < NS; ++k) store_codes<QD>(qrow, lane, k, codes[k]);
        store_row_scales<G, SF>(p, row, cols, lane, stage[wave]);
    }
}

using NormFn = void (*)(NormParams);

// One-wave-per-row variants by segments held per lane: 4 (rows up to 2048
// channels), 8 (up to 4096), 14 (up to 7168); wider rows take the
// workgroup-per-row kernel.
constexpr int kWaveNS[3] = {4, 8, 14};

struct NormTable {
    NormFn cast[4][4][2][3];     // [kernel: workgroup, one wave per row with NS 4/8/14][group][code format][variant]
    NormFn plain[4][2];          // [the same kernels][bf16 y, fp32 y]
    NormFn cast8[4][2][3];       // NS 14 in workgroups of 8 waves: [group][code format][variant]
    NormFn plain8[2];
};

template <int G, int QD, bool POW2, int SF>
void fill_norm_variant(NormTable &t, int gi, int vi)
{
    t.cast[0][gi][QD][vi] = rmsnorm_kernel<G, QD, POW2, SF, kOutCast>;
    t.cast[1][gi][QD][vi] = rmsnorm_wave_kernel<G, QD, POW2, SF, kOutCast, 4, 4>;
    t.cast[2][gi][QD][vi] = rmsnorm_wave_kernel<G, QD, POW2, SF, kOutCast, 8, 4>;
    t.cast[3][gi][QD][vi] = rmsnorm_wave_kernel<G, QD, POW2, SF, kOutCast, 14, 4>;
    t.cast8[gi][QD][vi] = rmsnorm_wave_kernel<G, QD, POW2, SF, kOutCast, 14, 8>;
}

template <int G, int QD>
void fill_norm(NormTable &t, int gi)
{
    fill_norm_variant<G, QD, false, kScaleF32>(t, gi, 0);
    fill_norm_variant<G, QD, true, kScaleF32>(t, gi, 1);
    fill_norm_variant<G, QD, true, kScaleUE8M0>(t, gi, 2);
}


NormTable make_norm_table()
{
    NormTable t;
    fill_norm<16, kE4M3>(t, 0);  fill_norm<16, kE2M1>(t, 0);
    fill_norm<32, kE4M3>(t, 1);  fill_norm<32, kE2M1>(t, 1);
    fill_norm<64, kE4M3>(t, 2);  fill_norm<64, kE2M1>(t, 2);
    fill_norm<128, kE4M3>(t, 3); fill_norm<128, kE2M1>(t, 3);
    t.plain[0][0] = rmsnorm_kernel<16, kE4M3, false, kScaleF32, kOutBF16>;
    t.plain[0][1] = rmsnorm_kernel<16, kE4M3, false, kScaleF32, kOutF32>;
    t.plain[1][0] = rmsnorm_wave_kernel<16, kE4M3, false, kScaleF32, kOutBF16, 4, 4>;
    t.plain[1][1] = rmsnorm_wave_kernel<16, kE4M3, false, kScaleF32, kOutF32, 4, 4>;
    t.plain[2][0] = rmsnorm_wave_kernel<16, kE4M3, false, kScaleF32, kOutBF16, 8, 4>;
    t.plain[2][1] = rmsnorm_wave_kernel<16, kE4M3, false, kScaleF32, kOutF32, 8, 4>;
    t.plain[3][0] = rmsnorm_wave_kernel<16, kE4M3, false, kScaleF32, kOutBF16, 14, 4>;
    t.plain[3][1] = rmsnorm_wave_kernel<16, kE4M3, false, kScaleF32, kOutF32, 14, 4>;
    t.plain8[0] = rmsnorm_wave_kernel<16, kE4M3, false, kScaleF32, kOutBF16, 14, 8>;
    t.plain8[1] = rmsnorm_wave_kernel<16, kE4M3, false, kScaleF32, kOutF32, 14, 8>;
    return t;
}

tk_status validate_norm(const void *x, int64_t rows, int64_t cols, int64_t x_ld, const void *weight, float eps)
{
    if (rows < 0 || cols <= 0 || x_ld < cols) return TK_ERROR_INVALID_VALUE;
    if (!(eps > 0.0f) || !(eps <= FLT_MAX)) return TK_ERROR_INVALID_VALUE;
    if (cols > kNormMaxCols) return TK_ERROR_UNSUPPORTED;
    if (!span_ok(rows, x_ld, cols, 2)) return TK_ERROR_INVALID_VALUE;
    if (rows == 0) return TK_SUCCESS;
    if (!x) return TK_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || (x_ld * 2) % 16 != 0 || (weight && !aligned(weight, 16))) return TK_ERROR_MISALIGNED;
    return TK_SUCCESS;
}

// Resident waves aimed for per CU by the persistent grids.
#ifndef TK_NORM_WAVES_PER_CU
#define TK_NORM_WAVES_PER_CU 32
#endif

// 0: workgroup-per-row kernel; 1..3: one wave per row holding 4/8/14 segments.
int norm_kernel_index(int64_t cols)
{
    for (int i = 0; i < 3; ++i)
        if (cols <= int64_t(kWaveNS[i]) * kSegCols) return i + 1;
    return 0;
}

tk_status launch_norm(const NormTable &t, int gi, int qd, int variant, int plain, const NormParams &p, int64_t s_words,
                      int cus, hipStream_t s)
{
    NormParams q = p;
    void *args[] = {&q};
    // Rows of up to 7168 channels: one wave per row (plain forward measured
    // 6 % faster than the workgroup kernel at 32768 x 7168, 3 % at 4096);
    // wider rows: one workgroup per row.
    const int ki = norm_kernel_index(p.cols);
    if (ki > 0) {
        // Workgroups of 4 waves, or of 8 for rows of 4097 to 7168 channels
        // when the rows fill between three and four of each SIMD's four wave
        // slots in one round (3072 < rows <= 4096 on 256 CUs): measured on
        // MI355X at 7168 channels, 4-wave workgroups take 2.8 us longer for
        // 3136 rows than for 3072 (13.3 -> 16.1 us), where 8-wave ones take
        // 14.2 us; across that range 8 waves were 2-16 % faster for every
        // code format, fp32 and UE8M0 scales, 5120 channels and the plain
        // forward (4096 x 7168 E4M3 G128: 18.0 -> 16.8 us; E2M1 G32 UE8M0
        // equal), and 4-16 % slower at 1024-3072 rows, 8 % just above 4096
        // (whole 8-wave workgroups waiting for free slots) and 3-6 % at
        // 8192-32768 rows.
        const int64_t slots = int64_t(cus) * kNormWaveSlotsPerCU;
        const bool eight = ki == 3 && p.rows * 4 > slots * 3 && p.rows <= slots;
        const int wpb = eight ? 8 : 4;
        int64_t blocks = (p.rows + wpb - 1) / wpb;                       // a wave for every row
        if (blocks > int64_t(0x7FFFFFFF)) blocks = int64_t(0x7FFFFFFF);  // taller inputs loop
        const NormFn fn = eight ? (plain >= 0 ? t.plain8[plain] : t.cast8[gi][qd][variant])
                                : (plain >= 0 ? t.plain[ki][plain] : t.cast[ki][gi][qd][variant]);
        const size_t lds = size_t(kWaveNS[ki - 1]) * kSegCols * 4u;      // fp32 weight row
        if (hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(uint32_t(blocks)), dim3(kWave * wpb),
                            args, lds, s) != hipSuccess)
            return TK_ERROR_LAUNCH;
        return TK_SUCCESS;
    }
    const NormFn fn = plain >= 0 ? t.plain[0][plain] : t.cast[0][gi][qd][variant];
    const int waves = int((p.cols + kNormU * kSegCols - 1) / (kNormU * kSegCols));
    int64_t per_cu = TK_NORM_WAVES_PER_CU / waves;
    if (per_cu < 1) per_cu = 1;
    int64_t blocks = int64_t(cus) * per_cu;
    if (blocks > p.rows) blocks = p.rows;
    if (hipLaunchKernel(reinterpret_cast<const void *>(fn), dim3(uint32_t(blocks)), dim3(kWave * waves), args,
                        size_t(s_words * 4), s) != hipSuccess)
        return TK_ERROR_LAUNCH;
    return TK_SUCCESS;
}

int norm_group_index(int32_t g) { return g == 16 ? 0 : g == 32 ? 1 : g == 64 ? 2 : 3; }

}  // namespace

extern "C" {

tk_status tk_rmsnorm(const void *x, int64_t rows, int64_t cols, int64_t x_ld, const void *weight, float eps, void *y,
                     int64_t y_ld, int32_t y_dtype, void *stream)
{
    if (y_dtype != TK_OUT_BF16 && y_dtype != TK_OUT_F32) return TK_ERROR_INVALID_VALUE;
    if (cols <= 0 || cols % 8 != 0 || y_ld < cols) return TK_ERROR_INVALID_VALUE;
    tk_status st = validate_norm(x, rows, cols, x_ld, weight, eps);
    if (st != TK_SUCCESS || rows == 0) return st;
    if (!y) return TK_ERROR_INVALID_VALUE;
    const int64_t ysize = y_dtype == TK_OUT_F32 ? 4 : 2;
    if (!span_ok(rows, y_ld, cols, ysize)) return TK_ERROR_INVALID_VALUE;
    if (!aligned(y, 16) || (y_ld * ysize) % 16 != 0) return TK_ERROR_MISALIGNED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    static const NormTable table = make_norm_table();
    NormParams p{static_cast<const uint16_t *>(x), rows, cols, x_ld, static_cast<const uint16_t *>(weight), eps, y,
                 y_ld, nullptr, 0};
    return launch_norm(table, 0, 0, 0, y_dtype == TK_OUT_F32 ? 1 : 0, p, 0, info->cus, static_cast<hipStream_t>(stream));
}

tk_status tk_rmsnorm_cast(const void *x, int64_t rows, int64_t cols, int64_t x_ld, const void *weight, float eps,
                          void *q, int64_t q_ld, void *scales, int64_t s_ld, int32_t group, int32_t out_dtype,
                          int32_t round_pow2, int32_t scale_fmt, void *stream)
{
    if (group != 16 && group != 32 && group != 64 && group != 128) return TK_ERROR_INVALID_VALUE;
    if (out_dtype != kE4M3 && out_dtype != kE2M1) return TK_ERROR_INVALID_VALUE;
    if (scale_fmt != kScaleF32 && scale_fmt != kScaleUE8M0) return TK_ERROR_INVALID_VALUE;
    if (cols <= 0 || cols % group != 0) return TK_ERROR_INVALID_VALUE;
    const int64_t ngroups = cols / group;
    if (scale_fmt == kScaleUE8M0 && (!round_pow2 || ngroups % 4 != 0)) return TK_ERROR_INVALID_VALUE;
    const int64_t q_cols = out_dtype == kE4M3 ? cols : cols / 2;
    const int64_t s_cols = scale_fmt == kScaleF32 ? ngroups : ngroups / 4;
    if (q_ld < q_cols || s_ld < s_cols) return TK_ERROR_INVALID_VALUE;
    tk_status st = validate_norm(x, rows, cols, x_ld, weight, eps);
    if (st != TK_SUCCESS || rows == 0) return st;
    if (!span_ok(rows, q_ld, q_cols, 1) || !span_ok(rows, s_ld, s_cols, 4)) return TK_ERROR_INVALID_VALUE;
    if (!q || !scales) return TK_ERROR_INVALID_VALUE;
    const int64_t qa = out_dtype == kE4M3 ? 8 : 4;
    if (!aligned(q, uintptr_t(qa)) || q_ld % qa != 0 || !aligned(scales, 4)) return TK_ERROR_MISALIGNED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    static const NormTable table = make_norm_table();
    const int variant = !round_pow2 ? 0 : (scale_fmt == kScaleF32 ? 1 : 2);
    NormParams p{static_cast<const uint16_t *>(x), rows, cols, x_ld, static_cast<const uint16_t *>(weight), eps, q,
                 q_ld, scales, s_ld};
    return launch_norm(table, norm_group_index(group), out_dtype, variant, -1, p, s_cols, info->cus,
                       static_cast<hipStream_t>(stream));
}

}  // extern "C"
