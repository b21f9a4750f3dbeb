// tk_device.h -- device helpers shared by the library's kernels (gfx950,
// wave64): formats, buffer-descriptor access, cross-lane reductions, and the
// conversion of 8 values with a known |max| to codes and a scale.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tk_quant.h"

namespace {

constexpr int kWave = 64;
constexpr int kSegCols = kWave * 8;   // columns per wave per segment

constexpr int kE4M3 = TK_QDTYPE_E4M3;
constexpr int kE2M1 = TK_QDTYPE_E2M1;
constexpr int kScaleF32 = TK_SCALE_F32;
constexpr int kScaleUE8M0 = TK_SCALE_UE8M0_X4;

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Buffer access.  dword 3 of a gfx9-family buffer descriptor is 0x00020000
// for raw (untyped, unswizzled) access; cache policy 2 sets the non-temporal
// bit (nt), so streamed lines do not displace other data in L2 / the Infinity
// Cache and a call's writes do not linger as dirty lines.

constexpr int kBufferDword3 = 0x00020000;
constexpr int kNonTemporal = 2;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_buffer(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, int(bytes), kBufferDword3);
}
__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, int(byte_off), 0, kNonTemporal);
}
__device__ __forceinline__ void store4(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, int(byte_off), 0, kNonTemporal);
}
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x2 v)
{
    __builtin_amdgcn_raw_buffer_store_b64(v, r, int(byte_off), 0, kNonTemporal);
}

// Scale rows are short (4 to 2048 bytes) and each is written in 4-to-64-byte
// pieces by several waves; plain write-back stores let L2 merge those pieces
// into whole lines before they go to memory.
#ifndef TK_SCALE_STORE_POLICY
#define TK_SCALE_STORE_POLICY 0
#endif
__device__ __forceinline__ void store_scale(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, uint32_t v)
{
    __builtin_amdgcn_raw_buffer_store_b32(v, r, int(byte_off), 0, TK_SCALE_STORE_POLICY);
}

// ---------------------------------------------------------------------------
// Workgroup order across the XCDs.  A launch's workgroups go to the MI355X's
// 8 XCDs round robin (workgroup b to XCD b % 8), and each XCD has its own L2.
// xcd_order renumbers the workgroups of a grid that takes n items once each
// so that every XCD gets runs of 2^L consecutive items: in each group of
// 8 * 2^L items, workgroup b takes item (b % 8) * 2^L + (b % (8 * 2^L)) / 8
// of the group.  The items of a last, partial group keep their own index,
// and L < 0 leaves every index alone, so this is a bijection on [0, n).
// The resident workgroups still cover one compact window of the tensor, but
// each XCD's share of it is contiguous instead of every eighth item.

__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t n, int L)
{
    if (L < 0) return b;
    const int64_t group = int64_t(8) << L;
    if (b >= n - (n & (group - 1))) return b;
    const int64_t in = b & (group - 1);
    return (b - in) + ((in & 7) << L) + (in >> 3);
}

// ---------------------------------------------------------------------------
// Cross-lane helpers.

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_mov(uint32_t v)
{
    // Row and bank masks full.  Lanes whose source falls outside their
    // 16-lane row (row_shl near the row end) keep 0; no result of such a lane
    // is used.
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
// row) and their |max| bits -> codes in registers plus the group's scale.

struct Quantized {
    u32x2 codes;    // E4M3: 8 bytes; E2M1: 8 nibbles in codes.x
    float s;        // the group's scale
    uint32_t e8;    // its biased exponent byte (power-of-two scales)
};

// Scale of a group from its |max| bits: s = max(a, 1e-4f) / D, rounded up to
// a power of two when POW2 (then e8 is its biased exponent and inv = 1/s,
// both exact).
template <int QD, bool POW2>
struct Scale {
    float s, inv;
    uint32_t e8;
};

// CARRY picks how E is formed from a's bits (the same E either way):
// comparing the significand field, or one addition whose carry does the
// rounding up (two VALU instructions fewer).  Measured on MI355X: the
// addition form made the memory-bound row-form cast 0.3 % slower at
// 32768 x 7168 (the timing of its memory traffic, not its arithmetic), so
// only RMSNorm + cast, whose VALU count matters, takes it.
template <int QD, bool POW2, bool CARRY = false>
__device__ __forceinline__ Scale<QD, POW2> group_scale(uint32_t amax_bits)
{
    constexpr float D = (QD == kE4M3) ? 448.0f : 6.0f;
    // max(a, 1e-4f) on the bits: amax_bits is the pattern of a finite |x| >= 0,
    // whose unsigned order is the numeric order (one integer max, where fmaxf
    // would first canonicalise its operand)
    const float a = __uint_as_float(max(amax_bits, 0x38D1B717u));   // 1e-4f
    Scale<QD, POW2> r;
    r.inv = 0.0f;
    r.e8 = 0;
    if constexpr (POW2) {
        // 2^ceil(log2 fl32(a / D)) without the division.  D = 7 * 2^6 (E4M3)
        // or 3 * 2 (E2M1): a / D is a power of two only for a = D * 2^k, and
        // otherwise lies more than half an fp32 unit from every power of two,
        // so fl32(a / D) is a power of two exactly when a / D is.  Hence
        // ceil(log2(a / D)) = e(a) - 8 + (m(a) > 1.75) for E4M3 and
        // e(a) - 2 + (m(a) > 1.5) for E2M1 (e, m: a's unbiased exponent and
        // significand).  a >= 1e-4 (exponent field 113) puts E in [105, 253],
        // so 2^(127-E) is normal too.
        const uint32_t b = __float_as_uint(a);
        if constexpr (CARRY) {
            // Adding 2^23 - T - 1 (T = 0x600000 or 0x400000, the significand
            // field of 1.75 or 1.5) carries into the exponent field exactly
            // when a's significand field exceeds T; the same addition takes
            // off the 8 or 2 (a's exponent field is at least 113, so nothing
            // wraps), and the mask leaves the bits of s = 2^(E - 127).
            constexpr uint32_t kRoundUp = QD == kE4M3 ? 0x1FFFFFu - (8u << 23) : 0x3FFFFFu - (2u << 23);
            const uint32_t s_bits = (b + kRoundUp) & 0x7F800000u;
            r.e8 = s_bits >> 23;
            r.s = __uint_as_float(s_bits);
            r.inv = __uint_as_float(0x7F000000u - s_bits);
        } else {
            const uint32_t E = QD == kE4M3 ? (b >> 23) - 8u + ((b & 0x7FFFFFu) > 0x600000u)
                                           : (b >> 23) - 2u + ((b & 0x7FFFFFu) > 0x400000u);
            r.e8 = E;
            r.s = __uint_as_float(E << 23);
            r.inv = __uint_as_float((254u - E) << 23);
        }
    } else {
        r.s = a / D;                       // IEEE fp32 division
    }
    return r;
}

// How a scale reaches the converter.  A quotient x / s by IEEE division is
// clamped to [-D, D]: fl32(a / D) may lie below a / D, so |x| / s can pass D
// by a rounding.  A power-of-two scale s = 2^e is at least a / D (fl32(a / D)
// is a power of two only when a / D is one, group_scale), so every |x| <= a
// gives |x| * 2^-e <= D and rounding cannot pass D either: a clamp there
// never binds.  Then x * 2^-e, the exact quotient x / 2^e rounded once as
// x / s is, goes to the converter as it is (kApplyMul), or x goes to the
// gfx950 scaled converters with s (kApplyScaledCvt: they divide by a
// power-of-two scale exactly and round once to nearest even, which the fused
// RMSNorm cast's parity tests check on every code value, midpoint and
// subnormal code at 26 scales).  kApplyClamp clamps power-of-two quotients
// too.  Measured on MI355X against kApplyClamp: SwiGLU + cast 1.9 % and the
// per-block cast 1.3-2.6 % faster with kApplyMul, RMSNorm + cast 3.1 % with
// kApplyScaledCvt; the plain bf16 cast, a memory-bound stream, 0.7 % slower
// without the clamp (an effect on the timing of its memory traffic), so it
// keeps kApplyClamp, as do the fp32-input cast and the cast-and-cast-back.
enum ApplyMode { kApplyClamp = 0, kApplyMul = 1, kApplyScaledCvt = 2 };

template <int QD, bool POW2, int MODE>
__device__ __forceinline__ float scaled(float x, float s, float inv)
{
    constexpr float D = (QD == kE4M3) ? 448.0f : 6.0f;
    if constexpr (POW2 && MODE != kApplyClamp) return x * inv;
    else return __builtin_amdgcn_fmed3f(POW2 ? x * inv : x / s, D, -D);
}

// 8 clamped values -> codes, nearest with ties to even, by the gfx950
// converters: E4M3 in 8 bytes, E2M1 in 8 nibbles of the first word (value
// 2i in the low nibble of byte i).  A converter writes only its half (byte)
// of the destination word and keeps the rest of the word it is given; every
// part of each word is written, so the first converter of a word is given
// the bits of its own first input, a register that dies there, rather than
// a zero that would take a move to make.
template <int QD>
__device__ __forceinline__ u32x2 encode8(const float (&v)[8])
{
    if constexpr (QD == kE4M3) {
        uint32_t lo = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[0], v[1], __float_as_int(v[0]), false));
        lo = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[2], v[3], int(lo), true));
        uint32_t hi = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[4], v[5], __float_as_int(v[4]), false));
        hi = uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(v[6], v[7], int(hi), true));
        return u32x2{lo, hi};
    } else {
        uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(v[0]), v[0], v[1], 1.0f, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[2], v[3], 1.0f, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[4], v[5], 1.0f, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[6], v[7], 1.0f, 3);
        return u32x2{r, 0u};
    }
}

// 8 values and their power-of-two scale s -> codes, by the scaled converters
// (x / s, nearest with ties to even; same packing and the same first
// destination words as encode8).
template <int QD>
__device__ __forceinline__ u32x2 encode8_pow2(const float (&x)[8], float s)
{
    if constexpr (QD == kE4M3) {
        typedef short s16x2 __attribute__((ext_vector_type(2)));
        s16x2 lo = __builtin_bit_cast(s16x2, x[0]), hi = __builtin_bit_cast(s16x2, x[4]);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[0], x[1], s, false);
        lo = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(lo, x[2], x[3], s, true);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, x[4], x[5], s, false);
        hi = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(hi, x[6], x[7], s, true);
        return u32x2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    } else {
        uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(__float_as_uint(x[0]), x[0], x[1], s, 0);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[2], x[3], s, 1);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[4], x[5], s, 2);
        r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, x[6], x[7], s, 3);
        return u32x2{r, 0u};
    }
}

// 8 values whose scale group has |max| bits amax_bits (already reduced over
// the group) -> codes and scale.
template <int QD, bool POW2, int MODE>
__device__ __forceinline__ Quantized quantize_values(const float (&x)[8], uint32_t amax_bits)
{
    const Scale<QD, POW2> sc = group_scale<QD, POW2, MODE == kApplyScaledCvt>(amax_bits);
    Quantized out;
    out.s = sc.s;
    out.e8 = sc.e8;
    if constexpr (POW2 && MODE == kApplyScaledCvt) {
        out.codes = encode8_pow2<QD>(x, sc.s);
    } else {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = scaled<QD, POW2, MODE>(x[i], sc.s, sc.inv);
        out.codes = encode8<QD>(v);
    }
    return out;
}

// Four consecutive groups' exponent bytes as one little-endian int32, valid
// on the first lane of the first group (groups of G columns, G/8 lanes each).
// For G <= 32 the four groups lie in one 16-lane DPP row and row_shl moves
// (lane i reads lane i + N) gather them without an LDS round trip.
template <int G>
__device__ __forceinline__ uint32_t pack_e8_word(uint32_t e8, int lane)
{
    constexpr int kLanesPerGroup = G / 8;
    uint32_t b1, b2, b3;
    if constexpr (G <= 32) {
        b1 = dpp_mov<0x100 + kLanesPerGroup>(e8);
        b2 = dpp_mov<0x100 + 2 * kLanesPerGroup>(e8);
        b3 = dpp_mov<0x100 + 3 * kLanesPerGroup>(e8);
    } else {
        b1 = shfl_u32(e8, lane + kLanesPerGroup);
        b2 = shfl_u32(e8, lane + 2 * kLanesPerGroup);
        b3 = shfl_u32(e8, lane + 3 * kLanesPerGroup);
    }
    return e8 | (b1 << 8) | (b2 << 16) | (b3 << 24);
}

// The same for a per-token group held by G/8 consecutive lanes: each lane
// brings its own 8 values' |max| bits, reduced here over the group.
template <int G, int QD, bool POW2, int MODE>
__device__ __forceinline__ Quantized quantize_segment(const float (&x)[8], uint32_t amax_bits)
{
    return quantize_values<QD, POW2, MODE>(x, group_max<G>(amax_bits));
}

// Code values back to fp32 (exact) with the hardware decoders, times s.
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int QD>
__device__ __forceinline__ void dequant_codes(u32x2 codes, float s, float (&y)[8])
{
    f32x2 d[4];
    if constexpr (QD == kE4M3) {
        d[0] = __builtin_amdgcn_cvt_pk_f32_fp8(int(codes.x), false);
        d[1] = __builtin_amdgcn_cvt_pk_f32_fp8(int(codes.x), true);
        d[2] = __builtin_amdgcn_cvt_pk_f32_fp8(int(codes.y), false);
        d[3] = __builtin_amdgcn_cvt_pk_f32_fp8(int(codes.y), true);
    } else {
        d[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.x, 1.0f, 0);
        d[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.x, 1.0f, 1);
        d[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.x, 1.0f, 2);
        d[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes.x, 1.0f, 3);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        y[2 * k] = d[k].x * s;
        y[2 * k + 1] = d[k].y * s;
    }
}

// 8 fp32 -> 8 bf16 (nearest, ties to even; v_cvt_pk_bf16_f32) in 16 bytes.
__device__ __forceinline__ u32x4 pack_bf16x8(const float (&y)[8])
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    u32x4 out;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const bf16x2 p = {__bf16(y[2 * k]), __bf16(y[2 * k + 1])};
        out[k] = __builtin_bit_cast(uint32_t, p);
    }
    return out;
}

__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, u32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(v, r, int(byte_off), 0, kNonTemporal);
}

__device__ __forceinline__ void widen8(const u32x4 &w, float (&x)[8])
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        x[2 * k] = __uint_as_float(w[k] << 16);
        x[2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
}

// |x| max of 8 bf16 as fp32 bits: bf16 magnitudes compare as unsigned 16-bit
// integers, two per packed max.
__device__ __forceinline__ uint32_t amax_bits_bf16x8(const u32x4 &w)
{
    const uint32_t m = 0x7FFF7FFFu;
    const u16x2 va = __builtin_bit_cast(u16x2, uint32_t(w[0] & m)), vb = __builtin_bit_cast(u16x2, uint32_t(w[1] & m));
    const u16x2 vc = __builtin_bit_cast(u16x2, uint32_t(w[2] & m)), vd = __builtin_bit_cast(u16x2, uint32_t(w[3] & m));
    const u16x2 t = __builtin_elementwise_max(__builtin_elementwise_max(va, vb), __builtin_elementwise_max(vc, vd));
    const uint32_t lo = t.x, hi = t.y;
    return max(lo, hi) << 16;
}

}  // namespace
