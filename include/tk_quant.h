/*
 * tk_quant.h -- C ABI of the MI355X (gfx950) per-token / per-group activation
 * cast and its fused SwiGLU form.
 *
 * The operation (sources on the pages):
 *   - "Tile Kernels" (PyPI project page, v2.0.0), Features: activations are
 *     cast per token to FP8 or FP4, and SwiGLU has a form fused with the cast.
 *   - "TileKernels" (aiwiki.ai), section Quantization: the per-token cast reads
 *     BF16, gives each group of G channels of a row its own scale (G one of
 *     16, 32, 64, 128), and can round scales up to powers of two and store
 *     them packed as UE8M0 bytes.
 *   - "TileKernels, TileLang kernels for MoE routing and low-precision
 *     quantization" (hysenlabs.com), section "Seven kernel families": the
 *     SwiGLU and the narrowing run in one pass, with no intermediate tensor
 *     written to memory.
 * For each row r and each group j of G consecutive channels
 * (columns jG .. jG+G-1):
 *     a   = max(max_i |x_i|, 1e-4f)                  (x_i widened from bf16)
 *     s   = a / D  (IEEE fp32 division; D = 448 for E4M3, 6 for E2M1)
 *     s   = 2^ceil(log2 s)  if round_pow2            (from s's exponent bits)
 *     q_i = RNE(clamp(x_i / s, -D, D))               (x_i / s: IEEE fp32)
 * with round-to-nearest-even onto the target grid, ties to the even code, and
 * the sign kept also on zero.  The SwiGLU form casts
 *     h_i = fl32(silu32(gate_i) * up_i),  silu32(g) = fp32 nearest to g/(1+e^-g)
 * (correctly rounded; the product is one fp32 multiply).  h is never written.
 *
 * Formats:
 *   TK_QDTYPE_E4M3: OCP FP8 E4M3FN, one byte per element, max 448.
 *   TK_QDTYPE_E2M1: FP4 E2M1, two per byte, element 2i in bits 0..3 and
 *                   element 2i+1 in bits 4..7; max 6.
 *   TK_SCALE_F32:      fp32 s per group, [rows, cols/G].
 *   TK_SCALE_UE8M0_X4: the biased exponent byte of s (s = 2^(byte-127)), four
 *                      groups per little-endian int32 (group 4k+b in byte b),
 *                      [rows, cols/G/4] int32.  Requires round_pow2 != 0.
 *
 * Ownership and execution: every pointer is a device pointer owned by the
 * caller.  Calls enqueue work on `stream` (a hipStream_t; NULL = the null
 * stream) and return without waiting; outputs are valid once the stream
 * reaches that point.  The library allocates no per-call memory.  All
 * argument checks run on the host before anything is enqueued: on error
 * nothing is launched and the outputs are untouched.  Each operand's span,
 * (rows - 1) * row stride + row length in bytes, must be at most 2^52 bytes
 * (TK_ERROR_INVALID_VALUE otherwise: no device holds that much, and the
 * limit keeps every offset the library forms inside int64).  Inputs with NaN or Inf,
 * and SwiGLU inputs whose product silu(gate) * up overflows fp32, give
 * unspecified codes and scales (outside the contract; no fault).
 */
#ifndef TK_QUANT_H
#define TK_QUANT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TK_ABI_VERSION 1

typedef enum tk_status {
    TK_SUCCESS = 0,
    TK_ERROR_INVALID_VALUE = 1, /* bad size, group, format or null pointer         */
    TK_ERROR_UNSUPPORTED = 2,   /* valid request this library does not provide     */
    TK_ERROR_MISALIGNED = 3,    /* a pointer or row stride breaks the alignment rule */
    TK_ERROR_LAUNCH = 4,        /* the HIP runtime refused the launch               */
    TK_ERROR_DEVICE = 5         /* no usable gfx950 device / runtime error          */
} tk_status;

typedef enum tk_qdtype { TK_QDTYPE_E4M3 = 0, TK_QDTYPE_E2M1 = 1 } tk_qdtype;
typedef enum tk_scale_fmt { TK_SCALE_F32 = 0, TK_SCALE_UE8M0_X4 = 1 } tk_scale_fmt;
typedef enum tk_out_dtype { TK_OUT_BF16 = 0, TK_OUT_F32 = 1 } tk_out_dtype;

/*
 * tk_per_token_cast -- cast bf16 activations to FP8 E4M3 or FP4 E2M1 codes
 * plus per-(row, group) scales.  ("TileKernels" (aiwiki.ai), Quantization.)
 *
 *   x        bf16 [rows, cols], row stride x_ld elements (x_ld >= cols).
 *   rows     >= 0; rows == 0 returns TK_SUCCESS and launches nothing.
 *   cols     > 0, a multiple of group (and of 4*group for TK_SCALE_UE8M0_X4).
 *   q        codes: uint8 [rows, cols] for E4M3 or [rows, cols/2] for E2M1,
 *            row stride q_ld bytes (q_ld >= cols resp. cols/2).
 *   scales   float [rows, cols/group] (TK_SCALE_F32) or int32
 *            [rows, cols/group/4] (TK_SCALE_UE8M0_X4); row stride s_ld
 *            elements of that type (s_ld >= the row length).
 *   group    16, 32, 64 or 128.
 *   out_dtype  TK_QDTYPE_E4M3 or TK_QDTYPE_E2M1.
 *   round_pow2 nonzero: scales rounded up to a power of two.
 *   scale_fmt  TK_SCALE_F32 or TK_SCALE_UE8M0_X4 (the latter needs round_pow2).
 *   stream   hipStream_t as void*.
 *
 * Alignment (TK_ERROR_MISALIGNED otherwise): x and 2*x_ld multiples of 16
 * bytes; q and q_ld multiples of 8 bytes (E4M3) or 4 bytes (E2M1); scales a
 * multiple of 4 bytes.  Output rows must not overlap the input or each other.
 */
tk_status tk_per_token_cast(const void *x, int64_t rows, int64_t cols, int64_t x_ld,
                            void *q, int64_t q_ld, void *scales, int64_t s_ld,
                            int32_t group, int32_t out_dtype, int32_t round_pow2,
                            int32_t scale_fmt, void *stream);

/*
 * tk_swiglu_per_token_cast -- fused SwiGLU + cast.  ("Tile Kernels" (PyPI,
 * v2.0.0), Features; "TileKernels, TileLang kernels for MoE routing and
 * low-precision quantization" (hysenlabs.com), Seven kernel families.)
 *
 *   gate_up  bf16 [rows, 2*cols], row stride x_ld elements (x_ld >= 2*cols);
 *            gate = columns [0, cols), up = columns [cols, 2*cols).
 *   All other arguments, layouts, alignment rules and errors are those of
 *   tk_per_token_cast with `cols` output channels; in addition 2*cols must
 *   keep the up half 16-byte aligned (cols a multiple of 8, which every
 *   valid group size implies).
 *
 * The first call on a device builds the library's correctly rounded silu32
 * table on that device (a one-time kernel followed by a wait on `stream`);
 * call tk_prepare_device() beforehand to keep that wait out of a region that
 * must not synchronise.  While `stream` is being captured into a graph and
 * the table is not yet built, the call returns TK_ERROR_UNSUPPORTED without
 * enqueueing anything.  A failed build is retried by the next call.
 */
tk_status tk_swiglu_per_token_cast(const void *gate_up, int64_t rows, int64_t cols, int64_t x_ld,
                                   void *q, int64_t q_ld, void *scales, int64_t s_ld,
                                   int32_t group, int32_t out_dtype, int32_t round_pow2,
                                   int32_t scale_fmt, void *stream);

/*
 * tk_per_token_cast_f32 -- the per-token cast of fp32 activations ("TileKernels"
 * (aiwiki.ai), Quantization: the casts accept FP32 activations as well as
 * BF16).  Identical to tk_per_token_cast except that x is
 * fp32 [rows, cols] with row stride x_ld elements (x and 4*x_ld multiples of
 * 16 bytes) and is used as it is (no widening).  Rows whose scale row exceeds
 * 32 KiB (more than 8192 scale words) return TK_ERROR_UNSUPPORTED.
 */
tk_status tk_per_token_cast_f32(const void *x, int64_t rows, int64_t cols, int64_t x_ld,
                                void *q, int64_t q_ld, void *scales, int64_t s_ld,
                                int32_t group, int32_t out_dtype, int32_t round_pow2,
                                int32_t scale_fmt, void *stream);

/*
 * tk_per_token_dequant -- codes + scales back to activations ("Tile Kernels"
 * (PyPI, v2.0.0), Features: casting and dequantization):
 *     y = fl32(value(code) * s)     (value(code) exact in fp32)
 * written as fp32 (TK_OUT_F32) or rounded to bf16, nearest with ties to even
 * (TK_OUT_BF16).  UE8M0 bytes decode to s = 2^(byte - 127).
 *
 *   q        codes as tk_per_token_cast writes them, row stride q_ld bytes.
 *   scales   fp32 [rows, cols/group] or int32 [rows, cols/group/4], row stride
 *            s_ld elements.
 *   group, in_dtype, scale_fmt  as for tk_per_token_cast (UE8M0 needs a
 *            multiple of 4 groups per row).
 *   y        bf16 or fp32 [rows, cols], row stride y_ld elements.
 *   y_dtype  TK_OUT_BF16 or TK_OUT_F32.
 * Alignment: q and q_ld multiples of 8 bytes (E4M3) or 4 bytes (E2M1);
 * scales 4 bytes; y and its row stride in bytes multiples of 16.
 * Errors as for tk_per_token_cast.
 */
tk_status tk_per_token_dequant(const void *q, int64_t rows, int64_t cols, int64_t q_ld,
                               const void *scales, int64_t s_ld, int32_t group, int32_t in_dtype,
                               int32_t scale_fmt, void *y, int64_t y_ld, int32_t y_dtype,
                               void *stream);

/*
 * tk_per_token_cast_back -- the cast-and-cast-back ("TileKernels"
 * (aiwiki.ai), Version 2.0.0): y = bf16 of the dequantized per-token cast of
 * x, bit-identical to tk_per_token_cast followed by tk_per_token_dequant with
 * TK_OUT_BF16, in one pass with no codes or scales written to memory.
 *
 *   x        bf16 [rows, cols], row stride x_ld elements.
 *   y        bf16 [rows, cols], row stride y_ld elements (may not alias x).
 *   group, out_dtype, round_pow2  as for tk_per_token_cast (the scale format
 *            does not change the values).
 * Alignment: x, y and both row strides in bytes multiples of 16.
 */
tk_status tk_per_token_cast_back(const void *x, int64_t rows, int64_t cols, int64_t x_ld,
                                 void *y, int64_t y_ld, int32_t group, int32_t out_dtype,
                                 int32_t round_pow2, void *stream);

/*
 * tk_per_block_cast -- the cast with one scale per block of block_rows x
 * block_cols elements ("Tile Kernels" (PyPI, v2.0.0), Features: per-block
 * FP8/FP4 casting).  Block (i, j) covers rows [i*block_rows,
 * min(rows, (i+1)*block_rows)) and columns [j*block_cols, (j+1)*block_cols);
 * a  = max(|x|) over the block, floored at 1e-4f, then s, pow2 and the codes
 * exactly as for tk_per_token_cast.
 *
 *   x, rows, cols, x_ld, q, q_ld, out_dtype, round_pow2, scale_fmt
 *            as for tk_per_token_cast (cols a multiple of block_cols; the last
 *            block row may be partial).
 *   scales   float [ceil(rows/block_rows), cols/block_cols] or int32
 *            [ceil(rows/block_rows), cols/block_cols/4] (UE8M0, four blocks of
 *            one block row per int32, block 4k+b in byte b); row stride s_ld
 *            elements.
 *   block_rows  1 .. 256 (larger: TK_ERROR_UNSUPPORTED); 1 is the per-token cast.
 *   block_cols  16, 32, 64 or 128.
 * Alignment and errors as for tk_per_token_cast.
 */
tk_status tk_per_block_cast(const void *x, int64_t rows, int64_t cols, int64_t x_ld,
                            void *q, int64_t q_ld, void *scales, int64_t s_ld,
                            int64_t block_rows, int64_t block_cols, int32_t out_dtype,
                            int32_t round_pow2, int32_t scale_fmt, void *stream);

/*
 * tk_per_channel_cast -- the cast with one scale per column (channel), the
 * |max| taken over all rows ("Tile Kernels" (PyPI, v2.0.0), Features: a scale
 * per channel); otherwise exactly the arithmetic of
 * tk_per_token_cast.  Equal to tk_per_block_cast with block_rows = rows and
 * block_cols = 1.
 *
 *   x, rows, cols, x_ld, q, q_ld, out_dtype, round_pow2, scale_fmt
 *            as for tk_per_token_cast, with cols any positive multiple of 8.
 *   scales   float [cols] (16-byte aligned) or int32 [cols/4] (UE8M0, column
 *            4k+b in byte b of word k; 8-byte aligned).
 *   workspace  device memory owned by the caller, 16-byte aligned, at least
 *            tk_per_channel_workspace_bytes(rows, cols) bytes; its contents
 *            on entry do not matter and are undefined afterwards.  Calls that
 *            share a workspace must be ordered on one stream.
 * The cast reads x twice (column maxima, then the codes), all on `stream`:
 * two kernels up to 64 MiB of x, three above (the column scales computed
 * between the two passes).  The workspace holds the column maxima of up to
 * 32 row chunks and then the column scales.  Errors as for tk_per_token_cast;
 * a missing or short workspace is TK_ERROR_INVALID_VALUE.
 * tk_per_channel_workspace_bytes returns 0 for rows or cols <= 0 and for sizes
 * the cast refuses whatever the strides (rows above 2^52, cols from 2^29).
 */
int64_t tk_per_channel_workspace_bytes(int64_t rows, int64_t cols);
tk_status tk_per_channel_cast(const void *x, int64_t rows, int64_t cols, int64_t x_ld,
                              void *q, int64_t q_ld, void *scales,
                              void *workspace, int64_t workspace_bytes, int32_t out_dtype,
                              int32_t round_pow2, int32_t scale_fmt, void *stream);

/*
 * tk_per_channel_cast_noalloc -- tk_per_channel_cast for callers that cannot
 * allocate device memory or hand in a workspace (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  Same
 * arguments, kernels and results as tk_per_channel_cast without the workspace
 * pair: the column maxima go to the library's own static device array of
 * tk_per_channel_noalloc_max_workspace_bytes() bytes (1088 KiB: the maxima
 * of 32 row chunks and the scales of up to 16384 columns), one per GPU, held
 * until the process ends.  The call
 * itself allocates nothing.  Inputs that need more than that
 * (tk_per_channel_workspace_bytes(rows, cols) above the maximum) return
 * TK_ERROR_UNSUPPORTED with nothing launched.  Every call on a GPU shares that
 * GPU's array, so calls that may overlap on one GPU (different streams, or
 * several host threads) race: order them on one stream.  Each call writes
 * every workspace entry it reads, so nothing needs clearing between calls.
 */
tk_status tk_per_channel_cast_noalloc(const void *x, int64_t rows, int64_t cols, int64_t x_ld,
                                      void *q, int64_t q_ld, void *scales, int32_t out_dtype,
                                      int32_t round_pow2, int32_t scale_fmt, void *stream);
int64_t tk_per_channel_noalloc_max_workspace_bytes(void);

/*
 * tk_rmsnorm -- RMSNorm forward ("TileKernels" (aiwiki.ai), Version 2.0.0:
 * RMSNorm forward, which can be followed by an FP8 cast in the same kernel).  For each row of C
 * values, with a per-channel weight w (or none, i.e. all ones) and eps > 0:
 *     ss  = sum_j x_j^2, the exact sum rounded once to fp32 (nearest-even)
 *     t   = fl32(fl32(ss / C) + eps)
 *     r   = fl32(1 / fl32(sqrt(t)))                 (IEEE division and sqrt)
 *     y_j = fl32(x_j * r), then fl32(y_j * w_j) with a weight
 * written as fp32 (TK_OUT_F32) or rounded to bf16, nearest-even (TK_OUT_BF16).
 *
 *   x        bf16 [rows, cols], row stride x_ld elements.
 *   cols     a multiple of 8, at most 16384 (larger: TK_ERROR_UNSUPPORTED).
 *   weight   bf16 [cols] (16-byte aligned), or NULL for no weight.
 *   eps      finite, > 0.
 *   y        bf16 or fp32 [rows, cols], row stride y_ld elements.
 * Alignment: x, y and both row strides in bytes multiples of 16.  Rows whose
 * sum of squares exceeds the fp32 range give r = 0 (y = +-0).
 */
tk_status tk_rmsnorm(const void *x, int64_t rows, int64_t cols, int64_t x_ld,
                     const void *weight, float eps, void *y, int64_t y_ld, int32_t y_dtype,
                     void *stream);

/*
 * tk_rmsnorm_cast -- RMSNorm forward fused with the per-token cast of its
 * fp32 output y (see tk_rmsnorm): codes and scales exactly as
 * tk_per_token_cast_f32 would produce from y, without y ever being written.
 * x, cols, weight, eps as for tk_rmsnorm (cols a multiple of group); q,
 * q_ld, scales, s_ld, group, out_dtype, round_pow2, scale_fmt, alignment and
 * errors as for tk_per_token_cast.
 */
tk_status tk_rmsnorm_cast(const void *x, int64_t rows, int64_t cols, int64_t x_ld,
                          const void *weight, float eps, void *q, int64_t q_ld,
                          void *scales, int64_t s_ld, int32_t group, int32_t out_dtype,
                          int32_t round_pow2, int32_t scale_fmt, void *stream);

/*
 * tk_silu32_bf16 -- diagnostic: out[i] = silu32(g[i]) for n bf16 gates, by the
 * same device lookup that tk_swiglu_per_token_cast uses for its gate half
 * (fp32 nearest to g / (1 + e^-g)).  g: bf16 [n] (2-byte aligned), out: fp32
 * [n] (4-byte aligned), both device pointers; 0 <= n <= 2^50.  Asynchronous on
 * `stream` after the first call on a device (see tk_swiglu_per_token_cast).
 */
tk_status tk_silu32_bf16(const void *g, void *out, int64_t n, void *stream);

/*
 * tk_copy_stream -- diagnostic: copy `bytes` bytes from src to dst with the
 * cast's memory instructions (16-byte non-temporal loads and stores, one pass,
 * grid-stride).  Used to calibrate hardware memory counters against a
 * transfer of known size and to measure the practical streaming ceiling.
 * src, dst: device pointers, 16-byte aligned, non-overlapping; bytes >= 0 and
 * a multiple of 16 (TK_ERROR_INVALID_VALUE / TK_ERROR_MISALIGNED otherwise).
 */
tk_status tk_copy_stream(const void *src, void *dst, int64_t bytes, void *stream);

/*
 * tk_stream_rw -- diagnostic: read `read_bytes` from src and write
 * `write_bytes` to dst with the row-form cast's memory instructions and
 * shape (non-temporal 16-byte loads, 4-byte stores per lane; workgroups of 7
 * waves, each wave reading 2 KiB and writing an equal share of dst).  The
 * written values are an xor of what was read (every load is kept); their
 * contents are otherwise meaningless.  Used as the
 * practical streaming ceiling of an operation with the same read and write
 * volumes.  Sizes multiples of 16, both nonzero (or both zero: nothing to
 * do), pointers 16-byte aligned (TK_ERROR_INVALID_VALUE /
 * TK_ERROR_MISALIGNED otherwise); sizes below 2^35 (TK_ERROR_UNSUPPORTED).
 */
tk_status tk_stream_rw(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes, void *stream);

/*
 * tk_prepare_device -- build the per-device tables used by the SwiGLU form on
 * the current HIP device (on the null stream), and wait until they are ready.
 * Idempotent; safe to call from several threads; after a failure the next
 * call tries again.
 */
tk_status tk_prepare_device(void);

/* Human-readable name of a status code (static storage; never NULL). */
const char *tk_status_string(int32_t status);

/* TK_ABI_VERSION of the built library. */
int32_t tk_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TK_QUANT_H */
