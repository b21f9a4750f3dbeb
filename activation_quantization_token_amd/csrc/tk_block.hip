// tk_block.hip -- gfx950 kernels and C ABI for the per-block and per-channel
// casts ("Tile Kernels" (PyPI, v2.0.0), Features: besides one scale per token
// group, the casts come with one scale per block or per channel).  The
// arithmetic is the per-token cast's
// (include/tk_quant.h) with the |max| taken over a block of rows x channels,
// or over a whole column.
//
// Per-block design.  A workgroup owns one block row (block_rows <= 256 rows)
// times one stripe of 512 columns.  Each of its waves loads RPW = 4, 8 or 16
// rows of the stripe (one 16-byte load, 8 bf16, per lane per row; 1 KiB contiguous
// per wave instruction) into registers, reduces |max| over its rows and over
// the G/8 lanes of each block column with DPP, and the waves combine their
// maxima through a small LDS table.  The data never leaves registers, so
// every element is read once and written once.
//
// Per-channel design.  The |max| of a column needs every row before any code
// can be written, so the cast takes two passes over x:
//   1. channel_amax_kernel: workgroups own (row chunk, 512-column stripe)
//      tiles and write the chunk's column maxima (bf16 magnitude bits) to a
//      caller-provided workspace [chunks, cols];
//   2. above 64 MiB of x, channel_scale_kernel (one workgroup per stripe)
//      reduces the chunk maxima to the column scales, writes them to the
//      output and to the workspace, and channel_rows_kernel converts one
//      whole row per workgroup in the row-form cast's shape, its lanes
//      reading their columns' scales from the workspace; the last rows go
//      first, since the rows the first pass read last are the likeliest still
//      in the 256 MB Infinity Cache.  Up to 64 MiB, channel_cast_kernel does
//      both in one launch: each workgroup reduces the chunk maxima of its
//      stripe (all chunk loads in flight at once, then an LDS max across
//      waves) to the stripe's scales, which one workgroup per stripe also
//      writes to the output, then converts its (chunk, stripe) tile.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tk_device.h"
#include "tk_host.h"

namespace {

constexpr int kMaxBlockWaves = 16;
constexpr int kMaxBlockRows = 256;

struct BlockParams {
    const uint16_t *x;   // bf16 bits
    int64_t rows, cols, x_ld;
    uint8_t *q;
    int64_t q_ld;
    void *s;
    int64_t s_ld;
    int64_t block_rows;
};

// RPW rows of the block per wave, held in registers (one 16-byte load each).
template <int BC, int QD, bool POW2, int SF, int RPW>
__global__ __launch_bounds__(kWave * kMaxBlockWaves) void block_cast_kernel(BlockParams p)
{
    constexpr int kBlockRowsPerWave = RPW;
    constexpr int kLanesPerBlock = BC / 8;
    constexpr int kBlocksPerStripe = kSegCols / BC;
    __shared__ uint32_t wave_max[kMaxBlockWaves][kBlocksPerStripe];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = int(blockDim.x) >> 6;
    const uint32_t cols = uint32_t(p.cols);
    const int64_t stripes = (p.cols + kSegCols - 1) / kSegCols;
    const int64_t bi = int64_t(blockIdx.x) / stripes;
    const uint32_t stripe = uint32_t(int64_t(blockIdx.x) - bi * stripes);
    const int64_t r0 = bi * p.block_rows;
    const int64_t r1 = r0 + p.block_rows < p.rows ? r0 + p.block_rows : p.rows;
    const int64_t wr0 = r0 + int64_t(wave) * kBlockRowsPerWave;   // this wave's first row
    const uint32_t col = stripe * uint32_t(kSegCols) + uint32_t(lane) * 8u;

    u32x4 w[kBlockRowsPerWave];
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < kBlockRowsPerWave; ++k) {
        w[k] = u32x4{0u, 0u, 0u, 0u};
        if (wr0 + k < r1) {                      // wave-uniform
            const __amdgpu_buffer_rsrc_t xrow = row_buffer(p.x + (wr0 + k) * p.x_ld, cols * 2u);
            w[k] = load16(xrow, col * 2u);
            m = max(m, amax_bits_bf16x8(w[k]));
        }
    }
    m = group_max<BC>(m);
    if (nw > 1) {
        if ((lane % kLanesPerBlock) == 0) wave_max[wave][lane / kLanesPerBlock] = m;
        __syncthreads();
        m = 0;
        for (int v = 0; v < nw; ++v) m = max(m, wave_max[v][lane / kLanesPerBlock]);
    }

    const Scale<QD, POW2> sc = group_scale<QD, POW2>(m);
#pragma unroll
    for (int k = 0; k < kBlockRowsPerWave; ++k) {
        if (wr0 + k < r1) {
            float x[8], v[8];
            widen8(w[k], x);
#pragma unroll
            for (int i = 0; i < 8; ++i) v[i] = scaled<QD, POW2, kApplyMul>(x[i], sc.s, sc.inv);
            const u32x2 codes = encode8<QD>(v);
            const uint32_t qbytes = QD == kE4M3 ? cols : cols / 2;
            const __amdgpu_buffer_rsrc_t qrow = row_buffer(p.q + (wr0 + k) * p.q_ld, qbytes);
            if constexpr (QD == kE4M3) store8(qrow, col, codes);
            else store4(qrow, col / 2, codes.x);
        }
    }

    if (wave == 0) {
        const uint32_t nbc = cols / BC;
        if constexpr (SF == kScaleF32) {
            const __amdgpu_buffer_rsrc_t srow = row_buffer(static_cast<float *>(p.s) + bi * p.s_ld, nbc * 4u);
            if ((lane % kLanesPerBlock) == 0) store_scale(srow, (col / BC) * 4u, __float_as_uint(sc.s));
        } else {
            const __amdgpu_buffer_rsrc_t srow = row_buffer(static_cast<uint32_t *>(p.s) + bi * p.s_ld, nbc);
            const uint32_t word = pack_e8_word<BC>(sc.e8, lane);
            if ((lane % (4 * kLanesPerBlock)) == 0) store_scale(srow, (col / (4 * BC)) * 4u, word);
        }
    }
}

// ---------------------------------------------------------------------------
// Per-channel cast.

#ifndef TK_CHANNEL_WPB
#define TK_CHANNEL_WPB 16
#endif
#ifndef TK_CHANNEL_UNROLL
#define TK_CHANNEL_UNROLL 4
#endif
constexpr int kChannelWPB = TK_CHANNEL_WPB;        // waves per workgroup
constexpr int kChannelUnroll = TK_CHANNEL_UNROLL;  // rows in flight per wave
constexpr int kChannelSmallUnroll = 2;             // the same for x of at most kChannelSmallBytes
// The first pass reads x with ordinary (allocating) loads, so that as much of
// x as the caches hold is still there for the second pass.
#ifndef TK_CHANNEL_P1_POLICY
#define TK_CHANNEL_P1_POLICY 0
#endif
constexpr int kChannelFirstPassPolicy = TK_CHANNEL_P1_POLICY;
constexpr int64_t kChannelMinChunkRows = 64;
constexpr int64_t kChannelCachedBytes = int64_t(128) << 20;   // half the 256 MiB Infinity Cache
constexpr int64_t kChannelSmallBytes = int64_t(64) << 20;
constexpr int64_t kChannelMaxChunks = 32;
static_assert(kChannelMaxChunks % kChannelWPB == 0, "each wave reduces the same number of chunks");

struct ChannelParams {
    const uint16_t *x;
    int64_t rows, cols, x_ld;
    uint8_t *q;
    int64_t q_ld;
    void *s;
    uint16_t *ws;          // [chunks, cols] bf16 magnitude bits
    int64_t chunk_rows, chunks;
    uint8_t *col_scales;   // per column: the biased exponent byte (power-of-two scales) or the fp32 scale
    int32_t xcd_log2;      // xcd_order run length over the row-form pass's workgroups
};

// Rows [c0, c1) of one 512-column stripe, visited by the waves of a workgroup
// in batches of U rows per wave (wave w takes rows c0 + w + k W, k < U, of a
// batch of U W rows).  Each batch's loads are issued before the previous
// batch is consumed, so U loads per lane are always in flight.
template <int U, int POLICY = kNonTemporal>
struct RowBatches {
    const uint16_t *x;
    int64_t x_ld, c0, c1;
    uint32_t row_bytes, byte_off;   // bytes of a row; this lane's offset in it
    int wave;

    __device__ __forceinline__ int64_t row(int64_t batch, int k) const
    {
        return c0 + batch * int64_t(U) * kChannelWPB + int64_t(k) * kChannelWPB + wave;
    }
    __device__ __forceinline__ void load(int64_t batch, u32x4 (&w)[U]) const
    {
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t r = row(batch, k);
            w[k] = u32x4{0u, 0u, 0u, 0u};
            if (batch >= 0 && r < c1)
                w[k] = __builtin_amdgcn_raw_buffer_load_b128(row_buffer(x + r * x_ld, row_bytes), int(byte_off), 0,
                                                             POLICY);
        }
    }
    __device__ __forceinline__ int64_t batches() const
    {
        const int64_t per = int64_t(U) * kChannelWPB;
        return c1 > c0 ? (c1 - c0 + per - 1) / per : 0;
    }
};

__device__ __forceinline__ void max_bf16x8(u16x2 (&mx)[4], const u32x4 &w)
{
    const u16x2 mag{0x7FFF, 0x7FFF};
#pragma unroll
    for (int j = 0; j < 4; ++j) mx[j] = __builtin_elementwise_max(mx[j], __builtin_bit_cast(u16x2, uint32_t(w[j])) & mag);
}

// Max of the 8 bf16 magnitudes per lane across the waves of the workgroup
// (every wave receives the result).  Ends with the LDS table free again.
__device__ __forceinline__ void workgroup_max(u16x2 (&mx)[4], u32x4 (&part)[kChannelWPB][kWave], int wave, int lane)
{
    u32x4 mine;
#pragma unroll
    for (int j = 0; j < 4; ++j) mine[j] = __builtin_bit_cast(uint32_t, mx[j]);
    part[wave][lane] = mine;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < kChannelWPB; ++v) {
        const u32x4 o = part[v][lane];
#pragma unroll
        for (int j = 0; j < 4; ++j) mx[j] = __builtin_elementwise_max(mx[j], __builtin_bit_cast(u16x2, uint32_t(o[j])));
    }
}

// Pass 1: the |max| of each column over one chunk of rows.
template <int U>
__global__ __launch_bounds__(kWave * kChannelWPB) void channel_amax_kernel(ChannelParams p)
{
    __shared__ u32x4 part[kChannelWPB][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t cols = uint32_t(p.cols);
    const int64_t stripes = (p.cols + kSegCols - 1) / kSegCols;
    const int64_t chunk = int64_t(blockIdx.x) / stripes;
    const uint32_t stripe = uint32_t(int64_t(blockIdx.x) - chunk * stripes);
    const int64_t c0 = chunk * p.chunk_rows;
    const int64_t c1 = c0 + p.chunk_rows < p.rows ? c0 + p.chunk_rows : p.rows;
    const uint32_t col = stripe * uint32_t(kSegCols) + uint32_t(lane) * 8u;
    const RowBatches<U, kChannelFirstPassPolicy> rb{p.x, p.x_ld, c0, c1, cols * 2u, col * 2u, wave};
    // Running maxima of |x| as bf16 magnitudes, two per word (unsigned
    // 16-bit order is numeric order for them).
    u16x2 mx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mx[j] = u16x2{0, 0};
    const int64_t nb = rb.batches();
    u32x4 w[U];
    rb.load(0, w);
    for (int64_t b = 0; b < nb; ++b) {
        u32x4 wn[U];
        rb.load(b + 1, wn);                 // all-zero past the chunk's end
#pragma unroll
        for (int k = 0; k < U; ++k) max_bf16x8(mx, w[k]);
#pragma unroll
        for (int k = 0; k < U; ++k) w[k] = wn[k];
    }
    workgroup_max(mx, part, wave, lane);
    if (wave == 0) {
        u32x4 out;
#pragma unroll
        for (int j = 0; j < 4; ++j) out[j] = __builtin_bit_cast(uint32_t, mx[j]);
        store16(row_buffer(p.ws + chunk * p.cols, cols * 2u), col * 2u, out);
    }
}

// Pass 2 for x of up to 64 MiB: the stripe's scales from the chunk maxima,
// then codes against the column scales, the chunks taken last first (the
// rows the first pass read last are the likeliest still cached).  The first
// batch of rows is loaded before the chunk maxima are reduced, so their
// latencies overlap.  P2_POLICY: the loads' cache policy (ordinary: x of
// this size stays in the Infinity Cache, where the first pass left it).
template <int QD, bool POW2, int SF, int P2_POLICY, int U>
__global__ __launch_bounds__(kWave * kChannelWPB) void channel_cast_kernel(ChannelParams p)
{
    __shared__ u32x4 part[kChannelWPB][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t cols = uint32_t(p.cols);
    const int64_t stripes = (p.cols + kSegCols - 1) / kSegCols;
    const int64_t chunk = p.chunks - 1 - int64_t(blockIdx.x) / stripes;
    const uint32_t stripe = uint32_t(int64_t(blockIdx.x) % stripes);
    const int64_t c0 = chunk * p.chunk_rows;
    const int64_t c1 = c0 + p.chunk_rows < p.rows ? c0 + p.chunk_rows : p.rows;
    const uint32_t col = stripe * uint32_t(kSegCols) + uint32_t(lane) * 8u;
    const RowBatches<U, P2_POLICY> rb{p.x, p.x_ld, c0, c1, cols * 2u, col * 2u, wave};
    const int64_t nb = rb.batches();
    u32x4 w[U];
    rb.load(0, w);

    // Column maxima of this lane's 8 columns over every chunk: wave w takes
    // chunks w, w + W, ... (all its loads issued before any is used).
    constexpr int kChunkLoads = int(kChannelMaxChunks) / kChannelWPB;
    u32x4 cw[kChunkLoads];
#pragma unroll
    for (int k = 0; k < kChunkLoads; ++k) {
        const int64_t c = wave + int64_t(k) * kChannelWPB;
        cw[k] = u32x4{0u, 0u, 0u, 0u};
        if (c < p.chunks) cw[k] = load16(row_buffer(p.ws + c * p.cols, cols * 2u), col * 2u);
    }
    u16x2 mx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mx[j] = u16x2{0, 0};
#pragma unroll
    for (int k = 0; k < kChunkLoads; ++k) max_bf16x8(mx, cw[k]);
    workgroup_max(mx, part, wave, lane);

    float s[8], inv[8];
    uint32_t e8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t amax_bits = uint32_t((i & 1) ? mx[i / 2].y : mx[i / 2].x) << 16;
        const Scale<QD, POW2> sc = group_scale<QD, POW2>(amax_bits);
        s[i] = sc.s;
        inv[i] = sc.inv;
        e8[i] = sc.e8;
    }
    if (blockIdx.x < stripes && wave == 0) {      // one workgroup per stripe
        if constexpr (SF == kScaleF32) {
            const __amdgpu_buffer_rsrc_t srow = row_buffer(p.s, cols * 4u);
            u32x4 a, b;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                a[i] = __float_as_uint(s[i]);
                b[i] = __float_as_uint(s[4 + i]);
            }
            __builtin_amdgcn_raw_buffer_store_b128(a, srow, int(col * 4u), 0, TK_SCALE_STORE_POLICY);
            __builtin_amdgcn_raw_buffer_store_b128(b, srow, int(col * 4u + 16u), 0, TK_SCALE_STORE_POLICY);
        } else {
            const __amdgpu_buffer_rsrc_t srow = row_buffer(p.s, cols);
            const u32x2 v{e8[0] | (e8[1] << 8) | (e8[2] << 16) | (e8[3] << 24),
                          e8[4] | (e8[5] << 8) | (e8[6] << 16) | (e8[7] << 24)};
            __builtin_amdgcn_raw_buffer_store_b64(v, srow, int(col), 0, TK_SCALE_STORE_POLICY);
        }
    }

    const uint32_t qbytes = QD == kE4M3 ? cols : cols / 2;
    for (int64_t i = 0; i < nb; ++i) {
        u32x4 wn[U];
        rb.load(i + 1, wn);                 // nothing past the last batch
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int64_t row = rb.row(i, k);
            if (row < c1) {
                float x[8], v[8];
                widen8(w[k], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = scaled<QD, POW2, kApplyMul>(x[i], s[i], inv[i]);
                const u32x2 codes = encode8<QD>(v);
                const __amdgpu_buffer_rsrc_t qrow = row_buffer(p.q + row * p.q_ld, qbytes);
                if constexpr (QD == kE4M3) store8(qrow, col, codes);
                else store4(qrow, col / 2, codes.x);
            }
        }
#pragma unroll
        for (int k = 0; k < U; ++k) w[k] = wn[k];
    }
}

// Column scales (between the two passes): one workgroup per 512-column
// stripe reduces the stripe's chunk maxima (each wave its share of the
// chunks, all loads in flight, then the LDS max across waves), writes the
// scales to `s` and, for the row-form cast pass, to col_scales: the biased
// exponent byte of each column's power-of-two scale, or its fp32 scale.
template <int QD, bool POW2, int SF>
__global__ __launch_bounds__(kWave * kChannelWPB) void channel_scale_kernel(ChannelParams p)
{
    __shared__ u32x4 part[kChannelWPB][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t cols = uint32_t(p.cols);
    const uint32_t col = blockIdx.x * uint32_t(kSegCols) + uint32_t(lane) * 8u;
    constexpr int kChunkLoads = int(kChannelMaxChunks) / kChannelWPB;
    u32x4 cw[kChunkLoads];
#pragma unroll
    for (int k = 0; k < kChunkLoads; ++k) {
        const int64_t c = wave + int64_t(k) * kChannelWPB;
        cw[k] = u32x4{0u, 0u, 0u, 0u};
        if (c < p.chunks) cw[k] = load16(row_buffer(p.ws + c * p.cols, cols * 2u), col * 2u);
    }
    u16x2 mx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) mx[j] = u16x2{0, 0};
#pragma unroll
    for (int k = 0; k < kChunkLoads; ++k) max_bf16x8(mx, cw[k]);
    workgroup_max(mx, part, wave, lane);
    if (wave != 0) return;
    float sv[8];
    uint32_t e8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t amax_bits = uint32_t((i & 1) ? mx[i / 2].y : mx[i / 2].x) << 16;
        const Scale<QD, POW2> sc = group_scale<QD, POW2>(amax_bits);
        sv[i] = sc.s;
        e8[i] = sc.e8;
    }
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i] = __float_as_uint(sv[i]);
        b[i] = __float_as_uint(sv[4 + i]);
    }
    const u32x2 bytes{e8[0] | (e8[1] << 8) | (e8[2] << 16) | (e8[3] << 24),
                      e8[4] | (e8[5] << 8) | (e8[6] << 16) | (e8[7] << 24)};
    if constexpr (SF == kScaleF32) {
        const __amdgpu_buffer_rsrc_t srow = row_buffer(p.s, cols * 4u);
        __builtin_amdgcn_raw_buffer_store_b128(a, srow, int(col * 4u), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(b, srow, int(col * 4u + 16u), 0, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b64(bytes, row_buffer(p.s, cols), int(col), 0, 0);
    }
    if constexpr (POW2) {
        __builtin_amdgcn_raw_buffer_store_b64(bytes, row_buffer(p.col_scales, cols), int(col), 0, 0);
    } else {
        const __amdgpu_buffer_rsrc_t crow = row_buffer(p.col_scales, cols * 4u);
        __builtin_amdgcn_raw_buffer_store_b128(a, crow, int(col * 4u), 0, 0);
        __builtin_amdgcn_raw_buffer_store_b128(b, crow, int(col * 4u + 16u), 0, 0);
    }
}

// Pass 2 in row form (x above 64 MiB): a workgroup converts one whole row,
// wave w taking the runs of two 512-column segments w, w + W, ... (one run
// per wave up to 16384 columns) with its lanes' 16 column scales read from
// the workspace.  Workgroups in XCD order, last rows first (the rows the
// first pass read last are the likeliest still cached).  Measured on MI355X
// against the (chunk, stripe) tile form: -2.1 % at 32768 x 7168, -1.5 % at
// 16384, -1.2 % at 8192, +3.7 % at 4096 (x of 56 MiB keeps the tile form).
template <int QD, bool POW2, int SF, int POL>
__global__ __launch_bounds__(1024) void channel_rows_kernel(ChannelParams p)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int nw = int(blockDim.x) >> 6;
    const uint32_t cols = uint32_t(p.cols);
    const uint32_t qbytes = QD == kE4M3 ? cols : cols / 2;
    const int runs = int((cols + 2 * kSegCols - 1) / (2 * kSegCols));
    for (int64_t i = blockIdx.x; i < p.rows; i += gridDim.x) {
        const int64_t row = p.rows - 1 - xcd_order(i, p.rows, p.xcd_log2);
        const __amdgpu_buffer_rsrc_t xrow = row_buffer(p.x + row * p.x_ld, cols * 2u);
        const __amdgpu_buffer_rsrc_t qrow = row_buffer(p.q + row * p.q_ld, qbytes);
        for (int run = wave; run < runs; run += nw) {
            const uint32_t col0 = uint32_t(run) * 2u * kSegCols + uint32_t(lane) * 8u;
            u32x4 w[2];
#pragma unroll
            for (int k = 0; k < 2; ++k)
                w[k] = __builtin_amdgcn_raw_buffer_load_b128(xrow, int((col0 + k * kSegCols) * 2u), 0, POL);
            // the lane's column scales: 2^-e from the exponent bytes, or s
            float sc[2][8];
            if constexpr (POW2) {
                const __amdgpu_buffer_rsrc_t crow = row_buffer(p.col_scales, cols);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const u32x2 e = __builtin_amdgcn_raw_buffer_load_b64(crow, int(col0 + k * kSegCols), 0, 0);
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        sc[k][i] = __uint_as_float((254u - ((e[i / 4] >> (8 * (i % 4))) & 0xFFu)) << 23);
                }
            } else {
                const __amdgpu_buffer_rsrc_t crow = row_buffer(p.col_scales, cols * 4u);
#pragma unroll
                for (int k = 0; k < 2; ++k) {
                    const u32x4 a = load16(crow, (col0 + k * kSegCols) * 4u);
                    const u32x4 b = load16(crow, (col0 + k * kSegCols) * 4u + 16u);
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        sc[k][i] = __uint_as_float(a[i]);
                        sc[k][4 + i] = __uint_as_float(b[i]);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                float x[8], v[8];
                widen8(w[k], x);
#pragma unroll
                for (int i = 0; i < 8; ++i) v[i] = scaled<QD, POW2, kApplyMul>(x[i], sc[k][i], sc[k][i]);
                const u32x2 codes = encode8<QD>(v);
                const uint32_t col = col0 + k * kSegCols;
                if constexpr (QD == kE4M3) store8(qrow, col, codes);
                else store4(qrow, col / 2, codes.x);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side.

using BlockFn = void (*)(BlockParams);
using ChannelFn = void (*)(ChannelParams);

struct BlockTable {
    BlockFn fn[3][4][2][3];      // [rows per wave 4/8/16][block_cols index][code format][variant]
};
struct ChannelTable {
    ChannelFn cast[2][3];        // [code format][variant]: x up to 64 MiB
    ChannelFn scale[2][3];       // [code format][variant]: above 64 MiB, then
    ChannelFn rows[2][3][2];     //   [code format][variant][x above 128 MiB (non-temporal loads), up to 128 MiB]
};

template <int BC, int QD, int RPW>
void fill_block_rpw(BlockFn (&t)[3])
{
    t[0] = block_cast_kernel<BC, QD, false, kScaleF32, RPW>;
    t[1] = block_cast_kernel<BC, QD, true, kScaleF32, RPW>;
    t[2] = block_cast_kernel<BC, QD, true, kScaleUE8M0, RPW>;
}

template <int BC, int QD>
void fill_block(BlockTable &t, int bci)
{
    fill_block_rpw<BC, QD, 4>(t.fn[0][bci][QD]);
    fill_block_rpw<BC, QD, 8>(t.fn[1][bci][QD]);
    fill_block_rpw<BC, QD, 16>(t.fn[2][bci][QD]);
}

BlockTable make_block_table()
{
    BlockTable t;
    fill_block<16, kE4M3>(t, 0);  fill_block<16, kE2M1>(t, 0);
    fill_block<32, kE4M3>(t, 1);  fill_block<32, kE2M1>(t, 1);
    fill_block<64, kE4M3>(t, 2);  fill_block<64, kE2M1>(t, 2);
    fill_block<128, kE4M3>(t, 3); fill_block<128, kE2M1>(t, 3);
    return t;
}

// Rows per wave for a launch (measured on MI355X over bf16 [32768, 7168] and
// [4096, 7168]): 4 up to 32-row blocks, 8 up to 64, and for 128-row blocks
// 16 once there are at least 8 tiles per CU (8 below: fewer, shorter waves
// finish a small grid sooner); 16 above 128 rows.
int block_rpw_index(int64_t block_rows, int64_t tiles, int cus)
{
    if (block_rows > 128) return 2;
    if (block_rows > 64) return tiles >= 8 * int64_t(cus) ? 2 : 1;
    return block_rows > 32 ? 1 : 0;
}

template <int QD>
void fill_channel(ChannelTable &t)
{
    t.cast[QD][0] = channel_cast_kernel<QD, false, kScaleF32, 0, kChannelSmallUnroll>;
    t.cast[QD][1] = channel_cast_kernel<QD, true, kScaleF32, 0, kChannelSmallUnroll>;
    t.cast[QD][2] = channel_cast_kernel<QD, true, kScaleUE8M0, 0, kChannelSmallUnroll>;
    t.scale[QD][0] = channel_scale_kernel<QD, false, kScaleF32>;
    t.scale[QD][1] = channel_scale_kernel<QD, true, kScaleF32>;
    t.scale[QD][2] = channel_scale_kernel<QD, true, kScaleUE8M0>;
    t.rows[QD][0][0] = channel_rows_kernel<QD, false, kScaleF32, kNonTemporal>;
    t.rows[QD][1][0] = channel_rows_kernel<QD, true, kScaleF32, kNonTemporal>;
    t.rows[QD][2][0] = channel_rows_kernel<QD, true, kScaleUE8M0, kNonTemporal>;
    t.rows[QD][0][1] = channel_rows_kernel<QD, false, kScaleF32, 0>;
    t.rows[QD][1][1] = channel_rows_kernel<QD, true, kScaleF32, 0>;
    t.rows[QD][2][1] = channel_rows_kernel<QD, true, kScaleUE8M0, 0>;
}

ChannelTable make_channel_table()
{
    ChannelTable t;
    fill_channel<kE4M3>(t);
    fill_channel<kE2M1>(t);
    return t;
}

int block_cols_index(int64_t bc) { return bc == 16 ? 0 : bc == 32 ? 1 : bc == 64 ? 2 : 3; }

// Checks shared by both casts: formats, sizes, the input and code layouts.
tk_status validate_common(const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *q, int64_t q_ld,
                          void *scales, int32_t out_dtype, int32_t round_pow2, int32_t scale_fmt)
{
    if (out_dtype != kE4M3 && out_dtype != kE2M1) return TK_ERROR_INVALID_VALUE;
    if (scale_fmt != kScaleF32 && scale_fmt != kScaleUE8M0) return TK_ERROR_INVALID_VALUE;
    if (scale_fmt == kScaleUE8M0 && !round_pow2) return TK_ERROR_INVALID_VALUE;
    if (rows < 0 || cols <= 0) return TK_ERROR_INVALID_VALUE;
    const int64_t q_cols = (out_dtype == kE4M3) ? cols : cols / 2;
    if (x_ld < cols || q_ld < q_cols) return TK_ERROR_INVALID_VALUE;
    if (cols >= (int64_t(1) << 29)) return TK_ERROR_UNSUPPORTED;   // row byte offsets are 32-bit
    if (!span_ok(rows, x_ld, cols, 2) || !span_ok(rows, q_ld, q_cols, 1)) return TK_ERROR_INVALID_VALUE;
    if (rows == 0) return TK_SUCCESS;
    if (!x || !q || !scales) return TK_ERROR_INVALID_VALUE;
    if (!aligned(x, 16) || (x_ld * 2) % 16 != 0) return TK_ERROR_MISALIGNED;
    const int64_t qa = (out_dtype == kE4M3) ? 8 : 4;
    if (!aligned(q, uintptr_t(qa)) || q_ld % qa != 0) return TK_ERROR_MISALIGNED;
    return TK_SUCCESS;
}

// The no-allocation variant's workspace: a file-scope array in device
// memory, one copy per GPU, kept until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in);
// it passes the device address that hipGetSymbolAddress gives, looked up once
// per device with that device current.  Every no-allocation call on a GPU
// shares that GPU's copy.
constexpr int64_t kNoAllocScratchBytes = int64_t(1088) << 10;   // 32 chunks x 16384 columns x 2 B + 4 B per column

}  // namespace

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

struct ScratchSlot {
    std::mutex mutex;
    std::atomic<void *> ptr{nullptr};
};
ScratchSlot g_scratch[kMaxDevices];

tk_status scratch_address(int dev, void **out)
{
    ScratchSlot &slot = g_scratch[dev];
    void *p = slot.ptr.load(std::memory_order_acquire);
    if (!p) {
        std::lock_guard<std::mutex> lock(slot.mutex);
        p = slot.ptr.load(std::memory_order_relaxed);
        if (!p) {
            if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return TK_ERROR_DEVICE;
            slot.ptr.store(p, std::memory_order_release);
        }
    }
    *out = p;
    return TK_SUCCESS;
}

int64_t channel_chunk_rows(int64_t rows)
{
    const int64_t r = (rows + kChannelMaxChunks - 1) / kChannelMaxChunks;
    return r > kChannelMinChunkRows ? r : kChannelMinChunkRows;
}

int64_t channel_chunks(int64_t rows)
{
    const int64_t cr = channel_chunk_rows(rows);
    return (rows + cr - 1) / cr;
}

// Workspace: the chunk maxima [chunks, cols] (bf16 bits), then from the next
// 256-byte boundary the column scales (4 bytes per column at most).
int64_t channel_maxima_bytes(int64_t rows, int64_t cols) { return (channel_chunks(rows) * cols * 2 + 255) / 256 * 256; }
int64_t channel_workspace_bytes(int64_t rows, int64_t cols) { return channel_maxima_bytes(rows, cols) + cols * 4; }

// The two passes of the per-channel cast on an argument-checked call, with
// `workspace` (device memory of at least tk_per_channel_workspace_bytes).
tk_status launch_channel(const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *q, int64_t q_ld, void *scales,
                         void *workspace, int32_t out_dtype, int32_t round_pow2, int32_t scale_fmt, hipStream_t s)
{
    static const ChannelTable table = make_channel_table();
    const int variant = !round_pow2 ? 0 : (scale_fmt == kScaleF32 ? 1 : 2);
    const int64_t chunk_rows = channel_chunk_rows(rows), chunks = channel_chunks(rows);
    const int64_t stripes = (cols + kSegCols - 1) / kSegCols;
    const int64_t tiles = chunks * stripes;
    if (tiles > int64_t(0x7FFFFFFF)) return TK_ERROR_UNSUPPORTED;
    const int64_t row_blocks = rows < int64_t(0x7FFFFFFF) ? rows : int64_t(0x7FFFFFFF);   // taller inputs loop
    ChannelParams p{static_cast<const uint16_t *>(x), rows, cols, x_ld, static_cast<uint8_t *>(q), q_ld, scales,
                    static_cast<uint16_t *>(workspace), chunk_rows, chunks,
                    static_cast<uint8_t *>(workspace) + channel_maxima_bytes(rows, cols),
                    xcd_run_log2(rows, row_blocks, cols * 2)};
    void *args[] = {&p};
    // Size classes of x.  Up to 64 MiB: both passes keep 2 rows in flight
    // per wave instead of 4 (-10 % at 4096 x 7168; 1 % slower at 8192 rows,
    // 2-5 % at 16384 and 32768), and the second pass is the tile form with
    // ordinary loads.  Above: the scale kernel and the row form, whose loads
    // are ordinary up to half the 256 MiB Infinity Cache and non-temporal
    // beyond (ordinary: +5 % at 16384 x 7168, +6 % at 32768).
    const int64_t x_bytes = rows * cols * 2;
    const bool small = x_bytes <= kChannelSmallBytes;
    const void *amax_fn = small ? reinterpret_cast<const void *>(channel_amax_kernel<kChannelSmallUnroll>)
                                : reinterpret_cast<const void *>(channel_amax_kernel<kChannelUnroll>);
    if (hipLaunchKernel(amax_fn, dim3(uint32_t(tiles)), dim3(kWave * kChannelWPB), args, 0, s) != hipSuccess)
        return TK_ERROR_LAUNCH;
    if (small) {
        if (hipLaunchKernel(reinterpret_cast<const void *>(table.cast[out_dtype][variant]), dim3(uint32_t(tiles)),
                            dim3(kWave * kChannelWPB), args, 0, s) != hipSuccess)
            return TK_ERROR_LAUNCH;
        return TK_SUCCESS;
    }
    const int64_t runs = (cols + 2 * kSegCols - 1) / (2 * kSegCols);
    const int waves = int(runs < 16 ? runs : 16);
    if (hipLaunchKernel(reinterpret_cast<const void *>(table.scale[out_dtype][variant]), dim3(uint32_t(stripes)),
                        dim3(kWave * kChannelWPB), args, 0, s) != hipSuccess)
        return TK_ERROR_LAUNCH;
    const int pol = x_bytes <= kChannelCachedBytes ? 1 : 0;
    if (hipLaunchKernel(reinterpret_cast<const void *>(table.rows[out_dtype][variant][pol]), dim3(uint32_t(row_blocks)),
                        dim3(kWave * waves), args, 0, s) != hipSuccess)
        return TK_ERROR_LAUNCH;
    return TK_SUCCESS;
}

}  // namespace

extern "C" {

tk_status tk_per_block_cast(const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *q, int64_t q_ld,
                            void *scales, int64_t s_ld, int64_t block_rows, int64_t block_cols, int32_t out_dtype,
                            int32_t round_pow2, int32_t scale_fmt, void *stream)
{
    if (block_cols != 16 && block_cols != 32 && block_cols != 64 && block_cols != 128) return TK_ERROR_INVALID_VALUE;
    if (block_rows <= 0) return TK_ERROR_INVALID_VALUE;
    if (cols <= 0 || cols % block_cols != 0) return TK_ERROR_INVALID_VALUE;
    const int64_t nbc = cols / block_cols;
    if (scale_fmt == kScaleUE8M0 && nbc % 4 != 0) return TK_ERROR_INVALID_VALUE;
    const int64_t s_cols = scale_fmt == kScaleUE8M0 ? nbc / 4 : nbc;
    if (s_ld < s_cols) return TK_ERROR_INVALID_VALUE;
    tk_status st = validate_common(x, rows, cols, x_ld, q, q_ld, scales, out_dtype, round_pow2, scale_fmt);
    if (st != TK_SUCCESS || rows == 0) return st;
    if (block_rows > kMaxBlockRows) return TK_ERROR_UNSUPPORTED;
    if (!span_ok((rows + block_rows - 1) / block_rows, s_ld, s_cols, 4)) return TK_ERROR_INVALID_VALUE;
    if (!aligned(scales, 4)) return TK_ERROR_MISALIGNED;
    // Blocks of one row are the per-token groups: same layouts, same values.
    if (block_rows == 1)
        return tk_per_token_cast(x, rows, cols, x_ld, q, q_ld, scales, s_ld, int32_t(block_cols), out_dtype,
                                 round_pow2, scale_fmt, stream);
    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    static const BlockTable table = make_block_table();
    const int variant = !round_pow2 ? 0 : (scale_fmt == kScaleF32 ? 1 : 2);
    const int64_t nbr = (rows + block_rows - 1) / block_rows;
    const int64_t stripes = (cols + kSegCols - 1) / kSegCols;
    const int64_t blocks = nbr * stripes;
    if (blocks > int64_t(0x7FFFFFFF)) return TK_ERROR_UNSUPPORTED;
    const int ri = block_rpw_index(block_rows, blocks, info->cus);
    const int64_t rpw = int64_t(4) << ri;
    const int64_t used_rows = block_rows < rows ? block_rows : rows;
    const int waves = int((used_rows + rpw - 1) / rpw);     // <= kMaxBlockWaves
    BlockParams p{static_cast<const uint16_t *>(x), rows, cols, x_ld, static_cast<uint8_t *>(q), q_ld, scales, s_ld,
                  block_rows};
    const int bci = block_cols_index(block_cols);
    hipStream_t s = static_cast<hipStream_t>(stream);
    void *args[] = {&p};
    if (hipLaunchKernel(reinterpret_cast<const void *>(table.fn[ri][bci][out_dtype][variant]), dim3(uint32_t(blocks)),
                        dim3(kWave * waves), args, 0, s) != hipSuccess)
        return TK_ERROR_LAUNCH;
    return TK_SUCCESS;
}

int64_t tk_per_channel_workspace_bytes(int64_t rows, int64_t cols)
{
    if (rows <= 0 || cols <= 0 || rows > kMaxSpanBytes || cols >= (int64_t(1) << 29)) return 0;
    return channel_workspace_bytes(rows, cols);
}

tk_status tk_per_channel_cast(const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *q, int64_t q_ld,
                              void *scales, void *workspace, int64_t workspace_bytes, int32_t out_dtype,
                              int32_t round_pow2, int32_t scale_fmt, void *stream)
{
    if (cols <= 0 || cols % 8 != 0) return TK_ERROR_INVALID_VALUE;
    tk_status st = validate_common(x, rows, cols, x_ld, q, q_ld, scales, out_dtype, round_pow2, scale_fmt);
    if (st != TK_SUCCESS || rows == 0) return st;
    if (!workspace || workspace_bytes < tk_per_channel_workspace_bytes(rows, cols)) return TK_ERROR_INVALID_VALUE;
    if (!aligned(scales, scale_fmt == kScaleF32 ? 16 : 8) || !aligned(workspace, 16)) return TK_ERROR_MISALIGNED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    return launch_channel(x, rows, cols, x_ld, q, q_ld, scales, workspace, out_dtype, round_pow2, scale_fmt,
                          static_cast<hipStream_t>(stream));
}

tk_status tk_per_channel_cast_noalloc(const void *x, int64_t rows, int64_t cols, int64_t x_ld, void *q, int64_t q_ld,
                                      void *scales, int32_t out_dtype, int32_t round_pow2, int32_t scale_fmt,
                                      void *stream)
{
    if (cols <= 0 || cols % 8 != 0) return TK_ERROR_INVALID_VALUE;
    tk_status st = validate_common(x, rows, cols, x_ld, q, q_ld, scales, out_dtype, round_pow2, scale_fmt);
    if (st != TK_SUCCESS || rows == 0) return st;
    if (tk_per_channel_workspace_bytes(rows, cols) > kNoAllocScratchBytes) return TK_ERROR_UNSUPPORTED;
    if (!aligned(scales, scale_fmt == kScaleF32 ? 16 : 8)) return TK_ERROR_MISALIGNED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    void *ws = nullptr;
    st = scratch_address(dev, &ws);
    if (st != TK_SUCCESS) return st;
    return launch_channel(x, rows, cols, x_ld, q, q_ld, scales, ws, out_dtype, round_pow2, scale_fmt,
                          static_cast<hipStream_t>(stream));
}

int64_t tk_per_channel_noalloc_max_workspace_bytes(void) { return kNoAllocScratchBytes; }

}  // extern "C"
