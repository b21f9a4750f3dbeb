// tk_diag.hip -- gfx950 streaming diagnostics behind the C ABI: a plain copy
// (the reference transfer for calibrating memory counters) and a read/write
// stream of given volumes (the practical ceiling of an operation that moves
// the same bytes).  They compute nothing of the cast.

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "tk_device.h"
#include "tk_host.h"

namespace {

constexpr int kCopyBlock = 256;

__global__ __launch_bounds__(kCopyBlock) void copy_stream_kernel(const u32x4 *src, u32x4 *dst, int64_t n16)
{
    const int64_t stride = int64_t(gridDim.x) * kCopyBlock;
    for (int64_t i = int64_t(blockIdx.x) * kCopyBlock + threadIdx.x; i < n16; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// A read/write stream shaped like the row-form cast: workgroups of 7 waves,
// each wave reading 2 KiB of src (two 1 KiB loads, 16 bytes per lane) and
// writing its share of dst, wpw bytes, in 4-byte stores per lane (256 bytes
// per wave instruction); all non-temporal.  The stores write an xor of what
// the wave read, so no load can be dropped.  Of the plain streams measured on
// MI355X at the cast's 4:1 and 2:1 read:write volumes (grid-stride loops of
// 2-8 KiB per wave step, one-shot waves of 1, 2 or 4 KiB, 4, 7 or 16 waves
// per workgroup), this shape was the fastest; its workgroups take the
// row-form cast's XCD order (xcd_order).
constexpr int kStreamWaves = 7;
constexpr int64_t kStreamWaveBytes = 2048;

__global__ __launch_bounds__(kWave * kStreamWaves) void stream_rw_kernel(const uint8_t *src, int64_t read_bytes,
                                                                       uint8_t *dst, int64_t write_bytes,
                                                                       int64_t wpw, int xcd_log2)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t wave = xcd_order(blockIdx.x, gridDim.x, xcd_log2) * kStreamWaves +
                         __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t r0 = wave * kStreamWaveBytes, w0 = wave * wpw;
    const int64_t rn = read_bytes - r0, wn = write_bytes - w0;
    const __amdgpu_buffer_rsrc_t r =
        row_buffer(src + (rn > 0 ? r0 : 0), uint32_t(rn <= 0 ? 0 : rn < kStreamWaveBytes ? rn : kStreamWaveBytes));
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 0, kNonTemporal);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, lane * 16, 1024, kNonTemporal);
    const uint32_t v = a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w;
    const __amdgpu_buffer_rsrc_t w = row_buffer(dst + (wn > 0 ? w0 : 0), uint32_t(wn <= 0 ? 0 : wn < wpw ? wn : wpw));
    for (int64_t j = 0; j < wpw; j += kWave * 4)
        __builtin_amdgcn_raw_buffer_store_b32(v ^ uint32_t(j), w, lane * 4 + int(j), 0, kNonTemporal);
}

}  // namespace

extern "C" {

tk_status tk_copy_stream(const void *src, void *dst, int64_t bytes, void *stream)
{
    if (bytes < 0 || bytes % 16 != 0) return TK_ERROR_INVALID_VALUE;
    if (bytes == 0) return TK_SUCCESS;
    if (!src || !dst) return TK_ERROR_INVALID_VALUE;
    if (!aligned(src, 16) || !aligned(dst, 16)) return TK_ERROR_MISALIGNED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    tk_status st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    const u32x4 *sp = static_cast<const u32x4 *>(src);
    u32x4 *dp = static_cast<u32x4 *>(dst);
    int64_t n16 = bytes / 16;
    int64_t blocks = (n16 + kCopyBlock - 1) / kCopyBlock;
    if (blocks > int64_t(info->cus) * 128) blocks = int64_t(info->cus) * 128;
    void *args[] = {&sp, &dp, &n16};
    if (hipLaunchKernel(reinterpret_cast<const void *>(copy_stream_kernel), dim3(uint32_t(blocks)),
                        dim3(kCopyBlock), args, 0, static_cast<hipStream_t>(stream)) != hipSuccess)
        return TK_ERROR_LAUNCH;
    return TK_SUCCESS;
}

tk_status tk_stream_rw(const void *src, int64_t read_bytes, void *dst, int64_t write_bytes, void *stream)
{
    if (read_bytes < 0 || write_bytes < 0 || read_bytes % 16 != 0 || write_bytes % 16 != 0)
        return TK_ERROR_INVALID_VALUE;
    if (read_bytes >= (int64_t(1) << 35) || write_bytes >= (int64_t(1) << 35)) return TK_ERROR_UNSUPPORTED;
    if (read_bytes == 0 || write_bytes == 0) return read_bytes == write_bytes ? TK_SUCCESS : TK_ERROR_INVALID_VALUE;
    if (!src || !dst) return TK_ERROR_INVALID_VALUE;
    if (!aligned(src, 16) || !aligned(dst, 16)) return TK_ERROR_MISALIGNED;
    int dev = 0;
    DeviceInfo *info = nullptr;
    tk_status st = device_info(&dev, &info);
    if (st != TK_SUCCESS) return st;
    // One wave per 2 KiB of the larger volume; each writes an equal share of
    // dst, rounded up to whole 256-byte wave stores (the last share is cut at
    // write_bytes by its descriptor).
    const int64_t larger = read_bytes > write_bytes ? read_bytes : write_bytes;
    const int64_t waves = (larger + kStreamWaveBytes - 1) / kStreamWaveBytes;
    const int64_t per_wave = (write_bytes + waves - 1) / waves;
    int64_t wpw = (per_wave + 255) / 256 * 256;
    const int64_t blocks = (waves + kStreamWaves - 1) / kStreamWaves;
    if (blocks > int64_t(0x7FFFFFFF)) return TK_ERROR_UNSUPPORTED;
    const uint8_t *sp = static_cast<const uint8_t *>(src);
    uint8_t *dp = static_cast<uint8_t *>(dst);
    int64_t rb = read_bytes, wb = write_bytes;
    // workgroups in the row-form cast's XCD order (14 KiB read each)
    int xl = xcd_run_log2(blocks, blocks, kStreamWaves * kStreamWaveBytes);
    void *args[] = {&sp, &rb, &dp, &wb, &wpw, &xl};
    if (hipLaunchKernel(reinterpret_cast<const void *>(stream_rw_kernel), dim3(uint32_t(blocks)),
                        dim3(kWave * kStreamWaves), args, 0, static_cast<hipStream_t>(stream)) != hipSuccess)
        return TK_ERROR_LAUNCH;
    return TK_SUCCESS;
}

}  // extern "C"
