// tk_host.h -- host helpers shared by the library's entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "tk_quant.h"

namespace {

constexpr int kMaxDevices = 64;

struct DeviceInfo {
    std::once_flag once;
    tk_status status = TK_ERROR_DEVICE;
    int cus = 0;
    // The SwiGLU form's silu32 table: built under table_mutex, table_ready
    // set only once the build has finished on the device, so that a failed
    // build is tried again by the next call.
    std::mutex table_mutex;
    std::atomic<bool> table_ready{false};
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

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Largest span accepted for an operand, (rows - 1) * ld + row length, in
// bytes: far beyond any device's memory, and small enough that every offset
// the host and the kernels form from rows, strides and sizes fits in int64.
constexpr int64_t kMaxSpanBytes = int64_t(1) << 52;

// Whether a [rows, row_elems] operand of elem-byte elements with a row stride
// of ld elements (ld >= row_elems >= 1) spans at most kMaxSpanBytes.
inline bool span_ok(int64_t rows, int64_t ld, int64_t row_elems, int64_t elem)
{
    if (rows <= 0) return true;
    const int64_t lim = kMaxSpanBytes / elem;
    return ld <= lim && rows - 1 <= (lim - row_elems) / ld;
}

// Run length (log2 of items) of xcd_order for a grid of `grid` workgroups
// over n items, each workgroup reading item_bytes of input: runs of about
// 1 MiB of input per XCD, 512 KiB when the whole input is at most 56 MiB
// (4096 x 7168 bf16), and -1 (no renumbering) when the grid loops over the
// items.  Measured on MI355X with the row-form cast at 7168 channels (one
// 14 KiB row per workgroup): runs of 64 rows 2.9 % faster than every-eighth-
// row order at 32768 rows and 2.4 % at 16384, runs of 32 rows 2 % at 4096;
// runs of 256 rows and more, and one contiguous eighth per XCD, were slower
// than no renumbering at all.  The fp32-input cast (-1.3 to -1.6 %), the
// cast-and-cast-back (-1.2 % at 32768 rows) and the stream ceiling use it;
// RMSNorm, per-block, per-channel and dequantization measured no gain (or a
// loss) and keep their order.
constexpr int64_t kXcdRunBytes = int64_t(1) << 20;
constexpr int64_t kXcdSmallRunBytes = int64_t(1) << 19;
constexpr int64_t kXcdSmallInputBytes = int64_t(4096) * 7168 * 2;

inline int xcd_run_log2(int64_t n, int64_t grid, int64_t item_bytes)
{
    if (grid != n || item_bytes <= 0) return -1;
    const int64_t target = n * item_bytes <= kXcdSmallInputBytes ? kXcdSmallRunBytes : kXcdRunBytes;
    int L = 0;
    while (L < 12 && (item_bytes << (L + 1)) <= target) ++L;
    return L;
}

}  // namespace
