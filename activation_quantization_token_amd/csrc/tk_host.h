// tk_host.h -- host helpers shared by the library's entry points.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <mutex>

#include "tk_quant.h"

namespace {

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

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

}  // namespace
