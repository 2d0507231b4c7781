// Internal interface of the reference copy (la_copy.hip), used by the C ABI
// layer (la_api.cpp). Not installed; callers use include/layeradam.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

// Enqueue dst[i] = src[i] for the n16 16-byte units of two disjoint, 16-byte
// aligned buffers, on `stream`. lds_per_cu / lds_per_block: the device's LDS
// sizes (0: unknown); wg_per_cu: resident workgroups per compute unit to aim
// for (-1: the kernel's default, 0: no cap).
hipError_t launch_copy_reference(void* dst, const void* src, int64_t n16, int lds_per_cu,
                                 int lds_per_block, int wg_per_cu, hipStream_t stream);

}  // namespace la
