// Internal interface of the measurement kernels (la_copy.hip): the reference
// copy and the direction probe, used by the C ABI layer (la_api.cpp). Not
// installed; callers use include/layeradam.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_internal.h"

namespace la {

// Enqueue dst[i] = src[i] for the n16 16-byte units of two disjoint, 16-byte
// aligned buffers, on `stream`. lds_per_cu / lds_per_block: the device's LDS
// sizes (0: unknown); wg_per_cu: resident workgroups per compute unit to aim
// for (-1: the kernel's default, 0: no cap); grid_cap: most workgroups of the
// launch (the kernel strides past it).
hipError_t launch_copy_reference(void* dst, const void* src, int64_t n16, int lds_per_cu,
                                 int lds_per_block, int wg_per_cu, int grid_cap,
                                 hipStream_t stream);

// Parts of the direction probe.
constexpr int kProbeReads = 0;   // read the R gradients and master, m, v; write nothing
constexpr int kProbeWrites = 1;  // write master, m, v (and the copy); read nothing

// Enqueue one part of the direction probe over `count` tensors (entries as
// for launch_layer_adam): the update's loads only, or its stores only, with
// the update's per-wave access pattern. The write part stores `fill` into
// master, m, v and its low 16 bits into the copy (unless out_dtype is
// kOutNone). shape.wg_per_cu: -1 for the part's default residency.
hipError_t launch_direction_probe(const TensorArgs* tensors, int count, int replicas,
                                  int out_dtype, int part, uint32_t fill, hipStream_t stream,
                                  const LaunchShape& shape);

}  // namespace la
