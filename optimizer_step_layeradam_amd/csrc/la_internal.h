// Internal interface between the C ABI layer (la_api.cpp) and the kernels
// (la_kernel.hip). Not installed; callers use include/layeradam.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace la {

constexpr int kMaxReplicas = 8;

// Compute-copy formats (the values of la_out_dtype).
constexpr int kOutBf16 = 0;
constexpr int kOutFp16 = 1;
constexpr int kOutNone = 2;
// Tensors per kernel launch: their pointers travel in the kernel arguments
// (about 104 bytes per tensor at R = 8).
constexpr int kTensorsPerLaunch = 16;

// Longest entry that may start unaligned (the head peeled off an element
// range that does not start at a multiple of 8 elements).
constexpr int kMaxUnalignedEntry = 7;

// The FP32 constants of one step, derived on the host.
struct Scalars {
  float b1, c1;   // beta1, 1 - beta1
  float b2, c2;   // beta2, 1 - beta2
  float alpha;    // lr / (1 - beta1^t)
  float q;        // sqrt(1 - beta2^t)
  float e;        // eps
  float d;        // 1 - lr * weight_decay
  float u;        // gradient unscale factor
};

// With the step count in device memory, the kernel derives alpha and q
// itself from these (the other constants come from the host as usual).
struct DeviceStep {
  const int64_t* t;  // null: alpha and q in Scalars are final
  double lr, beta1, beta2;
};

// One non-empty tensor, already validated (16-byte aligned, disjoint).
struct TensorArgs {
  float* p;
  float* m;
  float* v;
  uint16_t* w;
  const uint16_t* g[kMaxReplicas];
  int64_t numel;
};

struct LaunchShape {
  int grid_cap;        // upper bound on workgroups of one launch
  int lds_per_cu;      // LDS bytes of one compute unit (0: unknown)
  int lds_per_block;   // most LDS one workgroup may take (0: unknown)
  int wg_per_cu;       // resident workgroups per compute unit to aim for;
                       // -1: each kernel's own default, 0: no cap
};

// Enqueue the update of `count` (1..kTensorsPerLaunch) tensors in one launch.
// flag: overflow flag or null; skip: device flag that makes the kernel a
// no-op when non-zero, or null. An entry of at most kMaxUnalignedEntry
// elements may have pointers aligned to their element size only (every
// kernel takes its element-wise path for an entry shorter than one chunk);
// longer entries need 16-byte alignment of every pointer.
hipError_t launch_layer_adam(const TensorArgs* tensors, int count, int replicas,
                             bool fp16, int out_dtype, const Scalars& s,
                             const DeviceStep& dstep, int32_t* flag, const int32_t* skip,
                             hipStream_t stream, const LaunchShape& shape);

// Enqueue the stream probe over `count` tensors: the update's loads, stores
// and launch shape with no arithmetic (master, m, v written back unchanged;
// a 16-bit copy, unless out_dtype is kOutNone, written as the XOR of the
// replicas' bit patterns).
hipError_t launch_stream_probe(const TensorArgs* tensors, int count, int replicas,
                               int out_dtype, hipStream_t stream, const LaunchShape& shape);

// Enqueue the finite check of the aggregated gradients (sum of replicas times
// unscale) of `count` tensors; sets *flag to 1 if one is +-Inf or NaN.
hipError_t launch_check_gradients(const TensorArgs* tensors, int count, int replicas,
                                  bool fp16, float unscale, int32_t* flag,
                                  hipStream_t stream, const LaunchShape& shape);


}  // namespace la
