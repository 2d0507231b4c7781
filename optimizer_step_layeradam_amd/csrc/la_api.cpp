// la_api.cpp -- the C ABI of liblayeradam.so (declared in include/layeradam.h).
//
// Host side only: checks every argument before anything is enqueued, derives
// the FP32 constants of the step, splits the layer into launches of at most
// kTensorsPerLaunch tensors and enqueues them on the caller's stream.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <utility>
#include <vector>

#include "la_internal.h"
#include "layeradam.h"

namespace {

thread_local char g_error[512] = "";

la_status fail(la_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

la_status ok() {
  g_error[0] = '\0';
  return LA_OK;
}

// Per-device launch facts, read once per device: the LDS of one compute
// unit and the most one workgroup may take. (hipDeviceGetAttribute is cheap;
// caching keeps the per-call host path to a few hundred nanoseconds.)
constexpr int kMaxDevices = 64;
std::atomic<int> g_lds_reserve[kMaxDevices];  // bytes + 1; 0 = not read yet

// LDS to reserve per workgroup so that at most `per_cu` workgroups fit on a
// compute unit: floor(lds_per_cu / (per_cu + 1/2)), within the per-workgroup
// limit. 0 (no reservation) when no cap is wanted or the facts are missing.
int lds_reserve(int device, int per_cu) {
  if (per_cu <= 0 || device < 0 || device >= kMaxDevices) return 0;
  const int cached = g_lds_reserve[device].load(std::memory_order_relaxed);
  if (cached > 0) return cached - 1;
  int per_cu_bytes = 0, per_block_bytes = 0;
  int bytes = 0;
  if (hipDeviceGetAttribute(&per_cu_bytes, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                            device) == hipSuccess &&
      hipDeviceGetAttribute(&per_block_bytes, hipDeviceAttributeMaxSharedMemoryPerBlock,
                            device) == hipSuccess &&
      per_cu_bytes > 0 && per_block_bytes > 0) {
    bytes = static_cast<int>(2LL * per_cu_bytes / (2LL * per_cu + 1)) / 1024 * 1024;
    if (bytes > per_block_bytes) bytes = 0;  // cannot cap this way on this device
  }
  g_lds_reserve[device].store(bytes + 1, std::memory_order_relaxed);
  return bytes;
}

// Workgroups resident per compute unit. LAYERADAM_WORKGROUPS_PER_CU (0..64,
// read once) overrides the built-in target; 0 removes the cap.
int workgroups_per_cu() {
  static const int value = [] {
    const char* env = std::getenv("LAYERADAM_WORKGROUPS_PER_CU");
    if (env == nullptr) return la::target_workgroups_per_cu();
    const int v = std::atoi(env);
    return (v >= 0 && v <= 64) ? v : la::target_workgroups_per_cu();
  }();
  return value;
}

// One workgroup per chunk up to this many; the kernel strides past it.
constexpr int kMaxGrid = 1 << 30;

bool finite_nonneg(double x) { return std::isfinite(x) && x >= 0.0; }

struct Range {
  uintptr_t begin, end;  // [begin, end)
  const char* what;
  int tensor;
};

bool overlaps(const Range& a, const Range& b) { return a.begin < b.end && b.begin < a.end; }

// Counts, dtype and sizes; no pointers (enough for the byte accounting).
la_status check_counts(const la_layer_desc* layer) {
  if (layer == nullptr) return fail(LA_ERR_INVALID_ARGUMENT, "layer descriptor is NULL");
  if (layer->num_tensors < 0 || layer->num_tensors > LA_MAX_TENSORS)
    return fail(LA_ERR_INVALID_ARGUMENT, "num_tensors = %d, need 0..%d", layer->num_tensors,
                LA_MAX_TENSORS);
  if (layer->num_tensors > 0 && layer->tensors == nullptr)
    return fail(LA_ERR_INVALID_ARGUMENT, "tensors is NULL with num_tensors = %d",
                layer->num_tensors);
  if (layer->num_replicas < 1 || layer->num_replicas > LA_MAX_REPLICAS)
    return fail(LA_ERR_INVALID_ARGUMENT, "num_replicas = %d, need 1..%d", layer->num_replicas,
                LA_MAX_REPLICAS);
  if (layer->grad_dtype != LA_GRAD_BF16 && layer->grad_dtype != LA_GRAD_FP16)
    return fail(LA_ERR_UNSUPPORTED, "grad_dtype = %d, need LA_GRAD_BF16 or LA_GRAD_FP16",
                layer->grad_dtype);
  // Largest numel whose byte sizes and (2R + 26)-byte traffic stay far from
  // overflowing 64 bits, even summed over LA_MAX_TENSORS tensors.
  constexpr int64_t kMaxNumel = int64_t(1) << 48;
  for (int i = 0; i < layer->num_tensors; ++i) {
    const int64_t n = layer->tensors[i].numel;
    if (n < 0 || n > kMaxNumel)
      return fail(LA_ERR_INVALID_ARGUMENT, "tensor %d: numel = %lld out of range", i,
                  static_cast<long long>(n));
  }
  return LA_OK;
}

la_status check_layer(const la_layer_desc* layer) {
  la_status st = check_counts(layer);
  if (st != LA_OK) return st;
  for (int i = 0; i < layer->num_tensors; ++i) {
    const la_tensor_desc& t = layer->tensors[i];
    if (t.numel == 0) continue;
    const void* ptrs[4 + LA_MAX_REPLICAS] = {t.master, t.exp_avg, t.exp_avg_sq, t.weight_bf16};
    const char* names[4] = {"master", "exp_avg", "exp_avg_sq", "weight_bf16"};
    for (int r = 0; r < layer->num_replicas; ++r) ptrs[4 + r] = t.grads[r];
    for (int k = 0; k < 4 + layer->num_replicas; ++k) {
      const char* name = k < 4 ? names[k] : "grads";
      if (ptrs[k] == nullptr)
        return fail(LA_ERR_INVALID_ARGUMENT, "tensor %d: %s%s is NULL", i, name,
                    k < 4 ? "" : "[r]");
      if (reinterpret_cast<uintptr_t>(ptrs[k]) % LA_ALIGNMENT != 0)
        return fail(LA_ERR_MISALIGNED, "tensor %d: %s%s is not %d-byte aligned", i, name,
                    k < 4 ? "" : "[r]", LA_ALIGNMENT);
    }
  }
  return LA_OK;
}

// Written ranges must be pairwise disjoint and must not overlap any gradient
// or the flag. Sort the written ranges; check neighbours, then look every
// gradient range up by binary search.
la_status check_aliasing(const la_layer_desc* layer, const int32_t* flag) {
  std::vector<Range> written;
  std::vector<Range> read;
  written.reserve(4 * layer->num_tensors + 1);
  read.reserve(layer->num_replicas * layer->num_tensors);
  for (int i = 0; i < layer->num_tensors; ++i) {
    const la_tensor_desc& t = layer->tensors[i];
    if (t.numel == 0) continue;
    const uintptr_t n = static_cast<uintptr_t>(t.numel);
    auto add = [&](std::vector<Range>& v, const void* p, uintptr_t bytes, const char* what) {
      const uintptr_t b = reinterpret_cast<uintptr_t>(p);
      v.push_back({b, b + bytes, what, i});
    };
    add(written, t.master, 4 * n, "master");
    add(written, t.exp_avg, 4 * n, "exp_avg");
    add(written, t.exp_avg_sq, 4 * n, "exp_avg_sq");
    add(written, t.weight_bf16, 2 * n, "weight_bf16");
    for (int r = 0; r < layer->num_replicas; ++r) add(read, t.grads[r], 2 * n, "grads");
  }
  if (flag != nullptr) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(flag);
    written.push_back({b, b + 4, "overflow_flag", -1});
  }
  std::sort(written.begin(), written.end(),
            [](const Range& a, const Range& b) { return a.begin < b.begin; });
  for (size_t k = 1; k < written.size(); ++k) {
    if (overlaps(written[k - 1], written[k]))
      return fail(LA_ERR_ALIASING, "%s of tensor %d overlaps %s of tensor %d",
                  written[k - 1].what, written[k - 1].tensor, written[k].what,
                  written[k].tensor);
  }
  for (const Range& g : read) {
    // first written range that ends after g begins
    auto it = std::lower_bound(written.begin(), written.end(), g.begin,
                               [](const Range& w, uintptr_t x) { return w.end <= x; });
    // written ranges are disjoint and sorted, so their ends are sorted too
    if (it != written.end() && overlaps(*it, g))
      return fail(LA_ERR_ALIASING, "a gradient of tensor %d overlaps %s of tensor %d", g.tensor,
                  it->what, it->tensor);
  }
  return LA_OK;
}

la_status derive_scalars(const la_adam_params* hp, la::Scalars* s) {
  if (hp == nullptr) return fail(LA_ERR_INVALID_ARGUMENT, "hyperparameters are NULL");
  if (hp->step < 1)
    return fail(LA_ERR_INVALID_ARGUMENT, "step = %lld, need t >= 1",
                static_cast<long long>(hp->step));
  if (!(hp->beta1 >= 0.0 && hp->beta1 < 1.0))
    return fail(LA_ERR_INVALID_ARGUMENT, "beta1 = %g, need 0 <= beta1 < 1", hp->beta1);
  if (!(hp->beta2 >= 0.0 && hp->beta2 < 1.0))
    return fail(LA_ERR_INVALID_ARGUMENT, "beta2 = %g, need 0 <= beta2 < 1", hp->beta2);
  if (!finite_nonneg(hp->lr)) return fail(LA_ERR_INVALID_ARGUMENT, "lr = %g", hp->lr);
  if (!finite_nonneg(hp->eps)) return fail(LA_ERR_INVALID_ARGUMENT, "eps = %g", hp->eps);
  if (!finite_nonneg(hp->weight_decay))
    return fail(LA_ERR_INVALID_ARGUMENT, "weight_decay = %g", hp->weight_decay);
  if (!(std::isfinite(hp->grad_unscale) && hp->grad_unscale > 0.0))
    return fail(LA_ERR_INVALID_ARGUMENT, "grad_unscale = %g, need finite > 0",
                hp->grad_unscale);
  // Bias corrections of AdamW at the 1-based step t, in double; each FP32
  // constant is rounded once.
  const double t = static_cast<double>(hp->step);
  const double one_minus_beta1_t = 1.0 - std::pow(hp->beta1, t);
  const double one_minus_beta2_t = 1.0 - std::pow(hp->beta2, t);
  s->b1 = static_cast<float>(hp->beta1);
  s->c1 = static_cast<float>(1.0 - hp->beta1);
  s->b2 = static_cast<float>(hp->beta2);
  s->c2 = static_cast<float>(1.0 - hp->beta2);
  s->alpha = static_cast<float>(hp->lr / one_minus_beta1_t);
  s->q = static_cast<float>(std::sqrt(one_minus_beta2_t));
  s->e = static_cast<float>(hp->eps);
  s->d = static_cast<float>(1.0 - hp->lr * hp->weight_decay);
  s->u = static_cast<float>(hp->grad_unscale);
  return LA_OK;
}

}  // namespace

extern "C" {

LA_API la_status layer_adam_step(const la_layer_desc* layer, const la_adam_params* hp,
                                 int32_t* overflow_flag, void* hip_stream) {
  la_status st = check_layer(layer);
  if (st != LA_OK) return st;
  la::Scalars s;
  st = derive_scalars(hp, &s);
  if (st != LA_OK) return st;
  if (overflow_flag != nullptr && reinterpret_cast<uintptr_t>(overflow_flag) % 4 != 0)
    return fail(LA_ERR_MISALIGNED, "overflow_flag is not 4-byte aligned");
  st = check_aliasing(layer, overflow_flag);
  if (st != LA_OK) return st;

  // Non-empty tensors, in order.
  la::TensorArgs batch[la::kTensorsPerLaunch];
  int pending = 0;
  int launches = 0;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  la::LaunchShape shape{0, 0};

  auto flush = [&]() -> la_status {
    if (pending == 0) return LA_OK;
    if (shape.grid_cap == 0) {
      int device = 0;
      hipError_t e = hipGetDevice(&device);
      if (e != hipSuccess)
        return fail(LA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
      shape.grid_cap = kMaxGrid;
      shape.lds_bytes = lds_reserve(device, workgroups_per_cu());
    }
    hipError_t e = la::launch_layer_adam(batch, pending, layer->num_replicas,
                                         layer->grad_dtype == LA_GRAD_FP16, s, overflow_flag,
                                         stream, shape);
    if (e != hipSuccess)
      return fail(LA_ERR_HIP, "kernel launch %d failed: %s", launches, hipGetErrorString(e));
    ++launches;
    pending = 0;
    return LA_OK;
  };

  for (int i = 0; i < layer->num_tensors; ++i) {
    const la_tensor_desc& t = layer->tensors[i];
    if (t.numel == 0) continue;
    la::TensorArgs& a = batch[pending++];
    a.p = t.master;
    a.m = t.exp_avg;
    a.v = t.exp_avg_sq;
    a.w = t.weight_bf16;
    for (int r = 0; r < la::kMaxReplicas; ++r)
      a.g[r] = r < layer->num_replicas ? static_cast<const uint16_t*>(t.grads[r]) : nullptr;
    a.numel = t.numel;
    if (pending == la::kTensorsPerLaunch) {
      st = flush();
      if (st != LA_OK) return st;
    }
  }
  st = flush();
  if (st != LA_OK) return st;
  return ok();
}

LA_API int64_t la_state_bytes(const la_layer_desc* layer) {
  if (check_counts(layer) != LA_OK) return -1;
  int64_t n = 0;
  for (int i = 0; i < layer->num_tensors; ++i) n += layer->tensors[i].numel;
  // BF16/FP16 weights 2 + gradients 2 + FP32 master 4 + FP32 m and v 8
  return 16 * n;
}

LA_API int64_t la_traffic_bytes(const la_layer_desc* layer) {
  if (check_counts(layer) != LA_OK) return -1;
  int64_t n = 0;
  for (int i = 0; i < layer->num_tensors; ++i) n += layer->tensors[i].numel;
  // R gradient reads + master/m/v read and written + BF16 write
  return (2 * static_cast<int64_t>(layer->num_replicas) + 26) * n;
}

LA_API const char* la_last_error(void) { return g_error; }

LA_API const char* la_version(void) { return "layeradam 0.1.0 gfx950"; }

}  // extern "C"
