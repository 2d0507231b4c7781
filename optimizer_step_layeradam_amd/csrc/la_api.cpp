// la_api.cpp -- the C ABI of liblayeradam.so (declared in include/layeradam.h).
//
// Host side only: checks every argument before anything is enqueued, derives
// the FP32 constants of the step, turns the layer (or an element range of it)
// into kernel tensor entries, splits them into launches of at most
// kTensorsPerLaunch entries and enqueues them on the caller's stream.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "la_copy.h"
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
// unit and the most one workgroup may take (the kernels size their LDS
// reservation from them). hipDeviceGetAttribute is cheap; caching keeps the
// per-call host path to a few hundred nanoseconds.
constexpr int kMaxDevices = 64;
struct DeviceFacts {
  std::atomic<int> lds_per_cu{-1};   // -1: not read yet
  std::atomic<int> lds_per_block{-1};
};
DeviceFacts g_facts[kMaxDevices];

void device_facts(int device, int* per_cu, int* per_block) {
  *per_cu = *per_block = 0;
  if (device < 0 || device >= kMaxDevices) return;
  DeviceFacts& f = g_facts[device];
  int a = f.lds_per_cu.load(std::memory_order_relaxed);
  int b = f.lds_per_block.load(std::memory_order_relaxed);
  if (a < 0 || b < 0) {
    a = b = 0;
    if (hipDeviceGetAttribute(&a, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor,
                              device) != hipSuccess)
      a = 0;
    if (hipDeviceGetAttribute(&b, hipDeviceAttributeMaxSharedMemoryPerBlock, device) !=
        hipSuccess)
      b = 0;
    f.lds_per_block.store(b, std::memory_order_relaxed);
    f.lds_per_cu.store(a, std::memory_order_relaxed);
  }
  *per_cu = a;
  *per_block = b;
}

// Resident workgroups per compute unit: LAYERADAM_WORKGROUPS_PER_CU (0..64,
// read once) overrides every kernel's own default; 0 removes the cap; -1
// (unset or unparsable) keeps the defaults.
int workgroups_per_cu_override() {
  static const int value = [] {
    const char* env = std::getenv("LAYERADAM_WORKGROUPS_PER_CU");
    if (env == nullptr || *env == '\0') return -1;
    char* end = nullptr;
    const long v = std::strtol(env, &end, 10);
    return (*end == '\0' && v >= 0 && v <= 64) ? static_cast<int>(v) : -1;
  }();
  return value;
}

// One workgroup per chunk up to this many; the kernels stride past it.
constexpr int kMaxGrid = 1 << 30;

// Most workgroups of one launch: kMaxGrid, or LAYERADAM_MAX_GRID (1..kMaxGrid,
// read once), which lets a test drive the kernels' striding loops with
// layers of ordinary size.
int max_grid() {
  static const int value = [] {
    const char* env = std::getenv("LAYERADAM_MAX_GRID");
    if (env == nullptr || *env == '\0') return kMaxGrid;
    char* end = nullptr;
    const long v = std::strtol(env, &end, 10);
    return (*end == '\0' && v >= 1 && v <= kMaxGrid) ? static_cast<int>(v) : kMaxGrid;
  }();
  return value;
}

bool finite_nonneg(double x) { return std::isfinite(x) && x >= 0.0; }

bool aligned(const void* p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

// kUpdate: the update (state and copy written); kProbe: the stream probe
// (the same buffers, no arithmetic); kCheck: gradients read only;
// kReadProbe / kWriteProbe: the two parts of the direction probe (the
// update's loads only, its stores only; checked as the stream probe).
enum class Mode { kUpdate, kProbe, kCheck, kReadProbe, kWriteProbe };

// Counts, dtypes and sizes; no pointers (enough for the byte accounting).
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
  if (layer->out_dtype != LA_OUT_BF16 && layer->out_dtype != LA_OUT_FP16 &&
      layer->out_dtype != LA_OUT_NONE)
    return fail(LA_ERR_UNSUPPORTED, "out_dtype = %d, need LA_OUT_BF16, LA_OUT_FP16 or LA_OUT_NONE",
                layer->out_dtype);
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

// Every buffer the mode touches: present and 16-byte aligned.
la_status check_pointers(const la_layer_desc* layer, Mode mode) {
  const bool state = mode != Mode::kCheck;
  const bool out = state && layer->out_dtype != LA_OUT_NONE;
  for (int i = 0; i < layer->num_tensors; ++i) {
    const la_tensor_desc& t = layer->tensors[i];
    if (t.numel == 0) continue;
    struct {
      const void* p;
      const char* name;
      bool used;
    } bufs[4 + LA_MAX_REPLICAS] = {{t.master, "master", state},
                                   {t.exp_avg, "exp_avg", state},
                                   {t.exp_avg_sq, "exp_avg_sq", state},
                                   {t.weight_out, "weight_out", out}};
    for (int r = 0; r < layer->num_replicas; ++r) bufs[4 + r] = {t.grads[r], "grads[r]", true};
    for (int k = 0; k < 4 + layer->num_replicas; ++k) {
      if (!bufs[k].used) continue;
      if (bufs[k].p == nullptr)
        return fail(LA_ERR_INVALID_ARGUMENT, "tensor %d: %s is NULL", i, bufs[k].name);
      if (!aligned(bufs[k].p, LA_ALIGNMENT))
        return fail(LA_ERR_MISALIGNED, "tensor %d: %s is not %d-byte aligned", i, bufs[k].name,
                    LA_ALIGNMENT);
    }
  }
  return LA_OK;
}

struct Range {
  uintptr_t begin, end;  // [begin, end)
  const char* what;
  int tensor;
};

bool overlaps(const Range& a, const Range& b) { return a.begin < b.end && b.begin < a.end; }

// Written ranges must be pairwise disjoint and must not overlap any range
// that is only read (gradients, the skip flag). Sort the written ranges;
// check neighbours, then look every read range up by binary search.
la_status check_aliasing(const la_layer_desc* layer, Mode mode, const int32_t* flag,
                         const int32_t* skip, const int64_t* step = nullptr) {
  std::vector<Range> written;
  std::vector<Range> read;
  const bool state = mode != Mode::kCheck;
  const bool out = state && layer->out_dtype != LA_OUT_NONE;
  written.reserve(4 * layer->num_tensors + 1);
  read.reserve(layer->num_replicas * layer->num_tensors + 1);
  for (int i = 0; i < layer->num_tensors; ++i) {
    const la_tensor_desc& t = layer->tensors[i];
    if (t.numel == 0) continue;
    const uintptr_t n = static_cast<uintptr_t>(t.numel);
    auto add = [&](std::vector<Range>& v, const void* p, uintptr_t bytes, const char* what) {
      const uintptr_t b = reinterpret_cast<uintptr_t>(p);
      v.push_back({b, b + bytes, what, i});
    };
    if (state) {
      add(written, t.master, 4 * n, "master");
      add(written, t.exp_avg, 4 * n, "exp_avg");
      add(written, t.exp_avg_sq, 4 * n, "exp_avg_sq");
    }
    if (out) add(written, t.weight_out, 2 * n, "weight_out");
    for (int r = 0; r < layer->num_replicas; ++r) add(read, t.grads[r], 2 * n, "grads");
  }
  if (flag != nullptr) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(flag);
    written.push_back({b, b + 4, "the flag", -1});
  }
  if (skip != nullptr) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(skip);
    read.push_back({b, b + 4, "skip_if_nonzero", -1});
  }
  if (step != nullptr) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(step);
    read.push_back({b, b + 8, "step_on_device", -1});
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
    // first written range that ends after g begins (written ranges are
    // disjoint and sorted, so their ends are sorted too)
    auto it = std::lower_bound(written.begin(), written.end(), g.begin,
                               [](const Range& w, uintptr_t x) { return w.end <= x; });
    if (it != written.end() && overlaps(*it, g))
      return fail(LA_ERR_ALIASING, "%s of tensor %d overlaps %s of tensor %d", g.what, g.tensor,
                  it->what, it->tensor);
  }
  return LA_OK;
}

la_status check_unscale(double u) {
  if (!(std::isfinite(u) && u > 0.0))
    return fail(LA_ERR_INVALID_ARGUMENT, "grad_unscale = %g, need finite > 0", u);
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
  la_status st = check_unscale(hp->grad_unscale);
  if (st != LA_OK) return st;
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

int64_t total_numel(const la_layer_desc* layer) {
  int64_t n = 0;
  for (int i = 0; i < layer->num_tensors; ++i) n += layer->tensors[i].numel;
  return n;
}

// Collect the kernel entries of elements [begin, end) and launch them in
// batches. Within a tensor the sub-range starts at element s: the part before
// the next multiple of 8 (at most 7 elements, so always the element-wise
// path of the kernel) becomes its own entry, and the rest starts 16-byte
// aligned (32 bytes into FP32 arrays, 16 into 16-bit arrays).
// fill and wg_per_cu serve the direction probe only (its stored pattern, and
// its residency: -1 for the default).
la_status enqueue(const la_layer_desc* layer, Mode mode, const la::Scalars& s,
                  const la::DeviceStep& dstep, int64_t begin, int64_t end, int32_t* flag,
                  const int32_t* skip, void* hip_stream, uint32_t fill = 0,
                  int wg_per_cu = -1) {
  la::TensorArgs batch[la::kTensorsPerLaunch];
  int pending = 0;
  int launches = 0;
  hipStream_t stream = static_cast<hipStream_t>(hip_stream);
  la::LaunchShape shape{0, 0, 0, -1};
  const bool fp16 = layer->grad_dtype == LA_GRAD_FP16;
  const bool state = mode != Mode::kCheck;
  const bool out = state && layer->out_dtype != LA_OUT_NONE;

  auto flush = [&]() -> la_status {
    if (pending == 0) return LA_OK;
    if (shape.grid_cap == 0) {
      int device = 0;
      hipError_t e = hipGetDevice(&device);
      if (e != hipSuccess)
        return fail(LA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
      shape.grid_cap = max_grid();
      device_facts(device, &shape.lds_per_cu, &shape.lds_per_block);
      shape.wg_per_cu = wg_per_cu >= 0 ? wg_per_cu : workgroups_per_cu_override();
    }
    hipError_t e;
    switch (mode) {
      case Mode::kUpdate:
        e = la::launch_layer_adam(batch, pending, layer->num_replicas, fp16, layer->out_dtype, s,
                                  dstep, flag, skip, stream, shape);
        break;
      case Mode::kProbe:
        e = la::launch_stream_probe(batch, pending, layer->num_replicas, layer->out_dtype,
                                    stream, shape);
        break;
      case Mode::kReadProbe:
      case Mode::kWriteProbe:
        e = la::launch_direction_probe(
            batch, pending, layer->num_replicas, layer->out_dtype,
            mode == Mode::kReadProbe ? la::kProbeReads : la::kProbeWrites, fill, stream, shape);
        break;
      default:
        e = la::launch_check_gradients(batch, pending, layer->num_replicas, fp16, s.u, flag,
                                       stream, shape);
    }
    if (e != hipSuccess)
      return fail(LA_ERR_HIP, "kernel launch %d failed: %s", launches, hipGetErrorString(e));
    ++launches;
    pending = 0;
    return LA_OK;
  };
  auto add = [&](const la_tensor_desc& t, int64_t first, int64_t count) -> la_status {
    la::TensorArgs& a = batch[pending++];
    a.p = state ? t.master + first : nullptr;
    a.m = state ? t.exp_avg + first : nullptr;
    a.v = state ? t.exp_avg_sq + first : nullptr;
    a.w = out ? t.weight_out + first : nullptr;
    for (int r = 0; r < la::kMaxReplicas; ++r)
      a.g[r] = r < layer->num_replicas ? static_cast<const uint16_t*>(t.grads[r]) + first
                                       : nullptr;
    a.numel = count;
    return pending == la::kTensorsPerLaunch ? flush() : LA_OK;
  };

  int64_t offset = 0;  // layer element number of the tensor's first element
  for (int i = 0; i < layer->num_tensors; ++i) {
    const la_tensor_desc& t = layer->tensors[i];
    const int64_t lo = std::max(begin, offset), hi = std::min(end, offset + t.numel);
    offset += t.numel;
    if (lo >= hi) continue;
    int64_t first = lo - offset + t.numel;  // element within the tensor
    int64_t count = hi - lo;
    const int64_t head = std::min(count, (8 - first % 8) % 8);  // <= la::kMaxUnalignedEntry
    la_status st;
    if (head > 0) {
      if ((st = add(t, first, head)) != LA_OK) return st;
      first += head;
      count -= head;
    }
    if (count > 0 && (st = add(t, first, count)) != LA_OK) return st;
  }
  la_status st = flush();
  if (st != LA_OK) return st;
  return ok();
}

la_status update(const la_layer_desc* layer, const la_adam_params* hp, int64_t begin,
                 int64_t end, bool whole, int32_t* flag, const int32_t* skip,
                 const int64_t* step_on_device, void* hip_stream) {
  la_status st = check_counts(layer);
  if (st != LA_OK) return st;
  if ((st = check_pointers(layer, Mode::kUpdate)) != LA_OK) return st;
  la::Scalars s;
  la::DeviceStep dstep = {nullptr, 0.0, 0.0, 0.0};
  if (step_on_device != nullptr && hp != nullptr) {
    if (!aligned(step_on_device, 8))
      return fail(LA_ERR_MISALIGNED, "step_on_device is not 8-byte aligned");
    la_adam_params at_one = *hp;  // t comes from the device; check the rest
    at_one.step = 1;
    if ((st = derive_scalars(&at_one, &s)) != LA_OK) return st;
    dstep = {step_on_device, hp->lr, hp->beta1, hp->beta2};
  } else if ((st = derive_scalars(hp, &s)) != LA_OK) {
    return st;
  }
  if (flag != nullptr && !aligned(flag, 4))
    return fail(LA_ERR_MISALIGNED, "overflow_flag is not 4-byte aligned");
  if (skip != nullptr && !aligned(skip, 4))
    return fail(LA_ERR_MISALIGNED, "skip_if_nonzero is not 4-byte aligned");
  const int64_t n = total_numel(layer);
  if (whole) {
    begin = 0;
    end = n;
  } else if (begin < 0 || begin > end || end > n) {
    return fail(LA_ERR_INVALID_ARGUMENT, "element range [%lld, %lld) outside [0, %lld]",
                static_cast<long long>(begin), static_cast<long long>(end),
                static_cast<long long>(n));
  }
  if ((st = check_aliasing(layer, Mode::kUpdate, flag, skip, step_on_device)) != LA_OK)
    return st;
  return enqueue(layer, Mode::kUpdate, s, dstep, begin, end, flag, skip, hip_stream);
}

}  // namespace

extern "C" {

LA_API la_status layer_adam_step(const la_layer_desc* layer, const la_adam_params* hp,
                                 int32_t* overflow_flag, void* hip_stream) {
  return update(layer, hp, 0, 0, true, overflow_flag, nullptr, nullptr, hip_stream);
}

LA_API la_status layer_adam_step_range(const la_layer_desc* layer, const la_adam_params* hp,
                                       int64_t elem_begin, int64_t elem_end,
                                       int32_t* overflow_flag, void* hip_stream) {
  return update(layer, hp, elem_begin, elem_end, false, overflow_flag, nullptr, nullptr,
                hip_stream);
}

LA_API la_status layer_adam_step_gated(const la_layer_desc* layer, const la_adam_params* hp,
                                       const int32_t* skip_if_nonzero,
                                       int32_t* overflow_flag, void* hip_stream) {
  if (skip_if_nonzero == nullptr)
    return fail(LA_ERR_INVALID_ARGUMENT, "skip_if_nonzero is NULL");
  return update(layer, hp, 0, 0, true, overflow_flag, skip_if_nonzero, nullptr, hip_stream);
}

LA_API la_status layer_adam_step_device_step(const la_layer_desc* layer,
                                             const la_adam_params* hp,
                                             const int64_t* step_on_device,
                                             int32_t* overflow_flag, void* hip_stream) {
  if (step_on_device == nullptr)
    return fail(LA_ERR_INVALID_ARGUMENT, "step_on_device is NULL");
  return update(layer, hp, 0, 0, true, overflow_flag, nullptr, step_on_device, hip_stream);
}

LA_API la_status layer_adam_step_ex(const la_layer_desc* layer, const la_adam_params* hp,
                                    const la_step_options* opts, void* hip_stream) {
  const la_step_options defaults = {};
  const la_step_options& o = opts != nullptr ? *opts : defaults;
  if (o.use_range != 0 && o.use_range != 1)
    return fail(LA_ERR_INVALID_ARGUMENT, "use_range = %d, need 0 or 1", o.use_range);
  return update(layer, hp, o.elem_begin, o.elem_end, o.use_range == 0, o.overflow_flag,
                o.skip_if_nonzero, o.step_on_device, hip_stream);
}

LA_API la_status la_check_gradients(const la_layer_desc* layer, double grad_unscale,
                                    int32_t* found_nonfinite, void* hip_stream) {
  la_status st = check_counts(layer);
  if (st != LA_OK) return st;
  if ((st = check_pointers(layer, Mode::kCheck)) != LA_OK) return st;
  if ((st = check_unscale(grad_unscale)) != LA_OK) return st;
  if (found_nonfinite == nullptr)
    return fail(LA_ERR_INVALID_ARGUMENT, "found_nonfinite is NULL");
  if (!aligned(found_nonfinite, 4))
    return fail(LA_ERR_MISALIGNED, "found_nonfinite is not 4-byte aligned");
  if ((st = check_aliasing(layer, Mode::kCheck, found_nonfinite, nullptr)) != LA_OK) return st;
  la::Scalars s = {};
  s.u = static_cast<float>(grad_unscale);
  return enqueue(layer, Mode::kCheck, s, la::DeviceStep{nullptr, 0.0, 0.0, 0.0}, 0,
                 total_numel(layer), found_nonfinite, nullptr, hip_stream);
}

LA_API la_status la_stream_probe(const la_layer_desc* layer, void* hip_stream) {
  la_status st = check_counts(layer);
  if (st != LA_OK) return st;
  if ((st = check_pointers(layer, Mode::kProbe)) != LA_OK) return st;
  if ((st = check_aliasing(layer, Mode::kProbe, nullptr, nullptr)) != LA_OK) return st;
  return enqueue(layer, Mode::kProbe, la::Scalars{}, la::DeviceStep{nullptr, 0.0, 0.0, 0.0}, 0,
                 total_numel(layer), nullptr, nullptr, hip_stream);
}

LA_API la_status la_direction_probe(const la_layer_desc* layer, int32_t part,
                                    int64_t elem_begin, int64_t elem_end, uint32_t fill,
                                    int32_t workgroups_per_cu, void* hip_stream) {
  la_status st = check_counts(layer);
  if (st != LA_OK) return st;
  if ((st = check_pointers(layer, Mode::kProbe)) != LA_OK) return st;
  if (part != LA_PROBE_READS && part != LA_PROBE_WRITES)
    return fail(LA_ERR_INVALID_ARGUMENT, "part = %d, need LA_PROBE_READS or LA_PROBE_WRITES",
                part);
  if (workgroups_per_cu < -1 || workgroups_per_cu > 64)
    return fail(LA_ERR_INVALID_ARGUMENT, "workgroups_per_cu = %d, need -1..64",
                workgroups_per_cu);
  const int64_t n = total_numel(layer);
  if (elem_begin < 0 || elem_begin > elem_end || elem_end > n)
    return fail(LA_ERR_INVALID_ARGUMENT, "element range [%lld, %lld) outside [0, %lld]",
                static_cast<long long>(elem_begin), static_cast<long long>(elem_end),
                static_cast<long long>(n));
  if ((st = check_aliasing(layer, Mode::kProbe, nullptr, nullptr)) != LA_OK) return st;
  return enqueue(layer, part == LA_PROBE_READS ? Mode::kReadProbe : Mode::kWriteProbe,
                 la::Scalars{}, la::DeviceStep{nullptr, 0.0, 0.0, 0.0}, elem_begin, elem_end,
                 nullptr, nullptr, hip_stream, fill, workgroups_per_cu);
}

LA_API la_status la_copy_reference(void* dst, const void* src, int64_t bytes,
                                   void* hip_stream) {
  if (bytes < 0 || bytes % 16 != 0)
    return fail(LA_ERR_INVALID_ARGUMENT, "bytes = %lld, need a multiple of 16 >= 0",
                static_cast<long long>(bytes));
  if (bytes == 0) return ok();
  if (dst == nullptr || src == nullptr)
    return fail(LA_ERR_INVALID_ARGUMENT, "%s is NULL", dst == nullptr ? "dst" : "src");
  if (!aligned(dst, LA_ALIGNMENT) || !aligned(src, LA_ALIGNMENT))
    return fail(LA_ERR_MISALIGNED, "%s is not %d-byte aligned",
                aligned(dst, LA_ALIGNMENT) ? "src" : "dst", LA_ALIGNMENT);
  const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
  const uintptr_t n = static_cast<uintptr_t>(bytes);
  if (d < s + n && s < d + n) return fail(LA_ERR_ALIASING, "dst and src overlap");
  int device = 0;
  hipError_t e = hipGetDevice(&device);
  if (e != hipSuccess) return fail(LA_ERR_HIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  int lds_per_cu = 0, lds_per_block = 0;
  device_facts(device, &lds_per_cu, &lds_per_block);
  e = la::launch_copy_reference(dst, src, bytes / 16, lds_per_cu, lds_per_block,
                                workgroups_per_cu_override(), max_grid(),
                                static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess)
    return fail(LA_ERR_HIP, "copy launch failed: %s", hipGetErrorString(e));
  return ok();
}

LA_API int64_t la_state_bytes(const la_layer_desc* layer) {
  if (check_counts(layer) != LA_OK) return -1;
  // BF16/FP16 weights 2 + gradients 2 + FP32 master 4 + FP32 m and v 8
  return 16 * total_numel(layer);
}

LA_API int64_t la_traffic_bytes(const la_layer_desc* layer) {
  if (check_counts(layer) != LA_OK) return -1;
  // R gradient reads + master/m/v read and written + the compute copy
  const int64_t out = layer->out_dtype == LA_OUT_NONE ? 0 : 2;
  return (2 * static_cast<int64_t>(layer->num_replicas) + 24 + out) * total_numel(layer);
}

LA_API const char* la_last_error(void) { return g_error; }

LA_API const char* la_version(void) { return "layeradam 0.6.0 gfx950"; }

}  // extern "C"
