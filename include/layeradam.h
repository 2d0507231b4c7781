/*
 * layeradam.h -- C ABI of the LayerAdam library (liblayeradam.so, gfx950).
 *
 * One call updates one decoder layer: it sums the layer's R data-parallel
 * BF16/FP16 gradient replicas, applies one bias-corrected AdamW step to the
 * FP32 master weights and FP32 moments (m, v) in place, and writes the BF16
 * compute copy of the new master weights -- in one fused pass over HBM on the
 * caller's HIP stream.
 *
 * Where the operation is defined:
 *  - The state is the mixed-precision Adam state of "SlideDP: Scaling
 *    Host-Resident LLM Fine-Tuning Across Multiple GPUs", section 前置知识
 *    (preliminaries): BF16/FP16 weights and gradients 2N bytes each, FP32
 *    master 4N, FP32 Adam m and v 8N -- 16N bytes in all (la_state_bytes).
 *  - The same page, sections 核心方法 (core method) and 方法步骤详情
 *    (method details): one authoritative FP32 master and (m, v) per layer,
 *    updated once per iteration from one aggregated gradient (the replicas
 *    reduced on the GPU), after which the next BF16 delivery of the layer
 *    may go out. The page runs the update ("LayerAdam") on host CPUs; this
 *    library runs reduction, update and cast as one GPU kernel.
 *  - "An Efficient Heterogeneous Co-Design for Fine-Tuning on a Single GPU"
 *    (SlideFormer), technical summary 2.2: gradients in a BF16/FP16 buffer,
 *    FP32 -> BF16 conversion of the master for the compute copy, and
 *    preallocated fixed-size buffers (so the library allocates nothing).
 *    "AutoHete" (mhpn.cn), section 2.2: on-the-fly FP32 -> FP16 conversion
 *    (the FP16 compute copy).
 *  - The pages print no Adam formula. The update is PyTorch's AdamW, the
 *    optimizer of the FSDP2 runs SlideDP checks its loss against (section
 *    实验结果, results):
 *        g   = (G_0 + G_1 + ... + G_{R-1}) * grad_unscale   (left to right)
 *        m   = beta1*m + (1-beta1)*g
 *        v   = beta2*v + (1-beta2)*(g*g)
 *        p   = p*(1 - lr*weight_decay)
 *              - lr/(1-beta1^t) * m / (sqrt(v)/sqrt(1-beta2^t) + eps)
 *        w   = BF16(p) or FP16(p), round to nearest, ties to even
 *              (NaN -> 0x7FC0 / 0x7E00), or no compute copy at all
 *    in FP32, one rounding per operation and no fused multiply-add; the
 *    nine constants beta1, 1-beta1, beta2, 1-beta2, lr/(1-beta1^t),
 *    sqrt(1-beta2^t), eps, 1-lr*weight_decay and grad_unscale are computed
 *    on the host in double and rounded to FP32 once per call.
 *
 * Memory and ownership: every buffer is caller-owned memory the current HIP
 * device can address: its own memory, or pinned host memory mapped for it
 * (hipHostMalloc; pass the device-side address, hipHostGetDevicePointer).
 * With the master, m and v in pinned host memory the state stays host-
 * resident, as in the pages' setting ("SlideDP", 前置知识: host-resident
 * layer streaming), and the kernel streams it over the host link. The
 * library never allocates, never synchronises and keeps no pointer after a
 * call returns. Calls are asynchronous on the given stream; buffers must
 * stay alive until the stream reaches the work.
 *
 * Thread safety: calls may come from several host threads at once. The only
 * global state is a thread-local error message and, per device, the LDS
 * sizes the launch shape is derived from (read once, atomically).
 *
 * Environment (each read once per process; for measurement and testing, the
 * results do not depend on them): LAYERADAM_WORKGROUPS_PER_CU (0..64)
 * replaces every kernel's resident-workgroups-per-compute-unit default, 0
 * meaning no cap; LAYERADAM_MAX_GRID (1..2^30) lowers the most workgroups
 * one launch may have, past which the kernels stride.
 */
#ifndef LAYERADAM_H
#define LAYERADAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LA_API __attribute__((visibility("default")))

#define LA_MAX_REPLICAS 8   /* R in [1, 8]                                  */
#define LA_MAX_TENSORS 256  /* tensors per call (split into several launches) */
#define LA_ALIGNMENT 16     /* bytes; every non-empty buffer must be aligned  */

typedef enum {
  LA_OK = 0,
  LA_ERR_INVALID_ARGUMENT = 1, /* NULL where a pointer is needed, bad count,
                                  hyperparameter outside its domain        */
  LA_ERR_MISALIGNED = 2,       /* a buffer not 16-byte aligned              */
  LA_ERR_ALIASING = 3,         /* written ranges overlap each other or a
                                  gradient                                  */
  LA_ERR_UNSUPPORTED = 4,      /* unknown gradient dtype or copy format     */
  LA_ERR_HIP = 5               /* the HIP runtime refused the launch        */
} la_status;

typedef enum { LA_GRAD_BF16 = 0, LA_GRAD_FP16 = 1 } la_grad_dtype;

/* Format of the compute copy of the new master weights. */
typedef enum { LA_OUT_BF16 = 0, LA_OUT_FP16 = 1, LA_OUT_NONE = 2 } la_out_dtype;

/* One tensor of the layer. All arrays hold `numel` elements, contiguous.
 * master, exp_avg, exp_avg_sq are read and written in place; weight_out is
 * written only (BF16 or FP16 bit patterns, per the layer's out_dtype; not
 * used, and may be NULL, with LA_OUT_NONE); grads[0..R-1] are read only, in
 * the layer's gradient dtype. Gradient replicas may alias one another
 * (passing one buffer R times is legal); no written array may overlap any
 * other array of the call. numel == 0 tensors are skipped and their pointers
 * ignored. */
typedef struct {
  float *master;
  float *exp_avg;
  float *exp_avg_sq;
  uint16_t *weight_out;
  const void *grads[LA_MAX_REPLICAS];
  int64_t numel;
} la_tensor_desc;

/* The layer: a host array of num_tensors descriptors (0 <= num_tensors <=
 * LA_MAX_TENSORS; 0 is a no-op), the number of replicas R, their dtype
 * (la_grad_dtype) and the compute-copy format (la_out_dtype). The layer's
 * elements are numbered 0..N-1 across its tensors in order (tensor 0 first);
 * the range entry point uses that numbering. The descriptor array is read
 * during the call only. */
typedef struct {
  const la_tensor_desc *tensors;
  int32_t num_tensors;
  int32_t num_replicas;
  int32_t grad_dtype;
  int32_t out_dtype;
} la_layer_desc;

/* Hyperparameters of one step. step is the 1-based count of the update being
 * applied (t >= 1). Domains: 0 <= beta1, beta2 < 1; lr, eps, weight_decay
 * finite and >= 0; grad_unscale finite and > 0 (1.0 = none; 1/R gives the
 * mean of the replicas instead of their sum). */
typedef struct {
  double lr;
  double beta1;
  double beta2;
  double eps;
  double weight_decay;
  int64_t step;
  double grad_unscale;
} la_adam_params;

/* Enqueue one LayerAdam update of `layer` on `hip_stream` (a hipStream_t;
 * NULL = the null stream).
 *
 * overflow_flag: NULL, or a 4-byte-aligned int32 in device memory that the
 * kernel sets to 1 if some aggregated gradient element (after the unscale)
 * is +-Inf or NaN. The library never clears it: the caller zeroes it, may
 * share it across the layers of a step, and reads it after synchronising.
 * The update is applied either way; non-finite values propagate by IEEE
 * rules into m, v, master and the compute copy.
 *
 * Returns LA_OK once the work is enqueued. Every argument is checked on the
 * host before anything is enqueued; on any other status nothing is enqueued
 * and la_last_error() describes the problem. Device faults surface at the
 * caller's next synchronisation, not here. */
LA_API la_status layer_adam_step(const la_layer_desc *layer,
                                 const la_adam_params *hp,
                                 int32_t *overflow_flag, void *hip_stream);

/* The same update restricted to the layer's elements [elem_begin, elem_end)
 * (0 <= elem_begin <= elem_end <= N, numbering as in la_layer_desc). Calls
 * over a partition of [0, N) leave exactly the state one layer_adam_step
 * leaves, bit for bit: the update is elementwise. This is the per-chunk
 * release of "SlideDP: Scaling Host-Resident LLM Fine-Tuning Across Multiple
 * GPUs", sections 核心方法 and 方法步骤详情 (a chunk of the layer is updated
 * as soon as its reduced gradient is ready); a caller overlapping the update
 * with the gradient's producer makes the update stream wait on the
 * producer's event per chunk. Arguments are checked as for layer_adam_step
 * (the whole layer's buffers), plus the range. */
LA_API la_status layer_adam_step_range(const la_layer_desc *layer,
                                       const la_adam_params *hp,
                                       int64_t elem_begin, int64_t elem_end,
                                       int32_t *overflow_flag, void *hip_stream);

/* Pre-pass for overflow-gated steps: sets *found_nonfinite (a 4-byte-aligned
 * int32 in device memory) to 1 if some aggregated gradient element of the
 * layer -- the left-to-right sum of its R replicas times grad_unscale, in
 * FP32, exactly as the update forms it -- is +-Inf or NaN. Never clears it.
 * Reads only the gradients, 2R bytes per parameter; it may stop reading
 * once it sees the flag already set. grad_unscale must be finite and > 0.
 * The pages name FP16 gradients among the mixed-precision state ("SlideDP",
 * 前置知识) but give no overflow rule; this pre-pass and the gated step below
 * implement the usual loss-scaling reading: a step whose aggregated gradient
 * holds a non-finite value is skipped as a whole, decided on the device. */
LA_API la_status la_check_gradients(const la_layer_desc *layer,
                                    double grad_unscale,
                                    int32_t *found_nonfinite,
                                    void *hip_stream);

/* layer_adam_step that does nothing -- no state, compute copy or flag is
 * touched -- when the device int32 *skip_if_nonzero (4-byte aligned; may not
 * be NULL) holds a non-zero value when the kernel runs. With
 * la_check_gradients writing that flag for every layer first, a step whose
 * gradients overflowed is skipped without a host synchronisation (the
 * loss-scaling reading of the FP16-gradient state of "SlideDP", 前置知识,
 * described at la_check_gradients). The caller decides from the same flag,
 * once read, whether to count the step in t. */
LA_API la_status layer_adam_step_gated(const la_layer_desc *layer,
                                       const la_adam_params *hp,
                                       const int32_t *skip_if_nonzero,
                                       int32_t *overflow_flag,
                                       void *hip_stream);

/* layer_adam_step with the step count t read from device memory when the
 * kernel runs: *step_on_device (an 8-byte-aligned int64 in device memory;
 * may not be NULL) instead of hp->step, which is ignored. The two constants
 * that depend on t, lr/(1 - beta1^t) and sqrt(1 - beta2^t), are then formed
 * on the GPU in double and rounded to FP32 once, as the host does for the
 * other entry points (the device pow() may differ from the host's in the
 * last double ulp, which can move the master by at most about one FP32
 * ulp). A value below 1 makes the launch a no-op. This is the form to
 * capture in a HIP graph: the caller advances the device counter (e.g. with
 * a captured increment) and every replay applies the next step. */
LA_API la_status layer_adam_step_device_step(const la_layer_desc *layer,
                                             const la_adam_params *hp,
                                             const int64_t *step_on_device,
                                             int32_t *overflow_flag,
                                             void *hip_stream);

/* Options of layer_adam_step_ex. A zero-initialised struct means the whole
 * layer, t from hp->step, no overflow flag and no skip flag. */
typedef struct {
  int32_t use_range;               /* 0: the whole layer; 1: the elements
                                      [elem_begin, elem_end), as for
                                      layer_adam_step_range               */
  int64_t elem_begin;
  int64_t elem_end;
  int32_t *overflow_flag;          /* as for layer_adam_step; NULL: none   */
  const int32_t *skip_if_nonzero;  /* as for layer_adam_step_gated; NULL:
                                      never skipped                        */
  const int64_t *step_on_device;   /* as for layer_adam_step_device_step
                                      (hp->step ignored); NULL: hp->step   */
} la_step_options;

/* layer_adam_step with any combination of the options above in one call:
 * an element range (the per-chunk release of "SlideDP", 核心方法 and
 * 方法步骤详情), the overflow flag, the device skip flag of the gated step
 * (the loss-scaling reading of the FP16-gradient state of "SlideDP",
 * 前置知识, described at la_check_gradients) and the step count read from
 * device memory. Each option means exactly what it means for its own entry
 * point. Together they make a whole overflow-gated step of a layer
 * capturable in a HIP graph: la_check_gradients into a cleared flag, this
 * call with that flag as skip_if_nonzero and a device step count, then the
 * caller's own device-side increment of t when the flag is clear -- every
 * replay then applies the next step, or skips it, with no host
 * synchronisation. A launch whose skip flag is set reads nothing else (not
 * even the step count). opts NULL: all defaults. Arguments are checked as
 * for the entry points whose options are used, plus use_range (0 or 1);
 * nothing is enqueued on failure. */
LA_API la_status layer_adam_step_ex(const la_layer_desc *layer,
                                    const la_adam_params *hp,
                                    const la_step_options *opts,
                                    void *hip_stream);

/* Measurement aid, not part of the update: enqueue a plain copy of `bytes`
 * bytes from src to dst on `hip_stream`, with the update kernel's access
 * style (16-byte non-temporal loads and stores, one workgroup per chunk) but
 * one read and one write stream and no arithmetic -- the bandwidth a simple
 * two-stream pattern reaches on this GPU, to read the update's rate against.
 * bytes: a multiple of 16 (0 is a no-op); dst and src: device-addressable,
 * 16-byte aligned, not overlapping. Status and errors as for
 * layer_adam_step: checked on the host, nothing enqueued on failure. */
LA_API la_status la_copy_reference(void *dst, const void *src, int64_t bytes,
                                   void *hip_stream);

/* Measurement aid, not part of the update: the stream probe. Enqueue, on
 * `hip_stream`, a pass over `layer` that moves exactly the bytes a
 * layer_adam_step of the same layer moves, in exactly its launch shape (the
 * same tensor table, chunks, workgroups and residency), with no arithmetic:
 * it reads the R gradient replicas and master, m, v, writes master, m and v
 * back unchanged, and writes the compute copy (unless LA_OUT_NONE) as the
 * bitwise XOR of the replicas' 16-bit patterns -- so the copy is clobbered
 * until the next update rewrites it. Its rate is what HBM gives this mix of
 * R + 3 read and 4 write streams: the beta of the step-time bound
 * T >= max_j W_j / beta_j ("SlideDP", 研究动机 and 技术新颖性) measured for
 * the update's own access pattern. Like an update, it rewrites the layer's
 * state, so it must not overlap another call on the same buffers. Arguments
 * are checked as for layer_adam_step (no hyperparameters; the gradient dtype
 * does not matter); nothing is enqueued on failure. */
LA_API la_status la_stream_probe(const la_layer_desc *layer, void *hip_stream);

/* Parts of the direction probe. */
typedef enum { LA_PROBE_READS = 0, LA_PROBE_WRITES = 1 } la_probe_part;

/* Measurement aid, not part of the update: the stream probe split by
 * direction, over the layer's elements [elem_begin, elem_end) (numbering as
 * in la_layer_desc). LA_PROBE_READS issues exactly the loads an update of
 * that range issues -- the R gradient replicas, master, m and v, in the
 * update's per-wave pattern (one 64-lane wave per 256-element chunk) -- and
 * writes nothing. LA_PROBE_WRITES issues exactly its stores -- master, m and
 * v (each element the 32-bit pattern `fill`) and the compute copy (the low
 * 16 bits of `fill`; nothing with LA_OUT_NONE) -- and reads nothing, so it
 * overwrites the layer's state in the range. Timed alone, one after the
 * other, at once on two streams, or alternating over slices of the layer,
 * the two parts show the bandwidth HBM gives each direction of the update's
 * traffic and what interleaving the two directions costs: the per-resource
 * beta of the step-time bound T >= max_j W_j / beta_j ("SlideDP", 研究动机
 * and 技术新颖性) taken apart for HBM. workgroups_per_cu: resident one-wave
 * workgroups per compute unit, 1..64, 0 for no cap, -1 for the part's
 * default. Arguments are checked as for la_stream_probe, plus the part, the
 * residency and the range; nothing is enqueued on failure. Must not overlap
 * another call on the same buffers. */
LA_API la_status la_direction_probe(const la_layer_desc *layer, int32_t part,
                                    int64_t elem_begin, int64_t elem_end,
                                    uint32_t fill, int32_t workgroups_per_cu,
                                    void *hip_stream);

/* Bytes of mixed-precision Adam state the layer stands for: 16 per
 * parameter (2 BF16 weight + 2 gradient + 4 FP32 master + 8 FP32 m and v).
 * -1 if the descriptor is invalid. Host only. */
LA_API int64_t la_state_bytes(const la_layer_desc *layer);

/* Bytes one layer_adam_step moves to and from HBM in the ideal case:
 * (2R + 26) per parameter = R gradient reads + master, m, v read and written
 * + the 2-byte compute copy ((2R + 24) with LA_OUT_NONE). This is the W of
 * the one resource the update uses in the step-time bound T >= max_j W_j /
 * beta_j of "SlideDP: Scaling Host-Resident LLM Fine-Tuning Across Multiple
 * GPUs" (stated in 研究动机; 核心方法 builds its analytic step-time model on
 * it; 技术新颖性 gives the per-resource minimum duration W_j / beta_j): with
 * HBM the only resource, a launch takes at least these bytes over the HBM
 * bandwidth. -1 if the descriptor is invalid. Host only. */
LA_API int64_t la_traffic_bytes(const la_layer_desc *layer);

/* Message of the calling thread's last failed call ("" if none). The pointer
 * stays valid until that thread's next call into the library. */
LA_API const char *la_last_error(void);

/* Library version and the GPU target it was built for. */
LA_API const char *la_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LAYERADAM_H */
