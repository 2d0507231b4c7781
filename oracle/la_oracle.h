/*
 * la_oracle.h -- plain CPU reference ("oracle") for the per-layer
 * mixed-precision Adam update (LayerAdam).
 *
 * TEST INFRASTRUCTURE. This library exists to check the HIP path; it is not
 * part of the product. Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark may load it. It shares no source, header,
 * table or helper with the HIP library, and it never calls it.
 *
 * What it computes (one call = one update of one layer):
 *   g   = (dec(G_0) + dec(G_1) + ... + dec(G_{R-1})) * u     left fold, FP32
 *   m   = b1*m + c1*g
 *   v   = b2*v + c2*(g*g)
 *   den = sqrt(v)/q + e
 *   p   = p*d - alpha*(m/den)
 *   w   = round-to-nearest-even BF16 (or FP16) of p, or nothing
 * with b1, c1, b2, c2, alpha, q, e, d, u derived once per call in double and
 * rounded to FP32 (see lao_derive_scalars).
 *
 * Sources. The state this update works on -- FP32 master weights, FP32 Adam
 * first and second moments, BF16/FP16 compute weights and gradients -- is the
 * 16N-byte mixed-precision state of "SlideDP: Scaling Host-Resident LLM
 * Fine-Tuning Across Multiple GPUs", section "前置知识" (preliminaries:
 * the 16N-byte mixed-precision Adam state). The same page, "核心方法"
 * (core method) and "方法步骤详情" (method details), makes the update a
 * per-layer step on the single authoritative FP32 master and (m, v), fed by
 * the data-parallel gradient aggregated on the GPU before the update, with
 * the BF16 copy produced for the next forward pass; the SlideFormer page
 * ("An Efficient Heterogeneous Co-Design for Fine-Tuning on a Single GPU",
 * technical summary 2.2) keeps gradients in a BF16/FP16 buffer and casts
 * FP32 to BF16 for the compute copy. The pages print no update formula:
 * the Adam form is the AdamW of PyTorch (decoupled decay, bias corrections
 * 1 - beta^t, eps added after sqrt(v)/sqrt(1 - beta2^t)), the optimizer that
 * SlideDP's correctness check ("实验结果", loss parity with FSDP2) trains
 * against. Every reading taken where the pages are silent is listed in the
 * repository's design notes.
 *
 * Arithmetic: every operation above is one IEEE binary32 operation with
 * round-to-nearest-even; no fused multiply-add; sqrt and division correctly
 * rounded; subnormals kept. Built with gcc -O2 -ffp-contract=off.
 */
#ifndef LA_ORACLE_H
#define LA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LAO_MAX_REPLICAS 8

/* gradient element formats */
#define LAO_GRAD_BF16 0
#define LAO_GRAD_FP16 1

/* compute-copy formats */
#define LAO_OUT_BF16 0
#define LAO_OUT_FP16 1
#define LAO_OUT_NONE 2

/* One tensor of a layer, as host arrays of numel elements each. */
typedef struct {
  float *master;                          /* FP32, updated in place        */
  float *exp_avg;                         /* m, FP32, updated in place     */
  float *exp_avg_sq;                      /* v, FP32, updated in place     */
  uint16_t *weight_out;                   /* BF16/FP16 bits, written       */
  const uint16_t *grad[LAO_MAX_REPLICAS]; /* R replicas, BF16/FP16 bits    */
  int64_t numel;
} lao_tensor;

/* The FP32 constants of one call. */
typedef struct {
  float b1, c1;  /* beta1, 1 - beta1                       */
  float b2, c2;  /* beta2, 1 - beta2                       */
  float alpha;   /* lr / (1 - beta1^t)                     */
  float q;       /* sqrt(1 - beta2^t)                      */
  float e;       /* eps                                    */
  float d;       /* 1 - lr * weight_decay                  */
  float u;       /* gradient unscale factor                */
} lao_scalars;

/* Derive the per-call constants: each is computed in double from the double
 * hyperparameters and rounded to FP32 once. Returns 0, or -1 when an argument
 * is outside its domain (step < 1, beta outside [0,1), negative lr/eps/decay,
 * unscale not finite and positive). */
int lao_derive_scalars(double lr, double beta1, double beta2, double eps,
                       double weight_decay, int64_t step, double unscale,
                       lao_scalars *out);

/* Value of one gradient element: BF16 is the upper half of a binary32;
 * FP16 is IEEE binary16 (subnormals, Inf, NaN). Exact. */
float lao_decode(uint16_t bits, int dtype);

/* BF16 nearest to x, ties to the even significand; values past the largest
 * finite BF16 by half an ulp or more become +-Inf; every NaN becomes 0x7FC0. */
uint16_t lao_round_bf16(float x);

/* FP16 (IEEE binary16) nearest to x, ties to the even significand, with
 * binary16 subnormals; magnitudes at or past 65520 (half an ulp above the
 * largest finite 65504) become +-Inf; every NaN becomes 0x7E00. */
uint16_t lao_round_fp16(float x);

/* Aggregated gradient of element j: left fold over replicas 0..R-1 in FP32,
 * then one multiply by u. */
float lao_aggregate(const uint16_t *const *grad, int replicas, int dtype,
                    int64_t j, float u);

/* One LayerAdam update of every element of every tensor. out_dtype selects
 * the compute copy written to weight_out (LAO_OUT_NONE: none). If flag is not
 * NULL it is set to 1 when some aggregated gradient is +-Inf or NaN (never
 * cleared; the update is still applied). Returns 0, or -1 on invalid
 * arguments (then nothing is written). */
int lao_step(lao_tensor *tensors, int num_tensors, int replicas, int dtype,
             int out_dtype, double lr, double beta1, double beta2, double eps,
             double weight_decay, int64_t step, double unscale,
             int32_t *flag);

/* 1 if some aggregated gradient element (sum of the replicas times u, as in
 * lao_aggregate) of any tensor is +-Inf or NaN, else 0; -1 on invalid
 * arguments. Reads the gradients only. */
int lao_check_finite(const lao_tensor *tensors, int num_tensors, int replicas,
                     int dtype, double unscale);

/* Element-wise array forms of the helpers above, for tests. */
void lao_decode_array(const uint16_t *in, float *out, int64_t n, int dtype);
void lao_round_bf16_array(const float *in, uint16_t *out, int64_t n);
void lao_round_fp16_array(const float *in, uint16_t *out, int64_t n);
void lao_aggregate_array(const uint16_t *const *grad, int replicas, int dtype,
                         float u, float *out, int64_t n);

#ifdef __cplusplus
}
#endif

#endif /* LA_ORACLE_H */
