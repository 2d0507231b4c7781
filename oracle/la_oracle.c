/*
 * la_oracle.c -- plain, single-threaded CPU reference for the LayerAdam
 * update. TEST INFRASTRUCTURE ONLY (see la_oracle.h for what it computes and
 * which passages of the pages it follows).
 *
 * Written for a reader checking it by eye: one element at a time, one FP32
 * operation per statement, no blocking, no vectorisation tricks. Compiled
 * with -ffp-contract=off so that no multiply-add is fused.
 */
#include "la_oracle.h"

#include <math.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Per-call constants.                                                       */
/* The Adam constants (beta1, beta2, their complements, the bias corrections */
/* 1 - beta^t at the 1-based step t) and the decoupled decay factor          */
/* 1 - lr*wd; derived in double from the caller's double hyperparameters,   */
/* each rounded once to FP32.                                                */
/* ------------------------------------------------------------------------ */
int lao_derive_scalars(double lr, double beta1, double beta2, double eps,
                       double weight_decay, int64_t step, double unscale,
                       lao_scalars *out) {
  if (out == NULL) return -1;
  if (step < 1) return -1;
  if (!(beta1 >= 0.0 && beta1 < 1.0)) return -1;
  if (!(beta2 >= 0.0 && beta2 < 1.0)) return -1;
  if (!(lr >= 0.0) || !isfinite(lr)) return -1;
  if (!(eps >= 0.0) || !isfinite(eps)) return -1;
  if (!(weight_decay >= 0.0) || !isfinite(weight_decay)) return -1;
  if (!(unscale > 0.0) || !isfinite(unscale)) return -1;

  double t = (double)step;
  double bias_correction1 = 1.0 - pow(beta1, t);
  double bias_correction2 = 1.0 - pow(beta2, t);

  out->b1 = (float)beta1;
  out->c1 = (float)(1.0 - beta1);
  out->b2 = (float)beta2;
  out->c2 = (float)(1.0 - beta2);
  out->alpha = (float)(lr / bias_correction1);
  out->q = (float)sqrt(bias_correction2);
  out->e = (float)eps;
  out->d = (float)(1.0 - lr * weight_decay);
  out->u = (float)unscale;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Gradient element formats.                                                 */
/* ------------------------------------------------------------------------ */

/* BF16: the 16 most significant bits of an IEEE binary32. */
static float decode_bf16(uint16_t bits) {
  uint32_t word = (uint32_t)bits << 16;
  float x;
  memcpy(&x, &word, sizeof x);
  return x;
}

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Subnormals are f * 2^-24; normals are (1024 + f) * 2^(e - 25). */
static float decode_fp16(uint16_t bits) {
  int sign = bits >> 15;
  int exponent = (bits >> 10) & 0x1F;
  int fraction = bits & 0x3FF;
  float magnitude;
  if (exponent == 0)
    magnitude = ldexpf((float)fraction, -24);
  else if (exponent == 31)
    magnitude = fraction ? NAN : INFINITY;
  else
    magnitude = ldexpf((float)(1024 + fraction), exponent - 25);
  return sign ? -magnitude : magnitude;
}

float lao_decode(uint16_t bits, int dtype) {
  return dtype == LAO_GRAD_FP16 ? decode_fp16(bits) : decode_bf16(bits);
}

/* ------------------------------------------------------------------------ */
/* FP32 -> BF16, round to nearest, ties to even.                             */
/* Keep the upper 16 bits; the dropped lower 16 bits decide: above half an   */
/* ulp (0x8000) round the magnitude up, below it truncate, exactly half      */
/* round to the even upper part. A carry out of the significand moves to the */
/* next binade, and from the largest finite BF16 to Inf, as it should.       */
/* ------------------------------------------------------------------------ */
uint16_t lao_round_bf16(float x) {
  if (isnan(x)) return 0x7FC0;
  uint32_t word;
  memcpy(&word, &x, sizeof word);
  uint32_t kept = word >> 16;
  uint32_t dropped = word & 0xFFFFu;
  if (dropped > 0x8000u || (dropped == 0x8000u && (kept & 1u))) kept += 1u;
  return (uint16_t)kept;
}

/* ------------------------------------------------------------------------ */
/* FP32 -> FP16 (IEEE binary16), round to nearest, ties to even.             */
/* Written from the format: a normal binary16 is (1024 + f) * 2^(e - 25)     */
/* for biased exponent e in 1..30, a subnormal is f * 2^-24. Scale |x| so    */
/* that the binary16 significand becomes the integer part, round that       */
/* integer to nearest-even in double (exact: x has 24 significant bits),     */
/* and let a carry to 2048 move to the next binade (and from the top binade  */
/* to Inf).                                                                  */
/* ------------------------------------------------------------------------ */
uint16_t lao_round_fp16(float x) {
  if (isnan(x)) return 0x7E00;
  uint16_t sign = signbit(x) ? 0x8000 : 0x0000;
  double a = fabs((double)x);
  if (isinf(x)) return sign | 0x7C00;
  if (a < ldexp(1.0, -14)) {
    /* subnormal range: units of 2^-24; 1024 units is the smallest normal */
    double units = nearbyint(ldexp(a, 24));
    return sign | (uint16_t)units;
  }
  int e2;
  frexp(a, &e2);                 /* a = m * 2^e2 with m in [0.5, 1) */
  int unbiased = e2 - 1;         /* a in [2^unbiased, 2^(unbiased+1)) */
  double significand = nearbyint(ldexp(a, 10 - unbiased)); /* in [1024, 2048] */
  if (significand == 2048.0) {
    significand = 1024.0;
    unbiased += 1;
  }
  int biased = unbiased + 15;
  if (biased >= 31) return sign | 0x7C00;
  return sign | (uint16_t)(biased << 10) | (uint16_t)(significand - 1024.0);
}

/* ------------------------------------------------------------------------ */
/* Aggregated gradient of one element: the sum of the R data-parallel        */
/* replicas (SlideDP: one aggregated gradient per layer per iteration,       */
/* reduced on the GPU before the update), left to right, then the unscale    */
/* factor.                                                                   */
/* ------------------------------------------------------------------------ */
float lao_aggregate(const uint16_t *const *grad, int replicas, int dtype,
                    int64_t j, float u) {
  float g = lao_decode(grad[0][j], dtype);
  for (int r = 1; r < replicas; ++r) {
    float next = lao_decode(grad[r][j], dtype);
    g = g + next;
  }
  g = g * u;
  return g;
}

/* ------------------------------------------------------------------------ */
/* One update of one element.                                                */
/* ------------------------------------------------------------------------ */
static void update_element(const lao_scalars *s, float g, float *master,
                           float *exp_avg, float *exp_avg_sq,
                           uint16_t *weight_out, int out_dtype) {
  float m = *exp_avg;
  float v = *exp_avg_sq;
  float p = *master;

  /* first moment: m = beta1*m + (1-beta1)*g */
  float m_old_part = s->b1 * m;
  float m_new_part = s->c1 * g;
  m = m_old_part + m_new_part;

  /* second moment: v = beta2*v + (1-beta2)*g^2 */
  float g_squared = g * g;
  float v_old_part = s->b2 * v;
  float v_new_part = s->c2 * g_squared;
  v = v_old_part + v_new_part;

  /* bias-corrected denominator: sqrt(v)/sqrt(1-beta2^t) + eps */
  float root = sqrtf(v);
  float root_corrected = root / s->q;
  float denominator = root_corrected + s->e;

  /* decoupled weight decay, then the step lr/(1-beta1^t) * m/denominator */
  float ratio = m / denominator;
  float decayed = p * s->d;
  float step = s->alpha * ratio;
  p = decayed - step;

  *exp_avg = m;
  *exp_avg_sq = v;
  *master = p;
  if (out_dtype == LAO_OUT_BF16) *weight_out = lao_round_bf16(p);
  if (out_dtype == LAO_OUT_FP16) *weight_out = lao_round_fp16(p);
}

int lao_step(lao_tensor *tensors, int num_tensors, int replicas, int dtype,
             int out_dtype, double lr, double beta1, double beta2, double eps,
             double weight_decay, int64_t step, double unscale,
             int32_t *flag) {
  lao_scalars s;
  if (tensors == NULL && num_tensors != 0) return -1;
  if (num_tensors < 0) return -1;
  if (replicas < 1 || replicas > LAO_MAX_REPLICAS) return -1;
  if (dtype != LAO_GRAD_BF16 && dtype != LAO_GRAD_FP16) return -1;
  if (out_dtype != LAO_OUT_BF16 && out_dtype != LAO_OUT_FP16 && out_dtype != LAO_OUT_NONE)
    return -1;
  if (lao_derive_scalars(lr, beta1, beta2, eps, weight_decay, step, unscale,
                         &s) != 0)
    return -1;
  for (int t = 0; t < num_tensors; ++t) {
    if (tensors[t].numel < 0) return -1;
    if (tensors[t].numel == 0) continue;
    if (!tensors[t].master || !tensors[t].exp_avg || !tensors[t].exp_avg_sq)
      return -1;
    if (out_dtype != LAO_OUT_NONE && !tensors[t].weight_out) return -1;
    for (int r = 0; r < replicas; ++r)
      if (!tensors[t].grad[r]) return -1;
  }

  for (int t = 0; t < num_tensors; ++t) {
    lao_tensor *x = &tensors[t];
    for (int64_t j = 0; j < x->numel; ++j) {
      float g = lao_aggregate(x->grad, replicas, dtype, j, s.u);
      if (flag != NULL && !isfinite(g)) *flag = 1;
      update_element(&s, g, &x->master[j], &x->exp_avg[j], &x->exp_avg_sq[j],
                     out_dtype == LAO_OUT_NONE ? NULL : &x->weight_out[j],
                     out_dtype);
    }
  }
  return 0;
}

int lao_check_finite(const lao_tensor *tensors, int num_tensors, int replicas,
                     int dtype, double unscale) {
  if (tensors == NULL && num_tensors != 0) return -1;
  if (num_tensors < 0 || replicas < 1 || replicas > LAO_MAX_REPLICAS) return -1;
  if (dtype != LAO_GRAD_BF16 && dtype != LAO_GRAD_FP16) return -1;
  if (!(unscale > 0.0) || !isfinite(unscale)) return -1;
  float u = (float)unscale;
  int found = 0;
  for (int t = 0; t < num_tensors; ++t) {
    if (tensors[t].numel < 0) return -1;
    for (int r = 0; r < replicas && tensors[t].numel > 0; ++r)
      if (!tensors[t].grad[r]) return -1;
    for (int64_t j = 0; j < tensors[t].numel; ++j) {
      float g = lao_aggregate(tensors[t].grad, replicas, dtype, j, u);
      if (!isfinite(g)) found = 1;
    }
  }
  return found;
}

/* ------------------------------------------------------------------------ */
/* Array forms, for the tests.                                               */
/* ------------------------------------------------------------------------ */
void lao_decode_array(const uint16_t *in, float *out, int64_t n, int dtype) {
  for (int64_t i = 0; i < n; ++i) out[i] = lao_decode(in[i], dtype);
}

void lao_round_bf16_array(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = lao_round_bf16(in[i]);
}

void lao_round_fp16_array(const float *in, uint16_t *out, int64_t n) {
  for (int64_t i = 0; i < n; ++i) out[i] = lao_round_fp16(in[i]);
}

void lao_aggregate_array(const uint16_t *const *grad, int replicas, int dtype,
                         float u, float *out, int64_t n) {
  for (int64_t j = 0; j < n; ++j)
    out[j] = lao_aggregate(grad, replicas, dtype, j, u);
}
