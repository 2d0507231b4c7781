/*
 * la_c_abi_check.c -- the C ABI used from plain C, without Python or torch:
 * device buffers from hipMalloc, inputs drawn by the seeded generator
 * (libla_synth.so), the stream probe and the read part of the direction
 * probe, then one layer_adam_step on a side stream, results compared
 * element by element with the CPU oracle (libla_oracle.so). Test program;
 * exit status 0 when every master/m/v element is within 2 FP32 ulp of the
 * oracle (0 expected) and every BF16 element is identical.
 *
 * Build: gcc -std=c11 la_c_abi_check.c -I include -I oracle -D__HIP_PLATFORM_AMD__
 *        -I /opt/rocm/include -L ... -llayeradam -lla_oracle -lla_synth -lamdhip64
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "la_oracle.h"
#include "layeradam.h"

/* from libla_synth.so (synth/la_synth.c) */
void las_fill_normal_f32(uint64_t seed, uint64_t stream, float *out, int64_t n, double mean,
                         double std, int nthreads);
void las_fill_uniform_f32(uint64_t seed, uint64_t stream, float *out, int64_t n, double lo,
                          double hi, int nthreads);
void las_fill_normal_half(uint64_t seed, uint64_t stream, uint16_t *out, int64_t n, double std,
                          double scale, uint64_t outlier_stream, double outlier_prob,
                          double outlier_mult, int half_format, int nthreads);

#define NT 5
#define R 3
#define CHECK(x)                                                           \
  do {                                                                     \
    hipError_t e_ = (x);                                                   \
    if (e_ != hipSuccess) {                                                \
      fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));              \
      return 2;                                                            \
    }                                                                      \
  } while (0)

static int64_t ordered(float x) {
  int32_t b;
  memcpy(&b, &x, 4);
  return b < 0 ? -(int64_t)(b & 0x7FFFFFFF) : b;
}

int main(void) {
  const int64_t numel[NT] = {1, 2049, 4096 + 7, 100003, 70001};
  la_tensor_desc dev[NT];
  lao_tensor host[NT];
  float *hp[NT], *hm[NT], *hv[NT];
  uint16_t *hw[NT], *hg[NT][R];
  memset(dev, 0, sizeof dev);
  memset(host, 0, sizeof host);
  for (int t = 0; t < NT; ++t) {
    int64_t n = numel[t];
    hp[t] = malloc(4 * n);
    hm[t] = malloc(4 * n);
    hv[t] = malloc(4 * n);
    hw[t] = malloc(2 * n);
    las_fill_normal_f32(77, 64 * t + 0, hp[t], n, 0.0, 0.02, 4);
    las_fill_normal_f32(77, 64 * t + 1, hm[t], n, 0.0, 1e-4, 4);
    las_fill_uniform_f32(77, 64 * t + 2, hv[t], n, 0.0, 1e-6, 4);
    CHECK(hipMalloc((void **)&dev[t].master, 4 * n));
    CHECK(hipMalloc((void **)&dev[t].exp_avg, 4 * n));
    CHECK(hipMalloc((void **)&dev[t].exp_avg_sq, 4 * n));
    CHECK(hipMalloc((void **)&dev[t].weight_out, 2 * n));
    CHECK(hipMemcpy(dev[t].master, hp[t], 4 * n, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dev[t].exp_avg, hm[t], 4 * n, hipMemcpyHostToDevice));
    CHECK(hipMemcpy(dev[t].exp_avg_sq, hv[t], 4 * n, hipMemcpyHostToDevice));
    for (int r = 0; r < R; ++r) {
      void *g;
      hg[t][r] = malloc(2 * n);
      las_fill_normal_half(77, 64 * t + 8 + r, hg[t][r], n, 1e-3, 1.0, 64 * t + 24 + r, 0.01,
                           100.0, 0, 4);
      CHECK(hipMalloc(&g, 2 * n));
      CHECK(hipMemcpy(g, hg[t][r], 2 * n, hipMemcpyHostToDevice));
      dev[t].grads[r] = g;
      host[t].grad[r] = hg[t][r];
    }
    dev[t].numel = n;
    host[t].master = hp[t];
    host[t].exp_avg = hm[t];
    host[t].exp_avg_sq = hv[t];
    host[t].weight_out = hw[t];
    host[t].numel = n;
  }
  la_layer_desc layer = {dev, NT, R, LA_GRAD_BF16, LA_OUT_BF16};
  la_adam_params hyper = {1e-5, 0.9, 0.999, 1e-8, 0.01, 42, 1.0};
  int32_t *flag;
  CHECK(hipMalloc((void **)&flag, 4));
  CHECK(hipMemset(flag, 0, 4));
  hipStream_t stream;
  CHECK(hipStreamCreate(&stream));

  printf("%s; state %lld B, traffic %lld B\n", la_version(),
         (long long)la_state_bytes(&layer), (long long)la_traffic_bytes(&layer));
  /* the stream probe moves the update's bytes and leaves the state as it
     was, and the read part of the direction probe only reads: the step after
     them must still match the oracle */
  la_status st = la_stream_probe(&layer, stream);
  if (st != LA_OK) {
    fprintf(stderr, "la_stream_probe: %d %s\n", st, la_last_error());
    return 2;
  }
  int64_t total = 0;
  for (int t = 0; t < NT; ++t) total += numel[t];
  st = la_direction_probe(&layer, LA_PROBE_READS, 0, total, 0u, -1, stream);
  if (st != LA_OK) {
    fprintf(stderr, "la_direction_probe: %d %s\n", st, la_last_error());
    return 2;
  }
  st = layer_adam_step(&layer, &hyper, flag, stream);
  if (st != LA_OK) {
    fprintf(stderr, "layer_adam_step: %d %s\n", st, la_last_error());
    return 2;
  }
  /* the combined entry point from C: an empty range enqueues nothing, an
     unknown use_range is refused */
  la_step_options opt;
  memset(&opt, 0, sizeof opt);
  opt.use_range = 1;
  opt.elem_begin = opt.elem_end = 7;
  opt.overflow_flag = flag;
  st = layer_adam_step_ex(&layer, &hyper, &opt, stream);
  if (st != LA_OK) {
    fprintf(stderr, "layer_adam_step_ex: %d %s\n", st, la_last_error());
    return 2;
  }
  opt.use_range = 2;
  if (layer_adam_step_ex(&layer, &hyper, &opt, stream) != LA_ERR_INVALID_ARGUMENT ||
      strlen(la_last_error()) == 0) {
    fprintf(stderr, "use_range = 2 was not refused\n");
    return 2;
  }
  /* a refused call enqueues nothing and says why */
  la_adam_params bad = hyper;
  bad.step = 0;
  if (layer_adam_step(&layer, &bad, flag, stream) != LA_ERR_INVALID_ARGUMENT ||
      strlen(la_last_error()) == 0) {
    fprintf(stderr, "step = 0 was not refused\n");
    return 2;
  }
  CHECK(hipStreamSynchronize(stream));

  int32_t oflag = 0, gflag = -1;
  if (lao_step(host, NT, R, LAO_GRAD_BF16, LAO_OUT_BF16, hyper.lr, hyper.beta1, hyper.beta2,
               hyper.eps, hyper.weight_decay, hyper.step, hyper.grad_unscale, &oflag) != 0) {
    fprintf(stderr, "oracle refused\n");
    return 2;
  }
  CHECK(hipMemcpy(&gflag, flag, 4, hipMemcpyDeviceToHost));
  int64_t worst = 0, compared = 0, bf16_bad = 0;
  for (int t = 0; t < NT; ++t) {
    int64_t n = numel[t];
    float *gp = malloc(4 * n), *gm = malloc(4 * n), *gv = malloc(4 * n);
    uint16_t *gw = malloc(2 * n);
    CHECK(hipMemcpy(gp, dev[t].master, 4 * n, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(gm, dev[t].exp_avg, 4 * n, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(gv, dev[t].exp_avg_sq, 4 * n, hipMemcpyDeviceToHost));
    CHECK(hipMemcpy(gw, dev[t].weight_out, 2 * n, hipMemcpyDeviceToHost));
    for (int64_t j = 0; j < n; ++j) {
      int64_t d[3] = {llabs(ordered(gp[j]) - ordered(hp[t][j])),
                      llabs(ordered(gm[j]) - ordered(hm[t][j])),
                      llabs(ordered(gv[j]) - ordered(hv[t][j]))};
      for (int k = 0; k < 3; ++k)
        if (d[k] > worst) worst = d[k];
      if (gw[j] != hw[t][j]) ++bf16_bad;
    }
    compared += n;
    free(gp);
    free(gm);
    free(gv);
    free(gw);
  }
  printf("compared %lld elements: max %lld ulp, %lld BF16 mismatches, flag gpu %d oracle %d\n",
         (long long)compared, (long long)worst, (long long)bf16_bad, gflag, oflag);
  return (worst <= 2 && bf16_bad == 0 && gflag == oflag) ? 0 : 1;
}
