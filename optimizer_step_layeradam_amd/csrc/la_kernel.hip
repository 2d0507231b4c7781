// la_kernel.hip -- the fused LayerAdam kernel for gfx950.
//
// One pass over HBM per layer: for every parameter it reads R gradient
// replicas (2 bytes each) and the FP32 master, m and v (12 bytes), and
// writes master, m, v (12 bytes) and the BF16 copy (2 bytes) -- (2R + 26)
// bytes, the whole of the step's traffic. The arithmetic is the per-layer
// mixed-precision Adam update that "SlideDP: Scaling Host-Resident LLM
// Fine-Tuning Across Multiple GPUs" runs as its LayerAdam channel (sections
// 核心方法 and 方法步骤详情) fused with the GPU-side reduction of the data-
// parallel gradient that precedes it there; the BF16 cast is the FP32->BF16
// conversion the SlideFormer page (technical summary 2.2) does on the host.
//
// Work decomposition. Every tensor of a launch is cut into chunks of
// kChunk elements (the last chunk of a tensor may be partial). Workgroups
// walk the global chunk list with a grid stride, so one launch covers all
// tensors of the layer and the grid can be sized to the chip, not to the
// layer. A chunk is U tiles of 256 threads x 4 elements: each thread owns
// 4 consecutive elements per tile, so one wave's loads are contiguous
// 1 KiB (FP32, 16 B per lane) and 512 B (16-bit gradients, 8 B per lane)
// runs. A thread issues every load of its U tiles before any arithmetic,
// which keeps (12 + 2R) * 4 * U bytes per lane in flight.
//
// Arithmetic is IEEE binary32 with one rounding per operation: contraction
// into fused multiply-adds is switched off for this file, and division and
// sqrt are the correctly rounded forms (the HIP defaults).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_internal.h"

#pragma clang fp contract(off)

namespace la {
namespace {

constexpr int kBlock = 256;          // threads per workgroup (4 waves)
constexpr int kVec = 4;              // consecutive elements per thread per tile
constexpr int kUnroll = 2;           // tiles per chunk
constexpr int kChunk = kBlock * kVec * kUnroll;

template <int R>
struct KernelTensor {
  float* p;
  float* m;
  float* v;
  uint16_t* w;
  const uint16_t* g[R];
  int64_t numel;
};

template <int R>
struct KernelArgs {
  KernelTensor<R> t[kTensorsPerLaunch];
  int64_t chunk_end[kTensorsPerLaunch];  // cumulative chunk counts
  Scalars s;
  int32_t* flag;
  int32_t count;
};

// ---- gradient decode ------------------------------------------------------
// BF16 is the upper half of a binary32; FP16 widens exactly in hardware.
template <bool FP16>
__device__ __forceinline__ float decode_lo(uint32_t pair) {
  if constexpr (FP16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(pair)));
  } else {
    return __uint_as_float(pair << 16);
  }
}

template <bool FP16>
__device__ __forceinline__ float decode_hi(uint32_t pair) {
  if constexpr (FP16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(pair >> 16)));
  } else {
    return __uint_as_float(pair & 0xFFFF0000u);
  }
}

template <bool FP16>
__device__ __forceinline__ float decode_one(uint16_t bits) {
  if constexpr (FP16) {
    return static_cast<float>(__builtin_bit_cast(_Float16, bits));
  } else {
    return __uint_as_float(static_cast<uint32_t>(bits) << 16);
  }
}

// ---- FP32 -> BF16, round to nearest even ------------------------------------
// Adding 0x7FFF plus the lowest kept bit carries into the kept half exactly
// when the dropped half is above 0x8000, or equal to it with an odd kept half.
// NaN is tested first and becomes the canonical quiet NaN 0x7FC0.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t rounded = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  return __builtin_isnan(x) ? 0x7FC0u : rounded;
}

// ---- one element of the update ----------------------------------------------
struct Elem {
  float p, m, v;
};

__device__ __forceinline__ Elem adam_update(float g, float p, float m, float v,
                                            const Scalars& s) {
  const float m_new = s.b1 * m + s.c1 * g;
  const float v_new = s.b2 * v + s.c2 * (g * g);
  const float den = __builtin_sqrtf(v_new) / s.q + s.e;
  const float p_new = p * s.d - s.alpha * (m_new / den);
  return {p_new, m_new, v_new};
}

// ---- the kernel ---------------------------------------------------------------
template <int R, bool FP16, bool FLAG>
__global__ void __launch_bounds__(kBlock)
layer_adam_kernel(const KernelArgs<R> a) {
  const int tid = threadIdx.x;
  const int64_t total_chunks = a.chunk_end[a.count - 1];
  const Scalars s = a.s;
  bool bad = false;

  int t = 0;
  int64_t first_chunk_of_t = 0;
  for (int64_t c = blockIdx.x; c < total_chunks; c += gridDim.x) {
    while (c >= a.chunk_end[t]) {  // uniform: chunks only move forward
      first_chunk_of_t = a.chunk_end[t];
      ++t;
    }
    const KernelTensor<R>& T = a.t[t];
    const int64_t base = (c - first_chunk_of_t) * kChunk;
    const int64_t n = T.numel;

    float* __restrict__ p = T.p + base;
    float* __restrict__ m = T.m + base;
    float* __restrict__ v = T.v + base;
    uint16_t* __restrict__ w = T.w + base;
    const uint16_t* g[R];
#pragma unroll
    for (int r = 0; r < R; ++r) g[r] = T.g[r] + base;

    if (base + kChunk <= n) {
      // Full chunk: vector loads of every tile first, then the arithmetic.
      float4 P[kUnroll], M[kUnroll], V[kUnroll];
      uint2 G[kUnroll][R];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t off = static_cast<uint32_t>((u * kBlock + tid) * kVec);
        P[u] = *reinterpret_cast<const float4*>(p + off);
        M[u] = *reinterpret_cast<const float4*>(m + off);
        V[u] = *reinterpret_cast<const float4*>(v + off);
#pragma unroll
        for (int r = 0; r < R; ++r)
          G[u][r] = *reinterpret_cast<const uint2*>(g[r] + off);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t off = static_cast<uint32_t>((u * kBlock + tid) * kVec);
        float gs[kVec];
        gs[0] = decode_lo<FP16>(G[u][0].x);
        gs[1] = decode_hi<FP16>(G[u][0].x);
        gs[2] = decode_lo<FP16>(G[u][0].y);
        gs[3] = decode_hi<FP16>(G[u][0].y);
#pragma unroll
        for (int r = 1; r < R; ++r) {
          gs[0] = gs[0] + decode_lo<FP16>(G[u][r].x);
          gs[1] = gs[1] + decode_hi<FP16>(G[u][r].x);
          gs[2] = gs[2] + decode_lo<FP16>(G[u][r].y);
          gs[3] = gs[3] + decode_hi<FP16>(G[u][r].y);
        }
        const float pv[kVec] = {P[u].x, P[u].y, P[u].z, P[u].w};
        const float mv[kVec] = {M[u].x, M[u].y, M[u].z, M[u].w};
        const float vv[kVec] = {V[u].x, V[u].y, V[u].z, V[u].w};
        Elem e[kVec];
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          const float gk = gs[k] * s.u;
          if (FLAG) bad |= !__builtin_isfinite(gk);
          e[k] = adam_update(gk, pv[k], mv[k], vv[k], s);
        }
        *reinterpret_cast<float4*>(p + off) = make_float4(e[0].p, e[1].p, e[2].p, e[3].p);
        *reinterpret_cast<float4*>(m + off) = make_float4(e[0].m, e[1].m, e[2].m, e[3].m);
        *reinterpret_cast<float4*>(v + off) = make_float4(e[0].v, e[1].v, e[2].v, e[3].v);
        uint2 wb;
        wb.x = bf16_bits(e[0].p) | (bf16_bits(e[1].p) << 16);
        wb.y = bf16_bits(e[2].p) | (bf16_bits(e[3].p) << 16);
        *reinterpret_cast<uint2*>(w + off) = wb;
      }
    } else {
      // Last, partial chunk of a tensor: element by element, bounds-checked.
      const int64_t left = n - base;  // 1 .. kChunk - 1
#pragma unroll 1
      for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          const int64_t i = static_cast<int64_t>((u * kBlock + tid) * kVec + k);
          if (i < left) {
            float gk = decode_one<FP16>(g[0][i]);
#pragma unroll
            for (int r = 1; r < R; ++r) gk = gk + decode_one<FP16>(g[r][i]);
            gk = gk * s.u;
            if (FLAG) bad |= !__builtin_isfinite(gk);
            const Elem e = adam_update(gk, p[i], m[i], v[i], s);
            p[i] = e.p;
            m[i] = e.m;
            v[i] = e.v;
            w[i] = static_cast<uint16_t>(bf16_bits(e.p));
          }
        }
      }
    }
  }

  if (FLAG) {
    // Every lane reaches this point (the chunk loop is uniform per block).
    if (__any(bad) && __lane_id() == 0) atomicOr(a.flag, 1);
  }
}

template <int R, bool FP16, bool FLAG>
hipError_t launch_typed(const TensorArgs* ts, int count, const Scalars& s,
                        int32_t* flag, hipStream_t stream, const LaunchShape& shape) {
  KernelArgs<R> a = {};
  int64_t chunks = 0;
  for (int i = 0; i < count; ++i) {
    a.t[i].p = ts[i].p;
    a.t[i].m = ts[i].m;
    a.t[i].v = ts[i].v;
    a.t[i].w = ts[i].w;
    for (int r = 0; r < R; ++r) a.t[i].g[r] = ts[i].g[r];
    a.t[i].numel = ts[i].numel;
    chunks += (ts[i].numel + kChunk - 1) / kChunk;
    a.chunk_end[i] = chunks;
  }
  a.s = s;
  a.flag = flag;
  a.count = count;
  const int64_t grid = chunks < shape.grid_cap ? chunks : shape.grid_cap;
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&layer_adam_kernel<R, FP16, FLAG>),
                         dim3(static_cast<unsigned>(grid)), dim3(kBlock), args, 0, stream);
}

template <int R>
hipError_t launch_r(const TensorArgs* ts, int count, bool fp16, const Scalars& s,
                    int32_t* flag, hipStream_t stream, const LaunchShape& shape) {
  if (fp16) {
    return flag ? launch_typed<R, true, true>(ts, count, s, flag, stream, shape)
                : launch_typed<R, true, false>(ts, count, s, flag, stream, shape);
  }
  return flag ? launch_typed<R, false, true>(ts, count, s, flag, stream, shape)
              : launch_typed<R, false, false>(ts, count, s, flag, stream, shape);
}

}  // namespace

int64_t chunk_elements() { return kChunk; }

hipError_t launch_layer_adam(const TensorArgs* tensors, int count, int replicas,
                             bool fp16, const Scalars& s, int32_t* flag,
                             hipStream_t stream, const LaunchShape& shape) {
  switch (replicas) {
    case 1: return launch_r<1>(tensors, count, fp16, s, flag, stream, shape);
    case 2: return launch_r<2>(tensors, count, fp16, s, flag, stream, shape);
    case 3: return launch_r<3>(tensors, count, fp16, s, flag, stream, shape);
    case 4: return launch_r<4>(tensors, count, fp16, s, flag, stream, shape);
    case 5: return launch_r<5>(tensors, count, fp16, s, flag, stream, shape);
    case 6: return launch_r<6>(tensors, count, fp16, s, flag, stream, shape);
    case 7: return launch_r<7>(tensors, count, fp16, s, flag, stream, shape);
    case 8: return launch_r<8>(tensors, count, fp16, s, flag, stream, shape);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
