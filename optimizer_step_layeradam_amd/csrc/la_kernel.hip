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
// kChunk elements (the last chunk of a tensor may be partial); one launch
// covers all tensors of the layer. There is one workgroup per chunk: the
// dispatcher then keeps the workgroups in flight on a narrow, advancing
// window of every stream, which measured faster on MI355X than a
// persistent grid whose workgroups drift apart (the loop below still
// strides by the grid when the grid is capped). The launch also reserves
// LDS that the kernel never touches, so that a compute unit holds only two
// workgroups (four waves, one per SIMD) at a time: fewer requests in flight
// interleave the 2R + 8 streams less at the HBM, and that measured fastest.
// A chunk is U tiles of 128 threads x 4 elements: each thread owns 4
// consecutive elements per tile and a wave's U tiles are adjacent, so a wave
// reads U KiB runs of each FP32 stream (16 B per lane) and U/2 KiB runs of
// each 16-bit gradient stream (8 B per lane). A thread issues every load of
// its U tiles before any arithmetic, (12 + 2R) * 4 * U bytes per lane in
// flight. Every access carries the non-temporal hint: nothing is reused.
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

// Tile shape and cache hints. The defaults are the measured best on MI355X
// for the Qwen3-14B-shaped layer at R = 8; the macros exist so that other
// shapes can be built and compared.
#ifndef LA_BLOCK
#define LA_BLOCK 128
#endif
#ifndef LA_TILE_VEC
#define LA_TILE_VEC 4
#endif
#ifndef LA_TILE_UNROLL
#define LA_TILE_UNROLL 4
#endif
#ifndef LA_NT_LOADS
#define LA_NT_LOADS 1
#endif
#ifndef LA_NT_STORES
#define LA_NT_STORES 1
#endif
#ifndef LA_WAVE_CONTIG
#define LA_WAVE_CONTIG 1   // 1: each wave's tiles are adjacent in memory
#endif
#ifndef LA_STREAM_MAJOR
#define LA_STREAM_MAJOR 0  // 1: issue all tiles of one stream before the next stream
#endif
#ifndef LA_STORE_MAJOR
#define LA_STORE_MAJOR 0   // 1: compute every tile, then store stream by stream
#endif
#ifndef LA_WORKGROUPS_PER_CU
#define LA_WORKGROUPS_PER_CU 2  // resident workgroups per compute unit (0: no cap)
#endif

constexpr int kBlock = LA_BLOCK;        // threads per workgroup
constexpr int kVec = LA_TILE_VEC;       // consecutive elements per thread per tile (4 or 8)
constexpr int kUnroll = LA_TILE_UNROLL; // tiles per chunk
constexpr int kChunk = kBlock * kVec * kUnroll;
constexpr int kQuads = kVec / 4;        // 16-byte FP32 vectors per array per tile
static_assert(kVec == 4 || kVec == 8, "4 or 8 elements per thread per tile");
static_assert(kBlock % 64 == 0 && kBlock <= 1024, "whole waves");

// Native vector types (the non-temporal builtins need them).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t grad_words __attribute__((ext_vector_type(kVec / 2)));  // kVec 16-bit values

template <typename T>
__device__ __forceinline__ T load_stream(const T* p) {
  if constexpr (LA_NT_LOADS) return __builtin_nontemporal_load(p);
  else return *p;
}

template <typename T>
__device__ __forceinline__ void store_stream(T v, T* p) {
  if constexpr (LA_NT_STORES) __builtin_nontemporal_store(v, p);
  else *p = v;
}

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

// Element offset, within its chunk, of thread tid's first element in tile u.
// Tile-major: tile u covers [u * kBlock * kVec, (u + 1) * kBlock * kVec).
// Wave-contiguous: wave w owns kUnroll adjacent runs of 64 * kVec elements.
__device__ __forceinline__ uint32_t tile_offset(int u, int tid) {
  if constexpr (LA_WAVE_CONTIG) {
    return static_cast<uint32_t>((((tid >> 6) * kUnroll + u) * 64 + (tid & 63)) * kVec);
  } else {
    return static_cast<uint32_t>((u * kBlock + tid) * kVec);
  }
}

// Store one tile's results: master, m, v as 16-byte vectors, BF16 packed.
__device__ __forceinline__ void store_tile(const Elem* e, float* p, float* m, float* v,
                                           uint16_t* w, uint32_t off) {
#pragma unroll
  for (int q = 0; q < kQuads; ++q) {
    const Elem* x = e + 4 * q;
    store_stream(f32x4{x[0].p, x[1].p, x[2].p, x[3].p}, reinterpret_cast<f32x4*>(p + off) + q);
    store_stream(f32x4{x[0].m, x[1].m, x[2].m, x[3].m}, reinterpret_cast<f32x4*>(m + off) + q);
    store_stream(f32x4{x[0].v, x[1].v, x[2].v, x[3].v}, reinterpret_cast<f32x4*>(v + off) + q);
  }
  grad_words wb;
#pragma unroll
  for (int k = 0; k < kVec; k += 2) wb[k / 2] = bf16_bits(e[k].p) | (bf16_bits(e[k + 1].p) << 16);
  store_stream(wb, reinterpret_cast<grad_words*>(w + off));
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
      f32x4 P[kUnroll][kQuads], M[kUnroll][kQuads], V[kUnroll][kQuads];
      grad_words G[kUnroll][R];
      if constexpr (LA_STREAM_MAJOR) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int u = 0; u < kUnroll; ++u)
            G[u][r] = load_stream(reinterpret_cast<const grad_words*>(g[r] + tile_offset(u, tid)));
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int q = 0; q < kQuads; ++q)
            P[u][q] = load_stream(reinterpret_cast<const f32x4*>(p + tile_offset(u, tid)) + q);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int q = 0; q < kQuads; ++q)
            M[u][q] = load_stream(reinterpret_cast<const f32x4*>(m + tile_offset(u, tid)) + q);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int q = 0; q < kQuads; ++q)
            V[u][q] = load_stream(reinterpret_cast<const f32x4*>(v + tile_offset(u, tid)) + q);
      } else {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          const uint32_t off = tile_offset(u, tid);
#pragma unroll
          for (int q = 0; q < kQuads; ++q) {
            P[u][q] = load_stream(reinterpret_cast<const f32x4*>(p + off) + q);
            M[u][q] = load_stream(reinterpret_cast<const f32x4*>(m + off) + q);
            V[u][q] = load_stream(reinterpret_cast<const f32x4*>(v + off) + q);
          }
#pragma unroll
          for (int r = 0; r < R; ++r)
            G[u][r] = load_stream(reinterpret_cast<const grad_words*>(g[r] + off));
        }
      }
      Elem e[kUnroll][kVec];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          // left fold over the replicas, in replica order
          float gk = (k & 1) ? decode_hi<FP16>(G[u][0][k / 2]) : decode_lo<FP16>(G[u][0][k / 2]);
#pragma unroll
          for (int r = 1; r < R; ++r)
            gk = gk + ((k & 1) ? decode_hi<FP16>(G[u][r][k / 2]) : decode_lo<FP16>(G[u][r][k / 2]));
          gk = gk * s.u;
          if (FLAG) bad |= !__builtin_isfinite(gk);
          e[u][k] = adam_update(gk, P[u][k / 4][k % 4], M[u][k / 4][k % 4], V[u][k / 4][k % 4], s);
        }
        if constexpr (!LA_STORE_MAJOR) store_tile(e[u], p, m, v, w, tile_offset(u, tid));
      }
      if constexpr (LA_STORE_MAJOR) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int q = 0; q < kQuads; ++q) {
            const Elem* x = e[u] + 4 * q;
            store_stream(f32x4{x[0].p, x[1].p, x[2].p, x[3].p},
                         reinterpret_cast<f32x4*>(p + tile_offset(u, tid)) + q);
          }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int q = 0; q < kQuads; ++q) {
            const Elem* x = e[u] + 4 * q;
            store_stream(f32x4{x[0].m, x[1].m, x[2].m, x[3].m},
                         reinterpret_cast<f32x4*>(m + tile_offset(u, tid)) + q);
          }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
          for (int q = 0; q < kQuads; ++q) {
            const Elem* x = e[u] + 4 * q;
            store_stream(f32x4{x[0].v, x[1].v, x[2].v, x[3].v},
                         reinterpret_cast<f32x4*>(v + tile_offset(u, tid)) + q);
          }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
          grad_words wb;
#pragma unroll
          for (int k = 0; k < kVec; k += 2)
            wb[k / 2] = bf16_bits(e[u][k].p) | (bf16_bits(e[u][k + 1].p) << 16);
          store_stream(wb, reinterpret_cast<grad_words*>(w + tile_offset(u, tid)));
        }
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
  const int64_t grid = chunks < shape.grid_cap ? chunks : shape.grid_cap;  // >= 1
  void* args[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&layer_adam_kernel<R, FP16, FLAG>),
                         dim3(static_cast<unsigned>(grid)), dim3(kBlock), args, static_cast<unsigned>(shape.lds_bytes), stream);
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

int target_workgroups_per_cu() { return LA_WORKGROUPS_PER_CU; }

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
