// la_kernel.hip -- the fused LayerAdam kernels for gfx950.
//
// layer_adam_kernel: one pass over HBM per layer. For every parameter it
// reads R gradient replicas (2 bytes each) and the FP32 master, m and v
// (12 bytes), and writes master, m, v (12 bytes) and the 2-byte compute copy
// -- (2R + 26) bytes, the whole of the step's traffic. The arithmetic is the
// per-layer mixed-precision Adam update that "SlideDP: Scaling Host-Resident
// LLM Fine-Tuning Across Multiple GPUs" runs as its LayerAdam channel
// (sections 核心方法 and 方法步骤详情), fused with the GPU-side reduction of
// the data-parallel gradient that precedes it there; the BF16 cast is the
// FP32->BF16 conversion the SlideFormer page (technical summary 2.2) does on
// the host, the FP16 cast the on-the-fly FP32->FP16 conversion of the
// AutoHete page (section 2.2).
//
// check_kernel: the finite-check pre-pass of overflow-gated steps; reads the
// R gradients only (2R bytes per parameter).
//
// Work decomposition. Every tensor of a launch is cut into chunks of
// kChunk elements (the last chunk of a tensor may be partial); one launch
// covers all tensors of the layer. There is one workgroup per chunk: the
// dispatcher then keeps the workgroups in flight on a narrow, advancing
// window of every stream, which measured faster on MI355X than a
// persistent grid whose workgroups drift apart (the loop below still
// strides by the grid when the grid is capped). A workgroup is one wave of
// 64 lanes and a chunk one tile of 64 x 4 elements: each lane owns 4
// consecutive elements, so a wave reads a 1 KiB run of each FP32 stream
// (16 B per lane) and a 512 B run of each 16-bit gradient stream (8 B per
// lane), issues all R + 3 loads, computes, and issues its 4 stores. The
// launch also reserves LDS that the kernel never touches, so that a compute
// unit holds only a few of these waves at a time -- 11 at R = 1 down to 8 at
// R = 7, 8 (kResidency): about 40-55 KB of reads in flight per compute unit.
// More requests in flight interleave the R + 7 streams (R gradient reads;
// master, m, v read and written; the compute copy) worse at the HBM, fewer
// leave it idle; the table is the measured best per R on the 14B-shaped
// layer. Loads carry the non-temporal hint (nothing is reused); stores are
// written through the L2 to memory (buffer stores with the sc0, sc1 and nt
// policy bits), which measured 1-8 % faster than non-temporal write-back
// stores, the most where writes are the largest share of the traffic. Both
// are buffer instructions on a resource built per chunk from the uniform
// chunk base, so the per-lane offset is a 32-bit register.
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

// Tile shape, residency and cache policy. The defaults are the measured best
// on MI355X for the Qwen3-14B-shaped layer at R = 1..8 (and the other
// layers); the macros exist so that other shapes can be built and compared.
#ifndef LA_BLOCK
#define LA_BLOCK 64
#endif
#ifndef LA_TILE_VEC
#define LA_TILE_VEC 4
#endif
#ifndef LA_TILE_UNROLL
#define LA_TILE_UNROLL 1
#endif
#ifndef LA_NT_LOADS
#define LA_NT_LOADS 1
#endif
#ifndef LA_NT_STORES
#define LA_NT_STORES 1   // global stores only (LA_BUFFER_STORES 0)
#endif
// Update and probe: 1 issues their loads (stores) as buffer instructions
// with the cache-policy bits LA_LOAD_CPOL (LA_STORE_CPOL) -- 1 = sc0,
// 2 = nt, 16 = sc1 -- instead of global instructions with the non-temporal
// hint. Loads default to nt, stores to sc0 | sc1 | nt: written through to
// memory.
#ifndef LA_BUFFER_LOADS
#define LA_BUFFER_LOADS 1
#endif
#ifndef LA_BUFFER_STORES
#define LA_BUFFER_STORES 1
#endif
#ifndef LA_LOAD_CPOL
#define LA_LOAD_CPOL 2
#endif
#ifndef LA_STORE_CPOL
#define LA_STORE_CPOL 19
#endif
#ifndef LA_WAVE_CONTIG
#define LA_WAVE_CONTIG 1   // 1: each wave's tiles are adjacent in memory
#endif
// Update: resident workgroups per compute unit for every R (0: no cap);
// -1: the per-R table kResidency.
#ifndef LA_WORKGROUPS_PER_CU
#define LA_WORKGROUPS_PER_CU -1
#endif
// The finite check only reads: more requests in flight help it (measured
// 6.8-7.1 TB/s with 128-thread workgroups, 8 tiles per chunk and no
// residency cap, against 5.5 TB/s with a residency cap of one wave per SIMD).
#ifndef LA_CHECK_BLOCK
#define LA_CHECK_BLOCK 128      // finite check: threads per workgroup
#endif
#ifndef LA_CHECK_TILE_UNROLL
#define LA_CHECK_TILE_UNROLL 8  // finite check: tiles per chunk
#endif
#ifndef LA_CHECK_WORKGROUPS_PER_CU
#define LA_CHECK_WORKGROUPS_PER_CU 0  // finite check: resident workgroups per compute unit
#endif

constexpr int kBlock = LA_BLOCK;        // threads per workgroup
constexpr int kVec = LA_TILE_VEC;       // consecutive elements per thread per tile (4 or 8)
constexpr int kUnroll = LA_TILE_UNROLL; // tiles per chunk
constexpr int kChunk = kBlock * kVec * kUnroll;
constexpr int kQuads = kVec / 4;        // 16-byte FP32 vectors per array per tile
constexpr int kCheckBlock = LA_CHECK_BLOCK;
constexpr int kCheckUnroll = LA_CHECK_TILE_UNROLL;
constexpr int kCheckChunk = kCheckBlock * kVec * kCheckUnroll;
static_assert(kVec == 4 || kVec == 8, "4 or 8 elements per thread per tile");
static_assert(kBlock % 64 == 0 && kBlock <= 1024, "whole waves");
static_assert(kCheckBlock % 64 == 0 && kCheckBlock <= 1024, "whole waves");
static_assert(kChunk > kMaxUnalignedEntry && kCheckChunk > kMaxUnalignedEntry,
              "short unaligned entries must take the element-wise path");

// Update residency per replica count (index R), the measured best of 6..12
// per compute unit for one-tile chunks on the 14B-shaped layer.
constexpr int kResidency[kMaxReplicas + 1] = {0, 11, 10, 10, 9, 9, 9, 8, 8};

template <int R>
constexpr int update_workgroups_per_cu() {
  return LA_WORKGROUPS_PER_CU >= 0 ? LA_WORKGROUPS_PER_CU : kResidency[R];
}

// Native vector types (the non-temporal builtins need them).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t half_words __attribute__((ext_vector_type(kVec / 2)));  // kVec 16-bit values

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

// Buffer resource over a uniform base pointer: no stride, a range far past
// the one chunk the offsets address, and the fourth descriptor word of a raw
// 32-bit-format buffer on this architecture (data format field = 32 bits).
constexpr int kRsrcRange = 0x7fffffff;
constexpr int kRsrcWord3 = 0x00020000;

// T (16 or 8 bytes) at element `elem` of a uniform base pointer.
template <typename T, typename E>
__device__ __forceinline__ T load_at(const E* base, uint32_t elem) {
  static_assert(sizeof(T) == 16 || sizeof(T) == 8, "16- or 8-byte accesses");
  if constexpr (LA_BUFFER_LOADS) {
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<E*>(base), 0, kRsrcRange, kRsrcWord3);
    const uint32_t byte = elem * static_cast<uint32_t>(sizeof(E));
    if constexpr (sizeof(T) == 16)
      return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b128(r, byte, 0, LA_LOAD_CPOL));
    else
      return __builtin_bit_cast(T, __builtin_amdgcn_raw_buffer_load_b64(r, byte, 0, LA_LOAD_CPOL));
  } else {
    return load_stream(reinterpret_cast<const T*>(base + elem));
  }
}

template <typename T, typename E>
__device__ __forceinline__ void store_at(T x, E* base, uint32_t elem) {
  static_assert(sizeof(T) == 16 || sizeof(T) == 8, "16- or 8-byte accesses");
  if constexpr (LA_BUFFER_STORES) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(base, 0, kRsrcRange, kRsrcWord3);
    const uint32_t byte = elem * static_cast<uint32_t>(sizeof(E));
    if constexpr (sizeof(T) == 16)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, byte, 0,
                                             LA_STORE_CPOL);
    else
      __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, x), r, byte, 0,
                                            LA_STORE_CPOL);
  } else {
    store_stream(x, reinterpret_cast<T*>(base + elem));
  }
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
  int32_t* flag;         // overflow / found-non-finite flag, or null
  const int32_t* skip;   // update only: skip everything if *skip != 0; or null
  DeviceStep dstep;      // update only: step count in device memory, or t == null
  int32_t count;
  uint32_t key;          // probe only: XORed into the stored state; 0 from the host
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

// ---- FP32 -> compute copy ----------------------------------------------------
// BF16, round to nearest even: adding 0x7FFF plus the lowest kept bit carries
// into the kept half exactly when the dropped half is above 0x8000, or equal
// to it with an odd kept half. NaN is tested first -> canonical 0x7FC0.
__device__ __forceinline__ uint32_t bf16_bits(float x) {
  const uint32_t b = __float_as_uint(x);
  const uint32_t rounded = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
  return __builtin_isnan(x) ? 0x7FC0u : rounded;
}

// FP16: the hardware conversion rounds to nearest even (the default mode),
// keeps binary16 subnormals (FP16 denormals are on) and overflows to Inf;
// NaN -> canonical 0x7E00.
__device__ __forceinline__ uint32_t fp16_bits(float x) {
  const uint32_t h = __builtin_bit_cast(uint16_t, static_cast<_Float16>(x));
  return __builtin_isnan(x) ? 0x7E00u : h;
}

template <int OUT>
__device__ __forceinline__ uint32_t out_bits(float x) {
  if constexpr (OUT == kOutFp16) return fp16_bits(x);
  else return bf16_bits(x);
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

// Aggregated gradient of element k of a tile: left fold over the replicas in
// replica order, then the unscale factor.
template <int R, bool FP16>
__device__ __forceinline__ float aggregate(const half_words (&G)[R], int k, float u) {
  float g = (k & 1) ? decode_hi<FP16>(G[0][k / 2]) : decode_lo<FP16>(G[0][k / 2]);
#pragma unroll
  for (int r = 1; r < R; ++r)
    g = g + ((k & 1) ? decode_hi<FP16>(G[r][k / 2]) : decode_lo<FP16>(G[r][k / 2]));
  return g * u;
}

template <int R, bool FP16>
__device__ __forceinline__ float aggregate_one(const uint16_t* const (&g)[R], int64_t i,
                                               float u) {
  float x = decode_one<FP16>(g[0][i]);
#pragma unroll
  for (int r = 1; r < R; ++r) x = x + decode_one<FP16>(g[r][i]);
  return x * u;
}

// Element offset, within its chunk of TILES tiles of BLOCK threads, of
// thread tid's first element in tile u. Tile-major: tile u covers
// [u, u + 1) * BLOCK * kVec. Wave-contiguous: wave w owns TILES adjacent runs
// of 64 * kVec elements.
template <int BLOCK, int TILES>
__device__ __forceinline__ uint32_t tile_offset(int u, int tid) {
  if constexpr (LA_WAVE_CONTIG) {
    return static_cast<uint32_t>((((tid >> 6) * TILES + u) * 64 + (tid & 63)) * kVec);
  } else {
    return static_cast<uint32_t>((u * BLOCK + tid) * kVec);
  }
}

// One tile's results in store order: master, m, v as 16-byte vectors, the
// compute copy packed two values per 32-bit word.
struct TileOut {
  f32x4 P[kQuads], M[kQuads], V[kQuads];
  half_words W;
};

template <int OUT>
__device__ __forceinline__ void store_tile(const TileOut& y, float* p, float* m, float* v,
                                           uint16_t* w, uint32_t off) {
#pragma unroll
  for (int q = 0; q < kQuads; ++q) {
    store_at(y.P[q], p, off + 4 * q);
    store_at(y.M[q], m, off + 4 * q);
    store_at(y.V[q], v, off + 4 * q);
  }
  if constexpr (OUT != kOutNone) store_at(y.W, w, off);
}

// Tensor of chunk c. Chunks only move forward within a workgroup, so t and
// first_chunk_of_t carry over between iterations.
template <int R>
__device__ __forceinline__ void locate(const KernelArgs<R>& a, int64_t c, int& t,
                                       int64_t& first_chunk_of_t) {
  while (c >= a.chunk_end[t]) {  // uniform across the workgroup
    first_chunk_of_t = a.chunk_end[t];
    ++t;
  }
}

// ---- the update kernel ---------------------------------------------------------
// What a launch computes. kHostStep: the update with the constants the host
// derived. kDeviceStep: the same update with the step count read from device
// memory when the kernel runs (alpha and q then formed on the GPU); only
// these instantiations carry the double-precision pow. kProbe: no arithmetic
// at all -- the stream probe, which moves exactly the update's bytes (R
// gradient reads, master/m/v read and written back unchanged, the 16-bit copy
// written as the XOR of the replicas' bit patterns) in exactly its launch
// shape, to measure what HBM gives this stream mix.
constexpr int kHostStep = 0;
constexpr int kDeviceStep = 1;
constexpr int kProbe = 2;

// One tile of one lane: kVec elements of master, m, v and of every replica.
template <int R>
struct TileRegs {
  f32x4 P[kQuads], M[kQuads], V[kQuads];
  half_words G[R];
};

template <int R>
__device__ __forceinline__ void load_tile(TileRegs<R>& x, const float* p, const float* m,
                                          const float* v, const uint16_t* const (&g)[R],
                                          uint32_t off) {
#pragma unroll
  for (int q = 0; q < kQuads; ++q) {
    x.P[q] = load_at<f32x4>(p, off + 4 * q);
    x.M[q] = load_at<f32x4>(m, off + 4 * q);
    x.V[q] = load_at<f32x4>(v, off + 4 * q);
  }
#pragma unroll
  for (int r = 0; r < R; ++r)
    x.G[r] = load_at<half_words>(g[r], off);
}

// The update of one loaded tile.
template <int R, bool FP16, bool FLAG, int OUT>
__device__ __forceinline__ void update_tile(const TileRegs<R>& x, const Scalars& s, bool& bad,
                                            TileOut& y) {
  Elem e[kVec];
#pragma unroll
  for (int k = 0; k < kVec; ++k) {
    const float gk = aggregate<R, FP16>(x.G, k, s.u);
    if (FLAG) bad |= !__builtin_isfinite(gk);
    e[k] = adam_update(gk, x.P[k / 4][k % 4], x.M[k / 4][k % 4], x.V[k / 4][k % 4], s);
  }
#pragma unroll
  for (int q = 0; q < kQuads; ++q) {
    const Elem* z = e + 4 * q;
    y.P[q] = f32x4{z[0].p, z[1].p, z[2].p, z[3].p};
    y.M[q] = f32x4{z[0].m, z[1].m, z[2].m, z[3].m};
    y.V[q] = f32x4{z[0].v, z[1].v, z[2].v, z[3].v};
  }
  if constexpr (OUT != kOutNone) {
#pragma unroll
    for (int k = 0; k < kVec; k += 2)
      y.W[k / 2] = out_bits<OUT>(e[k].p) | (out_bits<OUT>(e[k + 1].p) << 16);
  }
}

// The probe's "arithmetic" for one loaded tile: master, m, v as loaded (XOR a
// key the host passes as 0, so the compiler cannot drop a store of the value
// it just loaded), the copy as the XOR of the replicas.
template <int R, int OUT>
__device__ __forceinline__ void probe_tile(const TileRegs<R>& x, uint32_t key, TileOut& y) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int q = 0; q < kQuads; ++q) {
    y.P[q] = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, x.P[q]) ^ key);
    y.M[q] = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, x.M[q]) ^ key);
    y.V[q] = __builtin_bit_cast(f32x4, __builtin_bit_cast(u32x4, x.V[q]) ^ key);
  }
  if constexpr (OUT != kOutNone) {
    y.W = x.G[0];
#pragma unroll
    for (int r = 1; r < R; ++r) y.W ^= x.G[r];
  }
}

template <int R, bool FP16, bool FLAG, int OUT, int MODE>
__global__ void __launch_bounds__(kBlock)
layer_adam_kernel(const KernelArgs<R> a) {
  if (a.skip != nullptr && *a.skip != 0) return;  // gated step: overflowed, skip
  const int tid = threadIdx.x;
  const int64_t total_chunks = a.chunk_end[a.count - 1];
  Scalars s = a.s;
  if constexpr (MODE == kDeviceStep) {
    // Step count in device memory: the bias corrections of AdamW at the
    // 1-based step t, in double, each constant rounded once to FP32.
    const int64_t t = *a.dstep.t;
    if (t < 1) return;
    const double td = static_cast<double>(t);
    s.alpha = static_cast<float>(a.dstep.lr / (1.0 - pow(a.dstep.beta1, td)));
    s.q = static_cast<float>(sqrt(1.0 - pow(a.dstep.beta2, td)));
  }
  bool bad = false;

  int t = 0;
  int64_t first_chunk_of_t = 0;
  for (int64_t c = blockIdx.x; c < total_chunks; c += gridDim.x) {
    locate(a, c, t, first_chunk_of_t);
    const KernelTensor<R>& T = a.t[t];
    const int64_t base = (c - first_chunk_of_t) * kChunk;
    const int64_t n = T.numel;

    float* __restrict__ p = T.p + base;
    float* __restrict__ m = T.m + base;
    float* __restrict__ v = T.v + base;
    uint16_t* __restrict__ w = OUT == kOutNone ? nullptr : T.w + base;
    const uint16_t* g[R];
#pragma unroll
    for (int r = 0; r < R; ++r) g[r] = T.g[r] + base;

    if (base + kChunk <= n) {
      // Full chunk: every load of the chunk, then per tile the arithmetic and
      // the stores.
      TileRegs<R> x[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
        load_tile<R>(x[u], p, m, v, g, tile_offset<kBlock, kUnroll>(u, tid));
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        TileOut y;
        if constexpr (MODE == kProbe) probe_tile<R, OUT>(x[u], a.key, y);
        else update_tile<R, FP16, FLAG, OUT>(x[u], s, bad, y);
        store_tile<OUT>(y, p, m, v, w, tile_offset<kBlock, kUnroll>(u, tid));
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
            if constexpr (MODE == kProbe) {
              p[i] = __uint_as_float(__float_as_uint(p[i]) ^ a.key);
              m[i] = __uint_as_float(__float_as_uint(m[i]) ^ a.key);
              v[i] = __uint_as_float(__float_as_uint(v[i]) ^ a.key);
              if constexpr (OUT != kOutNone) {
                uint16_t x = g[0][i];
#pragma unroll
                for (int r = 1; r < R; ++r) x ^= g[r][i];
                w[i] = x;
              }
            } else {
              const float gk = aggregate_one<R, FP16>(g, i, s.u);
              if (FLAG) bad |= !__builtin_isfinite(gk);
              const Elem e = adam_update(gk, p[i], m[i], v[i], s);
              p[i] = e.p;
              m[i] = e.m;
              v[i] = e.v;
              if constexpr (OUT != kOutNone) w[i] = static_cast<uint16_t>(out_bits<OUT>(e.p));
            }
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

// ---- the finite-check pre-pass -------------------------------------------------
template <int R, bool FP16>
__global__ void __launch_bounds__(kCheckBlock)
check_kernel(const KernelArgs<R> a) {
  // Already found (by an earlier layer or by other workgroups of this launch,
  // hence the atomic read): the answer cannot change.
  if (__hip_atomic_load(a.flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
  const int tid = threadIdx.x;
  const int64_t total_chunks = a.chunk_end[a.count - 1];
  const float u = a.s.u;
  bool bad = false;

  int t = 0;
  int64_t first_chunk_of_t = 0;
  for (int64_t c = blockIdx.x; c < total_chunks; c += gridDim.x) {
    locate(a, c, t, first_chunk_of_t);
    const KernelTensor<R>& T = a.t[t];
    const int64_t base = (c - first_chunk_of_t) * kCheckChunk;
    const int64_t n = T.numel;
    const uint16_t* g[R];
#pragma unroll
    for (int r = 0; r < R; ++r) g[r] = T.g[r] + base;

    if (base + kCheckChunk <= n) {
      half_words G[kCheckUnroll][R];
#pragma unroll
      for (int tile = 0; tile < kCheckUnroll; ++tile) {
        const uint32_t off = tile_offset<kCheckBlock, kCheckUnroll>(tile, tid);
#pragma unroll
        for (int r = 0; r < R; ++r)
          G[tile][r] = load_stream(reinterpret_cast<const half_words*>(g[r] + off));
      }
#pragma unroll
      for (int tile = 0; tile < kCheckUnroll; ++tile)
#pragma unroll
        for (int k = 0; k < kVec; ++k)
          bad |= !__builtin_isfinite(aggregate<R, FP16>(G[tile], k, u));
    } else {
      const int64_t left = n - base;
#pragma unroll 1
      for (int tile = 0; tile < kCheckUnroll; ++tile) {
#pragma unroll
        for (int k = 0; k < kVec; ++k) {
          const int64_t i = static_cast<int64_t>((tile * kCheckBlock + tid) * kVec + k);
          if (i < left) bad |= !__builtin_isfinite(aggregate_one<R, FP16>(g, i, u));
        }
      }
    }
  }
  if (__any(bad) && __lane_id() == 0) atomicOr(a.flag, 1);
}

// ---- launch --------------------------------------------------------------------
template <int R>
int64_t fill_args(KernelArgs<R>& a, const TensorArgs* ts, int count, int64_t chunk) {
  int64_t chunks = 0;
  for (int i = 0; i < count; ++i) {
    a.t[i].p = ts[i].p;
    a.t[i].m = ts[i].m;
    a.t[i].v = ts[i].v;
    a.t[i].w = ts[i].w;
    for (int r = 0; r < R; ++r) a.t[i].g[r] = ts[i].g[r];
    a.t[i].numel = ts[i].numel;
    chunks += (ts[i].numel + chunk - 1) / chunk;
    a.chunk_end[i] = chunks;
  }
  a.count = count;
  return chunks;
}

// LDS to reserve per workgroup so that at most `per_cu` workgroups fit on a
// compute unit: floor(lds_per_cu / (per_cu + 1/2)) in whole KiB, within the
// per-workgroup limit; 0 (no reservation) for no cap or unknown facts.
int lds_reservation(const LaunchShape& shape, int default_per_cu) {
  const int per_cu = shape.wg_per_cu < 0 ? default_per_cu : shape.wg_per_cu;
  if (per_cu <= 0 || shape.lds_per_cu <= 0 || shape.lds_per_block <= 0) return 0;
  const int bytes = static_cast<int>(2LL * shape.lds_per_cu / (2LL * per_cu + 1)) / 1024 * 1024;
  return bytes <= shape.lds_per_block ? bytes : 0;
}

hipError_t launch(const void* kernel, void* args, int64_t chunks, int block, int lds,
                  hipStream_t stream, const LaunchShape& shape) {
  const int64_t grid = chunks < shape.grid_cap ? chunks : shape.grid_cap;  // >= 1
  void* params[] = {args};
  return hipLaunchKernel(kernel, dim3(static_cast<unsigned>(grid)), dim3(block), params,
                         static_cast<unsigned>(lds), stream);
}

template <int R, bool FP16, bool FLAG, int OUT, int MODE>
hipError_t launch_update_typed(const TensorArgs* ts, int count, const Scalars& s,
                               const DeviceStep& dstep, int32_t* flag, const int32_t* skip,
                               hipStream_t stream, const LaunchShape& shape) {
  KernelArgs<R> a = {};
  const int64_t chunks = fill_args(a, ts, count, kChunk);
  a.s = s;
  a.dstep = dstep;
  a.flag = flag;
  a.skip = skip;
  a.key = 0;
  return launch(reinterpret_cast<const void*>(&layer_adam_kernel<R, FP16, FLAG, OUT, MODE>), &a,
                chunks, kBlock, lds_reservation(shape, update_workgroups_per_cu<R>()), stream,
                shape);
}

template <int R, bool FP16, int OUT>
hipError_t launch_update_flag(const TensorArgs* ts, int count, const Scalars& s,
                              const DeviceStep& d, int32_t* flag, const int32_t* skip,
                              hipStream_t stream, const LaunchShape& shape) {
  if (d.t != nullptr)
    return flag ? launch_update_typed<R, FP16, true, OUT, kDeviceStep>(ts, count, s, d, flag,
                                                                       skip, stream, shape)
                : launch_update_typed<R, FP16, false, OUT, kDeviceStep>(ts, count, s, d, flag,
                                                                        skip, stream, shape);
  return flag ? launch_update_typed<R, FP16, true, OUT, kHostStep>(ts, count, s, d, flag, skip,
                                                                   stream, shape)
              : launch_update_typed<R, FP16, false, OUT, kHostStep>(ts, count, s, d, flag, skip,
                                                                    stream, shape);
}

template <int R, bool FP16>
hipError_t launch_update_out(const TensorArgs* ts, int count, int out, const Scalars& s,
                             const DeviceStep& d, int32_t* flag, const int32_t* skip,
                             hipStream_t stream, const LaunchShape& shape) {
  switch (out) {
    case kOutBf16: return launch_update_flag<R, FP16, kOutBf16>(ts, count, s, d, flag, skip, stream, shape);
    case kOutFp16: return launch_update_flag<R, FP16, kOutFp16>(ts, count, s, d, flag, skip, stream, shape);
    case kOutNone: return launch_update_flag<R, FP16, kOutNone>(ts, count, s, d, flag, skip, stream, shape);
    default: return hipErrorInvalidValue;
  }
}

template <int R>
hipError_t launch_update_r(const TensorArgs* ts, int count, bool fp16, int out,
                           const Scalars& s, const DeviceStep& d, int32_t* flag,
                           const int32_t* skip, hipStream_t stream, const LaunchShape& shape) {
  return fp16 ? launch_update_out<R, true>(ts, count, out, s, d, flag, skip, stream, shape)
              : launch_update_out<R, false>(ts, count, out, s, d, flag, skip, stream, shape);
}

// The probe moves bit patterns only: the gradient format does not matter, and
// both 16-bit copy formats are one 2-byte store.
template <int R>
hipError_t launch_probe_r(const TensorArgs* ts, int count, int out, hipStream_t stream,
                          const LaunchShape& shape) {
  const Scalars none = {};
  const DeviceStep host = {nullptr, 0.0, 0.0, 0.0};
  return out == kOutNone
             ? launch_update_typed<R, false, false, kOutNone, kProbe>(ts, count, none, host,
                                                                      nullptr, nullptr, stream,
                                                                      shape)
             : launch_update_typed<R, false, false, kOutBf16, kProbe>(ts, count, none, host,
                                                                      nullptr, nullptr, stream,
                                                                      shape);
}

template <int R>
hipError_t launch_check_r(const TensorArgs* ts, int count, bool fp16, float u, int32_t* flag,
                          hipStream_t stream, const LaunchShape& shape) {
  KernelArgs<R> a = {};
  const int64_t chunks = fill_args(a, ts, count, kCheckChunk);
  a.s.u = u;
  a.flag = flag;
  const void* k = fp16 ? reinterpret_cast<const void*>(&check_kernel<R, true>)
                       : reinterpret_cast<const void*>(&check_kernel<R, false>);
  return launch(k, &a, chunks, kCheckBlock, lds_reservation(shape, LA_CHECK_WORKGROUPS_PER_CU),
                stream, shape);
}

}  // namespace

hipError_t launch_layer_adam(const TensorArgs* tensors, int count, int replicas, bool fp16,
                             int out_dtype, const Scalars& s, const DeviceStep& dstep,
                             int32_t* flag, const int32_t* skip, hipStream_t stream,
                             const LaunchShape& shape) {
  switch (replicas) {
#define LA_CASE(RR)                                                                        \
  case RR:                                                                                 \
    return launch_update_r<RR>(tensors, count, fp16, out_dtype, s, dstep, flag, skip,    \
                               stream, shape);
    LA_CASE(1) LA_CASE(2) LA_CASE(3) LA_CASE(4) LA_CASE(5) LA_CASE(6) LA_CASE(7) LA_CASE(8)
#undef LA_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_stream_probe(const TensorArgs* tensors, int count, int replicas,
                               int out_dtype, hipStream_t stream, const LaunchShape& shape) {
  switch (replicas) {
#define LA_CASE(RR) \
  case RR: return launch_probe_r<RR>(tensors, count, out_dtype, stream, shape);
    LA_CASE(1) LA_CASE(2) LA_CASE(3) LA_CASE(4) LA_CASE(5) LA_CASE(6) LA_CASE(7) LA_CASE(8)
#undef LA_CASE
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_check_gradients(const TensorArgs* tensors, int count, int replicas,
                                  bool fp16, float unscale, int32_t* flag, hipStream_t stream,
                                  const LaunchShape& shape) {
  switch (replicas) {
#define LA_CASE(RR) \
  case RR: return launch_check_r<RR>(tensors, count, fp16, unscale, flag, stream, shape);
    LA_CASE(1) LA_CASE(2) LA_CASE(3) LA_CASE(4) LA_CASE(5) LA_CASE(6) LA_CASE(7) LA_CASE(8)
#undef LA_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
