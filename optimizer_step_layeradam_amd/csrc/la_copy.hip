// la_copy.hip -- measurement kernels beside the update: a plain streaming
// copy, and the direction probe. Neither is part of the update.
//
// copy_kernel moves bytes the way the update does -- 16-byte non-temporal
// loads, 16-byte stores written through to memory, a wave's tiles adjacent
// in memory, every load of a workgroup issued before its first store, one
// workgroup per chunk so that the dispatcher keeps the workgroups in flight
// on a narrow advancing window -- but with one read and one write stream and
// no arithmetic. What it reaches is what this GPU's HBM gives a simple
// two-stream pattern; the update interleaves R + 7 streams (the library's
// stream probe measures that mix).
//
// direction_kernel splits the update's traffic by direction: its read part
// issues exactly the update's loads (the R gradient replicas and master, m,
// v: one 64-lane wave per 256-element chunk, 16 bytes of each FP32 array and
// 8 bytes of each replica per lane, non-temporal buffer loads) and stores
// nothing; its write part issues exactly the update's stores (master, m, v
// and the 16-bit copy, written through to memory) of a constant and loads
// nothing. Timed alone, in sequence, at once on two streams, or alternating
// over slices of a layer, the two parts show how fast HBM serves each
// direction of the update's traffic and what interleaving them costs -- the
// per-resource bandwidth beta of the step-time bound T >= max_j W_j / beta_j
// in "SlideDP: Scaling Host-Resident LLM Fine-Tuning Across Multiple GPUs"
// (研究动机 and 技术新颖性), taken apart for the one resource here.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "la_copy.h"

namespace la {
namespace {

// Defaults: the fastest copy measured on MI355X over 64-512 threads, 1-8
// units per thread, residency caps of 2-16 workgroups per compute unit or
// none, and non-temporal or written-through stores (2 and 8 GiB copies):
// one-wave workgroups of 4 units per lane, eight per compute unit, stores
// written through -- the same style as the update kernel's launch.
#ifndef LA_COPY_BLOCK
#define LA_COPY_BLOCK 64       // threads per workgroup
#endif
#ifndef LA_COPY_TILES
#define LA_COPY_TILES 4        // 16-byte units per thread per chunk
#endif
#ifndef LA_COPY_WORKGROUPS_PER_CU
#define LA_COPY_WORKGROUPS_PER_CU 8  // resident workgroups per compute unit (0: no cap)
#endif
// 1: stores as buffer instructions with the cache-policy bits
// LA_COPY_STORE_CPOL (1 = sc0, 2 = nt, 16 = sc1; 19 writes through to memory)
// instead of non-temporal global stores.
#ifndef LA_COPY_BUFFER_STORES
#define LA_COPY_BUFFER_STORES 1
#endif
#ifndef LA_COPY_STORE_CPOL
#define LA_COPY_STORE_CPOL 19
#endif

constexpr int kCopyBlock = LA_COPY_BLOCK;
constexpr int kCopyTiles = LA_COPY_TILES;
constexpr int64_t kCopyChunk = int64_t(kCopyBlock) * kCopyTiles;  // 16-byte units
constexpr int64_t kCopyMaxGrid = int64_t(1) << 30;
static_assert(kCopyBlock % 64 == 0 && kCopyBlock <= 1024, "whole waves");

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Unit of thread tid in tile u of a chunk: wave w owns kCopyTiles adjacent
// runs of 64 units.
__device__ __forceinline__ int64_t unit_offset(int u, int tid) {
  return ((int64_t(tid >> 6) * kCopyTiles + u) << 6) + (tid & 63);
}

__device__ __forceinline__ void store_unit(u32x4 x, u32x4* dst, int64_t i) {
  if constexpr (LA_COPY_BUFFER_STORES) {
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(dst, 0, 0x7fffffff,
                                                                      0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(x, r, static_cast<uint32_t>(i) * 16u, 0,
                                           LA_COPY_STORE_CPOL);
  } else {
    __builtin_nontemporal_store(x, dst + i);
  }
}

__global__ void __launch_bounds__(kCopyBlock)
copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, int64_t n16) {
  const int tid = threadIdx.x;
  const int64_t chunks = (n16 + kCopyChunk - 1) / kCopyChunk;
  for (int64_t c = blockIdx.x; c < chunks; c += gridDim.x) {
    const int64_t base = c * kCopyChunk;
    if (base + kCopyChunk <= n16) {
      u32x4 r[kCopyTiles];
#pragma unroll
      for (int u = 0; u < kCopyTiles; ++u)
        r[u] = __builtin_nontemporal_load(src + base + unit_offset(u, tid));
#pragma unroll
      for (int u = 0; u < kCopyTiles; ++u) store_unit(r[u], dst + base, unit_offset(u, tid));
    } else {
      // Last, partial chunk: unit by unit, bounds-checked, same cache policies.
#pragma unroll 1
      for (int u = 0; u < kCopyTiles; ++u) {
        const int64_t k = int64_t(u) * kCopyBlock + tid;
        if (base + k < n16) store_unit(__builtin_nontemporal_load(src + base + k), dst + base, k);
      }
    }
  }
}

// ---- the direction probe -----------------------------------------------------
// Default residency of both parts: eight one-wave workgroups per compute
// unit, the update's own at R = 7 and 8. Measured on MI355X (6-12 per CU and
// no cap): the writes alone are fastest at 7-8 on every layer shape, the
// reads alone at 6-8 (within 2 % of their best at 8), and the two parts at
// once on two streams at 8 each.
#ifndef LA_DIR_READ_WORKGROUPS_PER_CU
#define LA_DIR_READ_WORKGROUPS_PER_CU 8
#endif
#ifndef LA_DIR_WRITE_WORKGROUPS_PER_CU
#define LA_DIR_WRITE_WORKGROUPS_PER_CU 8
#endif

constexpr int kDirLanes = 64;                 // one wave per workgroup
constexpr int kDirVec = 4;                    // consecutive elements per lane
constexpr int kDirChunk = kDirLanes * kDirVec;  // 256 elements, the update's chunk
static_assert(kDirChunk > kMaxUnalignedEntry, "short entries take the element-wise path");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

template <int R>
struct DirTensor {
  uint32_t* p;  // master, m, v as 32-bit patterns
  uint32_t* m;
  uint32_t* v;
  uint16_t* w;  // the compute copy, or null
  const uint16_t* g[R];
  int64_t numel;
};

template <int R>
struct DirArgs {
  DirTensor<R> t[kTensorsPerLaunch];
  int64_t chunk_end[kTensorsPerLaunch];  // cumulative chunk counts
  int32_t count;
  uint32_t fill;  // write part: the pattern stored
};

// Buffer resource over a uniform base pointer (raw 32-bit format), as the
// update builds them.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}

constexpr int kLoadNt = 2;         // non-temporal
constexpr int kStoreThrough = 19;  // sc0 | sc1 | nt: written through to memory

template <int R, int PART>
__global__ void __launch_bounds__(kDirLanes)
direction_kernel(const DirArgs<R> a) {
  const int lane = threadIdx.x;
  const int64_t total_chunks = a.chunk_end[a.count - 1];
  const uint32_t fill = a.fill;
  uint32_t acc = 0;  // read part: every loaded word, folded, so that no load is dropped

  int t = 0;
  int64_t first_chunk_of_t = 0;
  for (int64_t c = blockIdx.x; c < total_chunks; c += gridDim.x) {
    while (c >= a.chunk_end[t]) {  // uniform across the wave
      first_chunk_of_t = a.chunk_end[t];
      ++t;
    }
    const DirTensor<R>& T = a.t[t];
    const int64_t base = (c - first_chunk_of_t) * kDirChunk;
    uint32_t* p = T.p + base;
    uint32_t* m = T.m + base;
    uint32_t* v = T.v + base;
    uint16_t* w = T.w == nullptr ? nullptr : T.w + base;

    if (base + kDirChunk <= T.numel) {
      const uint32_t off = static_cast<uint32_t>(lane) * kDirVec;  // element of the chunk
      if constexpr (PART == kProbeReads) {
        const u32x4 P = __builtin_amdgcn_raw_buffer_load_b128(rsrc(p), off * 4, 0, kLoadNt);
        const u32x4 M = __builtin_amdgcn_raw_buffer_load_b128(rsrc(m), off * 4, 0, kLoadNt);
        const u32x4 V = __builtin_amdgcn_raw_buffer_load_b128(rsrc(v), off * 4, 0, kLoadNt);
        u32x2 G[R];
#pragma unroll
        for (int r = 0; r < R; ++r)
          G[r] = __builtin_amdgcn_raw_buffer_load_b64(rsrc(T.g[r] + base), off * 2, 0, kLoadNt);
        u32x4 x = P ^ M ^ V;
#pragma unroll
        for (int r = 0; r < R; ++r) x.xy ^= G[r];
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
      } else {
        const u32x4 f4 = {fill, fill, fill, fill};
        __builtin_amdgcn_raw_buffer_store_b128(f4, rsrc(p), off * 4, 0, kStoreThrough);
        __builtin_amdgcn_raw_buffer_store_b128(f4, rsrc(m), off * 4, 0, kStoreThrough);
        __builtin_amdgcn_raw_buffer_store_b128(f4, rsrc(v), off * 4, 0, kStoreThrough);
        if (w != nullptr) {
          const uint32_t h = (fill & 0xFFFFu) * 0x10001u;
          const u32x2 h2 = {h, h};
          __builtin_amdgcn_raw_buffer_store_b64(h2, rsrc(w), off * 2, 0, kStoreThrough);
        }
      }
    } else {
      // Last, partial chunk of an entry: element by element, bounds-checked.
      const int64_t left = T.numel - base;  // 1 .. kDirChunk - 1
#pragma unroll
      for (int k = 0; k < kDirVec; ++k) {
        const int64_t i = static_cast<int64_t>(lane) * kDirVec + k;
        if (i < left) {
          if constexpr (PART == kProbeReads) {
            acc ^= p[i] ^ m[i] ^ v[i];
#pragma unroll
            for (int r = 0; r < R; ++r) acc ^= T.g[r][base + i];
          } else {
            p[i] = fill;
            m[i] = fill;
            v[i] = fill;
            if (w != nullptr) w[i] = static_cast<uint16_t>(fill);
          }
        }
      }
    }
  }
  if constexpr (PART == kProbeReads) asm volatile("" ::"v"(acc));  // keep every load
}

// LDS the kernels never touch, reserved so that at most `per_cu` workgroups
// fit on a compute unit: floor(lds_per_cu / (per_cu + 1/2)) in whole KiB
// (none for no cap or unknown sizes).
int reserved_lds(int per_cu, int lds_per_cu, int lds_per_block) {
  if (per_cu <= 0 || lds_per_cu <= 0 || lds_per_block <= 0) return 0;
  const int bytes = static_cast<int>(2LL * lds_per_cu / (2LL * per_cu + 1)) / 1024 * 1024;
  return bytes <= lds_per_block ? bytes : 0;
}

template <int R, int PART>
hipError_t launch_direction_typed(const TensorArgs* ts, int count, int out_dtype, uint32_t fill,
                                  hipStream_t stream, const LaunchShape& shape) {
  DirArgs<R> a = {};
  int64_t chunks = 0;
  for (int i = 0; i < count; ++i) {
    a.t[i].p = reinterpret_cast<uint32_t*>(ts[i].p);
    a.t[i].m = reinterpret_cast<uint32_t*>(ts[i].m);
    a.t[i].v = reinterpret_cast<uint32_t*>(ts[i].v);
    a.t[i].w = out_dtype == kOutNone ? nullptr : ts[i].w;
    for (int r = 0; r < R; ++r) a.t[i].g[r] = ts[i].g[r];
    a.t[i].numel = ts[i].numel;
    chunks += (ts[i].numel + kDirChunk - 1) / kDirChunk;
    a.chunk_end[i] = chunks;
  }
  a.count = count;
  a.fill = fill;
  const int per_cu = shape.wg_per_cu >= 0 ? shape.wg_per_cu
                     : PART == kProbeReads ? LA_DIR_READ_WORKGROUPS_PER_CU
                                           : LA_DIR_WRITE_WORKGROUPS_PER_CU;
  const int64_t grid = chunks < shape.grid_cap ? chunks : shape.grid_cap;
  void* params[] = {&a};
  return hipLaunchKernel(reinterpret_cast<const void*>(&direction_kernel<R, PART>),
                         dim3(static_cast<unsigned>(grid)), dim3(kDirLanes), params,
                         static_cast<unsigned>(reserved_lds(per_cu, shape.lds_per_cu,
                                                            shape.lds_per_block)),
                         stream);
}

}  // namespace

hipError_t launch_copy_reference(void* dst, const void* src, int64_t n16, int lds_per_cu,
                                 int lds_per_block, int wg_per_cu, int grid_cap,
                                 hipStream_t stream) {
  if (n16 <= 0) return hipSuccess;
  const int64_t chunks = (n16 + kCopyChunk - 1) / kCopyChunk;
  const int64_t cap = grid_cap >= 1 && grid_cap < kCopyMaxGrid ? grid_cap : kCopyMaxGrid;
  const int64_t grid = chunks < cap ? chunks : cap;
  const int per_cu = wg_per_cu < 0 ? LA_COPY_WORKGROUPS_PER_CU : wg_per_cu;
  const int lds = reserved_lds(per_cu, lds_per_cu, lds_per_block);
  u32x4* d = static_cast<u32x4*>(dst);
  const u32x4* s = static_cast<const u32x4*>(src);
  void* params[] = {&d, &s, &n16};
  return hipLaunchKernel(reinterpret_cast<const void*>(&copy_kernel),
                         dim3(static_cast<unsigned>(grid)), dim3(kCopyBlock), params,
                         static_cast<unsigned>(lds), stream);
}

hipError_t launch_direction_probe(const TensorArgs* tensors, int count, int replicas,
                                  int out_dtype, int part, uint32_t fill, hipStream_t stream,
                                  const LaunchShape& shape) {
  // The write part touches no gradient: one instantiation serves every R.
  if (part == kProbeWrites)
    return launch_direction_typed<1, kProbeWrites>(tensors, count, out_dtype, fill, stream,
                                                   shape);
  if (part != kProbeReads) return hipErrorInvalidValue;
  switch (replicas) {
#define LA_CASE(RR)                                                                     \
  case RR:                                                                              \
    return launch_direction_typed<RR, kProbeReads>(tensors, count, out_dtype, fill, stream, \
                                                   shape);
    LA_CASE(1) LA_CASE(2) LA_CASE(3) LA_CASE(4) LA_CASE(5) LA_CASE(6) LA_CASE(7) LA_CASE(8)
#undef LA_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace la
