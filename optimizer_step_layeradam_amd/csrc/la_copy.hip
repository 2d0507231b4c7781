// la_copy.hip -- a plain streaming copy, the bandwidth reference the update
// kernel is measured against.
//
// It moves bytes the way the update does -- 16-byte non-temporal loads,
// 16-byte stores written through to memory, a wave's tiles adjacent in
// memory, every load of a workgroup issued before its first store, one
// workgroup per chunk so that the dispatcher keeps the workgroups in flight
// on a narrow advancing window -- but with one read and one write stream and
// no arithmetic. What it reaches is what this GPU's HBM gives a simple
// two-stream pattern; the update interleaves R + 7 streams (the library's
// stream probe measures that mix).

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
#pragma unroll 1
      for (int u = 0; u < kCopyTiles; ++u) {
        const int64_t i = base + int64_t(u) * kCopyBlock + tid;
        if (i < n16) dst[i] = src[i];
      }
    }
  }
}

}  // namespace

hipError_t launch_copy_reference(void* dst, const void* src, int64_t n16, int lds_per_cu,
                                 int lds_per_block, int wg_per_cu, hipStream_t stream) {
  if (n16 <= 0) return hipSuccess;
  const int64_t chunks = (n16 + kCopyChunk - 1) / kCopyChunk;
  const int64_t grid = chunks < kCopyMaxGrid ? chunks : kCopyMaxGrid;
  // LDS the kernel never touches, reserved so that at most `per_cu`
  // workgroups fit on a compute unit (none for no cap or unknown sizes).
  const int per_cu = wg_per_cu < 0 ? LA_COPY_WORKGROUPS_PER_CU : wg_per_cu;
  int lds = 0;
  if (per_cu > 0 && lds_per_cu > 0 && lds_per_block > 0) {
    const int bytes = static_cast<int>(2LL * lds_per_cu / (2LL * per_cu + 1)) / 1024 * 1024;
    lds = bytes <= lds_per_block ? bytes : 0;
  }
  u32x4* d = static_cast<u32x4*>(dst);
  const u32x4* s = static_cast<const u32x4*>(src);
  void* params[] = {&d, &s, &n16};
  return hipLaunchKernel(reinterpret_cast<const void*>(&copy_kernel),
                         dim3(static_cast<unsigned>(grid)), dim3(kCopyBlock), params,
                         static_cast<unsigned>(lds), stream);
}

}  // namespace la
