// HBM reference kernels for measurement only (libpa_probe.so, loaded by the
// benchmark's --hbm-probe mode; not part of libpa's C ABI).  They give the
// practical ceilings the attention and store kernels are compared with:
//  * probe_read: a streaming read of a buffer, 16 bytes per lane per load,
//    each workgroup reading one contiguous stretch;
//  * probe_copy: a streaming copy (read + write), in the same stretches;
//  * probe_tiles: reads of whole 4 KB tiles in a seeded random order (the
//    access pattern of decode: one (block, kv head) tile per wave load).
// The reads and the copy's loads take the default cache policy or, with nt
// set, the non-temporal hint the decode's tile loads and the block copy's
// loads carry.
// Each kernel folds what it reads into one value per thread, stored only if
// it equals a key the data never holds, so no load can be dropped and
// nothing but the copy writes.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <bool NT>
__device__ __forceinline__ uint4 ld(const uint4* p) {
  if constexpr (NT) {
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
  } else {
    return *p;
  }
}

// Workgroup b streams the contiguous stretch [b n16 / grid, (b + 1) n16 / grid)
// of 16-byte chunks, each thread with eight loads in flight (the stretch is
// walked in rounds of 8 x 256 chunks; the remainder one chunk at a time).
template <bool NT>
__global__ void __launch_bounds__(256) probe_read(const uint4* __restrict__ src, size_t n16, uint32_t key,
                                                  uint32_t* __restrict__ sink) {
  const size_t lo = size_t(blockIdx.x) * n16 / gridDim.x, hi = size_t(blockIdx.x + 1) * n16 / gridDim.x;
  uint32_t acc = 0;
  size_t i = lo + threadIdx.x;
  for (; i + 7 * 256 < hi; i += 8 * 256) {
    uint4 x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = ld<NT>(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= x[u].x ^ x[u].y ^ x[u].z ^ x[u].w;
  }
  for (; i < hi; i += 256) {
    const uint4 a = ld<NT>(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == key) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

// Same stretches as probe_read, four 16-byte loads in flight per thread.
template <bool NT>
__global__ void __launch_bounds__(256) probe_copy(const uint4* __restrict__ src, uint4* __restrict__ dst, size_t n16) {
  const size_t lo = size_t(blockIdx.x) * n16 / gridDim.x, hi = size_t(blockIdx.x + 1) * n16 / gridDim.x;
  size_t i = lo + threadIdx.x;
  for (; i + 3 * 256 < hi; i += 4 * 256) {
    uint4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) x[u] = ld<NT>(src + i + u * 256);
#pragma unroll
    for (int u = 0; u < 4; ++u) dst[i + u * 256] = x[u];
  }
  for (; i < hi; i += 256) dst[i] = ld<NT>(src + i);
}

// Wave w reads tiles order[w], order[w + waves], ... (4 KB each: 64 lanes x
// 4 x 16 bytes).
template <bool NT>
__global__ void __launch_bounds__(256) probe_tiles(const uint4* __restrict__ src, const int32_t* __restrict__ order,
                                                   int32_t n_tiles, uint32_t key, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  const int waves = gridDim.x * 4;
  uint32_t acc = 0;
  for (int t = blockIdx.x * 4 + (threadIdx.x >> 6); t < n_tiles; t += waves) {
    const uint4* p = src + size_t(order[t]) * 256;
    const uint4 a = ld<NT>(p + lane), b = ld<NT>(p + lane + 64), c = ld<NT>(p + lane + 128), d = ld<NT>(p + lane + 192);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  if (acc == key) sink[blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace

// Host launchers (plain C, device pointers).  grid: workgroups of 256
// threads; sink: at least grid * 256 uint32 of device memory; nt: nonzero for
// loads with the non-temporal hint.
extern "C" int pa_probe_read(const void* src, size_t bytes, int grid, void* sink, int nt, void* stream) {
  hipLaunchKernelGGL(nt ? probe_read<true> : probe_read<false>, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), bytes / 16, 0xA5A5A5A5u,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

extern "C" int pa_probe_copy(const void* src, void* dst, size_t bytes, int grid, int nt, void* stream) {
  hipLaunchKernelGGL(nt ? probe_copy<true> : probe_copy<false>, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), static_cast<uint4*>(dst),
                     bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : -6;
}

// order: n_tiles int32 tile indices, each < bytes of src / 4096.
extern "C" int pa_probe_tiles(const void* src, const int32_t* order, int32_t n_tiles, int grid, void* sink, int nt,
                              void* stream) {
  hipLaunchKernelGGL(nt ? probe_tiles<true> : probe_tiles<false>, dim3(grid), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const uint4*>(src), order, n_tiles, 0xA5A5A5A5u,
                     static_cast<uint32_t*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -6;
}
