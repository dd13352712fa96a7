// Paged KV store (scatter of new K/V rows into their slots) and whole-block
// copy for copy-on-write, gfx950.
//
// Store: the nanoPD page names a "paged KV store op" beside its attention
// kernel; the serving-stack page, section 2.3, places a sequence's new token
// at offset length % block_size of its last block.  Here a slot is
// physical_block * block_size + offset.
// Copy: copy on write of a shared block before a forked sequence writes into
// it (nanoPD page, paged KV cache with CoW; serving-stack page 2.3, cow()).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// One workgroup = 64 consecutive tokens x one kv head.
//  K: 16-byte input chunks, mapped so that consecutive lanes cover one key
//     row: reads and writes are both contiguous.
//  V: lane = token, so that tokens landing at consecutive offsets of one
//     block write neighbouring elements of each transposed head-dim row.
template <int KV>
__global__ void __launch_bounds__(256) store_kv_kernel(StoreArgs a) {
  constexpr int IN_ES = (KV == KV_F32) ? 4 : 2;            // input element bytes
  constexpr int OUT_ES = (KV == KV_F32) ? 4 : (KV == KV_BF16 ? 2 : 1);
  constexpr int EPC = 16 / IN_ES;                          // elements per 16-byte chunk
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * 64;
  const int cpr = a.head_dim / EPC;                        // chunks per row
  const int H = a.num_kv_heads, D = a.head_dim, BS = a.block_size;

  const char* kin = static_cast<const char*>(a.k_new);
  const char* vin = static_cast<const char*>(a.v_new);
  char* kc = static_cast<char*>(a.k_cache);
  char* vc = static_cast<char*>(a.v_cache);
  float ksc = 1.f, vsc = 1.f;
  if constexpr (KV == KV_FP8) {
    ksc = a.k_scale[h];
    vsc = a.v_scale[h];
  }

  // ---- keys: contiguous rows
  for (int idx = threadIdx.x; idx < 64 * cpr; idx += 256) {
    const int t = t0 + idx / cpr;
    const int c = idx % cpr;
    if (t >= a.num_tokens) continue;
    const int slot = a.slot_mapping[t];
    if (slot < 0) continue;
    const int blk = slot / BS, off = slot % BS;
    const uint4 x = *reinterpret_cast<const uint4*>(kin + ((size_t(t) * H + h) * D + size_t(c) * EPC) * IN_ES);
    char* dst = kc + ((size_t(blk) * H + h) * BS + off) * size_t(D) * OUT_ES + size_t(c) * EPC * OUT_ES;
    if constexpr (KV != KV_FP8) {
      *reinterpret_cast<uint4*>(dst) = x;
    } else {
      const uint32_t w[4] = {x.x, x.y, x.z, x.w};
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t c0 = e4m3_encode(bf16_lo(w[e]) / ksc);
        const uint32_t c1 = e4m3_encode(bf16_hi(w[e]) / ksc);
        const uint32_t two = c0 | (c1 << 8);
        if (e < 2) lo |= two << (16 * e); else hi |= two << (16 * (e - 2));
      }
      *reinterpret_cast<uint2*>(dst) = make_uint2(lo, hi);
    }
  }

  // ---- values: transposed rows, lane = token
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int t = t0 + lane;
  int slot = -1;
  if (t < a.num_tokens) slot = a.slot_mapping[t];
  if (slot < 0) return;
  const int blk = slot / BS, off = slot % BS;
  char* vrow = vc + ((size_t(blk) * H + h) * D) * size_t(BS) * OUT_ES + size_t(off) * OUT_ES;
  for (int c = wave; c < cpr; c += 4) {
    const uint4 x = *reinterpret_cast<const uint4*>(vin + ((size_t(t) * H + h) * D + size_t(c) * EPC) * IN_ES);
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    const int d0 = c * EPC;
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int e = 0; e < 4; ++e)
        *reinterpret_cast<uint32_t*>(vrow + size_t(d0 + e) * BS * 4) = w[e];
    } else if constexpr (KV == KV_BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint16_t*>(vrow + size_t(d0 + 2 * e) * BS * 2) = uint16_t(w[e] & 0xFFFFu);
        *reinterpret_cast<uint16_t*>(vrow + size_t(d0 + 2 * e + 1) * BS * 2) = uint16_t(w[e] >> 16);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<uint8_t*>(vrow + size_t(d0 + 2 * e) * BS) = uint8_t(e4m3_encode(bf16_lo(w[e]) / vsc));
        *reinterpret_cast<uint8_t*>(vrow + size_t(d0 + 2 * e + 1) * BS) = uint8_t(e4m3_encode(bf16_hi(w[e]) / vsc));
      }
    }
  }
}

// One workgroup row per pair; 16-byte chunks of the block in both pools.
__global__ void __launch_bounds__(256) copy_blocks_kernel(CopyArgs a) {
  const int p = blockIdx.x;
  const int src = a.pairs[2 * p], dst = a.pairs[2 * p + 1];
  const size_t n16 = a.block_bytes / 16;
  const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_cache) + size_t(src) * a.block_bytes);
  uint4* kd = reinterpret_cast<uint4*>(static_cast<char*>(a.k_cache) + size_t(dst) * a.block_bytes);
  const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_cache) + size_t(src) * a.block_bytes);
  uint4* vd = reinterpret_cast<uint4*>(static_cast<char*>(a.v_cache) + size_t(dst) * a.block_bytes);
  for (size_t i = blockIdx.y * 256 + threadIdx.x; i < n16; i += size_t(gridDim.y) * 256) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
}

hipError_t launch_store_kv(const StoreArgs& a, int kv, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  dim3 grid((a.num_tokens + 63) / 64, a.num_kv_heads);
  switch (kv) {
    case KV_F32: hipLaunchKernelGGL(store_kv_kernel<KV_F32>, grid, dim3(256), 0, s, a); break;
    case KV_BF16: hipLaunchKernelGGL(store_kv_kernel<KV_BF16>, grid, dim3(256), 0, s, a); break;
    default: hipLaunchKernelGGL(store_kv_kernel<KV_FP8>, grid, dim3(256), 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_copy_blocks(const CopyArgs& a, int num_pairs, hipStream_t s) {
  if (num_pairs == 0) return hipSuccess;
  const size_t n16 = a.block_bytes / 16;
  const int ychunks = int((n16 + 255) / 256 < 8 ? (n16 + 255) / 256 : 8);
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(num_pairs, ychunks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
