// The store of one new token's K and V rows for one kv head into its slot
// (nanoPD page: the paged KV cache's store operation; serving-stack page,
// section 2.3: a sequence's new token goes to offset length % block_size of
// its last block), by one wavefront.  Shared by the row-store kernel and by
// the decode kernel's append form, which stores each sequence's new token
// before it reads the cache.
#pragma once
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// The token's input rows for head h: krow / vrow hold its D elements (f32
// for an f32 cache, bf16 otherwise; raw e4m3 codes for KV_FP8_RAW).  The key
// row is read as 16-byte chunks, the value row one element per lane (two for
// head_dim 128); a later store_new_row writes them.  Splitting the two lets a
// caller put other loads in flight with these before the one wait that both
// need.
struct NewRow {
  uint4 kx;
  uint32_t vx[2];
};

template <int KV>
__device__ __forceinline__ NewRow load_new_row(const char* krow, const char* vrow, int D) {
  constexpr int IN_ES = (KV == KV_F32) ? 4 : (KV == KV_FP8_RAW ? 1 : 2);   // input element bytes
  constexpr int EPC = 16 / IN_ES;                          // input elements per 16-byte chunk
  const int lane = threadIdx.x & 63;
  const int cpr = D / EPC;                                 // key chunks per row (<= 32)
  NewRow r;
  r.kx = *reinterpret_cast<const uint4*>(krow + size_t(min(lane, cpr - 1)) * 16);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int d = min(lane + 64 * i, D - 1);
    if constexpr (IN_ES == 4) r.vx[i] = *reinterpret_cast<const uint32_t*>(vrow + size_t(d) * 4);
    else if constexpr (IN_ES == 2) r.vx[i] = *reinterpret_cast<const uint16_t*>(vrow + size_t(d) * 2);
    else r.vx[i] = *reinterpret_cast<const uint8_t*>(vrow + d);
  }
  return r;
}

// The stores of a loaded row into its slot: the key row as 16-byte chunks,
// the value elements to their transposed places (head dim d at element
// d * block_size + offset of the tile).  A negative slot stores nothing.  An
// fp8 cache takes each bf16 value divided by the head's scale, rounded to the
// nearest e4m3 code.
template <int KV>
__device__ __forceinline__ void store_new_row(const NewRow& r, void* k_cache, void* v_cache, int slot, int h, int H,
                                              int D, int BS, float ksc, float vsc) {
  constexpr int IN_ES = (KV == KV_F32) ? 4 : (KV == KV_FP8_RAW ? 1 : 2);
  constexpr int OUT_ES = (KV == KV_F32) ? 4 : (KV == KV_BF16 ? 2 : 1);
  constexpr int EPC = 16 / IN_ES;
  const int lane = threadIdx.x & 63;
  const int cpr = D / EPC;
  const int vpl = D / 64;                                  // value elements per lane (1 or 2)
  if (slot < 0) return;
  const int blk = slot / BS, off = slot % BS;
  char* kdst = static_cast<char*>(k_cache) + ((size_t(blk) * H + h) * BS + off) * size_t(D) * OUT_ES;
  char* vdst = static_cast<char*>(v_cache) + (size_t(blk) * H + h) * size_t(D) * BS * OUT_ES + size_t(off) * OUT_ES;
  if (lane < cpr) {
    if constexpr (KV != KV_FP8) {
      *reinterpret_cast<uint4*>(kdst + size_t(lane) * 16) = r.kx;
    } else {
      const uint32_t w[4] = {r.kx.x, r.kx.y, r.kx.z, r.kx.w};
      uint32_t lo = 0, hi = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t c0 = e4m3_encode(bf16_lo(w[e]) / ksc);
        const uint32_t c1 = e4m3_encode(bf16_hi(w[e]) / ksc);
        const uint32_t two = c0 | (c1 << 8);
        if (e < 2) lo |= two << (16 * e); else hi |= two << (16 * (e - 2));
      }
      *reinterpret_cast<uint2*>(kdst + size_t(lane) * 8) = make_uint2(lo, hi);
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    if (i >= vpl) break;
    const int d = lane + 64 * i;
    char* p = vdst + size_t(d) * BS * OUT_ES;
    if constexpr (OUT_ES == 4) *reinterpret_cast<uint32_t*>(p) = r.vx[i];
    else if constexpr (OUT_ES == 2) *reinterpret_cast<uint16_t*>(p) = uint16_t(r.vx[i]);
    else if constexpr (KV == KV_FP8_RAW) *p = char(r.vx[i]);
    else *p = char(e4m3_encode(bf16_lo(r.vx[i]) / vsc));
  }
}

// Both in one: every load of the wave is issued before any store, so the wave
// pays one memory round trip.
template <int KV>
__device__ __forceinline__ void store_row(const char* krow, const char* vrow, void* k_cache, void* v_cache,
                                          int slot, int h, int H, int D, int BS, float ksc, float vsc) {
  store_new_row<KV>(load_new_row<KV>(krow, vrow, D), k_cache, v_cache, slot, h, H, D, BS, ksc, vsc);
}

}  // namespace pa
