// Matrix-core pieces shared by the chunked-prefill and verify kernels: the
// bf16 32x32x16 MFMA and the key-row permutation that lets the accumulators
// of S^T = K Q^T serve directly as the P^T operand of O^T = V^T P^T.
#pragma once

#include <hip/hip_runtime.h>

#include "pa_device.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// D = A B + C with A 32x16 (lane l: row l % 32, k 8 (l / 32) .. + 7), B 16x32
// (lane l: k 8 (l / 32) .. + 7, column l % 32), C/D 32x32 (register 4i + j:
// row 8i + 4 (l / 32) + j, column l % 32).
__device__ __forceinline__ f32x16_t mfma32(const uint4& a, const uint4& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

// MFMA row m of a key tile holds key swap_bits_2_3(m) (an involution).  Then
// accumulator register 8ks + e of S^T (row 8(2ks + e / 4) + 4h + e % 4)
// holds key 16ks + 8h + e, which is exactly the B-operand layout of P^T for
// the 16-key slice ks.
__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Eight consecutive cache elements as the raw load (16 bytes of bf16 or 8
// bytes of e4m3 codes) and their bf16 form, the MFMA operand.  Every e4m3
// value is exactly a bf16 value, so the conversion is exact; the per-head
// scale is applied outside the contraction.
template <int KV>
struct KvRaw {
  using T = uint4;                                      // bf16
  static constexpr int ES = 2;
  __device__ static __forceinline__ uint4 to_bf16(const uint4& x) { return x; }
};
template <>
struct KvRaw<KV_FP8> {
  using T = uint2;
  static constexpr int ES = 1;
  __device__ static __forceinline__ uint4 to_bf16(const uint2& x) {
    uint4 r;
    fp8x4_to_bf16x4(x.x, r.x, r.y);
    fp8x4_to_bf16x4(x.y, r.z, r.w);
    return r;
  }
};

}  // namespace pa
