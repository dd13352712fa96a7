// Device helpers shared by libpa's gfx950 kernels: element types, OCP e4m3
// encoding, DPP lane exchange, wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Two floats -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t f = {lo, hi};
  bf16x2_t b = __builtin_convertvector(f, bf16x2_t);
  return __builtin_bit_cast(uint32_t, b);
}

// Dot product of two packed bf16 pairs accumulated in fp32 (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c,
                                         false);
}

// Four e4m3fn codes (one dword) -> two packed bf16 pairs.  Every e4m3 value
// is exactly representable in bf16, so the conversion is exact.  gfx950
// converts a pair of codes straight to a bf16 pair (v_cvt_scalef32_pk_bf16_fp8,
// scale 1): two instructions per dword instead of two conversions to fp32
// and two packs, with the same bits for every code, NaN included.
__device__ __forceinline__ void fp8x4_to_bf16x4(uint32_t w, uint32_t& p01, uint32_t& p23) {
  p01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false));
  p23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true));
}

// OCP E4M3FN encoding of an fp32 value: round to nearest, ties to even;
// magnitudes of 448 and above (and infinities) saturate to 448; NaN -> 0x7F
// with the sign.  Written from the format's field definitions (bias 7,
// 3 mantissa bits, subnormal step 2^-9).
__device__ __forceinline__ uint32_t e4m3_encode(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return sign | 0x7Fu;       // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;      // >= 448.0f (incl. inf)
  const int e = int(a >> 23) - 127;               // unbiased fp32 exponent
  if (e >= -6) {                                  // normal e4m3 range
    const uint32_t mant = a & 0x7FFFFFu;
    uint32_t keep = mant >> 20;                   // top 3 mantissa bits
    const uint32_t rest = mant & 0xFFFFFu;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) keep += 1u;   // carry may bump the exponent
    return sign | ((uint32_t(e + 7) << 3) + keep);
  }
  // subnormal: value = m * 2^-9; x * 512 is exact, then round to an integer (ties to even)
  const float q = __uint_as_float(a) * 512.0f;
  return sign | uint32_t(__builtin_rintf(q));
}

// ---- DPP lane exchange (gfx9 encodings) --------------------------------
// quad_perm: lane i of each quad reads lane sel[i];  row_ror:n rotates a
// 16-lane row by n;  row_half_mirror reverses each 8-lane half row.
constexpr int DPP_QP_XOR1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int DPP_QP_XOR2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int DPP_QP_XOR3 = 0x1B;        // quad_perm [3,2,1,0]
constexpr int DPP_HALF_MIRROR = 0x141;   // lane i <-> 7 - i inside each 8 lanes
constexpr int DPP_ROW_ROR(int n) { return 0x120 + n; }

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Sum over aligned groups of N lanes (N in 2..64, power of two), result in
// every lane of the group.  Inside a 16-lane row DPP rotations are used.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp<DPP_QP_XOR1>(x);
  if constexpr (N >= 4) x += dpp<DPP_QP_XOR2>(x);
  if constexpr (N >= 8) x += dpp<DPP_HALF_MIRROR>(x);
  if constexpr (N >= 16) x += dpp<DPP_ROW_ROR(8)>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16);
  if constexpr (N >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Wave-uniform max / sum of one value per lane.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<DPP_ROW_ROR(1)>(x));
  x = fmaxf(x, dpp<DPP_ROW_ROR(2)>(x));
  x = fmaxf(x, dpp<DPP_ROW_ROR(4)>(x));
  x = fmaxf(x, dpp<DPP_ROW_ROR(8)>(x));
  float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

__device__ __forceinline__ float wave_sum(float x) {
  x += dpp<DPP_ROW_ROR(1)>(x);
  x += dpp<DPP_ROW_ROR(2)>(x);
  x += dpp<DPP_ROW_ROR(4)>(x);
  x += dpp<DPP_ROW_ROR(8)>(x);
  float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
  float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
  float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
  float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
  return (r0 + r1) + (r2 + r3);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---- buffer loads: a descriptor (SGPRs) covering one tile, a 32-bit lane
// offset and an immediate offset.  Reads past `bytes` return zero.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kBufferDword3 = 0x00020000;   // gfx9 family: 32-bit data format, untyped access

__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kBufferDword3);
}
// Cache policy of loads that stream data read once per launch: nt (the
// non-temporal hint).  The KV a decode reads is far larger than the caches
// and is not read again in the launch.  The hint only marks the lines as
// streaming; they are still looked up in the caches, so a line this wave
// has just stored is read back.  On the Qwen3-8B decode layer it cut the
// kernel from 64.7 to 59.1 us, on long context from 5.59 to 6.24 TB/s.
constexpr int kStreamLoad = 2;
// voff: the lane's offset (VGPR); soff: a wave-uniform constant offset,
// which the compiler folds into the instruction's immediate field.
__device__ __forceinline__ void buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint4& out) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamLoad);
  out = make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void buffer_load(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, uint2& out) {
  const u32x2_t v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamLoad);
  out = make_uint2(v.x, v.y);
}

// Order this wave's LDS writes before its following LDS reads by other lanes.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pa
