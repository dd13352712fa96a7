// Paged decode attention for gfx950: one query token per sequence, grouped
// query heads, keys and values read through the block table.
//
// What it computes (nanoPD page: hand-written gather-scatter attention over
// non-contiguous KV blocks; serving-stack page 2.2: one block-table lookup
// per KV read; PD-engineering page 6.2: 8 KV heads shared by 32 query
// heads): out[s][h] = sum_i softmax_i(scale <q[s][h], k_i>) v_i over the
// context of sequence s.
//
// How (a bandwidth kernel; the pages' CUDA design is not available and is
// not followed):
//  * Work items are (sequence, kv head, partition of part_tokens tokens);
//    one wavefront owns one item, so the G query heads of a kv head share
//    every byte of K and V that the item reads.  Waves are persistent and
//    take items from an atomic queue, which balances ragged lengths.
//  * The partition's block ids are loaded once into a VGPR and broadcast
//    with readlane; every K/V load is a coalesced 16-byte (8-byte for fp8)
//    per-lane load of a whole block tile, issued for a 64-token step before
//    any arithmetic on it.
//  * QK^T: a key row is spread over LPR lanes; each lane forms partial dot
//    products for the G heads with v_dot2_f32_bf16 (fp32 FMA for fp32
//    caches).  The G partials are reduced by a transpose-reduce inside
//    groups of G lanes (lane c holds head j ^ gray(c) in register j, so each
//    DPP step halves the registers without selects), then a plain DPP
//    all-reduce over the remaining lanes of the row.
//  * Softmax: scores go to LDS, are read back one token per lane, and the
//    running max / sum per head are updated once per 64-token step
//    (wave64 DPP reductions).  Probabilities are written to LDS as bf16.
//  * PV: V is stored transposed per block, so a 16-byte load holds 8
//    consecutive tokens of one head dimension; v_dot2_f32_bf16 with the bf16
//    probabilities accumulates in fp32 with no cross-lane reduction until
//    the end of the item.
//  * Loads are software-pipelined: the next step's K tile is issued right
//    after this step's scores, its V tile right after this step's PV, so a
//    wave always has one tile in flight while it computes.
//  * Split-K: an item of a multi-partition sequence writes (max, sum, acc)
//    to the workspace and a small reduce kernel merges the partitions by
//    log-sum-exp rescaling (the kernel boundary orders the two, which costs
//    less than a device-scope fence per item).  The queue counters reset
//    themselves, so the workspace needs zero-filling only once.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_DECODE_STEP_TOKENS
#define PA_DECODE_STEP_TOKENS 64
#endif
#ifndef PA_DECODE_WAVES_ATTR
#define PA_DECODE_WAVES_ATTR
#endif

namespace pa {

template <int KV, int D, int B, int G>
struct DecCfg {
  static constexpr bool F32 = KV == KV_F32;
  static constexpr int ES = F32 ? 4 : (KV == KV_BF16 ? 2 : 1);   // cache element bytes
  static constexpr int EPL = F32 ? 4 : 8;                         // key elements per lane load
  static constexpr int LBYTES = EPL * ES;                         // 16 (f32, bf16) or 8 (fp8)
  static constexpr int LPR = D / EPL;                             // lanes per key row
  static constexpr int RPL = 64 / LPR;                            // key rows per load
  static constexpr int TPL = F32 ? 4 : 8;                         // value tokens per lane load
  static constexpr int LPD = B / TPL;                             // lanes per transposed value row
  static constexpr int DPL = 64 / LPD;                            // head dims per value load
  static constexpr int KLB = B / RPL;                             // key loads per block
  static constexpr int VLB = D / DPL;                             // value loads per block
  static constexpr int CH = PA_DECODE_STEP_TOKENS > B ? PA_DECODE_STEP_TOKENS : B;   // tokens per step (<= 64)
  static constexpr int BPC = CH / B;                              // blocks per step
  using LoadT = typename std::conditional<LBYTES == 16, uint4, uint2>::type;
  static_assert(LPR >= G && LPR <= 64 && (64 % LPR) == 0, "key row mapping");
  static_assert(LPD >= 1 && LPD <= 64, "value row mapping");
  static_assert(D % DPL == 0 && B % RPL == 0, "tile mapping");
  static_assert(CH <= 64 && CH % B == 0, "a step is at most one token per lane");
};

template <int KV>
__device__ __forceinline__ void load_pairs(const uint4& x, uint32_t p[4]) {
  p[0] = x.x; p[1] = x.y; p[2] = x.z; p[3] = x.w;
}
template <int KV>
__device__ __forceinline__ void load_pairs(const uint2& x, uint32_t p[4]) {
  fp8x4_to_bf16x4(x.x, p[0], p[1]);
  fp8x4_to_bf16x4(x.y, p[2], p[3]);
}

template <int KV, int D, int B, int G>
__global__ void __launch_bounds__(256) PA_DECODE_WAVES_ATTR decode_kernel(DecodeArgs a) {
  using C = DecCfg<KV, D, B, G>;
  using LoadT = typename C::LoadT;
  extern __shared__ int s_prefix[];                       // [num_seqs + 1] partitions before each sequence
  __shared__ int s_tmp[256];
  __shared__ float s_score[4][C::CH * G];                 // [token][head] per wave
  __shared__ __attribute__((aligned(16))) uint32_t s_p[4][C::CH * G];   // probabilities per wave

  const int tid = threadIdx.x;
  const int S = a.num_seqs;
  const int PT = a.part_tokens;

  // ---- partitions per sequence -> exclusive prefix in LDS
  {
    const int per = (S + 255) / 256;
    const int i0 = tid * per, i1 = min(S, i0 + per);
    int local = 0;
    for (int i = i0; i < i1; ++i) local += max(1, (max(0, a.context_lens[i]) + PT - 1) / PT);
    s_tmp[tid] = local;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = tid >= off ? s_tmp[tid - off] : 0;
      __syncthreads();
      s_tmp[tid] += v;
      __syncthreads();
    }
    int run = tid ? s_tmp[tid - 1] : 0;
    for (int i = i0; i < i1; ++i) {
      s_prefix[i] = run;
      run += max(1, (max(0, a.context_lens[i]) + PT - 1) / PT);
    }
    if (tid == 255) s_prefix[S] = s_tmp[255];
    __syncthreads();
  }

  const int lane = tid & 63;
  const int w = tid >> 6;
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const int total_items = s_prefix[S] * Hkv;
  const int kr = lane / C::LPR, kcol = lane % C::LPR;     // key row within a load, element chunk
  const int gsub = kcol % G;
  const int gray = gsub ^ (gsub >> 1);                    // head held in register 0 after the reduce
  const int vs = lane % C::LPD, vd = lane / C::LPD;       // value token segment, head-dim row
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  constexpr uint64_t kTile = uint64_t(B) * D * C::ES;     // bytes of one (block, kv head) tile
  const uint32_t k_off = uint32_t((kr * D + kcol * C::EPL) * C::ES);
  const uint32_t v_off = uint32_t((vd * B + vs * C::TPL) * C::ES);

  int next = 0;
  if (lane == 0) next = atomicAdd(&a.counters[0], 1);
  for (;;) {
    const int item = __builtin_amdgcn_readlane(next, 0);
    if (item >= total_items) break;
    if (lane == 0) next = atomicAdd(&a.counters[0], 1);      // fetch the following item early
    const int gp = item / Hkv;
    const int kvh = item - gp * Hkv;
    int lo = 0, hi = S;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_prefix[mid] <= gp) lo = mid; else hi = mid;
    }
    const int seq = uniform(lo);
    const int part = uniform(gp - s_prefix[seq]);

    const int L = max(0, a.context_lens[seq]);
    const int np = max(1, (L + PT - 1) / PT);
    const int t_begin = part * PT;
    const int t_end = min(L, t_begin + PT);
    const int nblk = max(0, (t_end - t_begin + B - 1) / B);
    int tbl = 0;
    if (lane < nblk) tbl = a.block_table[size_t(seq) * a.max_blocks_per_seq + t_begin / B + lane];

    float sl = a.scale_log2;
    if constexpr (KV == KV_FP8) sl *= a.k_scale[kvh];

    // query of the G heads; register j holds head j ^ gray
    float qf[C::F32 ? G : 1][4];
    uint32_t qp[C::F32 ? 1 : G][4];
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int head = kvh * G + (j ^ gray);
      if constexpr (C::F32) {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(a.q) +
                                                          (size_t(seq) * Hq + head) * D + kcol * 4);
        qf[j][0] = v.x; qf[j][1] = v.y; qf[j][2] = v.z; qf[j][3] = v.w;
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                        (size_t(seq) * Hq + head) * D + kcol * 8);
        qp[j][0] = v.x; qp[j][1] = v.y; qp[j][2] = v.z; qp[j][3] = v.w;
      }
    }

    float m_run[G], l_lane[G], acc[G][C::VLB];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m_run[g] = -INFINITY;
      l_lane[g] = 0.f;
#pragma unroll
      for (int j = 0; j < C::VLB; ++j) acc[g][j] = 0.f;
    }

    // Loads are unconditional so that the compiler can count them exactly
    // (s_waitcnt vmcnt(n) instead of vmcnt(0) at every use): blocks past
    // the end of the partition re-read its last block, the prefetch of the
    // last step re-reads that step, and everything past t_end is masked.
    LoadT kreg[C::BPC][C::KLB];
    LoadT vreg[C::BPC][C::VLB];
    const int last_blk = max(nblk - 1, 0);
    const int nsteps = (t_end - t_begin + C::CH - 1) / C::CH;
    // uniform tile base (SGPRs) + one 32-bit lane offset + immediate offsets
    auto load_k = [&](int step) {
#pragma unroll
      for (int k = 0; k < C::BPC; ++k) {
        const uint32_t blk = uint32_t(__builtin_amdgcn_readlane(tbl, min(step * C::BPC + k, last_blk)));
        const auto r = tile_rsrc(kpool + (uint64_t(blk) * uint32_t(Hkv) + uint32_t(kvh)) * kTile, uint32_t(kTile));
#pragma unroll
        for (int i = 0; i < C::KLB; ++i) buffer_load(r, k_off + uint32_t(i * C::RPL * D * C::ES), kreg[k][i]);
      }
    };
    auto load_v = [&](int step) {
#pragma unroll
      for (int k = 0; k < C::BPC; ++k) {
        const uint32_t blk = uint32_t(__builtin_amdgcn_readlane(tbl, min(step * C::BPC + k, last_blk)));
        const auto r = tile_rsrc(vpool + (uint64_t(blk) * uint32_t(Hkv) + uint32_t(kvh)) * kTile, uint32_t(kTile));
#pragma unroll
        for (int j = 0; j < C::VLB; ++j) buffer_load(r, v_off + uint32_t(j * C::DPL * B * C::ES), vreg[k][j]);
      }
    };

    // Block ids and the query must be in registers before the first tile is
    // requested; an explicit wait here keeps the compiler from waiting on
    // every in-flight tile (vmcnt(0)) at the top of each step.
    __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0) only
    load_k(0);                                                // (re-reads block 0 when the item is empty)
    load_v(0);
    for (int st = 0; st < nsteps; ++st) {
      const int cs = t_begin + st * C::CH;
      const int nxt = min(st + 1, nsteps - 1);

      // ---- scores (tokens past t_end are masked in the softmax)
#pragma unroll
      for (int k = 0; k < C::BPC; ++k) {
#pragma unroll
        for (int i = 0; i < C::KLB; ++i) {
          float pt[G];
          if constexpr (C::F32) {
            const uint4 x = kreg[k][i];
            const float kf[4] = {__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z),
                                 __uint_as_float(x.w)};
#pragma unroll
            for (int j = 0; j < G; ++j)
              pt[j] = fmaf(kf[3], qf[j][3], fmaf(kf[2], qf[j][2], fmaf(kf[1], qf[j][1], kf[0] * qf[j][0])));
          } else {
            uint32_t kp[4];
            load_pairs<KV>(kreg[k][i], kp);
#pragma unroll
            for (int j = 0; j < G; ++j)
              pt[j] = dot2_bf16(kp[3], qp[j][3],
                                dot2_bf16(kp[2], qp[j][2], dot2_bf16(kp[1], qp[j][1], dot2_bf16(kp[0], qp[j][0], 0.f))));
          }
          if constexpr (G >= 8) {
#pragma unroll
            for (int x = 0; x < 4; ++x) pt[x] += dpp<DPP_HALF_MIRROR>(pt[x + 4]);
          }
          if constexpr (G >= 4) {
#pragma unroll
            for (int x = 0; x < 2; ++x) pt[x] += dpp<DPP_QP_XOR3>(pt[x + 2]);
          }
          if constexpr (G >= 2) pt[0] += dpp<DPP_QP_XOR1>(pt[1]);
          float sc = pt[0];
#pragma unroll
          for (int sp = G; sp < C::LPR; sp *= 2) {
            if constexpr (C::LPR == 16) {
              if (sp == 1) sc += dpp<DPP_ROW_ROR(1)>(sc);
              else if (sp == 2) sc += dpp<DPP_ROW_ROR(2)>(sc);
              else if (sp == 4) sc += dpp<DPP_ROW_ROR(4)>(sc);
              else sc += dpp<DPP_ROW_ROR(8)>(sc);
            } else {
              sc += __shfl_xor(sc, sp);
            }
          }
          if (kcol < G) s_score[w][(k * B + i * C::RPL + kr) * G + gray] = sc * sl;
        }
      }
      load_k(nxt);                                            // next step's keys fly during softmax + PV
      wave_lds_sync();

      // ---- online softmax over this step, one token per lane
      const bool valid = lane < C::CH && cs + lane < t_end;
      float pv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float sv = valid ? s_score[w][min(lane, C::CH - 1) * G + g] : -INFINITY;
        const float mn = fmaxf(m_run[g], wave_max(sv));
        const float al = exp2f(m_run[g] - mn);
        pv[g] = exp2f(sv - mn);
        l_lane[g] = fmaf(l_lane[g], al, pv[g]);
#pragma unroll
        for (int j = 0; j < C::VLB; ++j) acc[g][j] *= al;
        m_run[g] = mn;
      }
      if (lane < C::CH) {
        if constexpr (C::F32) {
#pragma unroll
          for (int g = 0; g < G; ++g) reinterpret_cast<float*>(s_p[w])[g * C::CH + lane] = pv[g];
        } else {
#pragma unroll
          for (int g = 0; g < G; ++g)
            reinterpret_cast<uint16_t*>(s_p[w])[g * C::CH + lane] = uint16_t(pack_bf16x2(pv[g], 0.f) & 0xFFFFu);
        }
      }
      wave_lds_sync();

      // ---- PV (values of tokens past t_end may be NaN poison: zeroed by select)
#pragma unroll
      for (int k = 0; k < C::BPC; ++k) {
        const int tok0 = k * B + vs * C::TPL;              // step-relative first token of this lane's segment
        const bool tail = cs + k * B + B > t_end;           // block holds tokens past the end
        if constexpr (C::F32) {
          float pf[G][4];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const float4 t = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(s_p[w]) + g * C::CH + tok0);
            pf[g][0] = t.x; pf[g][1] = t.y; pf[g][2] = t.z; pf[g][3] = t.w;
          }
#pragma unroll
          for (int j = 0; j < C::VLB; ++j) {
            const uint4 x = vreg[k][j];
            float v[4] = {__uint_as_float(x.x), __uint_as_float(x.y), __uint_as_float(x.z), __uint_as_float(x.w)};
            if (tail) {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = (cs + tok0 + e < t_end) ? v[e] : 0.f;
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
              acc[g][j] = fmaf(v[3], pf[g][3], fmaf(v[2], pf[g][2], fmaf(v[1], pf[g][1], fmaf(v[0], pf[g][0], acc[g][j]))));
          }
        } else {
          uint32_t pp[G][4];
#pragma unroll
          for (int g = 0; g < G; ++g) {
            const uint4 t = *reinterpret_cast<const uint4*>(reinterpret_cast<const uint16_t*>(s_p[w]) + g * C::CH + tok0);
            pp[g][0] = t.x; pp[g][1] = t.y; pp[g][2] = t.z; pp[g][3] = t.w;
          }
#pragma unroll
          for (int j = 0; j < C::VLB; ++j) {
            uint32_t vp[4];
            load_pairs<KV>(vreg[k][j], vp);
            if (tail) {
#pragma unroll
              for (int m = 0; m < 4; ++m) {
                const int t = cs + tok0 + 2 * m;
                vp[m] &= (t < t_end ? 0x0000FFFFu : 0u) | (t + 1 < t_end ? 0xFFFF0000u : 0u);
              }
            }
#pragma unroll
            for (int g = 0; g < G; ++g)
              acc[g][j] = dot2_bf16(vp[3], pp[g][3], dot2_bf16(vp[2], pp[g][2],
                          dot2_bf16(vp[1], pp[g][1], dot2_bf16(vp[0], pp[g][0], acc[g][j]))));
          }
        }
      }
      load_v(nxt);                                            // next step's values fly during its scores
    }

    // ---- finish the item
    float l[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      l[g] = wave_sum(l_lane[g]);
#pragma unroll
      for (int j = 0; j < C::VLB; ++j) acc[g][j] = group_sum<C::LPD>(acc[g][j]);
    }
    if constexpr (KV == KV_FP8) {
      const float vsc = a.v_scale[kvh];
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int j = 0; j < C::VLB; ++j) acc[g][j] *= vsc;
    }

    if (np == 1) {
      if (vs == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
          const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
          const size_t o = (size_t(seq) * Hq + kvh * G + g) * D + vd;
#pragma unroll
          for (int j = 0; j < C::VLB; ++j) {
            const float r = acc[g][j] * inv;
            if constexpr (C::F32) static_cast<float*>(a.out)[o + j * C::DPL] = r;
            else static_cast<uint16_t*>(a.out)[o + j * C::DPL] = uint16_t(pack_bf16x2(r, 0.f) & 0xFFFFu);
          }
        }
      }
    } else {
      // multi-partition sequence: publish this partition for the reduce kernel
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const size_t base = (size_t(seq) * Hq + kvh * G + g) * a.max_parts + part;
        if (lane == 0) {
          a.part_ml[2 * base] = m_run[g];
          a.part_ml[2 * base + 1] = l[g];
        }
        if (vs == 0) {
#pragma unroll
          for (int j = 0; j < C::VLB; ++j) a.part_acc[base * D + j * C::DPL + vd] = acc[g][j];
        }
      }
    }
  }

  // ---- the last wave to leave resets the queue for the next call
  if (lane == 0) {
    const int left = atomicAdd(&a.counters[1], 1);
    if (left == a.total_waves - 1) {
      atomicExch(&a.counters[0], 0);
      atomicExch(&a.counters[1], 0);
    }
  }
}

// Merge of the partitions of multi-partition sequences: one wave per
// (sequence, query head); out = sum_p e^(m_p - M) acc_p / sum_p e^(m_p - M) l_p.
template <int D, bool F32OUT>
__global__ void __launch_bounds__(256) decode_reduce_kernel(DecodeArgs a) {
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int Hq = a.num_q_heads;
  if (pair >= a.num_seqs * Hq) return;
  const int seq = pair / Hq, head = pair - seq * Hq;
  const int L = max(0, a.context_lens[seq]);
  const int np = max(1, (L + a.part_tokens - 1) / a.part_tokens);
  if (np == 1) return;                                   // written by the partition kernel
  const size_t base = size_t(pair) * a.max_parts;
  float M = -INFINITY;
  for (int p0 = 0; p0 < np; p0 += 64) {
    const int p = p0 + lane;
    const float mp = p < np ? a.part_ml[2 * (base + p)] : -INFINITY;
    M = fmaxf(M, wave_max(mp));
  }
  float Ls = 0.f;
  float o[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) o[i] = 0.f;
  for (int p0 = 0; p0 < np; p0 += 64) {
    const int p = p0 + lane;
    const float wp = p < np ? exp2f(a.part_ml[2 * (base + p)] - M) : 0.f;
    const float lp = p < np ? a.part_ml[2 * (base + p) + 1] : 0.f;
    Ls += wave_sum(wp * lp);
    const int cnt = min(64, np - p0);
    for (int q = 0; q < cnt; ++q) {
      const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wp), q));
      const float* src = a.part_acc + (base + p0 + q) * D;
#pragma unroll
      for (int i = 0; i < D / 64; ++i) o[i] = fmaf(wq, src[lane + 64 * i], o[i]);
    }
  }
  const float inv = 1.f / Ls;
  const size_t ob = size_t(pair) * D;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) {
    const float r = o[i] * inv;
    if constexpr (F32OUT) static_cast<float*>(a.out)[ob + lane + 64 * i] = r;
    else static_cast<uint16_t*>(a.out)[ob + lane + 64 * i] = uint16_t(pack_bf16x2(r, 0.f) & 0xFFFFu);
  }
}

template <int KV, int D, int B, int G>
hipError_t launch_decode_t(const DecodeArgs& a0, int64_t upper_items, hipStream_t s) {
  auto kern = decode_kernel<KV, D, B, G>;
  const size_t lds = size_t(a0.num_seqs + 1) * sizeof(int);
  static int cached_occ = -1;
  static size_t cached_lds = 0;
  if (cached_occ < 0 || cached_lds != lds) {
    int occ = 0;
    hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, 256, lds);
    if (e != hipSuccess) return e;
    cached_occ = occ > 0 ? occ : 1;
    cached_lds = lds;
  }
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  int64_t wgs = int64_t(cached_occ) * cus;
  const int64_t need = (upper_items + 3) / 4;
  if (need < wgs) wgs = need;
  if (wgs < 1) wgs = 1;
  DecodeArgs a = a0;
  a.total_waves = int32_t(wgs * 4);
  hipLaunchKernelGGL(kern, dim3(uint32_t(wgs)), dim3(256), lds, s, a);
  e = hipGetLastError();
  if (e != hipSuccess || a.max_parts <= 1) return e;
  const int64_t pairs = int64_t(a.num_seqs) * a.num_q_heads;
  hipLaunchKernelGGL((decode_reduce_kernel<D, KV == KV_F32>), dim3(uint32_t((pairs + 3) / 4)), dim3(256), 0, s, a);
  return hipGetLastError();
}

// Dispatch over the compiled (head_dim, block_size, group) set for one cache dtype.
template <int KV>
hipError_t launch_decode_kv(const DecodeArgs& a, int D, int B, int G, int64_t upper, hipStream_t s) {
#define PA_DEC_CASE(d, b, g) \
  if (D == d && B == b && G == g) return launch_decode_t<KV, d, b, g>(a, upper, s);
#define PA_DEC_G(d, b) PA_DEC_CASE(d, b, 1) PA_DEC_CASE(d, b, 2) PA_DEC_CASE(d, b, 4) PA_DEC_CASE(d, b, 8)
  PA_DEC_G(64, 16)
  PA_DEC_G(64, 32)
  PA_DEC_G(128, 16)
  PA_DEC_G(128, 32)
#undef PA_DEC_G
#undef PA_DEC_CASE
  return hipErrorInvalidValue;
}

}  // namespace pa
