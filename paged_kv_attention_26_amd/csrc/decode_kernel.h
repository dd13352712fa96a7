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
//  * Work is cut into units = (sequence, kv head, partition of part_tokens
//    tokens), ordered sequence-major.  Every wavefront takes an equal,
//    contiguous range of units (a static split of the whole batch, so ragged
//    lengths cannot unbalance the waves), and runs its online softmax across
//    consecutive partitions of one (sequence, kv head).  One wave serves the
//    G query heads of a kv head, so they share every byte of K and V read.
//  * A (sequence, kv head) whose units all fall in one wave's range is
//    written out directly.  Otherwise each wave that touched it writes a
//    partial (max, sum, acc) -- at most two per wave, for the first and the
//    last item of its range -- and a small reduce kernel merges them by
//    log-sum-exp rescaling.
//  * Block ids are fetched one 64-token step ahead of their use; every K/V
//    load is a raw buffer load of one (block, kv head) tile (a descriptor,
//    one lane offset, immediate offsets), 16 bytes per lane (8 for fp8).
//  * Loads are software-pipelined: the next step's K tile is issued right
//    after this step's scores, its V tile right after this step's PV, so a
//    wave keeps one step of K and V in flight while it computes.
//  * QK^T: a key row is spread over LPR lanes; each lane forms partial dot
//    products for the G heads with v_dot2_f32_bf16 (fp32 FMA for fp32
//    caches).  The G partials are reduced by a transpose-reduce inside
//    groups of G lanes (lane c holds head j ^ gray(c) in register j, so each
//    DPP step halves the registers without selects), then a plain DPP
//    all-reduce over the remaining lanes of the row.
//  * Softmax: raw scores go to LDS and are read back one token per lane; the
//    running max / sum per head are updated once per step (wave64 DPP
//    reductions), the positive scale applied inside exp2.  Probabilities go
//    to LDS as bf16.
//  * PV: V is stored transposed per block, so a 16-byte load holds 8
//    consecutive tokens of one head dimension; v_dot2_f32_bf16 with the bf16
//    probabilities accumulates in fp32 with no cross-lane reduction until
//    the end of the segment.
#pragma once

#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

#ifndef PA_DECODE_STEP_TOKENS
#define PA_DECODE_STEP_TOKENS 64
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
  // tokens per step: the configured step rounded up to whole blocks (<= 64)
  static constexpr int CH = ((PA_DECODE_STEP_TOKENS + B - 1) / B) * B;
  static constexpr int BPC = CH / B;                              // blocks per step
  using LoadT = typename std::conditional<LBYTES == 16, uint4, uint2>::type;
  static_assert(LPR >= G && LPR <= 64 && (64 % LPR) == 0, "key row mapping");
  static_assert(LPD >= 1 && LPD <= 64, "value row mapping");
  static_assert(D % DPL == 0 && B % RPL == 0, "tile mapping");
  static_assert(CH <= 64, "a step is at most one token per lane");
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

// Partitions of a sequence of L tokens (an empty sequence still owns one,
// which writes its zero output).
__device__ __forceinline__ int units_of(int L, int PT) { return max(1, (max(0, L) + PT - 1) / PT); }

// The wave whose range holds unit u when U units are split over W waves,
// wave w owning [floor(w U / W), floor((w + 1) U / W)).
__device__ __forceinline__ int owner_wave(int64_t u, int64_t U, int64_t W) {
  return int(((u + 1) * W + U - 1) / U - 1);
}

// Exclusive prefix of the partitions per sequence, built in LDS by the
// whole workgroup: s_prefix[s] = sum over s' < s, s_prefix[S] = total.
__device__ __forceinline__ void build_prefix(const int32_t* lens, int S, int PT, int* s_prefix, int* s_tmp) {
  const int tid = threadIdx.x;
  const int per = (S + 255) / 256;
  const int i0 = tid * per, i1 = min(S, i0 + per);
  int local = 0;
  for (int i = i0; i < i1; ++i) local += units_of(lens[i], PT);
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
    run += units_of(lens[i], PT);
  }
  if (tid == 255) s_prefix[S] = s_tmp[255];
  __syncthreads();
}

// Largest s with s_prefix[s] <= key (s_prefix strictly increasing, s_prefix[0] == 0).
__device__ __forceinline__ int find_seq(const int* s_prefix, int S, int key) {
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_prefix[mid] <= key) lo = mid; else hi = mid;
  }
  return uniform(lo);
}

// block_table and context_lens are separate restrict arguments so that the
// compiler may read them through the scalar cache (s_load) even though the
// kernel stores results: block ids then never wait behind in-flight tiles.
template <int KV, int D, int B, int G>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a, const int32_t* __restrict__ block_table,
                                                     const int32_t* __restrict__ context_lens) {
  using C = DecCfg<KV, D, B, G>;
  using LoadT = typename C::LoadT;
  extern __shared__ int s_prefix[];                       // [num_seqs + 1]
  __shared__ int s_tmp[256];
  __shared__ float s_score[4][C::CH * G];                 // [token][head] per wave
  __shared__ __attribute__((aligned(16))) uint32_t s_p[4][C::CH * G];   // probabilities per wave

  const int S = a.num_seqs;
  const int PT = a.part_tokens;
  build_prefix(context_lens, S, PT, s_prefix, s_tmp);

  const int lane = threadIdx.x & 63;
  const int w = uniform(threadIdx.x >> 6);                // wave-uniform, so all range math stays scalar
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const int64_t U = int64_t(s_prefix[S]) * Hkv;
  const int64_t W = min<int64_t>(a.total_waves, U);       // every range non-empty (see the reduce)
  const int wid = blockIdx.x * 4 + w;
  if (wid >= W) return;                                    // no work (no barrier follows)
  int64_t u = int64_t(wid) * U / W;
  const int64_t u_end = int64_t(wid + 1) * U / W;

  const int kr = lane / C::LPR, kcol = lane % C::LPR;     // key row within a load, element chunk
  const int gsub = kcol % G;
  const int gray = gsub ^ (gsub >> 1);                    // head held in register 0 after the reduce
  const int vs = lane % C::LPD, vd = lane / C::LPD;       // value token segment, head-dim row
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  constexpr uint64_t kTile = uint64_t(B) * D * C::ES;     // bytes of one (block, kv head) tile
  const uint32_t k_off = uint32_t((kr * D + kcol * C::EPL) * C::ES);
  const uint32_t v_off = uint32_t((vd * B + vs * C::TPL) * C::ES);

  // first unit of the range -> (sequence, kv head, partition)
  int seq = find_seq(s_prefix, S, int(u / Hkv));
  int kvh, part;
  {
    const int nu = units_of(context_lens[seq], PT);
    const int r = int(u - int64_t(s_prefix[seq]) * Hkv);
    kvh = uniform(r / nu);
    part = uniform(r - kvh * nu);
  }
  bool first = true;

  for (;;) {                                               // one (sequence, kv head) segment per pass
    const int L = max(0, context_lens[seq]);
    const int nu = units_of(L, PT);
    const int p_end = int(min<int64_t>(nu, part + (u_end - u)));
    const bool whole = part == 0 && p_end == nu;
    const int t_begin = part * PT;
    const int t_end = min(L, p_end * PT);
    const int last_blk = max((t_end + B - 1) / B - 1, 0);  // absolute index of the segment's last block
    const int blk0 = t_begin / B;
    const int32_t* trow = block_table + size_t(seq) * a.max_blocks_per_seq;
    const int nsteps = (t_end - t_begin + C::CH - 1) / C::CH;

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

    // block ids of a step (blocks past the segment re-read its last block;
    // everything past t_end is masked)
    auto step_ids = [&](int step, int (&ids)[C::BPC]) {
#pragma unroll
      for (int k = 0; k < C::BPC; ++k) ids[k] = uniform(trow[min(blk0 + step * C::BPC + k, last_blk)]);
    };
    LoadT kreg[C::BPC][C::KLB];
    LoadT vreg[C::BPC][C::VLB];
    auto load_k = [&](const int (&ids)[C::BPC]) {
#pragma unroll
      for (int k = 0; k < C::BPC; ++k) {
        const auto r = tile_rsrc(kpool + (uint64_t(uint32_t(ids[k])) * uint32_t(Hkv) + uint32_t(kvh)) * kTile,
                                 uint32_t(kTile));
#pragma unroll
        for (int i = 0; i < C::KLB; ++i) buffer_load(r, k_off, uint32_t(i * C::RPL * D * C::ES), kreg[k][i]);
      }
    };
    auto load_v = [&](const int (&ids)[C::BPC]) {
#pragma unroll
      for (int k = 0; k < C::BPC; ++k) {
        const auto r = tile_rsrc(vpool + (uint64_t(uint32_t(ids[k])) * uint32_t(Hkv) + uint32_t(kvh)) * kTile,
                                 uint32_t(kTile));
#pragma unroll
        for (int j = 0; j < C::VLB; ++j) buffer_load(r, v_off, uint32_t(j * C::DPL * B * C::ES), vreg[k][j]);
      }
    };

    int ids_cur[C::BPC], ids_nxt[C::BPC];
    if (nsteps > 0) {                                        // an empty sequence reads nothing
    step_ids(0, ids_cur);
    step_ids(min(1, max(nsteps - 1, 0)), ids_nxt);
    // The query and the first block ids must be in registers before the
    // first tile is requested; an explicit wait here keeps the compiler
    // from waiting on every in-flight tile (vmcnt(0)) at each step.
    __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0) only
    // Loads are unconditional so that the compiler counts them exactly
    // (vmcnt(n) rather than vmcnt(0) at every use); a prefetch past the
    // last step re-reads that step.
    __builtin_amdgcn_sched_barrier(0);
    load_k(ids_cur);                                          // keys before values, as in the loop
    __builtin_amdgcn_sched_barrier(0);
    load_v(ids_cur);
    __builtin_amdgcn_sched_barrier(0);
    for (int st = 0; st < nsteps; ++st) {
      const int cs = t_begin + st * C::CH;

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
          // every lane writes; the lanes of one (token, head) hold the same sum
          s_score[w][(k * B + i * C::RPL + kr) * G + gray] = sc;
        }
      }
      // The scheduler must not move loads across these phase boundaries: the
      // next step's K tile goes out after the scores and its V tile after
      // the PV, which is what lets each use wait for half the loads in flight.
      __builtin_amdgcn_sched_barrier(0);
      load_k(ids_nxt);                                        // next step's keys fly during softmax + PV
      __builtin_amdgcn_sched_barrier(0);
      wave_lds_sync();

      // ---- online softmax over this step, one token per lane
      const bool valid = lane < C::CH && cs + lane < t_end;
      float pv[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        // raw scores; the positive scale sl (log2 units) is applied inside exp2
        const float sv = valid ? s_score[w][min(lane, C::CH - 1) * G + g] : -INFINITY;
        const float mn = fmaxf(m_run[g], wave_max(sv));
        const float al = exp2f((m_run[g] - mn) * sl);
        pv[g] = exp2f(fmaf(sv, sl, -mn * sl));
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
        const int tok0 = k * B + vs * C::TPL;                // step-relative first token of this lane's segment
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
      __builtin_amdgcn_sched_barrier(0);
      load_v(ids_nxt);                                        // next step's values fly during its scores
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int k = 0; k < C::BPC; ++k) ids_cur[k] = ids_nxt[k];
      step_ids(min(st + 2, max(nsteps - 1, 0)), ids_nxt);     // ids one step ahead of their loads
    }
    }

    // ---- finish the segment
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

    if (whole) {
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
      // split (sequence, kv head): slot 0 holds the range's first item, slot 1 its last
      const size_t base = (size_t(wid) * 2 + (first ? 0 : 1)) * G;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (lane == 0) {
          a.part_ml[2 * (base + g)] = m_run[g] * sl;        // log2 units
          a.part_ml[2 * (base + g) + 1] = l[g];
        }
        if (vs == 0) {
#pragma unroll
          for (int j = 0; j < C::VLB; ++j) a.part_acc[(base + g) * D + j * C::DPL + vd] = acc[g][j];
        }
      }
    }

    u += p_end - part;
    if (u >= u_end) break;
    first = false;
    part = 0;
    if (++kvh == Hkv) {
      kvh = 0;
      ++seq;
    }
  }
}

// Merge of split (sequence, kv head) items: one wave per (sequence, query
// head) finds the waves whose ranges cut through its item and combines their
// partials, out = sum_w e^(m_w - M) acc_w / sum_w e^(m_w - M) l_w.
template <int D, int G, bool F32OUT>
__global__ void __launch_bounds__(256) decode_reduce_kernel(DecodeArgs a) {
  extern __shared__ int s_prefix[];
  __shared__ int s_tmp[256];
  const int S = a.num_seqs, PT = a.part_tokens;
  build_prefix(a.context_lens, S, PT, s_prefix, s_tmp);
  const int lane = threadIdx.x & 63;
  const int pair = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int Hq = a.num_q_heads, Hkv = a.num_kv_heads;
  if (pair >= S * Hq) return;
  const int seq = pair / Hq, head = pair - seq * Hq;
  const int kvh = head / G, g = head - kvh * G;
  const int64_t U = int64_t(s_prefix[S]) * Hkv;
  // As in the partition kernel: with at most U waves no range is empty, so
  // every wave from w0 to w1 holds a partial of this item.
  const int64_t W = min<int64_t>(a.total_waves, U);
  const int nu = units_of(a.context_lens[seq], PT);
  const int64_t u0 = int64_t(s_prefix[seq]) * Hkv + int64_t(kvh) * nu;
  const int w0 = owner_wave(u0, U, W);
  const int w1 = owner_wave(u0 + nu - 1, U, W);
  if (w0 == w1) return;                                    // written by the partition kernel
  const bool w0_starts_here = int64_t(w0) * U / W == u0;   // then the item is w0's first
  const int n = w1 - w0 + 1;
  auto slot_base = [&](int i) -> size_t {                  // partial of the i-th wave over the item
    const int wv = w0 + i;
    const int slot = (i > 0 || w0_starts_here) ? 0 : 1;
    return (size_t(wv) * 2 + slot) * G + g;
  };
  float M = -INFINITY;
  for (int p0 = 0; p0 < n; p0 += 64) {
    const int p = p0 + lane;
    const float mp = p < n ? a.part_ml[2 * slot_base(p)] : -INFINITY;
    M = fmaxf(M, wave_max(mp));
  }
  float Ls = 0.f;
  float o[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) o[i] = 0.f;
  for (int p0 = 0; p0 < n; p0 += 64) {
    const int p = p0 + lane;
    const float wp = p < n ? exp2f(a.part_ml[2 * slot_base(p)] - M) : 0.f;
    const float lp = p < n ? a.part_ml[2 * slot_base(p) + 1] : 0.f;
    Ls += wave_sum(wp * lp);
    const int cnt = min(64, n - p0);
    for (int q = 0; q < cnt; ++q) {
      const float wq = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wp), q));
      const float* src = a.part_acc + slot_base(p0 + q) * D;
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
hipError_t launch_decode_t(const DecodeArgs& a0, int64_t upper_units, hipStream_t s) {
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
  int64_t wgs = int64_t(cached_occ) * cus;                  // every resident wave gets a range
  if (wgs * 4 > kDecodeMaxWaves) wgs = kDecodeMaxWaves / 4;
  const int64_t need = (upper_units + 3) / 4;
  if (need < wgs) wgs = need;
  if (wgs < 1) wgs = 1;
  DecodeArgs a = a0;
  a.total_waves = int32_t(wgs * 4);
  hipLaunchKernelGGL(kern, dim3(uint32_t(wgs)), dim3(256), lds, s, a, a.block_table, a.context_lens);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t pairs = int64_t(a.num_seqs) * a.num_q_heads;
  hipLaunchKernelGGL((decode_reduce_kernel<D, G, KV == KV_F32>), dim3(uint32_t((pairs + 3) / 4)), dim3(256), lds, s,
                     a);
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
