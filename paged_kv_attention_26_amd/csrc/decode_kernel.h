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
//    tokens), ordered sequence-major.  Every wave finds its range from the
//    prefix of the units over the sequences: built in each wave's own
//    registers for at most 64 sequences, in LDS by the workgroup beyond.  Every wavefront takes an equal,
//    contiguous range of units (a static split of the whole batch, so ragged
//    lengths cannot unbalance the waves), and runs its online softmax across
//    consecutive partitions of one (sequence, kv head).  One wave serves the
//    G query heads of a kv head, so they share every byte of K and V read.
//  * A (sequence, kv head) whose units all fall in one wave's range is
//    written out directly.  Otherwise each wave that touched it writes a
//    partial (max, sum, acc) -- at most two per wave, for the first and the
//    last item of its range -- and counts itself in on the item: on its
//    first item as soon as that partial is stored (if its range goes on),
//    on its last item after the range.  The last of an item's waves to
//    arrive merges the partials by log-sum-exp rescaling, in the same
//    launch.
//  * A scalar cursor walks the steps of the range across items: block ids
//    are fetched one 64-token step ahead of their use, and every K/V load is
//    a raw buffer load of one (block, kv head) tile (a descriptor, one lane
//    offset, immediate offsets), 16 bytes per lane (8 for fp8).
//  * Loads are software-pipelined: the next step's K tile is issued right
//    after this step's scores, its V tile right after this step's PV, so a
//    wave keeps one step of K and V in flight while it computes -- also from
//    the last step of one item into the first of the next, whose query is
//    fetched along with them.  Past the range's last step the descriptors
//    are empty: those loads return zeros without touching memory.
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

#include <hip/hip_ext.h>

#include "pa_device.h"
#include "pa_internal.h"
#include "store_row.h"

#ifndef PA_DECODE_STEP_TOKENS
#define PA_DECODE_STEP_TOKENS 64
#endif

// A measurement build (PA_DECODE_TRACE) records per-wave time stamps of the
// decode kernel's phases (the 100 MHz constant clock of s_memrealtime) into
// DecodeArgs::trace; in the library itself the stamps compile to nothing.
// Record of wave w (16 uint32 at trace + 16 w): stamps of its start, unit
// prefix, first tiles issued, first step done, range done, end (after its
// merges and their stores); XCD (workgroup id mod 8), hardware XCC id,
// segments, steps, merged items (bits), pending items (bits), early
// count-in; stamps of the count-in done, first block ids requested and
// arrived.
#ifdef PA_DECODE_TRACE
#define PA_TRACE_STAMP(v) ((v) = uint32_t(__builtin_amdgcn_s_memrealtime()))
#else
#define PA_TRACE_STAMP(v) ((void)0)
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
  // tokens per step: the configured step rounded up to whole blocks (<= 64);
  // 32 for an fp32 cache at head_dim 128 with four or more heads per group,
  // whose 64-token K and V tiles alone would fill the 256 registers
  static constexpr int STEP = (F32 && D == 128 && G >= 4) ? 32 : PA_DECODE_STEP_TOKENS;
  static constexpr int CH = ((STEP + B - 1) / B) * B;
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
// whole workgroup: s_prefix[s] = sum over s' < s, s_prefix[S] = total.  The
// lengths themselves are kept in LDS too (s_len[s] = max(0, lens[s])), so
// that no wave goes back to memory for its sequences' lengths.
__device__ __forceinline__ void build_prefix(const int32_t* lens, int S, int PT, int* s_prefix, int* s_len,
                                             int* s_tmp) {
  const int tid = threadIdx.x;
  const int per = (S + 255) / 256;
  const int i0 = tid * per, i1 = min(S, i0 + per);
  int local = 0;
  for (int i = i0; i < i1; ++i) {
    const int L = max(0, lens[i]);
    s_len[i] = L;
    local += units_of(L, PT);
  }
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
    run += units_of(s_len[i], PT);
  }
  if (tid == 255) s_prefix[S] = s_tmp[255];
  __syncthreads();
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
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

// Cross-wave hand-off of split items.  Partials and arrival counters are only
// ever touched through agent-scope atomics, which the L2 of one XCD does not
// hold back from the other XCDs.  A wave waits until its partial stores have
// completed (vmcnt(0)) before it counts itself in, and the last wave to arrive
// reads the partials only after its counter increment has returned, so no
// cache write-back or invalidation is needed.
__device__ __forceinline__ void xstore(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float xload(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Count this wave in on up to two split items (counter c[i], n[i] waves
// each); last[i] is true for the last of an item's waves to arrive, which then
// owns its merge and leaves the counter at zero for the next call.  Both
// increments go out before either result is awaited.  early0: this wave
// already added itself to c0 (with no result); it only reads c0, and merges
// when the count is complete.
__device__ __forceinline__ void arrive_last2(int32_t* c0, int n0, bool h0, bool early0, int32_t* c1, int n1,
                                             bool h1, bool& last0, bool& last1) {
  int r0 = 0, r1 = 0;
  const bool l0 = (threadIdx.x & 63) == 0;
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);                      // this wave's partial stores are complete
  __builtin_amdgcn_sched_barrier(0);
  if (l0 && h0) {
    if (early0) r0 = __hip_atomic_load(c0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) - 1;
    else r0 = __hip_atomic_fetch_add(c0, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (l0 && h1) r1 = __hip_atomic_fetch_add(c1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  r0 = __builtin_amdgcn_readfirstlane(r0);
  r1 = __builtin_amdgcn_readfirstlane(r1);
  last0 = h0 && r0 == n0 - 1;
  last1 = h1 && r1 == n1 - 1;
  if (l0 && last0) __hip_atomic_store(c0, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (l0 && last1) __hip_atomic_store(c1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Merge of the n partials of one (sequence, kv head) split over waves
// w0 .. w0 + n - 1: out = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i
// (m in log2 units).  Wave w0 holds the item in slot 0 if the item opens its
// range, else in slot 1; every later wave holds it in slot 0.
template <int D, int G, bool F32OUT>
__device__ __forceinline__ void merge_split(const DecodeArgs& a, int seq, int kvh, int w0, int n, bool w0_first) {
  constexpr int PL = D / 64;
  const int lane = threadIdx.x & 63;
  float M[G], Ls[G], o[G][PL];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    M[g] = -INFINITY;
    Ls[g] = 0.f;
#pragma unroll
    for (int k = 0; k < PL; ++k) o[g][k] = 0.f;
  }
  constexpr int NB = G <= 4 ? 8 : 2;                       // partials whose loads are in flight at once
  for (int i0 = 0; i0 < n; i0 += NB) {
    float m[NB][G], l[NB][G], x[NB][G][PL];
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const int i = min(i0 + r, n - 1);
      const size_t base = (size_t(w0 + i) * 2 + ((i > 0 || w0_first) ? 0 : 1)) * G;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        m[r][g] = xload(a.part_ml + 2 * (base + g));
        l[r][g] = xload(a.part_ml + 2 * (base + g) + 1);
#pragma unroll
        for (int k = 0; k < PL; ++k) x[r][g][k] = xload(a.part_acc + (base + g) * D + lane + 64 * k);
      }
    }
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      if (i0 + r >= n) break;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const float mn = fmaxf(M[g], m[r][g]);
        const float co = exp2f(M[g] - mn), cn = exp2f(m[r][g] - mn);
        Ls[g] = fmaf(Ls[g], co, l[r][g] * cn);
#pragma unroll
        for (int k = 0; k < PL; ++k) o[g][k] = fmaf(o[g][k], co, x[r][g][k] * cn);
        M[g] = mn;
      }
    }
  }
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const float inv = 1.f / Ls[g];
    const size_t ob = (size_t(seq) * a.num_q_heads + kvh * G + g) * D + lane;
#pragma unroll
    for (int k = 0; k < PL; ++k) {
      const float r = o[g][k] * inv;
      if constexpr (F32OUT) static_cast<float*>(a.out)[ob + 64 * k] = r;
      else static_cast<uint16_t*>(a.out)[ob + 64 * k] = uint16_t(pack_bf16x2(r, 0.f) & 0xFFFFu);
    }
  }
}

// block_table and context_lens are separate restrict arguments so that the
// compiler may read them through the scalar cache (s_load) even though the
// kernel stores results: block ids then never wait behind in-flight tiles.
template <int KV, int D, int B, int G>
__global__ void __launch_bounds__(256) decode_kernel(DecodeArgs a, const int32_t* __restrict__ block_table,
                                                     const int32_t* __restrict__ context_lens) {
  using C = DecCfg<KV, D, B, G>;
  using LoadT = typename C::LoadT;
  extern __shared__ int s_prefix[];                       // [num_seqs + 1], then s_len [num_seqs]
  __shared__ int s_tmp[256];
  __shared__ float s_score[4][C::CH * G];                 // [token][head] per wave
  __shared__ __attribute__((aligned(16))) uint32_t s_p[4][C::CH * G];   // probabilities per wave

  const int S = a.num_seqs;
  const int PT = a.part_tokens;
  int* s_len = s_prefix + S + 1;
  const int lane = threadIdx.x & 63;
  // trace stamps: start, prefix, first tiles issued, first step done, range
  // done, end; segments, steps
  [[maybe_unused]] uint32_t tr_start = 0, tr_prefix = 0, tr_issue = 0, tr_step1 = 0, tr_range = 0, tr_end = 0;
  [[maybe_unused]] uint32_t tr_ids_req = 0, tr_ids = 0;   // first block ids requested, arrived
  [[maybe_unused]] uint32_t tr_arrived = 0;               // counted in on the split items
  [[maybe_unused]] uint32_t tr_nseg = 0, tr_nstep = 0;
  PA_TRACE_STAMP(tr_start);
  // The unit prefix over the sequences: for at most 64 sequences every wave
  // builds it in its own registers (lane i: sequence i's length and the
  // units before it), with no LDS and no barrier; larger batches build it in
  // LDS with the whole workgroup.
  const bool wave_prefix = S <= 64;
  int r_len = 0, r_ex = 0, total_units;
  if (wave_prefix) {
    r_len = lane < S ? max(0, context_lens[lane]) : 0;
    const int u = lane < S ? units_of(r_len, PT) : 0;
    const int incl = wave_incl_scan(u);
    r_ex = incl - u;
    total_units = uniform(__builtin_amdgcn_readlane(incl, 63));
  } else {
    build_prefix(context_lens, S, PT, s_prefix, s_len, s_tmp);
    total_units = s_prefix[S];
  }
  PA_TRACE_STAMP(tr_prefix);
  // length and first unit of sequence sq (wave-uniform)
  auto len_of = [&](int sq) -> int {
    return wave_prefix ? __builtin_amdgcn_readlane(r_len, sq) : uniform(s_len[sq]);
  };
  auto prefix_of = [&](int sq) -> int {
    return wave_prefix ? __builtin_amdgcn_readlane(r_ex, sq) : s_prefix[sq];
  };

  const int w = uniform(threadIdx.x >> 6);                // wave-uniform, so all range math stays scalar
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const int64_t U = int64_t(total_units) * Hkv;
  // at most U waves: every range is non-empty, so every wave from the first
  // to the last of a split item holds a partial of it
  const int64_t W = min<int64_t>(a.total_waves, U);
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

  // Scalar cursor over the steps of this wave's range.  It runs ahead of the
  // compute across (sequence, kv head) segments, so the first tiles of the
  // next segment are in flight while the current one finishes; past the
  // range it stays on the last step (a harmless re-read).
  struct Cursor {
    int64_t u;                  // first unit of the cursor's segment
    int seq, kvh, part, p_end;  // segment: partitions [part, p_end) of (seq, kvh)
    int blk, last_blk;          // first block of the step, last block of the segment
    int st, nsteps;
    bool live, any;             // any: some step of the range was ever found
  };
  auto seg_setup = [&](Cursor& c) {                          // derive the segment's steps
    const int L = len_of(c.seq);
    const int nu = units_of(L, PT);
    c.p_end = int(min<int64_t>(nu, c.part + (u_end - c.u)));
    const int t_begin = c.part * PT, t_end = min(L, c.p_end * PT);
    c.nsteps = (max(t_end - t_begin, 0) + C::CH - 1) / C::CH;
    c.blk = t_begin / B;
    c.last_blk = max((t_end + B - 1) / B - 1, 0);
    c.st = 0;
  };
  auto next_seg = [&](Cursor& c) -> bool {                   // false past the range
    c.u += c.p_end - c.part;
    if (c.u >= u_end) return false;
    c.part = 0;
    if (++c.kvh == Hkv) {
      c.kvh = 0;
      ++c.seq;
    }
    seg_setup(c);
    return true;
  };
  auto skip_empty = [&](Cursor& c) {                         // first segment with a step, else dead
    while (c.nsteps == 0) {
      Cursor t = c;
      if (!next_seg(t)) {
        c.live = false;
        return;
      }
      c = t;
    }
    c.any = true;
  };
  auto advance = [&](Cursor& c) {
    if (!c.live) return;
    if (c.st + 1 < c.nsteps) {
      ++c.st;
      c.blk += C::BPC;
      return;
    }
    Cursor t = c;
    if (!next_seg(t)) {
      c.live = false;
      return;
    }
    skip_empty(t);
    if (t.live) c = t;
    else c.live = false;
  };
  // block ids of the cursor's step (blocks past the segment re-read its last
  // block, and everything past the segment's end is masked); a range with no
  // token at all reads block 0, which always exists, and uses nothing of it
  auto cursor_ids = [&](const Cursor& c, int (&ids)[C::BPC]) {
    const int32_t* row = block_table + size_t(c.seq) * a.max_blocks_per_seq;
#pragma unroll
    for (int k = 0; k < C::BPC; ++k) ids[k] = c.any ? uniform(row[min(c.blk + k, c.last_blk)]) : 0;
  };

  LoadT kreg[C::BPC][C::KLB];
  LoadT vreg[C::BPC][C::VLB];
  // Bytes of a tile that the next loads may read: a whole tile while the
  // cursor is live, none past the range's last step.  Loads through an empty
  // descriptor return zeros without a memory access, so the wait that closes
  // the range has no tile in flight to wait for.
  uint32_t nx_bytes = uint32_t(kTile);
  auto load_k = [&](const int (&ids)[C::BPC], int kh) {
#pragma unroll
    for (int k = 0; k < C::BPC; ++k) {
      const auto r = tile_rsrc(kpool + (uint64_t(uint32_t(ids[k])) * uint32_t(Hkv) + uint32_t(kh)) * kTile,
                               nx_bytes);
#pragma unroll
      for (int i = 0; i < C::KLB; ++i) buffer_load(r, k_off, uint32_t(i * C::RPL * D * C::ES), kreg[k][i]);
    }
  };
  auto load_v = [&](const int (&ids)[C::BPC], int kh) {
#pragma unroll
    for (int k = 0; k < C::BPC; ++k) {
      const auto r = tile_rsrc(vpool + (uint64_t(uint32_t(ids[k])) * uint32_t(Hkv) + uint32_t(kh)) * kTile,
                               nx_bytes);
#pragma unroll
      for (int j = 0; j < C::VLB; ++j) buffer_load(r, v_off, uint32_t(j * C::DPL * B * C::ES), vreg[k][j]);
    }
  };

  // first unit of the range -> (sequence, kv head, partition)
  int seq;
  if (wave_prefix) {                                      // the last sequence whose prefix is <= the key
    const int key = int(u / Hkv);
    seq = uniform(__builtin_popcountll(__ballot(lane < S && r_ex <= key))) - 1;
  } else {
    seq = find_seq(s_prefix, S, int(u / Hkv));
  }
  int kvh, part;
  {
    const int nu = units_of(len_of(seq), PT);
    const int r = int(u - int64_t(prefix_of(seq)) * Hkv);
    kvh = uniform(r / nu);
    part = uniform(r - kvh * nu);
  }

  // query of the G heads of (sq, kh); register j holds head j ^ gray.  qf / qp
  // serve the segment being computed, qfn / qpn receive the next segment's.
  float qf[C::F32 ? G : 1][4], qfn[C::F32 ? G : 1][4];
  uint32_t qp[C::F32 ? 1 : G][4], qpn[C::F32 ? 1 : G][4];
  auto load_q = [&](auto& df, auto& dp, int sq, int kh) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const int head = kh * G + (j ^ gray);
      if constexpr (C::F32) {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(a.q) +
                                                          (size_t(sq) * Hq + head) * D + kcol * 4);
        df[j][0] = v.x; df[j][1] = v.y; df[j][2] = v.z; df[j][3] = v.w;
      } else {
        const uint4 v = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.q) +
                                                        (size_t(sq) * Hq + head) * D + kcol * 8);
        dp[j][0] = v.x; dp[j][1] = v.y; dp[j][2] = v.z; dp[j][3] = v.w;
      }
    }
  };

  // Pipeline: kreg / vreg hold the tiles of the step being computed; nx is
  // the cursor of the step whose tiles are loaded next, its ids already in
  // scalar registers.
  Cursor nx{u, seq, kvh, part, 0, 0, 0, 0, 0, true, false};
  seg_setup(nx);
  skip_empty(nx);
  PA_TRACE_STAMP(tr_ids_req);
  int ids_nx[C::BPC];
  cursor_ids(nx, ids_nx);
  int kvh_nx = nx.kvh;
  // Append: partitions are whole blocks, so the last block of a (sequence,
  // kv head), which receives the step's new token (position length - 1), is
  // read by one wave only, the one whose range holds the item's last
  // partition; that wave stores the token.  The first such item's rows are
  // fetched with the query, so the two share one wait.  The stores then go
  // out ahead of every tile load of the wave, and vector memory operations
  // complete in issue order, so each later step, whose loads are issued after
  // the wait for an earlier step's tiles, sees them; only a first step that
  // holds a stored token waits for the stores themselves.
  auto append_item = [&](int& sq, int& kh, int64_t& base) -> bool {   // next item to store, from (sq, kh)
    for (;;) {
      const int L = len_of(sq);
      const int nu = units_of(L, PT);
      if (base + nu > u_end) return false;                // its last partition lies past this range
      if (L > 0) return true;
      base += nu;
      if (base >= u_end) return false;
      if (++kh == Hkv) {
        kh = 0;
        ++sq;
      }
    }
  };
  constexpr int IN_ES = KV == KV_F32 ? 4 : 2;             // element bytes of k_new / v_new
  auto new_row = [&](int sq, int kh) {
    const size_t r = (size_t(sq) * Hkv + kh) * D * IN_ES;
    return load_new_row<KV>(static_cast<const char*>(a.k_new) + r, static_cast<const char*>(a.v_new) + r, D);
  };
  auto new_slot = [&](int sq) {                            // slot of position length - 1
    const int L = len_of(sq);
    return uniform(block_table[size_t(sq) * a.max_blocks_per_seq + (L - 1) / B]) * B + (L - 1) % B;
  };
  int ap_sq = seq, ap_kh = kvh;
  int64_t ap_base = u - part;                             // first unit of (ap_sq, ap_kh)
  const bool ap = a.k_new != nullptr && append_item(ap_sq, ap_kh, ap_base);
  load_q(qf, qp, seq, kvh);
  NewRow ap_row{};
  int ap_slot = -1;
  if (ap) {
    ap_row = new_row(ap_sq, ap_kh);
    ap_slot = new_slot(ap_sq);
  }
#ifdef PA_DECODE_TRACE
  __builtin_amdgcn_s_waitcnt(0xC07F);                       // lgkmcnt(0): the block ids are in
  PA_TRACE_STAMP(tr_ids);
#endif
  // The query and block ids must be in registers before the first tile is
  // requested; an explicit wait here keeps the compiler from waiting on every
  // in-flight tile (vmcnt(0)) at each step.
  __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0) only
  __builtin_amdgcn_sched_barrier(0);
  if (ap) {
    for (;;) {
      float ksc = 1.f, vsc = 1.f;
      if constexpr (KV == KV_FP8) {
        ksc = a.k_scale[ap_kh];
        vsc = a.v_scale[ap_kh];
      }
      store_new_row<KV>(ap_row, const_cast<void*>(a.k_cache), const_cast<void*>(a.v_cache), ap_slot, ap_kh, Hkv, D,
                        B, ksc, vsc);
      ap_base += units_of(len_of(ap_sq), PT);
      if (ap_base >= u_end) break;
      if (++ap_kh == Hkv) {
        ap_kh = 0;
        ++ap_sq;
      }
      if (!append_item(ap_sq, ap_kh, ap_base)) break;
      ap_row = new_row(ap_sq, ap_kh);
      ap_slot = new_slot(ap_sq);
    }
    // the first step holds the last block of an item stored above
    if (nx.live && nx.p_end == units_of(len_of(nx.seq), PT) && nx.blk + C::BPC > nx.last_blk)
      __builtin_amdgcn_s_waitcnt(0x0F70);
    __builtin_amdgcn_sched_barrier(0);
  }
  load_k(ids_nx, kvh_nx);                                   // keys before values, as in the loop
  __builtin_amdgcn_sched_barrier(0);
  load_v(ids_nx, kvh_nx);
  __builtin_amdgcn_sched_barrier(0);
  PA_TRACE_STAMP(tr_issue);
  advance(nx);
  cursor_ids(nx, ids_nx);
  kvh_nx = nx.kvh;
  nx_bytes = nx.live ? uint32_t(kTile) : 0u;

  // Split items this wave holds a partial of (at most two: the first and the
  // last of its range).  It counts itself in on them only once its whole range
  // is done, so that no segment switch waits for stores or atomics.
  struct Pending {
    int seq, kvh, w0, n, w1;
    bool w0_first;
  };
  Pending pend[2] = {{0, 0, 0, 1, 0, false}, {0, 0, 0, 1, 0, false}};
  bool has_pend[2] = {false, false};
  // A range's first item, when split and followed by more of the range, is
  // counted in on as soon as its partial is stored, with an add whose result
  // nobody waits for: the neighbour that finishes the item later usually
  // merges it, not this wave, which still has the rest of its range to
  // stream.  After its range this wave reads the counter: if it shows every
  // wave of the item, the wave merges too (a merge by two waves writes the
  // same bits twice; no merge is ever missed, since the wave whose add
  // completes the count also merges).
  bool early = false;

  bool first = true;
  bool q_ready = false;                                      // qfn / qpn hold this segment's query
  for (;;) {                                                 // one (sequence, kv head) segment per pass
    const int L = len_of(seq);
    const int nu = units_of(L, PT);
    const int p_end = int(min<int64_t>(nu, part + (u_end - u)));
    const bool whole = part == 0 && p_end == nu;
    const int t_begin = part * PT;
    const int t_end = min(L, p_end * PT);
    const int nsteps = (max(t_end - t_begin, 0) + C::CH - 1) / C::CH;
    // the next segment of the range (itself at the range's end): its query
    // is fetched during this segment's last step
    const bool has_next = u + (p_end - part) < u_end;
    const int nq_kvh = has_next ? (kvh + 1 == Hkv ? 0 : kvh + 1) : kvh;
    const int nq_seq = has_next && kvh + 1 == Hkv ? seq + 1 : seq;

    float sl = a.scale_log2;
    if constexpr (KV == KV_FP8) sl *= a.k_scale[kvh];

    if (!first) {
      if (q_ready) {
#pragma unroll
        for (int j = 0; j < (C::F32 ? G : 1); ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) qf[j][e] = qfn[j][e];
#pragma unroll
        for (int j = 0; j < (C::F32 ? 1 : G); ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) qp[j][e] = qpn[j][e];
      } else {                                               // after an empty segment
        load_q(qf, qp, seq, kvh);
        __builtin_amdgcn_s_waitcnt(0x0F70);
        __builtin_amdgcn_sched_barrier(0);
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

    // One 64-token step.  The last step of a segment also fetches the next
    // segment's query, ahead of the next tiles, so that the wait for those
    // tiles covers it.
    auto do_step = [&](int st, auto last_step) {
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
      if constexpr (decltype(last_step)::value) load_q(qfn, qpn, nq_seq, nq_kvh);
      load_k(ids_nx, kvh_nx);                                 // the next step's keys fly during softmax + PV
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
      load_v(ids_nx, kvh_nx);                                 // its values fly during its scores
      __builtin_amdgcn_sched_barrier(0);
      advance(nx);                                            // ids one step ahead of their loads
      cursor_ids(nx, ids_nx);
      kvh_nx = nx.kvh;
      nx_bytes = nx.live ? uint32_t(kTile) : 0u;
    };
    for (int st = 0; st + 1 < nsteps; ++st) {
      do_step(st, std::false_type{});
#ifdef PA_DECODE_TRACE
      if (tr_step1 == 0) PA_TRACE_STAMP(tr_step1);
#endif
    }
    q_ready = nsteps > 0;
    if (nsteps > 0) do_step(nsteps - 1, std::true_type{});
#ifdef PA_DECODE_TRACE
    if (tr_step1 == 0) PA_TRACE_STAMP(tr_step1);
    ++tr_nseg;
    tr_nstep += uint32_t(nsteps);
#endif

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
      const int slot = first ? 0 : 1;
      const size_t base = (size_t(wid) * 2 + slot) * G;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (lane == 0) {
          xstore(a.part_ml + 2 * (base + g), m_run[g] * sl);  // log2 units
          xstore(a.part_ml + 2 * (base + g) + 1, l[g]);
        }
        if (vs == 0) {
#pragma unroll
          for (int j = 0; j < C::VLB; ++j) xstore(a.part_acc + (base + g) * D + j * C::DPL + vd, acc[g][j]);
        }
      }
      const int64_t u0 = int64_t(prefix_of(seq)) * Hkv + int64_t(kvh) * nu;
      const int w0 = owner_wave(u0, U, W);
      const int w1 = owner_wave(u0 + nu - 1, U, W);
      pend[slot] = Pending{seq, kvh, w0, w1 - w0 + 1, w1, int64_t(w0) * U / W == u0};
      has_pend[slot] = true;
      if (slot == 0 && u + (p_end - part) < u_end) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        __builtin_amdgcn_s_waitcnt(0x0F70);                 // the partial stores are complete
        __builtin_amdgcn_sched_barrier(0);
        if (lane == 0) __hip_atomic_fetch_add(a.arrivals + w1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        early = true;
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

  PA_TRACE_STAMP(tr_range);
  [[maybe_unused]] uint32_t tr_merged = 0;
  // Count in on the split items; the last wave to arrive at one merges it.
  if (has_pend[0] || has_pend[1]) {
    bool last0, last1;
    arrive_last2(a.arrivals + pend[0].w1, pend[0].n, has_pend[0], early, a.arrivals + pend[1].w1, pend[1].n,
                 has_pend[1], last0, last1);
    PA_TRACE_STAMP(tr_arrived);
    if (last0) merge_split<D, G, C::F32>(a, pend[0].seq, pend[0].kvh, pend[0].w0, pend[0].n, pend[0].w0_first);
    if (last1) merge_split<D, G, C::F32>(a, pend[1].seq, pend[1].kvh, pend[1].w0, pend[1].n, pend[1].w0_first);
#ifdef PA_DECODE_TRACE
    tr_merged = (last0 ? 1u : 0u) | (last1 ? 2u : 0u);
#endif
  }
#ifdef PA_DECODE_TRACE
  __builtin_amdgcn_s_waitcnt(0);                            // the wave's last stores have completed
  PA_TRACE_STAMP(tr_end);
  if (a.trace && lane == 0) {
    // XCC_ID (hardware register 20, bits 3:0): the XCD this wave runs on
    const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);
    const uint32_t rec[16] = {tr_start, tr_prefix, tr_issue, tr_step1, tr_range, tr_end,
                              uint32_t(blockIdx.x & 7), xcc, tr_nseg, tr_nstep, tr_merged,
                              uint32_t(has_pend[0]) | (uint32_t(has_pend[1]) << 1), uint32_t(early),
                              tr_arrived, tr_ids_req, tr_ids};
#pragma unroll
    for (int i = 0; i < 16; ++i) a.trace[size_t(wid) * 16 + i] = rec[i];
  }
#endif
}

// A launch whose events take the kernel's own start and end timestamps.
template <typename K, typename... Args>
hipError_t launch_with_events(K kern, dim3 grid, dim3 block, size_t lds, hipStream_t s, const LaunchEvents& ev,
                              Args... args) {
  void* argv[] = {static_cast<void*>(&args)...};
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, argv, lds, s, ev.start, ev.stop, 0);
}

template <int KV, int D, int B, int G>
hipError_t launch_decode_t(const DecodeArgs& a0, int64_t upper_units, hipStream_t s, const LaunchEvents& ev) {
  auto kern = decode_kernel<KV, D, B, G>;
  const size_t lds = size_t(2 * a0.num_seqs + 1) * sizeof(int);
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
  if (ev.start || ev.stop)
    return launch_with_events(kern, dim3(uint32_t(wgs)), dim3(256), lds, s, ev, a, a.block_table, a.context_lens);
  hipLaunchKernelGGL(kern, dim3(uint32_t(wgs)), dim3(256), lds, s, a, a.block_table, a.context_lens);
  return hipGetLastError();
}

// Dispatch over the compiled (head_dim, block_size, group) set for one cache dtype.
template <int KV>
hipError_t launch_decode_kv(const DecodeArgs& a, int D, int B, int G, int64_t upper, hipStream_t s,
                            const LaunchEvents& ev) {
#define PA_DEC_CASE(d, b, g) \
  if (D == d && B == b && G == g) return launch_decode_t<KV, d, b, g>(a, upper, s, ev);
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
