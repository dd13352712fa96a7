// Attention of a chunk of a few tokens over a paged prefix on gfx950 matrix
// cores: the shape of speculative-decoding verification, where k draft
// tokens plus the last accepted one (k + 1 causal query positions per
// sequence) are checked in one pass over the cache.
//
// What it computes is exactly pa_prefill_chunk's result (serving-stack page,
// speculative decoding: the target model scores all draft tokens in one
// forward pass; nanoPD page, 分页KV缓存: speculative branches share blocks
// through copy-on-write): chunk row t of sequence j, at absolute position
// P_j + t, attends to keys 0 .. P_j + t read through the block table.  The
// launcher picks this kernel when a chunk has at most 32 / G tokens.
//
// How:
//  * An item is a (sequence, kv head); its units are its 32-key tiles.  A
//    workgroup of eight waves computes a stretch of consecutive units.  A
//    wave's 32 MFMA columns are the (query head, token) pairs of the group:
//    column n is head n / (32/G) and token n % (32/G), so every K/V byte
//    read serves all G heads and all tokens of the chunk.
//  * With a workspace, a launch fills the CUs once and its workgroups read
//    the batch's lengths.  Unless every item has a workgroup and none is
//    more than twice an equal share (then one workgroup per item is faster),
//    the units of the whole batch (sequence-major, then kv head, then tile)
//    are cut into equal stretches, one per workgroup, so that long and short
//    contexts finish together and few sequences still fill the chip.  An
//    item cut by a stretch boundary leaves a partial result (max, sum,
//    unnormalised output per column) in the workspace from each workgroup
//    that holds part of it; after its stretch, each of them counts itself in,
//    and the last merges the partials by log-sum-exp rescaling and writes the
//    output.  Without a workspace, one workgroup computes each item whole.
//  * A wave walks its tiles of the stretch with a cursor that crosses items:
//    the first tile of its next item, and that item's query, are requested
//    before the current item's cross-wave merge, as within an item.
//  * Inside a workgroup, the eight waves take the item's tiles t0 + w,
//    t0 + w + 8, ... of the stretch and keep an online softmax per column;
//    their eight partial results are merged through LDS by log-sum-exp
//    rescaling.
//  * Operands come straight from the paged pools (each tile is read by one
//    wave, so staging would not save bytes): K rows as the A operand of
//    S^T = K Q^T at MFMA row swap23(key), V^T (stored transposed per block)
//    as the A operand of O^T = V^T P^T.  The next tile's K is issued right
//    after this tile's S^T, its V right after this tile's PV; block ids come
//    through the scalar cache a tile earlier.
#include <algorithm>

#include "mfma_attn.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kVerifyWaves = 8;
constexpr int kVerifyThreads = kVerifyWaves * 64;
// Sequences of a split launch: their unit prefix (4 bytes each) shares LDS
// with the 139 KB of the cross-wave merge.
constexpr int kVerifySplitMaxSeqs = 4096;

namespace {

// The workgroup whose stretch holds unit u when U units are cut into W
// stretches, stretch g being [floor(g U / W), floor((g + 1) U / W)).
__device__ __forceinline__ int owner_group(int64_t u, int64_t U, int64_t W) {
  return int(((u + 1) * W + U - 1) / U - 1);
}

// Cross-workgroup hand-off of split items, as in decode: partials are
// written through this XCD's L2 to the point where every XCD reads them (the
// sc1 stores of agent-scope atomics) and read with agent-scope loads that
// bypass a stale L2 line; a workgroup counts itself in only after every one
// of its threads has seen its partial stores complete, and the merging
// workgroup loads the partials only after the count has returned.  The
// stores are 16 bytes wide: 4-byte write-through stores cost several times
// their bytes in HBM writes and read-modify-write reads.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void vstore4(float* p, const f32x4_t& v) {
  asm volatile("global_store_dwordx4 %0, %1, off sc1" : : "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void vstore2(float* p, float x, float y) {
  const uint64_t b = uint64_t(__float_as_uint(x)) | (uint64_t(__float_as_uint(y)) << 32);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), b, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// V operand loads with the non-temporal hint (nt): each of them reads 32
// rows x 32 contiguous bytes of a transposed V tile, whole lines, and no
// line is read twice in the launch (5.2% faster on the Qwen3-8B verify
// batch, 9.5% on the long-context prefixes).  The K operand loads keep the
// default policy: each reads 32 bytes of every 256-byte key row, so the four
// loads of one line would each fetch it again (with the hint on both, 28%
// slower).
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 stream_load(const uint2* p) {
  const u32x2_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ void vload2(const float* p, float& x, float& y) {
  const uint64_t b = __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
  x = __uint_as_float(uint32_t(b));
  y = __uint_as_float(uint32_t(b >> 32));
}

}  // namespace

template <int KV, int B, int G>
__global__ void __launch_bounds__(kVerifyThreads) verify_kernel(PrefillArgs a,
                                                               const int32_t* __restrict__ block_table,
                                                               const int32_t* __restrict__ cu_q_lens,
                                                               const int32_t* __restrict__ seq_lens) {
  constexpr int D = 128;
  constexpr int KT = 32;                         // keys per tile
  constexpr int NW = kVerifyWaves;
  constexpr int TS = 32 / G;                     // token slots per head among a wave's 32 columns
  constexpr int OROW = D + 4;                    // LDS floats per (wave, column) row of O^T, padded
  __shared__ float s_m[NW][32], s_l[NW][32];
  __shared__ __attribute__((aligned(16))) float s_o[NW][32][OROW];
  __shared__ int s_scan[kVerifyThreads];
  __shared__ int s_merge[5];                     // split items to merge: first workgroups (or -1), slots, counts
  extern __shared__ int s_prefix[];              // split launches: units before each sequence, [num_seqs + 1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int hh = lane >> 5;                      // lane half: k-slice of operands, row group of accumulators
  const int n = lane & 31;                       // MFMA column / operand row
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads, S = a.num_seqs;
  const bool split = a.part_acc != nullptr;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  using Raw = KvRaw<KV>;
  constexpr int ES = Raw::ES;                   // cache element bytes
  // Per-sequence lengths.  For batches of at most 64 sequences lane i loads
  // sequence i's once, and any sequence's are then a register read by lane
  // (no memory round trip in the wave's chain of dependent steps); larger
  // batches read memory (through the scalar cache).
  const bool lane_meta = S <= 64;
  int m_q0 = 0, m_ql = 0, m_kend = 0;
  if (lane_meta && lane < S) {
    m_q0 = cu_q_lens[lane];
    m_ql = cu_q_lens[lane + 1] - m_q0;
    m_kend = seq_lens[lane];
  }
  const int m_tiles = m_ql > 0 ? (max(m_kend, 0) + KT - 1) / KT : 0;
  auto q0_of = [&](int s) { return lane_meta ? __builtin_amdgcn_readlane(m_q0, s) : cu_q_lens[s]; };
  auto qlen_of = [&](int s) { return lane_meta ? __builtin_amdgcn_readlane(m_ql, s) : cu_q_lens[s + 1] - cu_q_lens[s]; };
  auto kend_of = [&](int s) { return lane_meta ? __builtin_amdgcn_readlane(m_kend, s) : seq_lens[s]; };
  // tiles of a sequence's items (none when its chunk is empty)
  auto tiles_of = [&](int s) {
    if (lane_meta) return __builtin_amdgcn_readlane(m_tiles, s);
    return cu_q_lens[s + 1] > cu_q_lens[s] ? (max(seq_lens[s], 0) + KT - 1) / KT : 0;
  };

  // ---- this workgroup's stretch [u, u_end) of units, its first item and tile
  int64_t u, u_end, U = 0, W = 0;
  int seq, kvh, tile0;
  bool cut = split;                              // stretches cut across items
  // batches of at most 64 sequences: lane i holds sequence i's tiles and the
  // units before it, built by each wave alone (no LDS, no barrier)
  const bool wave_prefix = S <= 64;
  int l_tiles = 0, l_excl = 0;
  if (split && wave_prefix) {
    l_tiles = m_tiles;
    int x = l_tiles * Hkv, mx = l_tiles;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
      mx = max(mx, __shfl_xor(mx, off));
    }
    l_excl = x - l_tiles * Hkv;
    U = uniform(__shfl(x, 63));
    const int64_t M = uniform(mx);
    if (U == 0) return;                          // whole workgroup; no barrier follows
    cut = !(int64_t(S) * Hkv <= int64_t(gridDim.x) && M * int64_t(gridDim.x) <= 2 * U);
  } else if (split) {
    // exclusive prefix of units (tiles x kv heads) per sequence, in LDS, and
    // the longest item's tiles
    const int per = (S + kVerifyThreads - 1) / kVerifyThreads;
    const int i0 = tid * per, i1 = min(S, i0 + per);
    int local = 0, lmax = 0;
    for (int i = i0; i < i1; ++i) {
      const int nt = tiles_of(i);
      local += nt * Hkv;
      lmax = max(lmax, nt);
    }
    s_scan[tid] = local;
    if (tid == 0) s_merge[0] = 0;
    __syncthreads();
    atomicMax(&s_merge[0], lmax);
    for (int off = 1; off < kVerifyThreads; off <<= 1) {
      const int v = tid >= off ? s_scan[tid - off] : 0;
      __syncthreads();
      s_scan[tid] += v;
      __syncthreads();
    }
    int run = tid ? s_scan[tid - 1] : 0;
    for (int i = i0; i < i1; ++i) {
      s_prefix[i] = run;
      run += tiles_of(i) * Hkv;
    }
    if (tid == kVerifyThreads - 1) s_prefix[S] = s_scan[kVerifyThreads - 1];
    __syncthreads();
    U = s_prefix[S];
    const int64_t M = s_merge[0];
    __syncthreads();                             // s_merge is written again below
    if (U == 0) return;                          // whole workgroup; no barrier follows
    // When every item has a workgroup of this launch and none is much longer
    // than an equal share (at most twice), one workgroup per item is faster:
    // the items that end early leave the memory system to the longer ones,
    // and no partial is stored or merged.
    cut = !(int64_t(S) * Hkv <= int64_t(gridDim.x) && M * int64_t(gridDim.x) <= 2 * U);
  }
  if (cut) {
    W = min<int64_t>(a.total_groups, U);
    if (int64_t(blockIdx.x) >= W) return;        // whole workgroup; no barrier follows
    u = int64_t(blockIdx.x) * U / W;
    u_end = int64_t(blockIdx.x + 1) * U / W;
    // the last sequence whose prefix is <= u (sequences without units share
    // the prefix of the next one, so this is one with units)
    int pre;
    if (wave_prefix) {
      seq = uniform(__builtin_popcountll(__ballot(lane < S && l_excl <= u))) - 1;
      pre = uniform(__shfl(l_excl, seq));
    } else {
      int lo = 0, hi = S;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_prefix[mid] <= u) lo = mid; else hi = mid;
      }
      seq = uniform(lo);
      pre = s_prefix[seq];
    }
    const int nt = tiles_of(seq);
    const int r = int(u - pre);
    kvh = uniform(r / nt);
    tile0 = uniform(r - kvh * nt);
  } else {
    if (int64_t(blockIdx.x) >= int64_t(S) * Hkv) return;   // whole workgroup
    seq = blockIdx.x / Hkv;
    kvh = blockIdx.x - seq * Hkv;
    tile0 = 0;
    u = 0;
    u_end = tiles_of(seq);
    if (u_end == 0) return;                      // empty chunk: whole workgroup
  }

  const int gq = n / TS, t = n % TS;             // this lane's column: head gq of the group, chunk token t
  const int my_key = swap23(n);                  // key of MFMA row n within a tile

  // A slot of this wave's tile stream through the stretch: tile kt of the
  // item (seq, kvh), whose tiles in this stretch are [tile0, t1) (segment k
  // of the stretch, starting at unit useg); kend = the sequence's keys.  A
  // dead slot (past the wave's last tile) keeps the last live one's tile,
  // which its loads re-read; every index stays inside the sequence.
  struct Slot {
    int64_t useg;
    int k, seq, kvh, tile0, t1, kt, kend;
    bool live;
  };
  auto seg_end = [&](int sq, int t0, int64_t us) {
    return int(min<int64_t>(tiles_of(sq), t0 + (u_end - us)));
  };
  // the stretch's next segment (false at its end)
  auto next_seg = [&](Slot& s) -> bool {
    const int64_t us = s.useg + (s.t1 - s.tile0);
    if (us >= u_end) return false;
    if (s.kvh + 1 < Hkv) {
      ++s.kvh;
    } else {
      s.kvh = 0;
      do ++s.seq; while (tiles_of(s.seq) == 0);         // one with units follows: us < u_end <= U
    }
    s.seq = uniform(s.seq);
    s.kvh = uniform(s.kvh);
    s.k += 1;
    s.tile0 = 0;
    s.useg = us;
    s.t1 = seg_end(s.seq, 0, us);
    s.kend = kend_of(s.seq);
    return true;
  };
  // this wave's first tile in s's segment, or in the first later one where it has one
  auto settle = [&](Slot& s) {
    Slot x = s;
    while (x.tile0 + w >= x.t1) {
      if (!next_seg(x)) {
        s.live = false;
        s.kt = s.t1 - 1;
        return;
      }
    }
    x.kt = x.tile0 + w;
    s = x;
  };
  // the slot after s
  auto advance = [&](Slot& s) {
    if (!s.live) return;
    if (s.kt + NW < s.t1) {
      s.kt += NW;
      return;
    }
    Slot x = s;
    if (!next_seg(x)) {
      s.live = false;
      return;
    }
    settle(x);
    if (x.live) s = x;
    else s.live = false;
  };

  // ---- Q^T of a slot's item as 8 B operands (k = 16 head dims each): row q0 + t, dims 16s + 8hh .. + 7
  uint4 qb[8];
  auto load_q = [&](const Slot& s) __attribute__((always_inline)) {
    const int q0 = q0_of(s.seq), ql = qlen_of(s.seq);
    const int row = q0 + min(t, ql - 1);
    const uint16_t* qr = static_cast<const uint16_t*>(a.q) + (size_t(row) * Hq + s.kvh * G + gq) * D + 8 * hh;
#pragma unroll
    for (int i = 0; i < 8; ++i) qb[i] = *reinterpret_cast<const uint4*>(qr + 16 * i);
  };
  // ---- operands of a slot's tile
  typename Raw::T ka[8], va[4][2];               // raw loads; converted to bf16 at their use
  auto tile_ids = [&](const Slot& s, int& id0, int& id1) __attribute__((always_inline)) {
    const int32_t* table = block_table + size_t(s.seq) * a.max_blocks_per_seq;
    const int kmax = s.kend - 1;
    const int b0 = s.kt * KT / B;
    id0 = table[min(b0, kmax / B)];
    id1 = table[min(b0 + 1, kmax / B)];
  };
  auto load_k = [&](const Slot& s, int id0, int id1) __attribute__((always_inline)) {
    const int kmax = s.kend - 1;
    const int k0 = s.kt * KT;
    const int key = min(k0 + my_key, kmax);
    const int bid = key / B == k0 / B ? id0 : id1;
    const char* kr = kpool + ((size_t(bid) * Hkv + s.kvh) * B + key % B) * (D * ES) + 8 * ES * hh;
#pragma unroll
    for (int i = 0; i < 8; ++i) ka[i] = *reinterpret_cast<const typename Raw::T*>(kr + 16 * ES * i);
  };
  auto load_v = [&](const Slot& s, int id0, int id1) __attribute__((always_inline)) {
    const int kmax = s.kend - 1;
    const int k0 = s.kt * KT;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kb = min(k0 + 16 * ks + 8 * hh, kmax & ~7);   // 8 keys of one block
      const int bid = kb / B == k0 / B ? id0 : id1;
      const char* vb = vpool + (size_t(bid) * Hkv + s.kvh) * size_t(D * B * ES) + (kb % B) * ES;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        va[dt][ks] = stream_load(reinterpret_cast<const typename Raw::T*>(vb + size_t(32 * dt + n) * (B * ES)));
    }
  };

  // cs walks the stretch's segments; cl is the slot whose tile is in ka / va
  // (landed or in flight), ci the slot after it, whose block ids are in id0 / id1
  Slot cs{u, 0, seq, kvh, tile0, 0, 0, kend_of(seq), true};
  cs.t1 = seg_end(seq, tile0, u);
  Slot cl = cs;
  settle(cl);
  int id0, id1;
  load_q(cl);
  tile_ids(cl, id0, id1);
  // The query must be in registers before the first tile is requested: then
  // the tile loop is entered with the same two groups of loads in flight as
  // from its back edge, and its waits stay graded (no vmcnt(0)).
  __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0) only
  __builtin_amdgcn_sched_barrier(0);
  load_k(cl, id0, id1);
  __builtin_amdgcn_sched_barrier(0);
  load_v(cl, id0, id1);
  __builtin_amdgcn_sched_barrier(0);
  Slot ci = cl;
  advance(ci);
  tile_ids(ci, id0, id1);

  // split items of this stretch: its first segment's and its last segment's
  bool split0 = false, split1 = false;
  int seq0 = 0, kvh0 = 0, seq1 = 0, kvh1 = 0;
  int64_t first0 = 0, first1 = 0;
  for (;;) {                                                // segment cs.k of the stretch
    const int q0 = q0_of(cs.seq);
    const int q_len = qlen_of(cs.seq);
    const int key_end = cs.kend;                            // keys 0 .. key_end - 1 (prefix and chunk)
    const int P = key_end - q_len;
    const int n_tiles = (key_end + KT - 1) / KT;
    const bool whole = cs.tile0 == 0 && cs.t1 == n_tiles;
    const int pos = P + t;                                  // this lane's column's absolute position
    // an fp8 code of kv head h means code * scale[h]: K's scale goes into the
    // softmax constant, V's onto the output
    const float c = KV == KV_FP8 ? a.scale_log2 * a.k_scale[cs.kvh] : a.scale_log2;
    const float v_mul = KV == KV_FP8 ? a.v_scale[cs.kvh] : 1.f;

    f32x16_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
    float m_run = -INFINITY, l_run = 0.f;
    if (cl.live && cl.k == cs.k) {                          // this wave has tiles in the segment
      for (;;) {
        const int k0 = cl.kt * KT;
        // ---- S^T = K Q^T; accumulator r = 4i + j is key k0 + swap23(8i + 4hh + j)
        f32x16_t sc = f32x16_t{};
#pragma unroll
        for (int st = 0; st < 8; ++st) sc = mfma32(Raw::to_bf16(ka[st]), qb[st], sc);
        const Slot nx = ci;
        const bool seg_done = !(nx.live && nx.k == cs.k);   // the next tile opens a later segment
        __builtin_amdgcn_sched_barrier(0);
        // its query goes out ahead of its tile (the query registers are free
        // after this S^T), so that the loop's waits stay graded
        if (seg_done && nx.live) load_q(nx);
        load_k(nx, id0, id1);                               // next tile's keys fly during softmax + PV
        __builtin_amdgcn_sched_barrier(0);
        if (k0 + KT - 1 > P) {                              // tile reaches the chunk: causal mask and end
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + swap23(8 * (r >> 2) + 4 * hh + (r & 3));
            sc[r] = (key <= pos && key < key_end) ? sc[r] : -INFINITY;
          }
        }
        float mt = sc[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
        mt = fmaxf(mt, __shfl_xor(mt, 32));
        // A wave's tiles can lie wholly past a column's position (causal mask),
        // so a column may still have no key at all: its max stays -inf, and
        // both factors below are guarded against -inf - -inf.
        const float m_new = fmaxf(m_run, mt);
        if (__any(m_new > m_run)) {
          const float al = m_new > m_run ? __builtin_amdgcn_exp2f((m_run - m_new) * c) : 1.f;
          l_run *= al;
#pragma unroll
          for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] *= al;
          m_run = m_new;
        }
        const float mc = m_run == -INFINITY ? 0.f : m_run * c;   // then every p is 0
        float p[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mc));
          l_run += p[r];
        }
        // P^T operands: key slice ks takes accumulators 8ks .. 8ks + 7 (keys k0 + 16ks + 8hh + 0..7)
        uint4 pb[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          pb[ks] = make_uint4(pack_bf16x2(p[8 * ks + 0], p[8 * ks + 1]), pack_bf16x2(p[8 * ks + 2], p[8 * ks + 3]),
                              pack_bf16x2(p[8 * ks + 4], p[8 * ks + 5]), pack_bf16x2(p[8 * ks + 6], p[8 * ks + 7]));
        uint4 vb16[4][2];
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) vb16[dt][ks] = Raw::to_bf16(va[dt][ks]);
        if (k0 + KT > key_end) {                            // zero V rows of keys past the end (NaN poison)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            const int kb = k0 + 16 * ks + 8 * hh;
            uint32_t msk[4];
#pragma unroll
            for (int e = 0; e < 4; ++e)
              msk[e] = (kb + 2 * e < key_end ? 0x0000FFFFu : 0u) | (kb + 2 * e + 1 < key_end ? 0xFFFF0000u : 0u);
#pragma unroll
            for (int dt = 0; dt < 4; ++dt) {
              vb16[dt][ks].x &= msk[0]; vb16[dt][ks].y &= msk[1]; vb16[dt][ks].z &= msk[2]; vb16[dt][ks].w &= msk[3];
            }
          }
        }
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          o[dt] = mfma32(vb16[dt][0], pb[0], o[dt]);
          o[dt] = mfma32(vb16[dt][1], pb[1], o[dt]);
        }
        __builtin_amdgcn_sched_barrier(0);
        load_v(nx, id0, id1);                               // its values fly during its S^T
        __builtin_amdgcn_sched_barrier(0);
        ci = nx;
        advance(ci);
        tile_ids(ci, id0, id1);                             // ids one tile ahead of their loads
        cl = nx;
        if (seg_done) break;
      }
    }

    // ---- merge the eight waves' partial results through LDS
    // accumulator r of d-tile dt is dim 32dt + 8(r/4) + 4hh + (r%4) of column n
    const float l_col = l_run + __shfl_xor(l_run, 32);
    if (hh == 0) {
      s_m[w][n] = m_run;
      s_l[w][n] = l_col;
    }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(&s_o[w][n][32 * dt + 8 * i + 4 * hh]) =
            make_float4(o[dt][4 * i], o[dt][4 * i + 1], o[dt][4 * i + 2], o[dt][4 * i + 3]);
    __syncthreads();
    // thread -> (column, 8 dims): (M, L, acc) = max_w m_w, sum_w 2^((m_w - M) c) l_w, sum_w 2^((m_w - M) c) o_w.
    // A column with no key in this part (its keys lie in later tiles) keeps
    // M = -inf, L = 0, acc = 0.
    static_assert(kVerifyThreads == 32 * D / 8, "one thread per 8 output dims of a column");
    const int col = tid >> 4, d0 = (tid & 15) * 8;
    const int cg = col / TS, ct = col % TS;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, s_m[v][col]);
    float L = 0.f, acc[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int v = 0; v < NW; ++v) {
        const float wt = __builtin_amdgcn_exp2f((s_m[v][col] - M) * c);   // 0 for a wave without keys
        L = fmaf(wt, s_l[v][col], L);
        const float4 x0 = *reinterpret_cast<const float4*>(&s_o[v][col][d0]);
        const float4 x1 = *reinterpret_cast<const float4*>(&s_o[v][col][d0 + 4]);
        acc[0] = fmaf(wt, x0.x, acc[0]); acc[1] = fmaf(wt, x0.y, acc[1]);
        acc[2] = fmaf(wt, x0.z, acc[2]); acc[3] = fmaf(wt, x0.w, acc[3]);
        acc[4] = fmaf(wt, x1.x, acc[4]); acc[5] = fmaf(wt, x1.y, acc[5]);
        acc[6] = fmaf(wt, x1.z, acc[6]); acc[7] = fmaf(wt, x1.w, acc[7]);
      }
    }
    const bool last_seg = cs.useg + (cs.t1 - cs.tile0) >= u_end;
    if (whole) {
      if (ct < q_len) {
        const float inv = v_mul / L;
        uint16_t* orow = static_cast<uint16_t*>(a.out) + (size_t(q0 + ct) * Hq + cs.kvh * G + cg) * D + d0;
        *reinterpret_cast<uint4*>(orow) =
            make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                       pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
      }
    } else {
      // partial of an item split between stretches (only a stretch's first or
      // last segment can be one): stored now, counted in after the stretch
      const int slot = cs.k == 0 ? 0 : 1;
      if (slot == 0) {
        split0 = true; seq0 = cs.seq; kvh0 = cs.kvh; first0 = cs.useg - cs.tile0;
      } else {
        split1 = true; seq1 = cs.seq; kvh1 = cs.kvh; first1 = cs.useg - cs.tile0;
      }
      if (ct < q_len) {
        const size_t base = (size_t(blockIdx.x) * 2 + slot) * 32 + col;
        if ((tid & 15) == 0) vstore2(a.part_ml + 2 * base, M, L);
        vstore4(a.part_acc + base * D + d0, f32x4_t{acc[0], acc[1], acc[2], acc[3]});
        vstore4(a.part_acc + base * D + d0 + 4, f32x4_t{acc[4], acc[5], acc[6], acc[7]});
      }
    }
    if (last_seg) break;
    __syncthreads();                                        // s_m / s_l / s_o are reused
    next_seg(cs);
  }

  // ---- count in on the split items; the last workgroup of each merges it
  if (split0 || split1) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0x0F70);                     // this thread's partial stores are complete
    __syncthreads();
    if (tid == 0) {
      // workgroup g0 holds an item in slot 0 if the item opens its stretch,
      // else in slot 1; every later workgroup holds it in slot 0
      int r0 = 0, r1 = 0, g00 = 0, g10 = 0, g01 = 0, g11 = 0;
      if (split0) {
        g00 = owner_group(first0, U, W);
        g10 = owner_group(first0 + tiles_of(seq0) - 1, U, W);
        r0 = __hip_atomic_fetch_add(a.arrivals + g10, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      if (split1) {
        g01 = owner_group(first1, U, W);
        g11 = owner_group(first1 + tiles_of(seq1) - 1, U, W);
        r1 = __hip_atomic_fetch_add(a.arrivals + g11, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      const bool m0 = split0 && r0 == g10 - g00;
      const bool m1 = split1 && r1 == g11 - g01;
      if (m0) __hip_atomic_store(a.arrivals + g10, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (m1) __hip_atomic_store(a.arrivals + g11, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_merge[0] = m0 ? g00 : -1;
      s_merge[1] = m1 ? g01 : -1;
      s_merge[2] = (first0 == int64_t(g00) * U / W ? 0 : 1) | (first1 == int64_t(g01) * U / W ? 0 : 2);
      s_merge[3] = g10 - g00 + 1;
      s_merge[4] = g11 - g01 + 1;
    }
    __syncthreads();
    const int col = tid >> 4, d0 = (tid & 15) * 8;
    const int cg = col / TS, ct = col % TS;
#pragma unroll 1
    for (int it = 0; it < 2; ++it) {
      const int g0 = s_merge[it];
      if (g0 < 0) continue;
      const int sq = it ? seq1 : seq0, kh = it ? kvh1 : kvh0;
      const int cnt = s_merge[3 + it];
      const int slot0 = (s_merge[2] >> it) & 1;
      const int q0 = q0_of(sq), q_len = qlen_of(sq);
      if (ct >= q_len) continue;
      const float c = KV == KV_FP8 ? a.scale_log2 * a.k_scale[kh] : a.scale_log2;
      const float v_mul = KV == KV_FP8 ? a.v_scale[kh] : 1.f;
      float Mt = -INFINITY, Lt = 0.f, x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = 0.f;
      // the first part holds key 0, which every column sees, so Mt is finite
      // from the first fold on and later parts without keys weigh 0; the
      // loads of four parts are in flight at once
      constexpr int NB = 4;
      for (int i0 = 0; i0 < cnt; i0 += NB) {
        float mi[NB], li[NB], xi[NB][8];
#pragma unroll
        for (int r = 0; r < NB; ++r) {
          const int i = min(i0 + r, cnt - 1);
          const size_t b = (size_t(g0 + i) * 2 + (i ? 0 : slot0)) * 32 + col;
          vload2(a.part_ml + 2 * b, mi[r], li[r]);
#pragma unroll
          for (int e = 0; e < 8; e += 2) vload2(a.part_acc + b * D + d0 + e, xi[r][e], xi[r][e + 1]);
        }
#pragma unroll
        for (int r = 0; r < NB; ++r) {
          if (i0 + r >= cnt) break;
          const float mn = fmaxf(Mt, mi[r]);
          const float co = __builtin_amdgcn_exp2f((Mt - mn) * c), cn = __builtin_amdgcn_exp2f((mi[r] - mn) * c);
          Lt = fmaf(Lt, co, li[r] * cn);
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = fmaf(x[e], co, xi[r][e] * cn);
          Mt = mn;
        }
      }
      const float inv = v_mul / Lt;
      uint16_t* orow = static_cast<uint16_t*>(a.out) + (size_t(q0 + ct) * Hq + kh * G + cg) * D + d0;
      *reinterpret_cast<uint4*>(orow) =
          make_uint4(pack_bf16x2(x[0] * inv, x[1] * inv), pack_bf16x2(x[2] * inv, x[3] * inv),
                     pack_bf16x2(x[4] * inv, x[5] * inv), pack_bf16x2(x[6] * inv, x[7] * inv));
    }
  }
}

hipError_t launch_verify_chunk(const PrefillArgs& a0, int kv_kind, int block_size, int group, hipStream_t s) {
  PrefillArgs a = a0;
  const int64_t items = int64_t(a.num_seqs) * a.num_kv_heads;
  if (items == 0) return hipSuccess;
  // the unit prefix must fit in LDS beside the merge, and its sums in 31 bits
  const int64_t upper = items * ((int64_t(a.max_seq_len) + 31) / 32);
  if (a.num_seqs > kVerifySplitMaxSeqs || upper > 0x7FFFFFFF) a.part_acc = nullptr;
  int64_t wgs = items;
  size_t lds = 0;
  if (a.part_acc) {
    static int cus = 0;
    if (cus == 0) {
      int dev = 0;
      hipError_t e = hipGetDevice(&dev);
      if (e != hipSuccess) return e;
      e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
      if (e != hipSuccess) return e;
    }
    // one workgroup per CU (the cross-wave merge's LDS allows no second),
    // at most kVerifyMaxGroups (the workspace's partial slots), at most the
    // units the launch can have
    wgs = std::min<int64_t>(std::min<int64_t>(cus, kVerifyMaxGroups), std::max<int64_t>(upper, 1));
    a.total_groups = int32_t(wgs);
    lds = size_t(a.num_seqs + 1) * sizeof(int);
  }
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
#define PA_VF(kv, b, g) \
  if (kv_kind == kv && block_size == b && group == g) { \
    hipLaunchKernelGGL((verify_kernel<kv, b, g>), dim3(uint32_t(wgs)), dim3(kVerifyThreads), lds, s, a, \
                       a.block_table, a.cu_q_lens, a.seq_lens); \
    return hipGetLastError(); \
  }
#define PA_VF_G(kv, b) PA_VF(kv, b, 1) PA_VF(kv, b, 2) PA_VF(kv, b, 4) PA_VF(kv, b, 8)
  PA_VF_G(KV_BF16, 16) PA_VF_G(KV_BF16, 32) PA_VF_G(KV_FP8, 16) PA_VF_G(KV_FP8, 32)
#undef PA_VF_G
#undef PA_VF
  return hipErrorInvalidValue;
}

}  // namespace pa
