// Chunked-prefill attention over a paged prefix on gfx950 matrix cores.
//
// What it computes (nanoPD page, "分块预填充": long prompts are cut into
// chunks interleaved with decode; PD-engineering page 6.1 and serving-stack
// page 5.2: chunks of a few hundred tokens): sequence j appends a chunk of
// q_len tokens after P cached tokens; chunk row t, at absolute position
// P + t, attends to keys 0 .. P + t read through the block table.  Its own
// K/V were stored by pa_store_kv before the call.
//
// How (QK^T and PV are dense contractions, so they run on MFMA; bf16 in,
// fp32 accumulate):
//  * A wave owns 32 query rows of one query head; the four waves of a
//    workgroup share a kv head (the G = 4 heads of a query tile, or more
//    tiles of fewer heads).  The workgroup stages each 32-key K / V^T tile
//    once into LDS, swizzled so that the MFMA operand reads are free of bank
//    conflicts.  A bf16 cache is loaded straight into LDS (16-byte loads to
//    LDS, no registers) through a ring of four buffers, and each wave issues
//    the next tile's S^T MFMAs among this tile's exponentials (the matrix
//    cores then work under the wave's own softmax); an fp8 cache is loaded
//    into registers, converted to bf16 and written to a ring of three
//    buffers, with the same interleave.  One barrier per tile.  Block ids come
//    through the scalar cache.  Two workgroups share each CU, so the two waves on a
//    SIMD belong to different workgroups and do not pass their barriers
//    together: one's softmax can overlap the other's MFMAs.
//  * Scores are formed transposed, S^T = K Q^T with v_mfma_f32_32x32x16_bf16
//    (keys are MFMA rows, queries columns): every lane then owns one query
//    column, and the softmax statistics and the rescaling of O^T stay in the
//    lane (one exchange with lane ^ 32 per key tile, v_permlane32_swap).
//    The row sum l adds the bf16 probabilities PV multiplies, two per
//    v_dot2 against ones.
//  * K rows are loaded into MFMA row m = swap_bits_2_3(key), which makes the
//    accumulator layout of S^T equal to the B-operand layout of P^T for
//    O^T = V^T P^T: probabilities go straight from accumulators to bf16
//    operands, without a pass through LDS.  V is stored transposed per
//    block, so its A operand (8 consecutive keys of one head dimension) is
//    one 16-byte load.
//  * Online softmax in base 2 with the scale folded into exp2's argument
//    (the hardware v_exp_f32; results that would be denormal flush to zero,
//    far below bf16 resolution of the sum); O^T is rescaled only when some
//    column's running max grows by more than 2^8 (probabilities stay <= 256).
//  * The causal mask is applied only on key tiles that reach the diagonal;
//    keys past the sequence are masked by select and their V rows zeroed,
//    so NaN in unused slots never reaches the result.  The V operands are
//    read and masked before the next tile's S^T MFMAs are issued, so that
//    those MFMAs and this tile's exponentials share one basic block and
//    the forced interleave takes effect.  The next tile's K operands are
//    read from LDS at the start of the step, so that their latency passes
//    under this tile's masking and maximum.
//  * Workgroups of one (sequence, kv head) are placed on the same XCD
//    (workgroup id mod 8), so all query tiles of a sequence share that
//    XCD's L2 copy of its K/V.
#include "mfma_attn.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

// x of this lane and of lane ^ 32, combined (gfx950 v_permlane32_swap: no
// LDS round trip).
__device__ __forceinline__ float max_lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS swizzle of a key row's 16-byte chunks: chunk c of key row r sits at
// c ^ kswz(r).  Lane n reads key row swap23(n), so the lanes of any group of
// 8 or 16 read chunk c ^ (n & 15): distinct bank groups, no conflicts.
__device__ __forceinline__ int kswz(int r) { return swap23(r) & 15; }

// Sequences of a launch are ordered by work when there are at most this many.
constexpr int kPrefillSortMax = 256;

// Waves per workgroup: the four heads of a query tile (or more tiles of
// fewer heads) share every staged K / V tile.
constexpr int kPrefillWaves = 4;

template <int KV, int B, int G>
__global__ void __launch_bounds__(kPrefillWaves * 64, 2) prefill_kernel(PrefillArgs a, const int32_t* __restrict__ block_table,
                                                        const int32_t* __restrict__ cu_q_lens,
                                                        const int32_t* __restrict__ seq_lens) {
  constexpr int D = 128;
  constexpr int QT = 32;                 // query rows per wave
  constexpr int KT = 32;                 // keys per tile
  constexpr int KROW = D * 2;            // LDS bytes per key row; 16-byte chunks XOR-swizzled by kswz(row)
  constexpr int KBUF = KT * KROW;
  // A bf16 cache is staged straight from memory into LDS (16-byte loads to
  // LDS) through a ring of four buffers; an fp8 cache goes through
  // registers, converted to bf16, into a ring of three.  Both use the same
  // unpadded layout.
  constexpr bool DIRECT = KV == KV_BF16;
  constexpr int RBUF = KBUF + D * KT * 2;                  // ring buffer: K tile, then V^T tile
  __shared__ __attribute__((aligned(16))) char smem[3][DIRECT ? 16 : RBUF];  // ring of three (fp8)
  __shared__ __attribute__((aligned(16))) char ring0[DIRECT ? RBUF : 16];
  __shared__ __attribute__((aligned(16))) char ring1[DIRECT ? RBUF : 16];
  __shared__ __attribute__((aligned(16))) char ring2[DIRECT ? RBUF : 16];
  __shared__ __attribute__((aligned(16))) char ring3[DIRECT ? RBUF : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int hh = lane >> 5;              // lane half: k-slice of operands, row group of accumulators
  const int n = lane & 31;               // query column / operand row
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;

  // ---- workgroup -> (sequence, kv head, group of 4 column tiles), XCD-aware:
  // the workgroups of one (sequence, kv head) run on one XCD (id mod 8) and
  // share its L2.  Sequences are taken heaviest first (work ~ q_len * (2P +
  // q_len)), so that the longest chains of key tiles start first.
  const int id = blockIdx.x;
  const int xcd = id & 7;
  const int k8 = id >> 3;
  const int pair = (k8 / a.wg_per_pair) * 8 + xcd;       // rank of the (sequence, kv head)
  const int S = a.num_seqs;
  if (pair >= S * Hkv) return;                           // whole workgroup
  const int grp = k8 % a.wg_per_pair;
  int seq = pair / Hkv;
  const int kvh = pair - seq * Hkv;
  if (S <= kPrefillSortMax) {
    __shared__ float s_work[kPrefillSortMax];
    __shared__ int s_order[kPrefillSortMax];
    for (int i = tid; i < S; i += kPrefillWaves * 64) {
      const float ql = float(cu_q_lens[i + 1] - cu_q_lens[i]);
      s_work[i] = ql * (2.f * (float(seq_lens[i]) - ql) + ql);
    }
    __syncthreads();
    for (int i = tid; i < S; i += kPrefillWaves * 64) {
      const float wi = s_work[i];
      int rank = 0;
      for (int j = 0; j < S; ++j) rank += (s_work[j] > wi) || (s_work[j] == wi && j < i);
      s_order[rank] = i;
    }
    __syncthreads();
    seq = s_order[seq];
  }
  const int q0 = cu_q_lens[seq];
  const int q_len = cu_q_lens[seq + 1] - q0;
  const int total = seq_lens[seq];
  const int P = total - q_len;
  // wave w serves query head kvh * G + (col % G) on query tile qt (heavy, late tiles first)
  auto tile_of = [&](int wv) { return a.num_qtiles - 1 - (grp * kPrefillWaves + wv) / G; };
  auto key_end_of = [&](int wv) {                        // keys the wave's last row needs; 0 if idle
    const int t = tile_of(wv);
    return (t >= 0 && t * QT < q_len) ? P + min(q_len, (t + 1) * QT) : 0;
  };
  // the workgroup streams the keys any of its waves needs
  int key_end_wg = 0;
#pragma unroll
  for (int wv = 0; wv < kPrefillWaves; ++wv) key_end_wg = max(key_end_wg, key_end_of(wv));
  if (key_end_wg <= 0) return;                           // whole workgroup
  const int n_tiles_wg = (key_end_wg + KT - 1) / KT;
  const int kmax = key_end_wg - 1;
  const int col = grp * kPrefillWaves + w;
  const int h_local = col % G;
  const int qt = tile_of(w);
  const int key_end = key_end_of(w);
  const int n_tiles = (key_end + KT - 1) / KT;          // 0 for an idle wave
  const int head = kvh * G + h_local;
  const int t = qt * QT + n;                            // this lane's chunk row
  const bool valid_q = key_end > 0 && t < q_len;
  const int pos = P + t;                                 // absolute position of the query
  const int32_t* table = block_table + size_t(seq) * a.max_blocks_per_seq;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  using Raw = KvRaw<KV>;
  constexpr int ES = Raw::ES;                   // cache element bytes
  // an fp8 code of kv head h means code * scale[h]: K's scale goes into the
  // softmax constant, V's onto the output
  const float c = KV == KV_FP8 ? a.scale_log2 * a.k_scale[kvh] : a.scale_log2;
  const float v_mul = KV == KV_FP8 ? a.v_scale[kvh] : 1.f;

  // ---- staging of one tile by the whole workgroup through registers (fp8):
  // each thread moves NCH chunks of 8 elements of K (chunk i: row i / 16,
  // column chunk i % 16) and NCH of V^T (the chunk that the ring layout below
  // puts at LDS position i), chunks tid and tid + 64 * kPrefillWaves.
  constexpr int NCH = KT * 16 / (kPrefillWaves * 64);
  static_assert(NCH * kPrefillWaves * 64 == KT * 16 && NCH * kPrefillWaves * 64 == D * 4 && NCH <= 2,
                "whole chunks of K and V per thread");
  static_assert(B == KT || 2 * B == KT, "a tile is one or two blocks");
  // Per-thread constants: the chunk's offset inside its block's tile, which
  // of the tile's two blocks holds it (block 16: keys 16..31 and 8-key
  // groups 2, 3), and its LDS address.  A tile past the last key reads the
  // last block again (tile_ids clamps), so every address stays inside an
  // allocated block; those keys are masked.
  constexpr uint64_t kBlockTile = uint64_t(B) * D * ES;    // bytes of one (block, kv head) tile
  // V^T position i holds keys 8 g .. 8 g + 7 of head dim (i % 256) / 2 (see
  // the ring layout): consecutive lanes write consecutive 16-byte positions,
  // free of bank conflicts.
  auto vphi = [](int r) { return (r >> 3) & 1; };
  auto v_dim = [](int i) { return (i & 255) >> 1; };
  auto v_grp = [&](int i) { return 2 * (i >> 8) + ((i & 1) ^ vphi(v_dim(i))); };
  auto k_lane = [&](int i) { return uint64_t((((i >> 4) % B) * D + (i & 15) * 8) * ES); };
  auto v_lane = [&](int i) { return uint64_t((v_dim(i) * B + (8 * v_grp(i)) % B) * ES); };
  auto k_hi = [&](int i) { return B != KT && (i >> 4) >= B; };
  auto v_hi = [&](int i) { return B != KT && 8 * v_grp(i) >= B; };
  auto k_lds = [&](int i) { return (i >> 4) * KROW + ((i & 15) ^ kswz(i >> 4)) * 16; };
  auto v_lds = [&](int i) { return KBUF + i * 16; };
  const int ci0 = tid, ci1 = tid + kPrefillWaves * 64;
  const uint64_t k_lane0 = k_lane(ci0), k_lane1 = k_lane(ci1), v_lane0 = v_lane(ci0), v_lane1 = v_lane(ci1);
  const bool k_hi0 = k_hi(ci0), k_hi1 = k_hi(ci1), v_hi0 = v_hi(ci0), v_hi1 = v_hi(ci1);
  const int k_lds0 = k_lds(ci0), k_lds1 = k_lds(ci1), v_lds0 = v_lds(ci0), v_lds1 = v_lds(ci1);
  // (macros over plain variables: two staging sets, kept in registers)
#define PA_STAGE_LOAD(P, KT_, ID0, ID1)                                                                   \
  do {                                                                                                \
    const uint64_t t0_ = (uint64_t(uint32_t(ID0)) * uint32_t(Hkv) + uint32_t(kvh)) * kBlockTile;       \
    const uint64_t t1_ = (uint64_t(uint32_t(ID1)) * uint32_t(Hkv) + uint32_t(kvh)) * kBlockTile;       \
    P##k0 = *reinterpret_cast<const typename Raw::T*>(kpool + (k_hi0 ? t1_ : t0_) + k_lane0);         \
    P##v0 = *reinterpret_cast<const typename Raw::T*>(vpool + (v_hi0 ? t1_ : t0_) + v_lane0);         \
    if constexpr (NCH > 1) {                                                                          \
      P##k1 = *reinterpret_cast<const typename Raw::T*>(kpool + (k_hi1 ? t1_ : t0_) + k_lane1);       \
      P##v1 = *reinterpret_cast<const typename Raw::T*>(vpool + (v_hi1 ? t1_ : t0_) + v_lane1);       \
    }                                                                                                 \
  } while (0)
#define PA_STAGE_STORE(P, BUF)                                                                        \
  do {                                                                                                \
    char* sb_ = smem[BUF];                                                                            \
    *reinterpret_cast<uint4*>(sb_ + k_lds0) = Raw::to_bf16(P##k0);                                    \
    *reinterpret_cast<uint4*>(sb_ + v_lds0) = Raw::to_bf16(P##v0);                                    \
    if constexpr (NCH > 1) {                                                                          \
      *reinterpret_cast<uint4*>(sb_ + k_lds1) = Raw::to_bf16(P##k1);                                  \
      *reinterpret_cast<uint4*>(sb_ + v_lds1) = Raw::to_bf16(P##v1);                                  \
    }                                                                                                 \
  } while (0)
  // block ids of a tile's (at most two) blocks, read through the scalar cache
  auto tile_ids = [&](int kt, int& id0, int& id1) __attribute__((always_inline)) {
    const int b0 = kt * KT / B;
    id0 = table[min(b0, kmax / B)];
    id1 = table[min(b0 + 1, kmax / B)];
  };

  // Ring layout (16-byte positions).  A load to LDS puts lane l's 16 bytes
  // at the wave's base + 16 l, so the layout is chosen per LDS position and
  // each lane loads the chunk that belongs there.  K: position 16 r + (c ^
  // kswz(r)) holds chunk c of key row r (rows of 256 bytes).  V^T: keys
  // 0..15 of every head dim in positions 0..255, keys 16..31 in 256..511, so
  // that each staging load (positions 256 j + tid) reads from one block at
  // block size 16: position 256 (g / 2) + 2 r + ((g & 1) ^ vphi(r)) holds
  // keys 8g .. 8g + 7 of head dim r.  The operand reads (lane n: dim 32 dt +
  // n, one g per half wave) then fall on distinct 16-byte bank groups in
  // every 8 and every 16 lanes.
  auto v_pos = [&](int r, int g) { return 256 * (g >> 1) + 2 * r + ((g & 1) ^ vphi(r)); };
  // thread tid fills positions tid and tid + 256 of each tile (lane l of wave
  // w writes position 256 j + 64 w + l); load j reads block j of the tile at
  // block size 16 (block 0 at 32), at a per-thread 32-bit offset
  uint32_t dk_off[2], dv_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int pk = tid + 256 * j;
    const int row = pk >> 4, colc = (pk & 15) ^ kswz(row);
    dk_off[j] = uint32_t(((row % B) * D + colc * 8) * 2);
    const int dim = tid >> 1, g = 2 * j + ((tid & 1) ^ vphi(tid >> 1));
    dv_off[j] = uint32_t((dim * B + (8 * g) % B) * 2);
  }
  auto direct_stage = [&](char* base, int id0, int id1) __attribute__((always_inline)) {
    const uint64_t t0_ = (uint64_t(uint32_t(id0)) * uint32_t(Hkv) + uint32_t(kvh)) * kBlockTile;
    const uint64_t t1_ = B == KT ? t0_ : (uint64_t(uint32_t(id1)) * uint32_t(Hkv) + uint32_t(kvh)) * kBlockTile;
    const char* kb0 = kpool + t0_;
    const char* kb1 = kpool + t1_;
    const char* vb0 = vpool + t0_;
    const char* vb1 = vpool + t1_;
    __builtin_amdgcn_global_load_lds(kb0 + dk_off[0], (__attribute__((address_space(3))) void*)(base + 64 * w * 16), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb0 + dv_off[0], (__attribute__((address_space(3))) void*)(base + KBUF + 64 * w * 16), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(kb1 + dk_off[1], (__attribute__((address_space(3))) void*)(base + (256 + 64 * w) * 16), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vb1 + dv_off[1], (__attribute__((address_space(3))) void*)(base + KBUF + (256 + 64 * w) * 16), 16, 0, 0);
  };

  // ---- Q^T as 8 B operands (k = 16 head dims each): row q0 + t, dims 16s + 8hh .. + 7
  uint4 qb[8];
  {
    const int row = q0 + max(0, min(t, q_len - 1));
    const uint16_t* qr = static_cast<const uint16_t*>(a.q) + (size_t(row) * Hq + head) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qb[s] = *reinterpret_cast<const uint4*>(qr + 16 * s);
  }

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;
  const int my_key = swap23(n);                          // key of MFMA row n within a tile
  const int first_row_pos = P + qt * QT;                 // smallest query position of the tile

  // Two staging register sets: a tile's global loads are issued two tiles
  // before its own MFMAs and written to LDS one tile before them, so about
  // two tiles of MFMA work cover each load's latency.  Tiles past the last
  // re-read the last one.
  // A tile in three parts.  read_k + qk_mfma: S^T = K Q^T (A: lane row n =
  // key k0 + my_key, dims 16s + 8hh).  mask_rescale: causal and end masks,
  // the tile maximum and the lazy rescale.  probs_pv: probabilities and
  // O^T += V^T P^T, with the next tile's S^T MFMAs issued among its
  // exponentials.  Every wave runs every tile of its workgroup: a tile past
  // a wave's own keys is masked whole (probabilities 0, V rows zeroed),
  // which leaves its results bit for bit as they would be without it.
  auto read_k = [&](const char* sb, uint4 (&ka)[8]) __attribute__((always_inline)) {
#pragma unroll
    for (int s = 0; s < 8; ++s)
      ka[s] = *reinterpret_cast<const uint4*>(sb + my_key * KROW + ((2 * s + hh) ^ kswz(my_key)) * 16);
  };
  auto qk_mfma = [&](const uint4 (&ka)[8]) __attribute__((always_inline)) -> f32x16_t {
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int st = 0; st < 8; ++st) sc = mfma32(ka[st], qb[st], sc);
    return sc;
  };
  auto qk_tile = [&](const char* sb) __attribute__((always_inline)) -> f32x16_t {
    uint4 ka[8];
    read_k(sb, ka);
    return qk_mfma(ka);
  };
  auto mask_rescale = [&](int kt, f32x16_t& sc) __attribute__((always_inline)) {
      const int k0 = kt * KT;
      // accumulator r = 4i + j holds MFMA row 8i + 4hh + j, i.e. key k0 + swap23(8i + 4hh + j)
      if (k0 + KT - 1 > first_row_pos) {                 // tile reaches the diagonal or the end
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + swap23(8 * (r >> 2) + 4 * hh + (r & 3));
          sc[r] = (key <= pos && key < key_end) ? sc[r] : -INFINITY;
        }
      }
      float mt = sc[0];
#pragma unroll
      for (int r = 1; r < 16; ++r) mt = fmaxf(mt, sc[r]);
      mt = max_lane_xor32(mt);
      const float m_new = fmaxf(m_run, mt);
      // O^T and l are rescaled only when some column's maximum grew by more
      // than 2^8 in exp2 units: until then the stale maximum keeps every
      // probability <= 256, which bf16 and fp32 hold at full relative
      // precision, and the final division by l is unchanged.  The first tile
      // always rescales (m_run = -inf), and it holds key 0, unmasked in
      // every column, so m_run is finite from then on.
      if (__any((m_new - m_run) * c > 8.f)) {
        const float al = __builtin_amdgcn_exp2f((m_run - m_new) * c);
        l_run *= al;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= al;
        m_run = m_new;
      }
  };
  // V^T operands of tile kt (d-tile dt: dims 32dt + n; key slice ks: keys
  // k0 + 16ks + 8hh .. + 7), with the rows of keys past the wave's keys
  // zeroed (NaN poison past the sequence).
  auto v_operands = [&](int kt, const char* sb, uint4 (&va)[4][2]) __attribute__((always_inline)) {
      const int k0 = kt * KT;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          va[dt][ks] = *reinterpret_cast<const uint4*>(sb + KBUF + v_pos(32 * dt + n, 2 * ks + hh) * 16);
      if (k0 + KT > key_end) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int kb = k0 + 16 * ks + 8 * hh;
          uint32_t msk[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            msk[e] = (kb + 2 * e < key_end ? 0x0000FFFFu : 0u) | (kb + 2 * e + 1 < key_end ? 0xFFFF0000u : 0u);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) {
            va[dt][ks].x &= msk[0]; va[dt][ks].y &= msk[1]; va[dt][ks].z &= msk[2]; va[dt][ks].w &= msk[3];
          }
        }
      }
  };
  // Probabilities of tile kt and O^T += V^T P^T (V operands va, read and
  // masked by the caller before the tile maximum, so that their LDS latency
  // passes under it and the masking branch does not split the MFMAs from
  // the exponentials), with the next tile's S^T (from its K operands
  // ka_next, read earlier) issued among the exponentials.
  auto probs_pv = [&](const f32x16_t& sc, const uint4 (&va)[4][2], f32x16_t& s_next,
                      const uint4 (&ka_next)[8]) __attribute__((always_inline)) {
      s_next = qk_mfma(ka_next);
      float p[16];
      const float mc = m_run * c;
#pragma unroll
      for (int r = 0; r < 16; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(sc[r], c, -mc));
      // P^T operands: key slice ks takes accumulators 8ks .. 8ks + 7 (keys k0 + 16ks + 8hh + 0..7)
      uint4 pb[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        pb[ks] = make_uint4(pack_bf16x2(p[8 * ks + 0], p[8 * ks + 1]), pack_bf16x2(p[8 * ks + 2], p[8 * ks + 3]),
                            pack_bf16x2(p[8 * ks + 4], p[8 * ks + 5]), pack_bf16x2(p[8 * ks + 6], p[8 * ks + 7]));
      // l sums the probabilities PV uses: the bf16 pairs, two per v_dot2
      constexpr uint32_t kOnes = 0x3F803F80u;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        l_run = dot2_bf16(pb[ks].x, kOnes, l_run);
        l_run = dot2_bf16(pb[ks].y, kOnes, l_run);
        l_run = dot2_bf16(pb[ks].z, kOnes, l_run);
        l_run = dot2_bf16(pb[ks].w, kOnes, l_run);
      }
      // twelve MFMAs (the next tile's eight S^T, then the first key slice's
      // four PV) each followed by a few vector or transcendental
      // instructions of this tile (the exponentials count: mask 0x002 alone
      // leaves them out), so that the matrix cores work under this wave's
      // own softmax.  Five per MFMA for a bf16 cache, four for fp8 (measured
      // best of 4-6 on the mixed batch).
      constexpr int kValuPerMfma = DIRECT ? 5 : 4;
#pragma unroll
      for (int r = 0; r < 12; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x402, kValuPerMfma, 1);
      }
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        o[dt] = mfma32(va[dt][0], pb[0], o[dt]);
        o[dt] = mfma32(va[dt][1], pb[1], o[dt]);
      }
  };
  const int last = n_tiles_wg - 1;
  int j0, j1;
  if constexpr (DIRECT) {
    // Ring of four buffers.  Step kt processes tile kt (its S^T was issued
    // one step earlier) and issues tile kt + 1's S^T, so tile kt + 1 must be
    // in LDS when step kt starts, and tile kt + 3 is requested into the
    // buffer that held tile kt - 1, which every wave finished reading before
    // the barrier that opens step kt.  A thread has four loads per tile, so
    // once only its four newest (tile kt + 2) are in flight (vmcnt(4)), its
    // part of tile kt + 1 is in LDS, and after the barrier all of it is.  The
    // barrier is a plain s_barrier between compiler-only fences: a
    // __syncthreads() would also wait for tile kt + 2.  Each buffer is a
    // distinct array named statically, so the compiler does not take loads
    // into one for writes to the one being read (it would wait for them
    // before every LDS read).
#define PA_RING_SYNC()                                                                                 \
    __builtin_amdgcn_s_waitcnt(0x0F74); /* vmcnt(4) */                                                 \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);                                                           \
    __builtin_amdgcn_s_barrier();                                                                      \
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    tile_ids(0, j0, j1);
    direct_stage(ring0, j0, j1);
    tile_ids(min(1, last), j0, j1);
    direct_stage(ring1, j0, j1);
    tile_ids(min(2, last), j0, j1);
    direct_stage(ring2, j0, j1);
    tile_ids(min(3, last), j0, j1);
    __builtin_amdgcn_s_waitcnt(0x0F78);                     // vmcnt(8): tile 0 is in LDS
    __syncthreads();                                          // (once: also settles the query loads)
    f32x16_t s_cur = qk_tile(ring0);
#define PA_RING_STEP(KT_, CUR, NXT, LD)                                                                \
    PA_RING_SYNC()                                                                                     \
    direct_stage(LD, j0, j1);                                                                          \
    tile_ids(min((KT_) + 4, last), j0, j1);                                                            \
    {                                                                                                  \
      f32x16_t s_nxt;                                                                                  \
      uint4 ka_n[8];                                                                                   \
      uint4 va[4][2];                                                                                  \
      read_k(NXT, ka_n);                 /* next tile's K and this tile's V operands: their latency */ \
      v_operands((KT_), CUR, va);        /* under the tile maximum */                                 \
      mask_rescale((KT_), s_cur);                                                                      \
      probs_pv(s_cur, va, s_nxt, ka_n);                                                                \
      s_cur = s_nxt;                                                                                   \
    }
    for (int kt = 0; kt < n_tiles_wg; kt += 4) {
      PA_RING_STEP(kt, ring0, ring1, ring3)
      if (kt + 1 >= n_tiles_wg) break;
      PA_RING_STEP(kt + 1, ring1, ring2, ring0)
      if (kt + 2 >= n_tiles_wg) break;
      PA_RING_STEP(kt + 2, ring2, ring3, ring1)
      if (kt + 3 >= n_tiles_wg) break;
      PA_RING_STEP(kt + 3, ring3, ring0, ring2)
    }
#undef PA_RING_STEP
#undef PA_RING_SYNC
    __builtin_amdgcn_s_waitcnt(0x0F70);                     // vmcnt(0): no load into LDS outlives the loop
  } else {
  // Ring of three buffers filled through registers (fp8 codes converted to
  // bf16 on the way): step kt computes tile kt + 1's S^T among tile kt's
  // exponentials, then writes tile kt + 2 (loaded one step earlier) into the
  // buffer that held tile kt - 1, and requests tile kt + 3 into the register
  // set that tile kt + 2 leaves.
  typename Raw::T sa_k0{}, sa_v0{}, sb_k0{}, sb_v0{}, sa_k1{}, sa_v1{}, sb_k1{}, sb_v1{};
  tile_ids(0, j0, j1);
  PA_STAGE_LOAD(sa_, 0, j0, j1);
  tile_ids(min(1, last), j0, j1);
  PA_STAGE_LOAD(sb_, min(1, last), j0, j1);
  tile_ids(min(2, last), j0, j1);
  PA_STAGE_STORE(sa_, 0);                                    // tile 0
  PA_STAGE_LOAD(sa_, min(2, last), j0, j1);
  tile_ids(min(3, last), j0, j1);
  PA_STAGE_STORE(sb_, 1);                                    // tile 1
  __syncthreads();
  f32x16_t s_cur = qk_tile(smem[0]);
#define PA_FP8_STEP(KT_, LD, ST, CUR, NXT, SBUF)                                                       \
  PA_STAGE_LOAD(LD, 0, j0, j1);                              /* tile KT_ + 3 */                        \
  tile_ids(min((KT_) + 4, last), j0, j1);                                                             \
  {                                                                                                   \
    f32x16_t s_nxt;                                                                                   \
    uint4 ka_n[8];                                                                                    \
    uint4 va[4][2];                                                                                   \
    read_k(NXT, ka_n);                                                                                \
    v_operands((KT_), CUR, va);                                                                       \
    mask_rescale((KT_), s_cur);                                                                       \
    probs_pv(s_cur, va, s_nxt, ka_n);                                                                 \
    s_cur = s_nxt;                                                                                    \
  }                                                                                                   \
  PA_STAGE_STORE(ST, SBUF);                                  /* tile KT_ + 2 */                        \
  __syncthreads();
  for (int kt = 0; kt < n_tiles_wg; kt += 6) {
    PA_FP8_STEP(kt, sb_, sa_, smem[0], smem[1], 2)
    if (kt + 1 >= n_tiles_wg) break;
    PA_FP8_STEP(kt + 1, sa_, sb_, smem[1], smem[2], 0)
    if (kt + 2 >= n_tiles_wg) break;
    PA_FP8_STEP(kt + 2, sb_, sa_, smem[2], smem[0], 1)
    if (kt + 3 >= n_tiles_wg) break;
    PA_FP8_STEP(kt + 3, sa_, sb_, smem[0], smem[1], 2)
    if (kt + 4 >= n_tiles_wg) break;
    PA_FP8_STEP(kt + 4, sb_, sa_, smem[1], smem[2], 0)
    if (kt + 5 >= n_tiles_wg) break;
    PA_FP8_STEP(kt + 5, sa_, sb_, smem[2], smem[0], 1)
  }
#undef PA_FP8_STEP
  }
#undef PA_STAGE_LOAD
#undef PA_STAGE_STORE

  // ---- normalise and store: accumulator r of d-tile dt is dim 32dt + 8(r/4) + 4hh + (r%4)
  const float l = sum_lane_xor32(l_run);
  if (!valid_q) return;
  const float inv = v_mul / l;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + (size_t(q0 + t) * Hq + head) * D + 4 * hh;
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 4 * i;
      *reinterpret_cast<uint2*>(orow + 32 * dt + 8 * i) =
          make_uint2(pack_bf16x2(o[dt][r] * inv, o[dt][r + 1] * inv), pack_bf16x2(o[dt][r + 2] * inv, o[dt][r + 3] * inv));
    }
}

hipError_t launch_prefill_chunk(const PrefillArgs& a0, int kv_kind, int block_size, int group, hipStream_t s) {
  // chunks of at most 32 / G tokens (speculative verification) fill the MFMA
  // columns with (head, token) pairs instead of 32 rows of one head
  if (int64_t(a0.max_q_len) * group <= 32) return launch_verify_chunk(a0, kv_kind, block_size, group, s);
  PrefillArgs a = a0;
  a.num_qtiles = (a.max_q_len + 31) / 32;
  a.wg_per_pair = (group * a.num_qtiles + kPrefillWaves - 1) / kPrefillWaves;
  const int64_t pairs = int64_t(a.num_seqs) * a.num_kv_heads;
  const int64_t wgs = ((pairs + 7) / 8) * 8 * a.wg_per_pair;
  if (wgs == 0) return hipSuccess;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
#define PA_PF(kv, b, g) \
  if (kv_kind == kv && block_size == b && group == g) { \
    hipLaunchKernelGGL((prefill_kernel<kv, b, g>), dim3(uint32_t(wgs)), dim3(kPrefillWaves * 64), 0, s, a, \
                       a.block_table, a.cu_q_lens, a.seq_lens); \
    return hipGetLastError(); \
  }
#define PA_PF_G(kv, b) PA_PF(kv, b, 1) PA_PF(kv, b, 2) PA_PF(kv, b, 4) PA_PF(kv, b, 8)
  PA_PF_G(KV_BF16, 16) PA_PF_G(KV_BF16, 32) PA_PF_G(KV_FP8, 16) PA_PF_G(KV_FP8, 32)
#undef PA_PF_G
#undef PA_PF
  return hipErrorInvalidValue;
}

}  // namespace pa
