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
//  * One workgroup of eight waves per (sequence, kv head).  A wave's 32 MFMA
//    columns are the (query head, token) pairs of the group: column n is head
//    n / (32/G) and token n % (32/G).  Every K/V byte read serves all G heads
//    and all tokens of the chunk.
//  * The eight waves take the 32-key tiles kt = w, w + 8, ... and each keeps
//    an online softmax per column; their eight partial results are merged
//    through LDS at the end by log-sum-exp rescaling.  No workspace.
//  * Operands come straight from the paged pools (each tile is read by one
//    wave, so staging would not save bytes): K rows as the A operand of
//    S^T = K Q^T at MFMA row swap23(key), V^T (stored transposed per block)
//    as the A operand of O^T = V^T P^T.  The next tile's K is issued right
//    after this tile's S^T, its V right after this tile's PV; block ids come
//    through the scalar cache a tile earlier.
#include "mfma_attn.h"
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

constexpr int kVerifyWaves = 8;

template <int KV, int B, int G>
__global__ void __launch_bounds__(kVerifyWaves * 64) verify_kernel(PrefillArgs a,
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = uniform(tid >> 6);
  const int hh = lane >> 5;                      // lane half: k-slice of operands, row group of accumulators
  const int n = lane & 31;                       // MFMA column / operand row
  const int Hkv = a.num_kv_heads, Hq = a.num_q_heads;
  const int seq = blockIdx.x / Hkv, kvh = blockIdx.x - seq * Hkv;
  const int q0 = cu_q_lens[seq];
  const int q_len = cu_q_lens[seq + 1] - q0;
  if (q_len <= 0) return;                        // whole workgroup
  const int key_end = seq_lens[seq];             // keys 0 .. key_end - 1 (prefix and chunk)
  const int P = key_end - q_len;
  const int kmax = key_end - 1;
  const int n_tiles = (key_end + KT - 1) / KT;
  const int last = n_tiles - 1;
  const int gq = n / TS, t = n % TS;             // this lane's column: head gq of the group, chunk token t
  const int pos = P + t;                         // its absolute position
  const int head = kvh * G + gq;
  const int32_t* table = block_table + size_t(seq) * a.max_blocks_per_seq;
  const char* kpool = static_cast<const char*>(a.k_cache);
  const char* vpool = static_cast<const char*>(a.v_cache);
  using Raw = KvRaw<KV>;
  constexpr int ES = Raw::ES;                   // cache element bytes
  // an fp8 code of kv head h means code * scale[h]: K's scale goes into the
  // softmax constant, V's onto the output
  const float c = KV == KV_FP8 ? a.scale_log2 * a.k_scale[kvh] : a.scale_log2;
  const float v_mul = KV == KV_FP8 ? a.v_scale[kvh] : 1.f;

  // ---- Q^T as 8 B operands (k = 16 head dims each): row q0 + t, dims 16s + 8hh .. + 7
  uint4 qb[8];
  {
    const int row = q0 + min(t, q_len - 1);
    const uint16_t* qr = static_cast<const uint16_t*>(a.q) + (size_t(row) * Hq + head) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qb[s] = *reinterpret_cast<const uint4*>(qr + 16 * s);
  }

  // ---- operands of a tile (tiles past the last re-read the last one)
  typename Raw::T ka[8], va[4][2];               // raw loads; converted to bf16 at their use
  const int my_key = swap23(n);                  // key of MFMA row n within a tile
  auto tile_ids = [&](int kt, int& id0, int& id1) __attribute__((always_inline)) {
    const int b0 = kt * KT / B;
    id0 = table[min(b0, kmax / B)];
    id1 = table[min(b0 + 1, kmax / B)];
  };
  auto load_k = [&](int kt, int id0, int id1) __attribute__((always_inline)) {
    const int k0 = kt * KT;
    const int key = min(k0 + my_key, kmax);
    const int bid = key / B == k0 / B ? id0 : id1;
    const char* kr = kpool + ((size_t(bid) * Hkv + kvh) * B + key % B) * (D * ES) + 8 * ES * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) ka[s] = *reinterpret_cast<const typename Raw::T*>(kr + 16 * ES * s);
  };
  auto load_v = [&](int kt, int id0, int id1) __attribute__((always_inline)) {
    const int k0 = kt * KT;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int kb = min(k0 + 16 * ks + 8 * hh, kmax & ~7);   // 8 keys of one block
      const int bid = kb / B == k0 / B ? id0 : id1;
      const char* vb = vpool + (size_t(bid) * Hkv + kvh) * size_t(D * B * ES) + (kb % B) * ES;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        va[dt][ks] = *reinterpret_cast<const typename Raw::T*>(vb + size_t(32 * dt + n) * (B * ES));
    }
  };

  f32x16_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = f32x16_t{};
  float m_run = -INFINITY, l_run = 0.f;

  int id0, id1;
  tile_ids(min(w, last), id0, id1);
  // The query must be in registers before the first tile is requested: then
  // the loop is entered, from here or from its back edge, with the same two
  // groups of loads in flight, and its waits stay graded (no vmcnt(0)).
  __builtin_amdgcn_s_waitcnt(0x0F70);                       // vmcnt(0) only
  __builtin_amdgcn_sched_barrier(0);
  load_k(min(w, last), id0, id1);
  __builtin_amdgcn_sched_barrier(0);
  load_v(min(w, last), id0, id1);
  __builtin_amdgcn_sched_barrier(0);
  tile_ids(min(w + NW, last), id0, id1);                    // ids of each wave's next tile
  for (int kt = w; kt < n_tiles; kt += NW) {
    const int k0 = kt * KT;
    const int nxt = min(kt + NW, last);
    // ---- S^T = K Q^T; accumulator r = 4i + j is key k0 + swap23(8i + 4hh + j)
    f32x16_t sc = f32x16_t{};
#pragma unroll
    for (int st = 0; st < 8; ++st) sc = mfma32(Raw::to_bf16(ka[st]), qb[st], sc);
    __builtin_amdgcn_sched_barrier(0);
    load_k(nxt, id0, id1);                                  // next tile's keys fly during softmax + PV
    __builtin_amdgcn_sched_barrier(0);
    if (k0 + KT - 1 > P) {                                  // tile reaches the chunk: causal mask and end
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
    if (k0 + KT > key_end) {                                // zero V rows of keys past the end (NaN poison)
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
    load_v(nxt, id0, id1);                                  // its values fly during its S^T
    __builtin_amdgcn_sched_barrier(0);
    tile_ids(min(kt + 2 * NW, last), id0, id1);
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
  // thread -> (column, 8 dims): out = sum_w 2^((m_w - M) c) o_w / sum_w 2^((m_w - M) c) l_w
  static_assert(NW * 64 == 32 * D / 8, "one thread per 8 output dims of a column");
  const int col = tid >> 4, d0 = (tid & 15) * 8;
  const int cg = col / TS, ct = col % TS;
  if (ct >= q_len) return;                                  // slot without a token (no barrier follows)
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < NW; ++v) M = fmaxf(M, s_m[v][col]);
  float L = 0.f, acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const float wt = __builtin_amdgcn_exp2f((s_m[v][col] - M) * c);   // 0 for a wave without tiles
    L = fmaf(wt, s_l[v][col], L);
    const float4 x0 = *reinterpret_cast<const float4*>(&s_o[v][col][d0]);
    const float4 x1 = *reinterpret_cast<const float4*>(&s_o[v][col][d0 + 4]);
    acc[0] = fmaf(wt, x0.x, acc[0]); acc[1] = fmaf(wt, x0.y, acc[1]);
    acc[2] = fmaf(wt, x0.z, acc[2]); acc[3] = fmaf(wt, x0.w, acc[3]);
    acc[4] = fmaf(wt, x1.x, acc[4]); acc[5] = fmaf(wt, x1.y, acc[5]);
    acc[6] = fmaf(wt, x1.z, acc[6]); acc[7] = fmaf(wt, x1.w, acc[7]);
  }
  const float inv = v_mul / L;
  uint16_t* orow = static_cast<uint16_t*>(a.out) + (size_t(q0 + ct) * Hq + kvh * G + cg) * D + d0;
  *reinterpret_cast<uint4*>(orow) = make_uint4(pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                                               pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv));
}

hipError_t launch_verify_chunk(const PrefillArgs& a, int kv_kind, int block_size, int group, hipStream_t s) {
  const int64_t wgs = int64_t(a.num_seqs) * a.num_kv_heads;
  if (wgs == 0) return hipSuccess;
  if (wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
#define PA_VF(kv, b, g) \
  if (kv_kind == kv && block_size == b && group == g) { \
    hipLaunchKernelGGL((verify_kernel<kv, b, g>), dim3(uint32_t(wgs)), dim3(kVerifyWaves * 64), 0, s, a, \
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
