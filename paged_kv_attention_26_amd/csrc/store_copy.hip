// Paged KV store (scatter of new K/V rows into their slots) and whole-block
// copy for copy-on-write, gfx950.
//
// Store: the nanoPD page lists a store operation for the paged KV cache
// beside its attention kernel; the serving-stack page, section 2.3, places a
// sequence's new token at offset length % block_size of its last block.
// Here a slot is physical_block * block_size + offset.
// Pack: the inverse gather, a request's cached K/V out of its blocks into
// contiguous token rows, the form in which the prefill side hands KV to the
// decode side (nanoPD page, 异步KV传输; PD-engineering page section 3).
// Copy: copy on write of a shared block before a forked sequence writes into
// it (nanoPD page, paged KV cache with CoW; serving-stack page 2.3, cow()).
#include "pa_device.h"
#include "pa_internal.h"
#include "store_row.h"

namespace pa {

// 16-byte loads with the non-temporal hint (nt), for data a launch reads
// once with each line read whole by one instruction: the block copy's
// source blocks (5.39 -> 6.02 TB/s) and the tile store's key input rows
// (16 lanes take a head's 256-byte slice of a token row; 4.95 -> 5.03 TB/s).
// The store's value input loads take one 16-byte chunk of a token row per
// lane, eight instructions to a line, and keep the default policy: with the
// hint on them too the store lost a third of its bandwidth.  Stores keep the
// default policy (with the hint both kernels measured slower).
__device__ __forceinline__ uint4 stream_load(const uint4* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// One workgroup = 64 consecutive tokens x one kv head.
//  K: 16-byte input chunks, mapped so that consecutive lanes cover one key
//     row: reads and writes are both contiguous.
//  V: read with lane = token.  Tokens that land at consecutive offsets of one
//     block form a run; the first RMAX runs of the workgroup are placed in
//     an LDS tile [head dim][run, offset in block] of cache elements and
//     leave in 16-byte pieces of transposed block rows (one store per piece
//     a run covers whole; element stores for the pieces at its ends), so the
//     lanes of a wave cover whole block rows one after another.  Tokens of
//     later runs (a workgroup of scattered single tokens) are written
//     element by element straight from registers.
template <int KV>
__global__ void __launch_bounds__(256) store_kv_kernel(StoreArgs a) {
  constexpr int IN_ES = (KV == KV_F32) ? 4 : (KV == KV_FP8_RAW ? 1 : 2);   // input element bytes
  constexpr int OUT_ES = (KV == KV_F32) ? 4 : (KV == KV_BF16 ? 2 : 1);
  constexpr int EPC = 16 / IN_ES;                          // elements per 16-byte chunk
  constexpr int TPG = 16 / OUT_ES;                         // tokens per 16-byte piece of a block row
  constexpr int COLS = OUT_ES == 4 ? 64 : 128;             // LDS columns: RMAX runs x block size
  constexpr int ROWB = COLS * OUT_ES + 16;                 // LDS bytes per head-dim row (padded)
  __shared__ __attribute__((aligned(16))) char s_vt[128 * ROWB];
  __shared__ int s_rblk[64], s_rlo[64], s_rhi[64];        // per staged run: block, offsets [lo, hi)
  const int H = a.num_kv_heads, D = a.head_dim, BS = a.block_size;
  // Workgroup -> (64-token tile, kv head), XCD-aware: workgroup i runs on XCD
  // i mod 8, and each XCD takes a contiguous stretch of tiles (all heads of a
  // tile, then the next tile), so that the two workgroups sharing a block that
  // a run straddles usually meet in one L2 and the block's lines go to memory
  // whole, and an XCD reads whole input rows.
  const int ntiles = (a.num_tokens + 63) / 64;
  const int per_xcd = int(gridDim.x) / 8;
  const int idx = int(blockIdx.x % 8) * per_xcd + int(blockIdx.x / 8);
  if (idx >= ntiles * H) return;                           // padding workgroup, before any barrier
  const int tile = idx / H;
  const int h = idx - tile * H;
  const int t0 = tile * 64;
  const int cpr = a.head_dim / EPC;                        // chunks per row

  const char* kin = static_cast<const char*>(a.k_new);
  const char* vin = static_cast<const char*>(a.v_new);
  char* kc = static_cast<char*>(a.k_cache);
  char* vc = static_cast<char*>(a.v_cache);
  float ksc = 1.f, vsc = 1.f;
  if constexpr (KV == KV_FP8) {
    ksc = a.k_scale[h];
    vsc = a.v_scale[h];
  }

  // Every load of a thread goes out before its first store (the stores could
  // alias the inputs as far as the compiler knows, so a load-store loop would
  // keep one load in flight per thread).  Loads are unconditional, clamped to
  // the workgroup's last token; only the stores are guarded.
  const int nt = min(64, a.num_tokens - t0);
  const int nkc = nt * cpr;                                // key chunks of the workgroup
  constexpr int KI = (64 * 128 / EPC) / 256;               // key chunks per thread at head_dim 128
  uint4 kx[KI];
  int ks[KI];
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int idx = min(int(threadIdx.x) + 256 * i, nkc - 1);
    kx[i] = stream_load(reinterpret_cast<const uint4*>(kin + ((size_t(t0 + idx / cpr) * H + h) * D + size_t(idx % cpr) * EPC) * IN_ES));
    ks[i] = a.slot_mapping[t0 + idx / cpr];
  }
  // values: lane = token, wave w takes chunks w, w + 4, ...
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int tv = t0 + min(lane, nt - 1);
  constexpr int VI = (128 / EPC) / 4;                      // value chunks per lane at head_dim 128
  const int vslot = a.slot_mapping[tv];
  uint4 vx[VI];
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int c = min(wave + 4 * i, cpr - 1);
    vx[i] = *reinterpret_cast<const uint4*>(vin + ((size_t(tv) * H + h) * D + size_t(c) * EPC) * IN_ES);
  }

  // ---- keys: contiguous rows
#pragma unroll
  for (int i = 0; i < KI; ++i) {
    const int idx = threadIdx.x + 256 * i;
    if (idx >= nkc) break;
    const int c = idx % cpr;
    const int slot = ks[i];
    if (slot < 0) continue;
    const int blk = slot / BS, off = slot % BS;
    const uint4 x = kx[i];
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

  // ---- runs of the values' slots (every wave derives them from the slots
  // it loaded; wave 0 records each staged run's block and offsets)
  const int BS_ = BS;
  const int RMAX = COLS / BS_;
  const int slot = lane < nt ? vslot : -1;
  int prev = __shfl(slot, (lane + 63) & 63);
  if (lane == 0) prev = -1;
  const bool live = slot >= 0;
  const int off = live ? slot % BS_ : 0;
  const bool starts = live && (prev < 0 || slot != prev + 1 || off == 0);
  const uint64_t sb = __ballot(starts);
  const uint64_t lb = __ballot(live);
  const int r = __popcll(sb & ((2ull << lane) - 1ull)) - 1;  // run index of this token
  const bool staged = live && r < RMAX;
  const int nrun = min(__popcll(sb), RMAX);
  if (wave == 0 && staged) {
    const bool ends = lane == 63 || !((lb >> (lane + 1)) & 1ull) || ((sb >> (lane + 1)) & 1ull);
    if (starts) {
      s_rblk[r] = slot / BS_;
      s_rlo[r] = off;
    }
    if (ends) s_rhi[r] = off + 1;
  }

  // ---- values into LDS, encoded: s_vt[d * ROWB + (r * BS + off) * OUT_ES];
  // tokens of runs past the staged ones go out element by element
  char* col = s_vt + (staged ? r * BS_ + off : 0) * OUT_ES;
  char* vrow = vc + ((size_t(live ? slot / BS_ : 0) * H + h) * D) * size_t(BS_) * OUT_ES + size_t(off) * OUT_ES;
#pragma unroll
  for (int i = 0; i < VI; ++i) {
    const int c = wave + 4 * i;
    if (c >= cpr) break;
    const uint4 x = vx[i];
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint8_t e8[16];
    uint32_t e32[4];
    uint16_t e16[8];
    if constexpr (KV == KV_F32) {
#pragma unroll
      for (int e = 0; e < 4; ++e) e32[e] = w[e];
    } else if constexpr (KV == KV_BF16) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        e16[2 * e] = uint16_t(w[e] & 0xFFFFu);
        e16[2 * e + 1] = uint16_t(w[e] >> 16);
      }
    } else if constexpr (KV == KV_FP8_RAW) {
#pragma unroll
      for (int e = 0; e < 16; ++e) e8[e] = uint8_t(w[e >> 2] >> (8 * (e & 3)));
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        e8[2 * e] = uint8_t(e4m3_encode(bf16_lo(w[e]) / vsc));
        e8[2 * e + 1] = uint8_t(e4m3_encode(bf16_hi(w[e]) / vsc));
      }
    }
    const int d0 = c * EPC;
    if (staged) {
      char* p = col + size_t(d0) * ROWB;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if constexpr (OUT_ES == 4) *reinterpret_cast<uint32_t*>(p + e * ROWB) = e32[e];
        else if constexpr (OUT_ES == 2) *reinterpret_cast<uint16_t*>(p + e * ROWB) = e16[e];
        else p[e * ROWB] = char(e8[e]);
      }
    } else if (live) {
      char* q = vrow + size_t(d0) * BS_ * OUT_ES;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        if constexpr (OUT_ES == 4) *reinterpret_cast<uint32_t*>(q + e * BS_ * 4) = e32[e];
        else if constexpr (OUT_ES == 2) *reinterpret_cast<uint16_t*>(q + e * BS_ * 2) = e16[e];
        else q[e * BS_] = char(e8[e]);
      }
    }
  }
  __syncthreads();

  // ---- staged runs out: item = (run, head-dim row, 16-byte piece of the
  // block row); consecutive items walk the pieces of a row, then the rows
  const int ppr = BS_ / TPG;                               // pieces per block row
  const int items = nrun * ppr * D;
  for (int it = threadIdx.x; it < items; it += 256) {
    const int k = it % ppr;
    const int d = (it / ppr) % D;
    const int rr = it / (ppr * D);
    const int lo = s_rlo[rr], hi = s_rhi[rr];
    const int c0 = k * TPG, c1 = c0 + TPG;
    if (hi <= c0 || c1 <= lo) continue;                    // piece outside the run
    const char* src = s_vt + d * ROWB + rr * BS_ * OUT_ES;
    char* dst = vc + ((size_t(s_rblk[rr]) * H + h) * D + d) * size_t(BS_) * OUT_ES;
    if (lo <= c0 && c1 <= hi) {
      *reinterpret_cast<uint4*>(dst + c0 * OUT_ES) = *reinterpret_cast<const uint4*>(src + c0 * OUT_ES);
    } else {
      for (int o = max(lo, c0); o < min(hi, c1); ++o) {
        if constexpr (OUT_ES == 4) *reinterpret_cast<uint32_t*>(dst + 4 * o) = *reinterpret_cast<const uint32_t*>(src + 4 * o);
        else if constexpr (OUT_ES == 2) *reinterpret_cast<uint16_t*>(dst + 2 * o) = *reinterpret_cast<const uint16_t*>(src + 2 * o);
        else dst[o] = src[o];
      }
    }
  }
}

// Stores of at most this many tokens take one wave per (token, kv head);
// larger ones take the 64-token tiles above, which group each block's run
// of slots.
constexpr int kStoreRowsMaxTokens = 128;

// The store of a few scattered tokens (a decode step: one new token per
// sequence), where the time is latency, not bandwidth.  One wave per (token,
// kv head), so a 32-token step spreads over 256 waves instead of eight
// workgroups (the wave's work is store_row).
template <int KV>
__global__ void __launch_bounds__(256) store_rows_kernel(StoreArgs a) {
  const int H = a.num_kv_heads, D = a.head_dim;
  const int64_t pair = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (pair >= int64_t(a.num_tokens) * H) return;           // no barrier in this kernel
  const int t = int(pair / H), h = int(pair - int64_t(t) * H);
  constexpr int IN_ES = (KV == KV_F32) ? 4 : (KV == KV_FP8_RAW ? 1 : 2);   // input element bytes
  const char* krow = static_cast<const char*>(a.k_new) + (size_t(t) * H + h) * D * IN_ES;
  const char* vrow = static_cast<const char*>(a.v_new) + (size_t(t) * H + h) * D * IN_ES;
  float ksc = 1.f, vsc = 1.f;
  if constexpr (KV == KV_FP8) {
    ksc = a.k_scale[h];
    vsc = a.v_scale[h];
  }
  store_row<KV>(krow, vrow, a.k_cache, a.v_cache, a.slot_mapping[t], h, H, D, a.block_size, ksc, vsc);
}

// One workgroup row per pair; 16-byte chunks of the block in both pools,
// loaded with the non-temporal hint.
__global__ void __launch_bounds__(256) copy_blocks_kernel(CopyArgs a) {
  const int p = blockIdx.x;
  const int src = a.pairs[2 * p], dst = a.pairs[2 * p + 1];
  const size_t n16 = a.block_bytes / 16;
  const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_cache) + size_t(src) * a.block_bytes);
  uint4* kd = reinterpret_cast<uint4*>(static_cast<char*>(a.k_cache) + size_t(dst) * a.block_bytes);
  const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_cache) + size_t(src) * a.block_bytes);
  uint4* vd = reinterpret_cast<uint4*>(static_cast<char*>(a.v_cache) + size_t(dst) * a.block_bytes);
  for (size_t i = blockIdx.y * 256 + threadIdx.x; i < n16; i += size_t(gridDim.y) * 256) {
    kd[i] = stream_load(ks + i);
    vd[i] = stream_load(vs + i);
  }
}

// One (block, kv head) tile: block index bi of sequence seq's table.  K rows
// leave as they are (16-byte chunks, contiguous on both sides); the
// transposed V tile goes through LDS and leaves as token rows.
template <int ES>
__device__ __forceinline__ void pack_tile(const PackArgs& a, int seq, int bi, int h, char* s_v) {
  constexpr int EPC = 16 / ES;                             // elements per 16-byte chunk
  constexpr int NI = (ES == 1) ? 1 : (ES == 2 ? 2 : 4);   // chunks per thread at most (block 32, d 128)
  const int H = a.num_kv_heads, D = a.head_dim, BS = a.block_size;
  const int L = a.seq_lens[seq];
  const int ntok = min(BS, L - bi * BS);                   // >= 1: the tile is a used block
  const int blk = a.block_table[size_t(seq) * a.max_blocks_per_seq + bi];
  const size_t row0 = size_t(a.cu_rows[seq]) + size_t(bi) * BS;
  const int cpr = D / EPC;                                 // 16-byte chunks per token row
  const int cpv = BS / EPC;                                // 16-byte chunks per transposed V row
  const char* ktile = static_cast<const char*>(a.k_cache) + (size_t(blk) * H + h) * size_t(BS) * D * ES;
  const char* vtile = static_cast<const char*>(a.v_cache) + (size_t(blk) * H + h) * size_t(D) * BS * ES;
  char* ko = static_cast<char*>(a.k_out);
  char* vo = static_cast<char*>(a.v_out);
  const int nk = ntok * cpr, nv = D * cpv;
  // every load of the thread goes out before its first store.  Loads are
  // unconditional, clamped to the last chunk, so that they all fly
  // together; only the stores are guarded.
  // (chunks in plain named registers: no array or lambda capture, which
  // inside the tile loop would go to private memory)
  uint4 k0{}, k1{}, k2{}, k3{}, v0{}, v1{}, v2{}, v3{};
#define PA_PK_LOAD(I)                                                                                     \
  if constexpr (NI > I) {                                                                                 \
    const int ck = min(int(threadIdx.x) + 256 * I, nk - 1);                                              \
    k##I = *reinterpret_cast<const uint4*>(ktile + (size_t(ck / cpr) * D) * ES + (ck % cpr) * 16);        \
    const int cv = min(int(threadIdx.x) + 256 * I, nv - 1);                                              \
    v##I = *reinterpret_cast<const uint4*>(vtile + (size_t(cv / cpv) * BS + (cv % cpv) * EPC) * ES);     \
  }
#define PA_PK_STORE(I)                                                                                    \
  if constexpr (NI > I) {                                                                                 \
    const int c = threadIdx.x + 256 * I;                                                                  \
    if (c < nk)                                                                                           \
      *reinterpret_cast<uint4*>(ko + ((row0 + c / cpr) * H + h) * size_t(D) * ES + (c % cpr) * 16) = k##I; \
    if (c < nv) {                                                                                         \
      const int dim = c / cpv, t0 = (c % cpv) * EPC;                                                      \
      const uint32_t w_[4] = {v##I.x, v##I.y, v##I.z, v##I.w};                                            \
      _Pragma("unroll") for (int e = 0; e < EPC; ++e) {                                                   \
        char* dst = s_v + (size_t(t0 + e) * D + dim) * ES;                                                \
        if constexpr (ES == 4) *reinterpret_cast<uint32_t*>(dst) = w_[e];                                 \
        else if constexpr (ES == 2) *reinterpret_cast<uint16_t*>(dst) = uint16_t(w_[e >> 1] >> (16 * (e & 1))); \
        else *reinterpret_cast<uint8_t*>(dst) = uint8_t(w_[e >> 2] >> (8 * (e & 3)));                    \
      }                                                                                                   \
    }                                                                                                     \
  }
  PA_PK_LOAD(0) PA_PK_LOAD(1) PA_PK_LOAD(2) PA_PK_LOAD(3)
  PA_PK_STORE(0) PA_PK_STORE(1) PA_PK_STORE(2) PA_PK_STORE(3)
#undef PA_PK_LOAD
#undef PA_PK_STORE
  __syncthreads();
  for (int c = threadIdx.x; c < nk; c += 256) {
    const int tok = c / cpr, cc = c % cpr;
    *reinterpret_cast<uint4*>(vo + ((row0 + tok) * H + h) * size_t(D) * ES + cc * 16) =
        *reinterpret_cast<const uint4*>(s_v + (size_t(tok) * D) * ES + cc * 16);
  }
  __syncthreads();                                         // s_v is rewritten by the next tile
}

// Tiles are (block, kv head) pairs of the sequences' used blocks (at most
// max_blocks_used per sequence, the blocks of max_seq_len), numbered
// sequence by sequence, block by block, kv head fastest (the heads of one
// block are neighbours in both caches).  Each workgroup first lays out, in
// LDS, the prefix of used blocks over the sequences, then walks the tiles
// with a grid-sized stride: no workgroup is launched for a block past a
// sequence's end.
template <int ES>
__global__ void __launch_bounds__(256) pack_kv_kernel(PackArgs a, int num_seqs, int max_blocks_used) {
  __shared__ __attribute__((aligned(16))) char s_v[32 * 128 * ES];   // [token][dim], at most B 32 x d 128
  __shared__ int s_tmp[256];
  extern __shared__ int s_pre[];                           // [num_seqs + 1] used blocks before each sequence
  const int S = num_seqs;
  const int H = a.num_kv_heads, BS = a.block_size;
  {
    const int per = (S + 255) / 256;
    const int i0 = threadIdx.x * per, i1 = min(S, i0 + per);
    int local = 0;
    for (int i = i0; i < i1; ++i) local += min((max(0, a.seq_lens[i]) + BS - 1) / BS, max_blocks_used);
    s_tmp[threadIdx.x] = local;
    __syncthreads();
    for (int off = 1; off < 256; off <<= 1) {
      const int v = int(threadIdx.x) >= off ? s_tmp[threadIdx.x - off] : 0;
      __syncthreads();
      s_tmp[threadIdx.x] += v;
      __syncthreads();
    }
    int run = threadIdx.x ? s_tmp[threadIdx.x - 1] : 0;
    for (int i = i0; i < i1; ++i) {
      s_pre[i] = run;
      run += min((max(0, a.seq_lens[i]) + BS - 1) / BS, max_blocks_used);
    }
    if (threadIdx.x == 255) s_pre[S] = s_tmp[255];
    __syncthreads();
  }
  const int64_t tiles = int64_t(s_pre[S]) * H;
  for (int64_t tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
    const int tb = int(tile / H), h = int(tile - int64_t(tb) * H);
    int lo = 0, hi = S;                                    // largest seq with s_pre[seq] <= tb
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_pre[mid] <= tb) lo = mid; else hi = mid;
    }
    pack_tile<ES>(a, lo, tb - s_pre[lo], h, s_v);
  }
}

hipError_t launch_pack_kv(const PackArgs& a, int es, int num_seqs, int max_blocks_used, hipStream_t s) {
  if (num_seqs == 0 || max_blocks_used == 0) return hipSuccess;
  // enough workgroups to fill the chip several times over, never more than
  // the tiles there can be
  const int64_t upper = int64_t(num_seqs) * max_blocks_used * a.num_kv_heads;
  const int64_t wgs = upper < 8192 ? upper : 8192;
  const size_t lds = size_t(num_seqs + 1) * sizeof(int);
  switch (es) {
    case 4: hipLaunchKernelGGL(pack_kv_kernel<4>, dim3(uint32_t(wgs)), dim3(256), lds, s, a, num_seqs, max_blocks_used); break;
    case 2: hipLaunchKernelGGL(pack_kv_kernel<2>, dim3(uint32_t(wgs)), dim3(256), lds, s, a, num_seqs, max_blocks_used); break;
    default: hipLaunchKernelGGL(pack_kv_kernel<1>, dim3(uint32_t(wgs)), dim3(256), lds, s, a, num_seqs, max_blocks_used); break;
  }
  return hipGetLastError();
}

hipError_t launch_store_kv(const StoreArgs& a, int kv, hipStream_t s) {
  if (a.num_tokens == 0) return hipSuccess;
  if (a.num_tokens <= kStoreRowsMaxTokens) {                // a few scattered tokens: latency-bound
    dim3 grid(uint32_t((int64_t(a.num_tokens) * a.num_kv_heads + 3) / 4));
    switch (kv) {
      case KV_F32: hipLaunchKernelGGL(store_rows_kernel<KV_F32>, grid, dim3(256), 0, s, a); break;
      case KV_BF16: hipLaunchKernelGGL(store_rows_kernel<KV_BF16>, grid, dim3(256), 0, s, a); break;
      case KV_FP8_RAW: hipLaunchKernelGGL(store_rows_kernel<KV_FP8_RAW>, grid, dim3(256), 0, s, a); break;
      default: hipLaunchKernelGGL(store_rows_kernel<KV_FP8>, grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
  }
  const int64_t work = int64_t((a.num_tokens + 63) / 64) * a.num_kv_heads;
  if (work > 0x7FFFFFF0ll) return hipErrorInvalidValue;
  dim3 grid(uint32_t((work + 7) / 8 * 8));
  switch (kv) {
    case KV_F32: hipLaunchKernelGGL(store_kv_kernel<KV_F32>, grid, dim3(256), 0, s, a); break;
    case KV_BF16: hipLaunchKernelGGL(store_kv_kernel<KV_BF16>, grid, dim3(256), 0, s, a); break;
    case KV_FP8_RAW: hipLaunchKernelGGL(store_kv_kernel<KV_FP8_RAW>, grid, dim3(256), 0, s, a); break;
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
