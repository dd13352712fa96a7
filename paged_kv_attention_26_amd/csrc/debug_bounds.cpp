// Checks of the values inside index arrays: pa_check_* take host arrays;
// with PA_DEBUG_BOUNDS=1 in the environment every call runs them on its own
// device arrays first, for debugging.  Release calls never look at
// these values: an out-of-range slot, block id or length is undefined
// behaviour there.  In this mode each call first copies its index arrays to
// the host on its stream, waits for them, and rejects the call with
// PA_ERR_BOUNDS -- before any kernel is launched -- naming the first bad
// entry.  The copies synchronise the stream, so this mode is not for code
// under graph capture.
#include <cmath>
#include <cstdlib>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

// ---- checks of host arrays (the C ABI's pa_check_*) ------------------------
extern "C" {

int pa_check_slots(const pa_kv_cache* c, const int32_t* slots, int32_t n) {
  if (!c) return pa::set_error(PA_ERR_NULL, "cache descriptor is NULL");
  if (n > 0 && !slots) return pa::set_error(PA_ERR_NULL, "slots is NULL");
  const int64_t cap = int64_t(c->num_blocks) * c->block_size;
  for (int32_t t = 0; t < n; ++t)
    if (slots[t] >= cap)
      return pa::set_error(PA_ERR_BOUNDS, "slot_mapping[%d] = %d is past the pool's %lld slots", t, slots[t],
                           (long long)cap);
  return PA_OK;
}

int pa_check_copy_pairs(const pa_kv_cache* c, const int32_t* pairs, int32_t n) {
  if (!c) return pa::set_error(PA_ERR_NULL, "cache descriptor is NULL");
  if (n > 0 && !pairs) return pa::set_error(PA_ERR_NULL, "pairs is NULL");
  if (c->num_blocks <= 0) return pa::set_error(PA_ERR_SHAPE, "num_blocks must be > 0");
  std::vector<char> is_dst(size_t(c->num_blocks), 0), is_src(size_t(c->num_blocks), 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t src = pairs[2 * size_t(i)], dst = pairs[2 * size_t(i) + 1];
    if (src < 0 || src >= c->num_blocks || dst < 0 || dst >= c->num_blocks)
      return pa::set_error(PA_ERR_BOUNDS, "pair %d (%d, %d) outside [0, %d)", i, src, dst, c->num_blocks);
    if (is_dst[size_t(dst)]) return pa::set_error(PA_ERR_BOUNDS, "block %d is the dst of two pairs", dst);
    is_dst[size_t(dst)] = 1;
    is_src[size_t(src)] = 1;
  }
  for (int32_t b = 0; b < c->num_blocks; ++b)
    if (is_dst[size_t(b)] && is_src[size_t(b)])
      return pa::set_error(PA_ERR_BOUNDS, "block %d is both a src and a dst", b);
  return PA_OK;
}

int pa_check_tables(const pa_kv_cache* c, const int32_t* table, int32_t max_blocks, const int32_t* lens,
                    int32_t num_seqs, int32_t max_len) {
  if (!c) return pa::set_error(PA_ERR_NULL, "cache descriptor is NULL");
  if (num_seqs > 0 && (!table || !lens)) return pa::set_error(PA_ERR_NULL, "table / lens is NULL");
  if (c->block_size <= 0) return pa::set_error(PA_ERR_SHAPE, "block_size must be > 0");
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int32_t L = lens[s];
    if (L < 0 || L > max_len)
      return pa::set_error(PA_ERR_BOUNDS, "length of sequence %d = %d outside [0, %d]", s, L, max_len);
    const int64_t nb = (int64_t(L) + c->block_size - 1) / c->block_size;
    if (nb > max_blocks)
      return pa::set_error(PA_ERR_BOUNDS, "sequence %d: %d tokens need %lld blocks, its table row holds %d", s, L,
                           (long long)nb, max_blocks);
    for (int64_t i = 0; i < nb; ++i) {
      const int32_t b = table[size_t(s) * size_t(max_blocks) + size_t(i)];
      if (b < 0 || b >= c->num_blocks)
        return pa::set_error(PA_ERR_BOUNDS, "block_table[%d][%lld] = %d outside [0, %d)", s, (long long)i, b,
                             c->num_blocks);
    }
  }
  return PA_OK;
}

int pa_check_chunks(const pa_kv_cache* c, const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t max_q_len) {
  if (!c) return pa::set_error(PA_ERR_NULL, "cache descriptor is NULL");
  if (!cu_q_lens || (num_seqs > 0 && !seq_lens)) return pa::set_error(PA_ERR_NULL, "cu_q_lens / seq_lens is NULL");
  if (cu_q_lens[0] != 0) return pa::set_error(PA_ERR_BOUNDS, "cu_q_lens[0] = %d, not 0", cu_q_lens[0]);
  for (int32_t j = 0; j < num_seqs; ++j) {
    const int32_t q = cu_q_lens[j + 1] - cu_q_lens[j];
    if (q < 0 || q > max_q_len)
      return pa::set_error(PA_ERR_BOUNDS, "chunk %d has %d rows, outside [0, %d]", j, q, max_q_len);
    if (seq_lens[j] < q)
      return pa::set_error(PA_ERR_BOUNDS, "seq_lens[%d] = %d is shorter than its chunk of %d", j, seq_lens[j], q);
  }
  return PA_OK;
}

int pa_check_scales(const pa_kv_cache* c, const float* k_scale, const float* v_scale) {
  if (!c) return pa::set_error(PA_ERR_NULL, "cache descriptor is NULL");
  if (!k_scale || !v_scale) return pa::set_error(PA_ERR_NULL, "k_scale / v_scale is NULL");
  for (int h = 0; h < c->num_kv_heads; ++h) {
    if (!(std::isfinite(k_scale[h]) && k_scale[h] > 0.f))
      return pa::set_error(PA_ERR_BOUNDS, "k_scale[%d] = %g is not finite and > 0", h, k_scale[h]);
    if (!(std::isfinite(v_scale[h]) && v_scale[h] > 0.f))
      return pa::set_error(PA_ERR_BOUNDS, "v_scale[%d] = %g is not finite and > 0", h, v_scale[h]);
  }
  return PA_OK;
}

}  // extern "C"

// ---- PA_DEBUG_BOUNDS: the same checks on a call's device arrays -------------
namespace pa {
namespace {

template <typename T>
hipError_t fetch(std::vector<T>& host, const void* dev, size_t n, hipStream_t s) {
  host.resize(n);
  if (n == 0) return hipSuccess;
  hipError_t e = hipMemcpyAsync(host.data(), dev, n * sizeof(T), hipMemcpyDeviceToHost, s);
  if (e != hipSuccess) return e;
  return hipStreamSynchronize(s);
}

int hip_err(hipError_t e) {
  return set_error(PA_ERR_HIP, "PA_DEBUG_BOUNDS: copying an index array to the host: %s", hipGetErrorString(e));
}

}  // namespace

bool debug_bounds_on() {
  const char* v = std::getenv("PA_DEBUG_BOUNDS");
  return v && v[0] && !(v[0] == '0' && v[1] == 0);
}

int debug_check_scales(const pa_kv_cache* c, hipStream_t s) {
  if (c->dtype != PA_FP8_E4M3) return PA_OK;
  std::vector<float> ks, vs;
  hipError_t e = fetch(ks, c->k_scale, size_t(c->num_kv_heads), s);
  if (e == hipSuccess) e = fetch(vs, c->v_scale, size_t(c->num_kv_heads), s);
  if (e != hipSuccess) return hip_err(e);
  return pa_check_scales(c, ks.data(), vs.data());
}

int debug_check_store(const pa_kv_cache* c, const int32_t* slots, int32_t n, hipStream_t s) {
  std::vector<int32_t> h;
  hipError_t e = fetch(h, slots, size_t(n), s);
  if (e != hipSuccess) return hip_err(e);
  const int rc = pa_check_slots(c, h.data(), n);
  return rc ? rc : debug_check_scales(c, s);
}

int debug_check_copy(const pa_kv_cache* c, const int32_t* pairs, int32_t n, hipStream_t s) {
  std::vector<int32_t> h;
  hipError_t e = fetch(h, pairs, size_t(n) * 2, s);
  if (e != hipSuccess) return hip_err(e);
  return pa_check_copy_pairs(c, h.data(), n);
}

int debug_check_decode(const pa_kv_cache* c, const int32_t* table, int32_t max_blocks, const int32_t* lens,
                       int32_t S, int32_t max_ctx, hipStream_t s) {
  std::vector<int32_t> hl, ht;
  hipError_t e = fetch(hl, lens, size_t(S), s);
  if (e == hipSuccess) e = fetch(ht, table, size_t(S) * size_t(max_blocks), s);
  if (e != hipSuccess) return hip_err(e);
  const int rc = pa_check_tables(c, ht.data(), max_blocks, hl.data(), S, max_ctx);
  return rc ? rc : debug_check_scales(c, s);
}

int debug_check_prefill(const pa_kv_cache* c, const int32_t* cu, const int32_t* seq_lens, const int32_t* table,
                        int32_t max_blocks, int32_t S, int32_t max_q, int32_t max_seq, hipStream_t s) {
  std::vector<int32_t> hc, hs, ht;
  hipError_t e = fetch(hc, cu, size_t(S) + 1, s);
  if (e == hipSuccess) e = fetch(hs, seq_lens, size_t(S), s);
  if (e == hipSuccess) e = fetch(ht, table, size_t(S) * size_t(max_blocks), s);
  if (e != hipSuccess) return hip_err(e);
  int rc = pa_check_chunks(c, hc.data(), hs.data(), S, max_q);
  if (!rc) rc = pa_check_tables(c, ht.data(), max_blocks, hs.data(), S, max_seq);
  return rc ? rc : debug_check_scales(c, s);
}

int debug_check_pack(const pa_kv_cache* c, const int32_t* table, int32_t max_blocks, const int32_t* seq_lens,
                     const int32_t* cu_rows, int32_t S, int32_t max_seq, hipStream_t s) {
  std::vector<int32_t> hs, hr, ht;
  hipError_t e = fetch(hs, seq_lens, size_t(S), s);
  if (e == hipSuccess) e = fetch(hr, cu_rows, size_t(S), s);
  if (e == hipSuccess) e = fetch(ht, table, size_t(S) * size_t(max_blocks), s);
  if (e != hipSuccess) return hip_err(e);
  for (int32_t j = 0; j < S; ++j)
    if (hr[size_t(j)] < 0) return set_error(PA_ERR_BOUNDS, "cu_rows[%d] = %d < 0", j, hr[size_t(j)]);
  return pa_check_tables(c, ht.data(), max_blocks, hs.data(), S, max_seq);
}

}  // namespace pa
