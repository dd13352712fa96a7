// libpa C ABI: argument validation, dtype/shape dispatch and launches.
// Every check runs on the host before the first HIP call, so a rejected
// call launches nothing and touches no device state.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/pa.h"
#include "pa_internal.h"

namespace pa {
hipError_t launch_decode_f32(const DecodeArgs&, int, int, int, int64_t, hipStream_t, const LaunchEvents&);
hipError_t launch_decode_bf16(const DecodeArgs&, int, int, int, int64_t, hipStream_t, const LaunchEvents&);
hipError_t launch_decode_fp8(const DecodeArgs&, int, int, int, int64_t, hipStream_t, const LaunchEvents&);
}  // namespace pa

namespace {

thread_local char g_err[512] = "";
// events armed by pa_decode_time_next for this thread's next pa_decode call
thread_local pa::LaunchEvents g_decode_events;
#ifdef PA_DECODE_TRACE
// trace buffer armed by pa_decode_trace_next (measurement build only)
thread_local uint32_t* g_decode_trace = nullptr;
#endif

template <typename... A>
int fail(int code, const char* fmt, A... args) {
  snprintf(g_err, sizeof(g_err), fmt, args...);
  return code;
}
int fail(int code, const char* msg) {
  snprintf(g_err, sizeof(g_err), "%s", msg);
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Largest partition: unit counts and token offsets stay far inside int32.
constexpr int32_t kMaxPartition = 1 << 28;
constexpr int kMaxSeqs = 8192;  // the decode kernel keeps a prefix over sequences in LDS

int elem_bytes(int dt) { return dt == PA_F32 ? 4 : dt == PA_BF16 ? 2 : 1; }

int check_cache(const pa_kv_cache* c) {
  if (!c) return fail(PA_ERR_NULL, "cache descriptor is NULL");
  if (!c->k_cache || !c->v_cache) return fail(PA_ERR_NULL, "k_cache / v_cache is NULL");
  if (c->dtype != PA_F32 && c->dtype != PA_BF16 && c->dtype != PA_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "unknown cache dtype %d", c->dtype);
  if (c->num_blocks <= 0 || c->num_kv_heads <= 0) return fail(PA_ERR_SHAPE, "num_blocks / num_kv_heads must be > 0");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(PA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", c->head_dim);
  if (c->block_size != 16 && c->block_size != 32)
    return fail(PA_ERR_UNSUPPORTED, "block_size %d not supported (16 or 32)", c->block_size);
  if (c->dtype == PA_FP8_E4M3) {
    if (!c->k_scale || !c->v_scale) return fail(PA_ERR_NULL, "fp8 cache needs k_scale and v_scale");
  } else if (c->k_scale || c->v_scale) {
    return fail(PA_ERR_DTYPE, "k_scale / v_scale are only for an fp8 cache");
  }
  return PA_OK;
}

int io_dtype_for(int cache_dtype) { return cache_dtype == PA_F32 ? PA_F32 : PA_BF16; }

// partition_tokens 0: no split -- one partition spans the longest context,
// so every (sequence, kv head) is one unit and no wave shares one.
// Otherwise a positive multiple of block_size.
int resolve_partition(int32_t p, int32_t block_size, int32_t max_context_len, int32_t* out) {
  if (p < 0) return fail(PA_ERR_SHAPE, "partition_tokens %d < 0", p);
  if (p == 0) {
    const int64_t whole = (int64_t(max_context_len > 0 ? max_context_len : 1) + 63) / 64 * 64;
    *out = int32_t(whole < kMaxPartition ? whole : kMaxPartition);
    return PA_OK;
  }
  if (p % block_size != 0 || p > kMaxPartition)
    return fail(PA_ERR_SHAPE, "partition_tokens %d must be a multiple of block_size %d and at most %d", p,
                block_size, kMaxPartition);
  *out = p;
  return PA_OK;
}

}  // namespace

namespace pa {

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

DecodeWorkspace decode_workspace_layout(int64_t D) {
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  const size_t slots = size_t(kDecodeMaxWaves) * 2 * kDecodeMaxGroup;   // two partials per wave
  DecodeWorkspace w;
  w.arrivals_off = 0;
  w.ml_off = up(size_t(kDecodeMaxWaves) * sizeof(int32_t));
  w.acc_off = w.ml_off + up(slots * 2 * sizeof(float));
  w.total = w.acc_off + up(slots * size_t(D) * sizeof(float));
  return w;
}

hipError_t launch_decode(const DecodeArgs& a, int kv, int D, int B, int G, int64_t upper, hipStream_t s,
                         const LaunchEvents& ev) {
  switch (kv) {
    case KV_F32: return launch_decode_f32(a, D, B, G, upper, s, ev);
    case KV_BF16: return launch_decode_bf16(a, D, B, G, upper, s, ev);
    default: return launch_decode_fp8(a, D, B, G, upper, s, ev);
  }
}

}  // namespace pa

extern "C" {

const char* pa_last_error(void) { return g_err; }

int pa_store_kv(const pa_kv_cache* cache, const void* k_new, const void* v_new, int32_t in_dtype,
                const int32_t* slot_mapping, int32_t num_tokens, void* hip_stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (num_tokens < 0) return fail(PA_ERR_SHAPE, "num_tokens %d < 0", num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !slot_mapping) return fail(PA_ERR_NULL, "k_new / v_new / slot_mapping is NULL");
  const bool raw_fp8 = cache->dtype == PA_FP8_E4M3 && in_dtype == PA_FP8_E4M3;   // codes as they are
  if (in_dtype != io_dtype_for(cache->dtype) && !raw_fp8)
    return fail(PA_ERR_DTYPE, "store into a %s cache takes %s input",
                cache->dtype == PA_F32 ? "f32" : cache->dtype == PA_BF16 ? "bf16" : "fp8",
                cache->dtype == PA_F32 ? "f32" : cache->dtype == PA_BF16 ? "bf16" : "bf16 or fp8");
  pa::StoreArgs a{cache->k_cache, cache->v_cache, cache->k_scale, cache->v_scale, k_new, v_new, slot_mapping,
                  num_tokens, cache->num_kv_heads, cache->block_size, cache->head_dim};
  const int kv = cache->dtype == PA_F32    ? pa::KV_F32
                 : cache->dtype == PA_BF16 ? pa::KV_BF16
                 : raw_fp8                 ? pa::KV_FP8_RAW
                                           : pa::KV_FP8;
  if (pa::debug_bounds_on()) {
    rc = pa::debug_check_store(cache, slot_mapping, num_tokens, static_cast<hipStream_t>(hip_stream));
    if (rc) return rc;
  }
  hipError_t e = pa::launch_store_kv(a, kv, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "pa_store_kv launch");
  g_err[0] = 0;
  return PA_OK;
}

int pa_copy_blocks(const pa_kv_cache* cache, const int32_t* src_dst, int32_t num_pairs, void* hip_stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (num_pairs < 0) return fail(PA_ERR_SHAPE, "num_pairs %d < 0", num_pairs);
  if (num_pairs == 0) return PA_OK;
  if (!src_dst) return fail(PA_ERR_NULL, "src_dst is NULL");
  pa::CopyArgs a{cache->k_cache, cache->v_cache, src_dst,
                 size_t(cache->num_kv_heads) * cache->block_size * cache->head_dim * elem_bytes(cache->dtype)};
  if (pa::debug_bounds_on()) {
    rc = pa::debug_check_copy(cache, src_dst, num_pairs, static_cast<hipStream_t>(hip_stream));
    if (rc) return rc;
  }
  hipError_t e = pa::launch_copy_blocks(a, num_pairs, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "pa_copy_blocks launch");
  g_err[0] = 0;
  return PA_OK;
}

int pa_pack_kv(const pa_kv_cache* cache, const int32_t* block_table, int32_t max_blocks_per_seq,
               const int32_t* seq_lens, const int32_t* cu_rows, int32_t num_seqs, int32_t max_seq_len, void* k_out,
               void* v_out, void* hip_stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (num_seqs < 0 || num_seqs > kMaxSeqs) return fail(PA_ERR_SHAPE, "num_seqs %d outside 0..%d", num_seqs, kMaxSeqs);
  if (max_seq_len < 0) return fail(PA_ERR_SHAPE, "max_seq_len %d < 0", max_seq_len);
  const int64_t blocks = (int64_t(max_seq_len) + cache->block_size - 1) / cache->block_size;
  if (max_blocks_per_seq < blocks || max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d < %lld blocks of max_seq_len", max_blocks_per_seq,
                (long long)blocks);
  if (blocks > 65535) return fail(PA_ERR_UNSUPPORTED, "max_seq_len %d: more than 65535 blocks", max_seq_len);
  if (num_seqs == 0 || max_seq_len == 0) return PA_OK;
  if (!block_table || !seq_lens || !cu_rows || !k_out || !v_out)
    return fail(PA_ERR_NULL, "block_table / seq_lens / cu_rows / k_out / v_out is NULL");
  pa::PackArgs a{cache->k_cache, cache->v_cache, block_table, seq_lens, cu_rows, k_out, v_out,
                 cache->num_kv_heads, cache->block_size, cache->head_dim, max_blocks_per_seq};
  if (pa::debug_bounds_on()) {
    rc = pa::debug_check_pack(cache, block_table, max_blocks_per_seq, seq_lens, cu_rows, num_seqs, max_seq_len,
                              static_cast<hipStream_t>(hip_stream));
    if (rc) return rc;
  }
  hipError_t e = pa::launch_pack_kv(a, int(elem_bytes(cache->dtype)), num_seqs, int(blocks),
                                    static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "pa_pack_kv launch");
  g_err[0] = 0;
  return PA_OK;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                                 int32_t partition_tokens) {
  if (num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 || partition_tokens < 0) return 0;
  return pa::decode_workspace_layout(head_dim).total;
}

}  // extern "C"

namespace {

// pa_decode, and pa_decode_append (append: the new rows k_new / v_new are
// stored first; name: the entry point, for messages).
int decode_call(const char* name, bool append, const pa_kv_cache* cache, const void* k_new, const void* v_new, const void* q,
                int32_t q_dtype, void* out, int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads, float scale,
                const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                int32_t max_context_len, int32_t partition_tokens, void* workspace, size_t workspace_bytes_given,
                void* hip_stream) {
  const pa::LaunchEvents ev = g_decode_events;             // armed for this call only
  g_decode_events = pa::LaunchEvents{};
  int rc = check_cache(cache);
  if (rc) return rc;
  if (num_seqs < 0 || num_seqs > kMaxSeqs) return fail(PA_ERR_SHAPE, "num_seqs %d outside 0..%d", num_seqs, kMaxSeqs);
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                cache->num_kv_heads);
  const int G = num_q_heads / cache->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PA_ERR_UNSUPPORTED, "query group %d not in {1,2,4,8}", G);
  const int io = io_dtype_for(cache->dtype);
  if (q_dtype != io || out_dtype != io)
    return fail(PA_ERR_DTYPE, "decode over this cache takes %s q and out", io == PA_F32 ? "f32" : "bf16");
  if (max_context_len < 0) return fail(PA_ERR_SHAPE, "max_context_len %d < 0", max_context_len);
  const int64_t need_blocks = (int64_t(max_context_len) + cache->block_size - 1) / cache->block_size;
  if (max_blocks_per_seq < need_blocks || max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d < %lld blocks of max_context_len", max_blocks_per_seq,
                (long long)need_blocks);
  if (!(std::isfinite(scale)) || !(scale > 0.f)) return fail(PA_ERR_SHAPE, "scale must be finite and > 0");
  int32_t P = 0;
  rc = resolve_partition(partition_tokens, cache->block_size, max_context_len, &P);
  if (rc) return rc;
  if (num_seqs == 0) return PA_OK;
  if (!q || !out || !block_table || !context_lens || !workspace)
    return fail(PA_ERR_NULL, "q / out / block_table / context_lens / workspace is NULL");
  if (append && (!k_new || !v_new)) return fail(PA_ERR_NULL, "%s: k_new / v_new is NULL", name);
  const pa::DecodeWorkspace lay = pa::decode_workspace_layout(cache->head_dim);
  if (workspace_bytes_given < lay.total)
    return fail(PA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes_given, lay.total);
  char* ws = static_cast<char*>(workspace);
  pa::DecodeArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.q = q;
  a.out = out;
  a.block_table = block_table;
  a.context_lens = context_lens;
  a.arrivals = reinterpret_cast<int32_t*>(ws + lay.arrivals_off);
  a.part_ml = reinterpret_cast<float*>(ws + lay.ml_off);
  a.part_acc = reinterpret_cast<float*>(ws + lay.acc_off);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.part_tokens = P;
#ifdef PA_DECODE_TRACE
  a.trace = g_decode_trace;                                // armed for this call only
  g_decode_trace = nullptr;
#endif
  const int kv = cache->dtype == PA_F32 ? pa::KV_F32 : cache->dtype == PA_BF16 ? pa::KV_BF16 : pa::KV_FP8;
  const int64_t max_parts = max_context_len > 0 ? (int64_t(max_context_len) + P - 1) / P : 1;
  const int64_t upper_units = int64_t(num_seqs) * cache->num_kv_heads * max_parts;
  if (pa::debug_bounds_on()) {
    rc = pa::debug_check_decode(cache, block_table, max_blocks_per_seq, context_lens, num_seqs, max_context_len,
                                static_cast<hipStream_t>(hip_stream));
    if (rc) return rc;
  }
  hipError_t e = pa::launch_decode(a, kv, cache->head_dim, cache->block_size, G, upper_units,
                                   static_cast<hipStream_t>(hip_stream), ev);
  if (e == hipErrorInvalidValue) return fail(PA_ERR_UNSUPPORTED, "no decode kernel for this shape");
  if (e != hipSuccess) return hip_fail(e, name);
  g_err[0] = 0;
  return PA_OK;
}

}  // namespace

extern "C" {

int pa_decode(const pa_kv_cache* cache, const void* q, int32_t q_dtype, void* out, int32_t out_dtype,
              int32_t num_seqs, int32_t num_q_heads, float scale, const int32_t* block_table,
              int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
              int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* hip_stream) {
  return decode_call("pa_decode", false, cache, nullptr, nullptr, q, q_dtype, out, out_dtype, num_seqs, num_q_heads, scale,
                     block_table, max_blocks_per_seq, context_lens, max_context_len, partition_tokens, workspace,
                     workspace_bytes, hip_stream);
}

int pa_decode_append(const pa_kv_cache* cache, const void* k_new, const void* v_new, const void* q, int32_t q_dtype,
                     void* out, int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads, float scale,
                     const int32_t* block_table, int32_t max_blocks_per_seq, const int32_t* context_lens,
                     int32_t max_context_len, int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                     void* hip_stream) {
  return decode_call("pa_decode_append", true, cache, k_new, v_new, q, q_dtype, out, out_dtype, num_seqs, num_q_heads,
                     scale, block_table, max_blocks_per_seq, context_lens, max_context_len, partition_tokens,
                     workspace, workspace_bytes, hip_stream);
}

int pa_decode_time_next(void* start_event, void* stop_event) {
  g_decode_events = pa::LaunchEvents{static_cast<hipEvent_t>(start_event), static_cast<hipEvent_t>(stop_event)};
  g_err[0] = 0;
  return PA_OK;
}

#ifdef PA_DECODE_TRACE
// Measurement build only (libpa_trace.so): the next pa_decode call on this
// thread writes 16 uint32 of time stamps per wave into buf (device memory of
// at least 4096 * 64 bytes).
int pa_decode_trace_next(void* buf) {
  g_decode_trace = static_cast<uint32_t*>(buf);
  g_err[0] = 0;
  return PA_OK;
}
#endif

int pa_prefill_chunk(const pa_kv_cache* cache, const void* q, int32_t q_dtype, void* out, int32_t out_dtype,
                     int32_t num_seqs, int32_t num_q_heads, float scale, const int32_t* cu_q_lens,
                     const int32_t* seq_lens, const int32_t* block_table, int32_t max_blocks_per_seq,
                     int32_t max_q_len, int32_t max_seq_len, void* workspace, size_t workspace_bytes,
                     void* hip_stream) {
  int rc = check_cache(cache);
  if (rc) return rc;
  if (num_seqs < 0) return fail(PA_ERR_SHAPE, "num_seqs %d < 0", num_seqs);
  if (num_q_heads <= 0 || num_q_heads % cache->num_kv_heads)
    return fail(PA_ERR_SHAPE, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                cache->num_kv_heads);
  const int G = num_q_heads / cache->num_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PA_ERR_UNSUPPORTED, "query group %d not in {1,2,4,8}", G);
  if (cache->dtype != PA_BF16 && cache->dtype != PA_FP8_E4M3)
    return fail(PA_ERR_DTYPE, "pa_prefill_chunk needs a bf16 or fp8 cache");
  if (q_dtype != PA_BF16 || out_dtype != PA_BF16) return fail(PA_ERR_DTYPE, "pa_prefill_chunk takes bf16 q and out");
  if (cache->head_dim != 128) return fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk supports head_dim 128");
  if (max_q_len < 0 || max_seq_len < max_q_len)
    return fail(PA_ERR_SHAPE, "need 0 <= max_q_len (%d) <= max_seq_len (%d)", max_q_len, max_seq_len);
  const int64_t need_blocks = (int64_t(max_seq_len) + cache->block_size - 1) / cache->block_size;
  if (max_blocks_per_seq < need_blocks || max_blocks_per_seq <= 0)
    return fail(PA_ERR_SHAPE, "max_blocks_per_seq %d < %lld blocks of max_seq_len", max_blocks_per_seq,
                (long long)need_blocks);
  if (!(std::isfinite(scale)) || !(scale > 0.f)) return fail(PA_ERR_SHAPE, "scale must be finite and > 0");
  if (num_seqs == 0 || max_q_len == 0) return PA_OK;
  if (!q || !out || !cu_q_lens || !seq_lens || !block_table)
    return fail(PA_ERR_NULL, "q / out / cu_q_lens / seq_lens / block_table is NULL");
  pa::PrefillArgs a{};
  a.k_cache = cache->k_cache;
  a.v_cache = cache->v_cache;
  a.k_scale = cache->k_scale;
  a.v_scale = cache->v_scale;
  a.q = q;
  a.out = out;
  a.cu_q_lens = cu_q_lens;
  a.seq_lens = seq_lens;
  a.block_table = block_table;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = cache->num_kv_heads;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.max_q_len = max_q_len;
  a.max_seq_len = max_seq_len;
  if (workspace) {
    const pa::DecodeWorkspace lay = pa::decode_workspace_layout(cache->head_dim);
    if (workspace_bytes < lay.total)
      return fail(PA_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, lay.total);
    char* ws = static_cast<char*>(workspace);
    a.arrivals = reinterpret_cast<int32_t*>(ws + lay.arrivals_off);
    a.part_ml = reinterpret_cast<float*>(ws + lay.ml_off);
    a.part_acc = reinterpret_cast<float*>(ws + lay.acc_off);
  }
  const int kv = cache->dtype == PA_BF16 ? pa::KV_BF16 : pa::KV_FP8;
  if (pa::debug_bounds_on()) {
    rc = pa::debug_check_prefill(cache, cu_q_lens, seq_lens, block_table, max_blocks_per_seq, num_seqs, max_q_len,
                                 max_seq_len, static_cast<hipStream_t>(hip_stream));
    if (rc) return rc;
  }
  hipError_t e = pa::launch_prefill_chunk(a, kv, cache->block_size, G, static_cast<hipStream_t>(hip_stream));
  if (e == hipErrorInvalidValue) return fail(PA_ERR_UNSUPPORTED, "no prefill kernel for this shape");
  if (e != hipSuccess) return hip_fail(e, "pa_prefill_chunk launch");
  g_err[0] = 0;
  return PA_OK;
}

}  // extern "C"
