// Launch arguments and launcher entry points shared between libpa's C ABI
// layer (api.cpp) and its kernels.  Host-visible plain structs only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

// Cache element kinds the kernels are compiled for.
// KV_FP8 stores bf16 input as e4m3 codes; KV_FP8_RAW stores e4m3 codes as they are.
enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2, KV_FP8_RAW = 3 };

struct StoreArgs {
  void* k_cache;
  void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const void* k_new;
  const void* v_new;
  const int32_t* slot_mapping;
  int32_t num_tokens, num_kv_heads, block_size, head_dim;
};

struct CopyArgs {
  void* k_cache;
  void* v_cache;
  const int32_t* pairs;
  size_t block_bytes;  // bytes of one block in one pool
};

struct PackArgs {
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* cu_rows;
  void* k_out;
  void* v_out;
  int32_t num_kv_heads, block_size, head_dim, max_blocks_per_seq;
};

struct DecodeArgs {
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;
  const float* v_scale;
  const void* q;
  void* out;
  const int32_t* block_table;
  const int32_t* context_lens;
  float* part_ml;     // [total_waves][2][G][2]  (running max in log2 units, sum) of split items
  float* part_acc;    // [total_waves][2][G][head_dim]
  int32_t* arrivals;  // [kDecodeMaxWaves] per split item (keyed by its last wave); zero between calls
  float scale_log2;   // softmax scale * log2(e)
  int32_t num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq;
  int32_t part_tokens, total_waves;  // total_waves is set by the launcher
  // the step's new token of each (sequence, kv head), [num_seqs][Hkv][head_dim]
  // in the cache's input dtype, stored at position context_len - 1 before
  // the attention reads it; null: nothing is stored
  const void* k_new;
  const void* v_new;
  // [total_waves][16] per-wave time stamps, written only by kernels built
  // with PA_DECODE_TRACE (a measurement build); null otherwise
  uint32_t* trace;
};

// Upper bound on the waves one decode launch uses (the workspace is sized for it).
constexpr int kDecodeMaxWaves = 4096;
constexpr int kDecodeMaxGroup = 8;
// Upper bound on the workgroups of a split verify launch: two partials of 32
// columns each, and one arrival counter, per workgroup in the same workspace.
constexpr int kVerifyMaxGroups = 1024;
static_assert(kVerifyMaxGroups * 2 * 32 <= kDecodeMaxWaves * 2 * kDecodeMaxGroup, "verify partial slots");
static_assert(kVerifyMaxGroups <= kDecodeMaxWaves, "verify arrival counters");

struct PrefillArgs {
  const void* k_cache;
  const void* v_cache;
  const float* k_scale;  // [num_kv_heads] for an fp8 cache, else unused
  const float* v_scale;
  const void* q;
  void* out;
  const int32_t* cu_q_lens;
  const int32_t* seq_lens;
  const int32_t* block_table;
  float scale_log2;  // softmax scale * log2(e)
  int32_t num_seqs, num_q_heads, num_kv_heads, max_blocks_per_seq, max_q_len, max_seq_len;
  int32_t num_qtiles, wg_per_pair;  // filled by the launcher
  // Verify launches with a workspace (the decode workspace's layout): the
  // partial results of items split between workgroups, [group][2][32 columns]
  // (max, sum) and [group][2][32][head_dim], and one arrival counter per item,
  // keyed by its last workgroup.  part_acc == nullptr: no split.
  float* part_ml;
  float* part_acc;
  int32_t* arrivals;
  int32_t total_groups;  // filled by the launcher
};

struct DecodeWorkspace {
  size_t arrivals_off, ml_off, acc_off, total;
};

// Record the message of a failed call for pa_last_error(); returns code.
int set_error(int code, const char* fmt, ...);

DecodeWorkspace decode_workspace_layout(int64_t head_dim);

// PA_DEBUG_BOUNDS=1 in the environment: host checks of the values in device
// index arrays (debug_bounds.cpp).  Each returns PA_OK, or PA_ERR_BOUNDS /
// PA_ERR_HIP with the message set; they synchronise the stream.
bool debug_bounds_on();
int debug_check_scales(const pa_kv_cache* c, hipStream_t s);
int debug_check_store(const pa_kv_cache* c, const int32_t* slots, int32_t n, hipStream_t s);
int debug_check_copy(const pa_kv_cache* c, const int32_t* pairs, int32_t n, hipStream_t s);
int debug_check_decode(const pa_kv_cache* c, const int32_t* table, int32_t max_blocks, const int32_t* lens,
                       int32_t S, int32_t max_ctx, hipStream_t s);
int debug_check_prefill(const pa_kv_cache* c, const int32_t* cu, const int32_t* seq_lens, const int32_t* table,
                        int32_t max_blocks, int32_t S, int32_t max_q, int32_t max_seq, hipStream_t s);
int debug_check_pack(const pa_kv_cache* c, const int32_t* table, int32_t max_blocks, const int32_t* seq_lens,
                     const int32_t* cu_rows, int32_t S, int32_t max_seq, hipStream_t s);

hipError_t launch_store_kv(const StoreArgs& a, int kv_kind, hipStream_t s);
hipError_t launch_copy_blocks(const CopyArgs& a, int num_pairs, hipStream_t s);
// elem_bytes 1, 2 or 4; grid num_seqs x max_blocks_used.
hipError_t launch_pack_kv(const PackArgs& a, int elem_bytes, int num_seqs, int max_blocks_used, hipStream_t s);
// Returns hipErrorInvalidValue for a combination without a compiled kernel.
// Events a launch records with its kernel's own start and end timestamps
// (hipExtLaunchKernel); both null: a plain launch.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

hipError_t launch_decode(const DecodeArgs& a, int kv_kind, int head_dim, int block_size, int group,
                         int64_t upper_units, hipStream_t s, const LaunchEvents& ev);
// bf16 cache, head_dim 128; hipErrorInvalidValue for an uncompiled combination.
// kv_kind: KV_BF16 or KV_FP8 (bf16 queries and output in both cases).
hipError_t launch_prefill_chunk(const PrefillArgs& a, int kv_kind, int block_size, int group, hipStream_t s);
// Chunks of at most 32 / group tokens; called by launch_prefill_chunk.
hipError_t launch_verify_chunk(const PrefillArgs& a, int kv_kind, int block_size, int group, hipStream_t s);

}  // namespace pa
