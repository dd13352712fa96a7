/*
 * pa.h -- C ABI of libpa: paged attention over a block-table-indexed KV cache
 * for AMD Instinct MI355X (gfx950).
 *
 * The method (nanoPD page "自定义CUDA分页注意力内核" and "分页KV缓存"; serving-stack
 * page section 2.2 "分页思想"): the KV cache is cut into fixed-size blocks of
 * block_size tokens; each sequence keeps a block table mapping its logical
 * block i to a physical block; every KV read goes through that table once.
 * New tokens are written to their slots (physical_block * block_size +
 * offset); forked sequences share blocks and copy a shared block before
 * writing into it (copy on write); decode attends one query per sequence to
 * all of its cached tokens; a prefill chunk attends causally to its paged
 * prefix plus itself.
 *
 * Conventions for every call below
 *  - All pointers are DEVICE pointers unless marked "host".  The caller owns
 *    every buffer; the library never allocates or frees device memory.
 *  - Calls are asynchronous on the given HIP stream (NULL = the default
 *    stream).  Nothing is synchronised inside the library.
 *  - Return value: 0 on success, or a negative PA_ERR_* code; the message of
 *    the last failure on the calling thread is returned by pa_last_error().
 *    Arguments are validated on the host before any HIP call, so a rejected
 *    call launches nothing.
 *  - Values inside device arrays (slots, block ids, lengths, fp8 scales) are
 *    NOT checked: a slot >= num_blocks * block_size, a block id >=
 *    num_blocks or a context length above max_blocks_per_seq * block_size
 *    reads or writes out of bounds (undefined behaviour), exactly like an
 *    out-of-range index.  With PA_DEBUG_BOUNDS=1 in the environment, every
 *    call first copies its index arrays (and fp8 scales) to the host on its
 *    stream, waits, and rejects the call with PA_ERR_BOUNDS, launching
 *    nothing, if a value is out of range: slots past the pool, block ids of
 *    a sequence's used blocks outside [0, num_blocks), lengths outside
 *    [0, max], chunk bounds that do not fit, copy pairs whose dst repeats or
 *    is also a src, fp8 scales that are not finite and > 0.  (The copies
 *    synchronise the stream: not for code under graph capture.)
 *  - No C++ exception crosses this interface.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  PA_FP8_E4M3 is the OCP 8-bit float E4M3FN (bias 7, max
 * +-448, no infinities, NaN = 0x7F / 0xFF), the FP8 KV format of the
 * PD-engineering page, section 6.2 (KV 缓存的精度压缩). */
typedef enum { PA_F32 = 0, PA_BF16 = 1, PA_FP8_E4M3 = 2 } pa_dtype;

enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                         */
  PA_ERR_SHAPE = -2,       /* inconsistent sizes (num_q_heads % num_kv_heads, ...)*/
  PA_ERR_DTYPE = -3,       /* unsupported dtype combination                      */
  PA_ERR_UNSUPPORTED = -4, /* head_dim / block_size / group size not compiled   */
  PA_ERR_WORKSPACE = -5,   /* workspace smaller than pa_decode_workspace_bytes() */
  PA_ERR_HIP = -6,         /* a HIP runtime call or kernel launch failed         */
  PA_ERR_NO_BLOCKS = -7,   /* block manager: the pool has no free block          */
  PA_ERR_PENDING = -8,     /* block manager: copy pairs are queued (take them)   */
  PA_ERR_BOUNDS = -9       /* PA_DEBUG_BOUNDS: a device index is out of range    */
};

/* A paged KV cache (the pools are device memory owned by the caller).
 *
 * Layout, per pool, row-major:
 *   k_cache[num_blocks][num_kv_heads][block_size][head_dim]
 *       -- one token's key row of one kv head is contiguous;
 *   v_cache[num_blocks][num_kv_heads][head_dim][block_size]
 *       -- V IS STORED TRANSPOSED inside each block (NOT [block_size]
 *          [head_dim] like the K pool): one head-dim column of a block's
 *          tokens is contiguous.  A V pool laid out like the K pool gives
 *          silently wrong attention; write V only through pa_store_kv /
 *          pa_copy_blocks, or in this layout.
 * Token t of a sequence lives in physical block table[t / block_size] at
 * offset t % block_size.
 *
 * dtype: PA_F32, PA_BF16 or PA_FP8_E4M3.  For PA_FP8_E4M3 a stored code c of
 * kv head h means c * k_scale[h] (keys) or c * v_scale[h] (values);
 * k_scale / v_scale are device arrays of num_kv_heads fp32, each FINITE AND
 * > 0 (the attention kernels fold them into positive softmax constants), and
 * must be NULL for the other dtypes.
 * Supported: head_dim in {64, 128}; block_size in {16, 32}. */
typedef struct {
  void* k_cache;
  void* v_cache;
  const float* k_scale;
  const float* v_scale;
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;
  int32_t head_dim;
  int32_t dtype; /* pa_dtype */
} pa_kv_cache;

/* Store new K/V rows into their slots (nanoPD page, the paged-KV store of the
 * paged_attention extension; serving-stack page section 2.3: a token goes to
 * its sequence's last block at offset length % block_size).
 *
 *   k_new, v_new : [num_tokens][num_kv_heads][head_dim] of in_dtype, contiguous.
 *   slot_mapping : [num_tokens] int32; slot = block * block_size + offset;
 *                  a negative slot skips that token.
 * For every token t with slot >= 0 and every kv head h:
 *   k_cache[slot / bs][h][slot % bs][:] = enc(k_new[t][h][:])
 *   v_cache[slot / bs][h][:][slot % bs] = enc(v_new[t][h][:])
 * enc is the identity when in_dtype == cache dtype (F32->F32, BF16->BF16,
 * FP8_E4M3->FP8_E4M3: codes as they are, e.g. rows from pa_pack_kv;
 * bit-exact).  Into an FP8 cache, BF16 input is quantised:
 * enc(x) = e4m3fn_round_nearest_even_saturate(float(x) / scale[h]) with an
 * IEEE fp32 division; magnitudes above 448 saturate to +-448, NaN stays NaN.
 * Two tokens with the same slot in one call: which one lands is unspecified.
 * num_tokens == 0 is a no-op. */
int pa_store_kv(const pa_kv_cache* cache, const void* k_new, const void* v_new, int32_t in_dtype,
                const int32_t* slot_mapping, int32_t num_tokens, void* hip_stream);

/* Copy whole blocks (copy on write for forked / beam sequences: nanoPD page,
 * section 分页KV缓存, where copy on write serves beam search and
 * speculative-decoding branches; serving-stack page section 2.3, cow()).
 *   src_dst : [num_pairs][2] int32 pairs (src, dst); for each pair
 *             k_cache[dst] = k_cache[src] and v_cache[dst] = v_cache[src]
 *             (all kv heads, the whole block, bit-exact).
 * The dst ids must be distinct and must not appear as a src in the same
 * call (then the copy order cannot matter).  num_pairs == 0 is a no-op. */
int pa_copy_blocks(const pa_kv_cache* cache, const int32_t* src_dst, int32_t num_pairs,
                   void* hip_stream);

/* Gather sequences' cached K/V out of the paged pools into contiguous token
 * rows: the prefill side's half of the KV hand-off to a decode instance
 * (nanoPD page, 异步KV传输; PD-engineering page section 3).  The receiving
 * side stores the rows with pa_store_kv and its own slot_mapping (for an
 * fp8 cache with in_dtype FP8_E4M3, codes unchanged).
 *   block_table : [num_seqs][max_blocks_per_seq] int32, as for pa_decode
 *   seq_lens    : [num_seqs] int32, tokens of each sequence (0 allowed)
 *   cu_rows     : [num_seqs] int32, first output row of each sequence
 *   k_out, v_out: [rows][num_kv_heads][head_dim] of the cache dtype
 * For every sequence s, token i < seq_lens[s] and kv head h (bit-exact):
 *   k_out[cu_rows[s] + i][h][:] = k_cache[table[s][i / bs]][h][i % bs][:]
 *   v_out[cu_rows[s] + i][h][:] = v_cache[table[s][i / bs]][h][:][i % bs]
 * max_seq_len is a host upper bound of seq_lens (sizes the launch; at most
 * 65535 blocks).  Rows of different sequences must not overlap. */
int pa_pack_kv(const pa_kv_cache* cache, const int32_t* block_table, int32_t max_blocks_per_seq,
               const int32_t* seq_lens, const int32_t* cu_rows, int32_t num_seqs, int32_t max_seq_len,
               void* k_out, void* v_out, void* hip_stream);

/* Bytes of device workspace pa_decode needs (host call, no HIP): two partial
 * results per wavefront for at most 4096 wavefronts and 8 query heads per kv
 * head, about 34 MB at head_dim 128 whatever the batch (one size serves
 * every shape, so one buffer serves every call on a stream).  Returns 0 for
 * negative sizes. */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_context_len, int32_t partition_tokens);

/* Paged decode attention: one query token per sequence, grouped-query heads
 * (PD-engineering page section 6.2: 8 KV heads shared by 32 query heads;
 * query head h reads kv head h / (num_q_heads / num_kv_heads)).
 *
 *   q   : [num_seqs][num_q_heads][head_dim] of q_dtype
 *   out : [num_seqs][num_q_heads][head_dim] of out_dtype
 *   block_table  : [num_seqs][max_blocks_per_seq] int32 physical block ids;
 *                  entries past a sequence's last block are never read.
 *   context_lens : [num_seqs] int32, tokens to attend to, including the one
 *                  just stored.  A length of 0 gives an output of 0.
 *   max_context_len : host upper bound of context_lens (sizes the launch).
 *   out[s][h] = sum_i softmax_i(scale * <q[s][h], k_i>) * v_i over tokens
 *   i < context_lens[s], accumulated in fp32.  scale must be finite and > 0
 *   (the softmax scale, 1/sqrt(head_dim) for the pages' attention).
 *
 * Work is cut into partitions of partition_tokens tokens of one (sequence,
 * kv head): a positive multiple of block_size (64 is the fastest on
 * MI355X), or 0 for no split (one partition spans max_context_len, so no
 * (sequence, kv head) is shared between wavefronts).  Every wavefront of the
 * launch takes an equal, contiguous run of partitions and keeps a running
 * max / sum across the partitions of one (sequence, kv head); where runs cut
 * a (sequence, kv head) apart, their partial results are merged by
 * log-sum-exp rescaling, in the same kernel, by whichever of those
 * wavefronts finishes last.
 * The result does not depend on partition_tokens or on the split beyond
 * fp32 rounding.
 *
 * dtypes: F32 cache -> q, out F32; BF16 cache -> q, out BF16;
 * FP8 cache -> q, out BF16.
 *
 * workspace: device memory of at least pa_decode_workspace_bytes() bytes
 * holding partial results and one arrival counter per split item.  It must
 * be zero-filled before its first use (hipMemset once); every completed call
 * leaves the counters at zero again, so the same workspace serves any number
 * of later calls, of any shape, on one stream.  Two calls that may run at
 * the same time must not share a workspace. */
int pa_decode(const pa_kv_cache* cache, const void* q, int32_t q_dtype, void* out, int32_t out_dtype,
              int32_t num_seqs, int32_t num_q_heads, float scale, const int32_t* block_table,
              int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
              int32_t partition_tokens, void* workspace, size_t workspace_bytes, void* hip_stream);

/* A decode step's store and attention in one launch (nanoPD page: the paged
 * KV cache's store operation beside its attention kernel; serving-stack page,
 * section 2.3: a sequence's new token goes to offset length % block_size of
 * its last block): the same results, bit for bit, as
 *   pa_store_kv(k_new, v_new, slots) followed by pa_decode(...)
 * where token s of the store is sequence s's new token, at position
 * context_lens[s] - 1, in the slot the block table gives for that position:
 *   slot = block_table[s][(L-1) / block_size] * block_size + (L-1) % block_size.
 *
 *   k_new, v_new : [num_seqs][num_kv_heads][head_dim] device rows in the
 *                  cache's input dtype (F32 for an F32 cache, BF16 for BF16
 *                  and FP8 caches; an FP8 cache stores value / scale[h]
 *                  rounded to e4m3, as pa_store_kv does).
 * Sequences with context_lens[s] == 0 store nothing.  All other arguments,
 * the workspace rules and the errors are those of pa_decode; NULL k_new or
 * v_new is PA_ERR_NULL.  The block of the new token must be allocated in the
 * table (as for pa_store_kv).  pa_decode_time_next arms this call as it arms
 * pa_decode. */
int pa_decode_append(const pa_kv_cache* cache, const void* k_new, const void* v_new, const void* q,
                     int32_t q_dtype, void* out, int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads,
                     float scale, const int32_t* block_table, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t max_context_len, int32_t partition_tokens,
                     void* workspace, size_t workspace_bytes, void* hip_stream);

/* pa_decode without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops or harnesses
 * that forbid allocation).  Arguments, results and errors as for pa_decode.
 * The split-K partials and arrival counters live in a device array inside
 * the library (34 095 104 bytes, the workspace pa_decode needs at its
 * largest: head_dim 128, groups of 8, 4096 wavefronts); each GPU the library
 * runs on holds its own copy until the process ends.  The first call on a
 * device looks its copy up and clears the counters (a small kernel on the
 * given stream); no call allocates or frees memory.  Every call on one GPU
 * shares that GPU's array, which keeps the last call's contents (each
 * completed call leaves the counters at zero): two calls that may run at
 * the same time on one GPU -- on different streams, or from different
 * threads -- RACE and give undefined results. */
int pa_decode_noalloc(const pa_kv_cache* cache, const void* q, int32_t q_dtype, void* out, int32_t out_dtype,
                      int32_t num_seqs, int32_t num_q_heads, float scale, const int32_t* block_table,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                      int32_t partition_tokens, void* hip_stream);

/* Timing hook for measurement (no counterpart in the pages): the next
 * pa_decode call made on this thread records start_event and stop_event
 * (hipEvent_t, created by the caller with timing enabled, either may be
 * NULL) with its kernel's own start and end timestamps, through
 * hipExtLaunchKernel, instead of marker packets placed around the call in the
 * stream, which add several microseconds of their own to the window and to
 * the stream.  One call arms one pa_decode (or pa_decode_append) call: that call disarms it at
 * entry, whether it then launches or not (a call rejected by its checks, or
 * one with num_seqs == 0, leaves the events untouched).  Passing NULL, NULL
 * disarms.  Returns PA_OK. */
int pa_decode_time_next(void* start_event, void* stop_event);

/* Chunked-prefill attention (nanoPD page "分块预填充"; PD-engineering page
 * section 6.1; serving-stack page section 5.2): sequence j appends a chunk
 * of q_len_j = cu_q_lens[j+1] - cu_q_lens[j] tokens, already stored in the
 * cache by pa_store_kv, after P_j = seq_lens[j] - q_len_j cached tokens.
 * Chunk row t (absolute position P_j + t) attends to tokens 0 .. P_j + t.
 *
 *   q   : [cu_q_lens[num_seqs]][num_q_heads][head_dim] BF16
 *   out : same shape, BF16
 *   cu_q_lens : [num_seqs + 1] int32, non-decreasing, cu_q_lens[0] == 0
 *   seq_lens  : [num_seqs] int32, tokens of the sequence including the chunk
 *   block_table : [num_seqs][max_blocks_per_seq] int32
 *   max_q_len, max_seq_len : host upper bounds (size the launch)
 * scale must be finite and > 0.
 * QK^T and PV run on bf16 matrix cores with fp32 accumulation; the
 * probabilities are rounded to bf16 for PV.  Supported: BF16 or FP8_E4M3
 * cache (q and out BF16 either way; an fp8 code of kv head h stands for
 * code * k_scale[h] or code * v_scale[h], converted to bf16 exactly, the
 * scales applied outside the contraction), head_dim 128.  ONLY THAT SUBSET:
 * an F32 cache (or F32 q / out) is rejected with PA_ERR_DTYPE and head_dim
 * 64 with PA_ERR_UNSUPPORTED (decode, store, copy and pack take all three
 * cache dtypes at both head dims).
 * Chunks of at most 32 / (num_q_heads / num_kv_heads) tokens -- the shape of
 * speculative-decoding verification, k draft tokens plus one -- run on a
 * kernel whose matrix-core columns are the (query head, token) pairs of a
 * kv head (serving-stack page, speculative decoding).
 *
 * workspace (optional, used by that verification kernel only): NULL, or
 * device memory of at least pa_decode_workspace_bytes() bytes with the same
 * rules as pa_decode's workspace (zero-filled before its first use; every
 * completed call leaves it ready for the next; one buffer serves pa_decode
 * and pa_prefill_chunk calls that run one after another on a stream; calls
 * that may run at the same time need their own).  Without a workspace, one
 * workgroup computes each (sequence, kv head) whole, so a batch of unequal
 * contexts waits for its longest and a batch of few sequences leaves most
 * CUs idle.  With one, the kernel reads the batch's lengths and, unless every
 * (sequence, kv head) has a workgroup and none is more than twice an equal
 * share, cuts the verification keys of the whole batch into equal stretches,
 * one per CU; a (sequence, kv head) cut between stretches is merged by
 * log-sum-exp rescaling in the same kernel (at most 4096 sequences; larger
 * batches run as without).  The results agree within fp32 rounding.  A
 * non-NULL workspace smaller than pa_decode_workspace_bytes() is rejected
 * with PA_ERR_WORKSPACE. */
int pa_prefill_chunk(const pa_kv_cache* cache, const void* q, int32_t q_dtype, void* out,
                     int32_t out_dtype, int32_t num_seqs, int32_t num_q_heads, float scale,
                     const int32_t* cu_q_lens, const int32_t* seq_lens, const int32_t* block_table,
                     int32_t max_blocks_per_seq, int32_t max_q_len, int32_t max_seq_len,
                     void* workspace, size_t workspace_bytes, void* hip_stream);

/* Checks of index arrays held in HOST memory (no HIP), the same checks that
 * PA_DEBUG_BOUNDS=1 runs on every call's device arrays.  Each returns PA_OK
 * or PA_ERR_BOUNDS (pa_last_error() names the first bad entry); NULL
 * arrays give PA_ERR_NULL.
 *   pa_check_slots      : slot_mapping[n] -- every slot < num_blocks * block_size
 *                         (negative slots are skips)
 *   pa_check_copy_pairs : src_dst[n][2] -- ids in [0, num_blocks), dst ids
 *                         distinct, no dst also a src
 *   pa_check_tables     : lens[num_seqs] in [0, max_len], and the first
 *                         ceil(len / block_size) entries of each
 *                         table[num_seqs][max_blocks] row in [0, num_blocks)
 *   pa_check_chunks     : cu_q_lens[num_seqs + 1] starts at 0, every chunk
 *                         has 0 .. max_q_len rows and seq_lens[j] >= its rows
 *   pa_check_scales     : k_scale / v_scale [num_kv_heads] finite and > 0 */
int pa_check_slots(const pa_kv_cache* cache, const int32_t* slot_mapping, int32_t n);
int pa_check_copy_pairs(const pa_kv_cache* cache, const int32_t* src_dst, int32_t n);
int pa_check_tables(const pa_kv_cache* cache, const int32_t* table, int32_t max_blocks, const int32_t* lens,
                    int32_t num_seqs, int32_t max_len);
int pa_check_chunks(const pa_kv_cache* cache, const int32_t* cu_q_lens, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t max_q_len);
int pa_check_scales(const pa_kv_cache* cache, const float* k_scale, const float* v_scale);

/* Message of the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

/* ------------------------------------------------------------------------
 * Host block manager (host memory only, no HIP): the paged allocator whose
 * decisions the kernels above consume as data (serving-stack page section
 * 2.3: allocate / incref / free / cow / append / fork / release).
 *  - the free list starts as free_order (host, a permutation of
 *    0..num_blocks-1; NULL = 0,1,2,...); allocation takes the LAST entry of
 *    the list and freed blocks are appended to its end;
 *  - appending to a sequence whose length is a multiple of block_size takes
 *    a new block; otherwise a shared tail block (reference count > 1) is
 *    first copied: a new block is taken, the pair (old, new) is queued for
 *    pa_copy_blocks and the old block loses one reference.
 *  - ORDER: a queued pair is a copy that has not run.  pa_bm_fork and
 *    pa_bm_release fail with PA_ERR_PENDING while pairs are queued (a fork
 *    then could make a queued pair's dst shared again, so that the next
 *    append queues a copy out of it -- a chain pa_copy_blocks cannot run --
 *    and a release could free a queued pair's block and hand it out again).
 *    Take the pairs with pa_bm_take_copies, and on the stream run
 *    pa_copy_blocks with them and then pa_store_kv of the slots handed out
 *    so far, before the copies and stores of later appends.
 * All ids are int32; functions returning int return PA_ERR_* on failure.
 * Not thread-safe: one manager per thread. */
typedef struct pa_block_manager pa_block_manager;

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order);
void pa_bm_destroy(pa_block_manager* bm);
/* New empty sequence; returns its id (>= 0). */
int32_t pa_bm_seq_new(pa_block_manager* bm);
/* Append n tokens to seq, writing their slots to slots_out (host, [n]).
 * Returns the number appended: n, or fewer when the pool ran out (then
 * pa_last_error() says so and the sequence keeps the tokens appended). */
int32_t pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t n, int32_t* slots_out);
/* Fork: a new sequence sharing every block of seq; returns its id. */
int32_t pa_bm_fork(pa_block_manager* bm, int32_t seq);
/* Drop every block reference of seq; the id stays valid and empty. */
int pa_bm_release(pa_block_manager* bm, int32_t seq);
/* Move up to max_pairs queued (src, dst) copy pairs to pairs_out (host,
 * [max_pairs][2]); returns how many were moved (oldest first). */
int32_t pa_bm_take_copies(pa_block_manager* bm, int32_t* pairs_out, int32_t max_pairs);
int32_t pa_bm_seq_len(const pa_block_manager* bm, int32_t seq);
/* Copy seq's block table to table_out (host, [max_entries]); returns the
 * number of blocks it holds (which may exceed max_entries). */
int32_t pa_bm_block_table(const pa_block_manager* bm, int32_t seq, int32_t* table_out,
                          int32_t max_entries);
int32_t pa_bm_used_blocks(const pa_block_manager* bm);
int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block);

/* Prefix cache (serving-stack page, section 4: 前缀缓存, its hash-chain
 * route and minimal implementation).  Off (capacity 0) on creation.
 *  - a key names one FULL block of block_size token ids together with the
 *    key of the block before it, so equal keys mean equal prefixes; keys
 *    are exact (no digest), so distinct prefixes never share a block;
 *  - the cache holds one reference of its own on every cached block: a
 *    cached block outlives the sequences that computed it, stays counted in
 *    pa_bm_used_blocks, and returns to the free list when it is evicted and
 *    no sequence holds it;
 *  - at most capacity_blocks entries; inserting past that evicts the least
 *    recently used entry (a lookup hit and an insert count as uses; blocks
 *    of one chain are used front to back, so a chain loses its front first
 *    and its later entries stop being reachable until the front returns);
 *  - a lookup that covers at least one block counts as a hit, else a miss.
 * The token ids are opaque int32 values; they are not stored in the KV
 * cache and the library never reads device memory here. */
/* Set the capacity in blocks (0 turns the cache off and evicts every entry;
 * lowering it evicts least recently used entries down to the new size). */
int pa_bm_prefix_cache_set_capacity(pa_block_manager* bm, int32_t capacity_blocks);
/* Longest cached prefix of token_ids (host, [n]): walks its full blocks
 * front to back and stops at the first one not cached.  Writes up to
 * max_blocks of the hit's physical blocks to blocks_out (host) and returns
 * the hit length in tokens (a multiple of block_size). */
int32_t pa_bm_prefix_lookup(pa_block_manager* bm, const int32_t* token_ids, int32_t n,
                            int32_t* blocks_out, int32_t max_blocks);
/* New sequence starting from the longest cached prefix of token_ids: it
 * shares those blocks (one more reference each) and its length is the hit
 * (pa_bm_seq_len); the caller appends the remaining tokens with
 * pa_bm_append, whose first slot opens a new block.  Returns its id. */
int32_t pa_bm_seq_new_prefixed(pa_block_manager* bm, const int32_t* token_ids, int32_t n);
/* Record the full blocks of token_ids (host, [n], n <= the sequence's
 * length: the ids of seq's first n tokens) with seq's block table; blocks
 * whose key is already cached keep the cached entry.  Returns the number of
 * entries added. */
int32_t pa_bm_prefix_insert(pa_block_manager* bm, int32_t seq, const int32_t* token_ids, int32_t n);
/* out (host, int64[4]) = hits, misses, cached blocks, capacity. */
int pa_bm_prefix_stats(const pa_block_manager* bm, int64_t* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
