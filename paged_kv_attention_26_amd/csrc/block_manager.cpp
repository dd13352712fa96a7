// Host block manager of libpa (host memory only; no HIP calls).
//
// The paged allocator whose decisions the kernels consume as data, after the
// serving-stack page, section 2.3 (手写一个 Block Manager) and section 2.2
// (分页思想): fixed-size blocks with a reference count, a free list,
// allocation that reports exhaustion, copy on write of a shared block, fork
// by sharing every block, and a block table per sequence.
//
// It also keeps the optional prefix cache of section 4 (前缀缓存) of the same
// page: full blocks keyed by a chain (parent key, the block's token ids),
// longest-prefix lookup that stops at the first uncached block, and
// least-recently-used eviction at a capacity counted in blocks.  Keys are
// exact (the parent's key and the ids themselves, interned), not digests, so
// two different prefixes never share a block.
#include <unordered_map>
#include <vector>

#include "../../include/pa.h"
#include "pa_internal.h"

using pa::set_error;
#define bm_fail set_error

struct pa_block_manager {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> ref;       // per block
  std::vector<int32_t> free_ids;  // allocation pops the back
  struct Seq {
    std::vector<int32_t> table;
    int32_t length = 0;
  };
  std::vector<Seq> seqs;
  std::vector<int32_t> copies;    // queued (src, dst) pairs, flattened
  size_t copies_head = 0;

  int32_t allocate() {
    if (free_ids.empty()) return -1;
    const int32_t b = free_ids.back();
    free_ids.pop_back();
    ref[b] = 1;
    return b;
  }
  void release_block(int32_t b) {
    if (--ref[b] == 0) free_ids.push_back(b);
  }
  // Copy on write: keep an unshared block, else take a private copy.
  int32_t cow(int32_t b) {
    if (ref[b] == 1) return b;
    const int32_t n = allocate();
    if (n < 0) return -1;
    copies.push_back(b);
    copies.push_back(n);
    release_block(b);
    return n;
  }
  bool valid_seq(int32_t s) const { return s >= 0 && size_t(s) < seqs.size(); }
  size_t queued_copies() const { return (copies.size() - copies_head) / 2; }

  // ---- prefix cache --------------------------------------------------------
  // A node is one interned chain key.  It stays interned while its block is
  // cached or some interned key names it as parent, so a key is found again
  // (same node) exactly when a digest of the same chain would be.
  struct KeyHash {
    size_t operator()(const std::vector<int32_t>& v) const {
      uint64_t h = 1469598103934665603ull;
      for (int32_t x : v) h = (h ^ uint32_t(x)) * 1099511628211ull;
      return size_t(h ^ (h >> 29));
    }
  };
  struct Node {
    std::vector<int32_t> key;  // [parent node, ids of the block...]
    int32_t block = -1;        // cached physical block, -1 when not cached
    int32_t children = 0;      // interned keys naming this node as parent
    int32_t prev = -1, next = -1;  // links of the LRU list while cached
  };
  std::unordered_map<std::vector<int32_t>, int32_t, KeyHash> intern;
  std::vector<Node> nodes;
  std::vector<int32_t> free_nodes;
  // Cached nodes in an intrusive list, least recently used at the head.
  int32_t lru_head = -1, lru_tail = -1, cached = 0;
  int32_t capacity = 0;            // 0: prefix cache off
  int64_t hits = 0, misses = 0;
  std::vector<int32_t> scratch_key;

  const std::vector<int32_t>& make_key(int32_t parent, const int32_t* ids) {
    scratch_key.resize(size_t(block_size) + 1);
    scratch_key[0] = parent;
    for (int32_t i = 0; i < block_size; ++i) scratch_key[size_t(i) + 1] = ids[i];
    return scratch_key;
  }
  int32_t find(int32_t parent, const int32_t* ids) {
    auto it = intern.find(make_key(parent, ids));
    return it == intern.end() ? -1 : it->second;
  }
  int32_t find_or_add(int32_t parent, const int32_t* ids) {
    const int32_t f = find(parent, ids);
    if (f >= 0) return f;
    int32_t n;
    if (!free_nodes.empty()) {
      n = free_nodes.back();
      free_nodes.pop_back();
    } else {
      n = int32_t(nodes.size());
      nodes.emplace_back();
    }
    Node& nd = nodes[size_t(n)];
    nd.key = scratch_key;
    nd.block = -1;
    nd.children = 0;
    intern.emplace(nd.key, n);
    if (parent >= 0) nodes[size_t(parent)].children += 1;
    return n;
  }
  // Forget keys that are neither cached nor anyone's parent, walking up.
  void unintern(int32_t n) {
    while (n >= 0 && nodes[size_t(n)].block < 0 && nodes[size_t(n)].children == 0) {
      Node& nd = nodes[size_t(n)];
      const int32_t parent = nd.key[0];
      intern.erase(nd.key);
      nd.key.clear();
      free_nodes.push_back(n);
      if (parent >= 0) nodes[size_t(parent)].children -= 1;
      n = parent;
    }
  }
  void lru_unlink(int32_t n) {
    Node& nd = nodes[size_t(n)];
    (nd.prev >= 0 ? nodes[size_t(nd.prev)].next : lru_head) = nd.next;
    (nd.next >= 0 ? nodes[size_t(nd.next)].prev : lru_tail) = nd.prev;
    nd.prev = nd.next = -1;
  }
  void lru_push_back(int32_t n) {
    Node& nd = nodes[size_t(n)];
    nd.prev = lru_tail;
    nd.next = -1;
    (lru_tail >= 0 ? nodes[size_t(lru_tail)].next : lru_head) = n;
    lru_tail = n;
  }
  void touch(int32_t n) {
    lru_unlink(n);
    lru_push_back(n);
  }
  // Cache block b under node n (one reference of the cache's own).
  void cache_block(int32_t n, int32_t b) {
    nodes[size_t(n)].block = b;
    ref[size_t(b)] += 1;
    lru_push_back(n);
    cached += 1;
  }
  void evict_lru() {
    const int32_t v = lru_head;
    lru_unlink(v);
    cached -= 1;
    release_block(nodes[size_t(v)].block);
    nodes[size_t(v)].block = -1;
    unintern(v);
  }
  // Longest cached prefix of ids[0, n): appends its blocks to out.
  int32_t lookup(const int32_t* ids, int32_t n, std::vector<int32_t>& out) {
    int32_t parent = -1, hit = 0;
    for (int32_t i = 0; i + block_size <= n; i += block_size) {
      const int32_t nd = find(parent, ids + i);
      if (nd < 0 || nodes[size_t(nd)].block < 0) break;
      out.push_back(nodes[size_t(nd)].block);
      touch(nd);
      hit += block_size;
      parent = nd;
    }
    if (hit > 0) hits += 1; else misses += 1;
    return hit;
  }
};

extern "C" {

pa_block_manager* pa_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order) {
  if (num_blocks <= 0 || block_size <= 0) {
    bm_fail(PA_ERR_SHAPE, "num_blocks and block_size must be > 0");
    return nullptr;
  }
  auto* bm = new pa_block_manager;
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(size_t(num_blocks), 0);
  bm->free_ids.resize(size_t(num_blocks));
  std::vector<char> seen(size_t(num_blocks), 0);
  for (int32_t i = 0; i < num_blocks; ++i) {
    const int32_t b = free_order ? free_order[i] : i;
    if (b < 0 || b >= num_blocks || seen[size_t(b)]) {
      delete bm;
      bm_fail(PA_ERR_SHAPE, "free_order is not a permutation of 0..%d", num_blocks - 1);
      return nullptr;
    }
    seen[size_t(b)] = 1;
    bm->free_ids[size_t(i)] = b;
  }
  return bm;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

int32_t pa_bm_seq_new(pa_block_manager* bm) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  bm->seqs.emplace_back();
  return int32_t(bm->seqs.size() - 1);
}

int32_t pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t n, int32_t* slots_out) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (!bm->valid_seq(seq)) return bm_fail(PA_ERR_SHAPE, "unknown sequence %d", seq);
  if (n < 0) return bm_fail(PA_ERR_SHAPE, "n %d < 0", n);
  if (n > 0 && !slots_out) return bm_fail(PA_ERR_NULL, "slots_out is NULL");
  auto& s = bm->seqs[size_t(seq)];
  const int32_t B = bm->block_size;
  for (int32_t i = 0; i < n; ++i) {
    if (s.length % B == 0) {
      const int32_t b = bm->allocate();
      if (b < 0) {
        bm_fail(PA_ERR_NO_BLOCKS, "sequence %d: no free block after %d of %d tokens", seq, i, n);
        return i;
      }
      s.table.push_back(b);
    } else {
      const int32_t b = bm->cow(s.table.back());
      if (b < 0) {
        bm_fail(PA_ERR_NO_BLOCKS, "sequence %d: no free block for copy-on-write after %d of %d tokens", seq, i, n);
        return i;
      }
      s.table.back() = b;
    }
    slots_out[i] = s.table.back() * B + s.length % B;
    s.length += 1;
  }
  return n;
}

int32_t pa_bm_fork(pa_block_manager* bm, int32_t seq) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (!bm->valid_seq(seq)) return bm_fail(PA_ERR_SHAPE, "unknown sequence %d", seq);
  if (bm->queued_copies())
    return bm_fail(PA_ERR_PENDING, "fork of sequence %d while %zu copy pairs are queued", seq, bm->queued_copies());
  pa_block_manager::Seq child = bm->seqs[size_t(seq)];
  for (int32_t b : child.table) bm->ref[size_t(b)] += 1;
  bm->seqs.push_back(std::move(child));
  return int32_t(bm->seqs.size() - 1);
}

int pa_bm_release(pa_block_manager* bm, int32_t seq) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (!bm->valid_seq(seq)) return bm_fail(PA_ERR_SHAPE, "unknown sequence %d", seq);
  if (bm->queued_copies())
    return bm_fail(PA_ERR_PENDING, "release of sequence %d while %zu copy pairs are queued", seq,
                   bm->queued_copies());
  auto& s = bm->seqs[size_t(seq)];
  for (int32_t b : s.table) bm->release_block(b);
  s.table.clear();
  s.length = 0;
  return PA_OK;
}

int32_t pa_bm_take_copies(pa_block_manager* bm, int32_t* pairs_out, int32_t max_pairs) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (max_pairs < 0) return bm_fail(PA_ERR_SHAPE, "max_pairs < 0");
  const size_t avail = (bm->copies.size() - bm->copies_head) / 2;
  const size_t n = avail < size_t(max_pairs) ? avail : size_t(max_pairs);
  if (n > 0 && !pairs_out) return bm_fail(PA_ERR_NULL, "pairs_out is NULL");
  for (size_t i = 0; i < 2 * n; ++i) pairs_out[i] = bm->copies[bm->copies_head + i];
  bm->copies_head += 2 * n;
  if (bm->copies_head == bm->copies.size()) {
    bm->copies.clear();
    bm->copies_head = 0;
  }
  return int32_t(n);
}

int32_t pa_bm_seq_len(const pa_block_manager* bm, int32_t seq) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (!bm->valid_seq(seq)) return bm_fail(PA_ERR_SHAPE, "unknown sequence %d", seq);
  return bm->seqs[size_t(seq)].length;
}

int32_t pa_bm_block_table(const pa_block_manager* bm, int32_t seq, int32_t* table_out, int32_t max_entries) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (!bm->valid_seq(seq)) return bm_fail(PA_ERR_SHAPE, "unknown sequence %d", seq);
  const auto& t = bm->seqs[size_t(seq)].table;
  const int32_t n = int32_t(t.size());
  for (int32_t i = 0; i < n && i < max_entries; ++i) table_out[i] = t[size_t(i)];
  return n;
}

int32_t pa_bm_used_blocks(const pa_block_manager* bm) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  return bm->num_blocks - int32_t(bm->free_ids.size());
}

int32_t pa_bm_ref_count(const pa_block_manager* bm, int32_t block) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (block < 0 || block >= bm->num_blocks) return bm_fail(PA_ERR_SHAPE, "block %d out of range", block);
  return bm->ref[size_t(block)];
}

int pa_bm_prefix_cache_set_capacity(pa_block_manager* bm, int32_t capacity_blocks) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (capacity_blocks < 0) return bm_fail(PA_ERR_SHAPE, "capacity_blocks %d < 0", capacity_blocks);
  while (bm->cached > capacity_blocks) bm->evict_lru();
  bm->capacity = capacity_blocks;
  return PA_OK;
}

int32_t pa_bm_prefix_lookup(pa_block_manager* bm, const int32_t* token_ids, int32_t n,
                            int32_t* blocks_out, int32_t max_blocks) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (bm->capacity == 0) return bm_fail(PA_ERR_SHAPE, "prefix cache is off (capacity 0)");
  if (n < 0 || max_blocks < 0) return bm_fail(PA_ERR_SHAPE, "n %d or max_blocks %d < 0", n, max_blocks);
  if (n > 0 && !token_ids) return bm_fail(PA_ERR_NULL, "token_ids is NULL");
  std::vector<int32_t> blocks;
  const int32_t hit = bm->lookup(token_ids, n, blocks);
  if (!blocks.empty() && max_blocks > 0 && !blocks_out) return bm_fail(PA_ERR_NULL, "blocks_out is NULL");
  for (size_t i = 0; i < blocks.size() && i < size_t(max_blocks); ++i) blocks_out[i] = blocks[i];
  return hit;
}

int32_t pa_bm_seq_new_prefixed(pa_block_manager* bm, const int32_t* token_ids, int32_t n) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (bm->capacity == 0) return bm_fail(PA_ERR_SHAPE, "prefix cache is off (capacity 0)");
  if (n < 0) return bm_fail(PA_ERR_SHAPE, "n %d < 0", n);
  if (n > 0 && !token_ids) return bm_fail(PA_ERR_NULL, "token_ids is NULL");
  pa_block_manager::Seq s;
  s.length = bm->lookup(token_ids, n, s.table);
  for (int32_t b : s.table) bm->ref[size_t(b)] += 1;
  bm->seqs.push_back(std::move(s));
  return int32_t(bm->seqs.size() - 1);
}

int32_t pa_bm_prefix_insert(pa_block_manager* bm, int32_t seq, const int32_t* token_ids, int32_t n) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (bm->capacity == 0) return bm_fail(PA_ERR_SHAPE, "prefix cache is off (capacity 0)");
  if (!bm->valid_seq(seq)) return bm_fail(PA_ERR_SHAPE, "unknown sequence %d", seq);
  const auto& s = bm->seqs[size_t(seq)];
  if (n < 0 || n > s.length)
    return bm_fail(PA_ERR_SHAPE, "n %d outside the %d tokens of sequence %d", n, s.length, seq);
  if (n > 0 && !token_ids) return bm_fail(PA_ERR_NULL, "token_ids is NULL");
  const int32_t B = bm->block_size;
  int32_t parent = -1, added = 0;
  for (int32_t j = 0; (j + 1) * B <= n; ++j) {
    const int32_t nd = bm->find_or_add(parent, token_ids + size_t(j) * B);
    if (bm->nodes[size_t(nd)].block < 0) {
      if (bm->cached >= bm->capacity) {
        // nd may be an older key whose cached descendants outlived it; the
        // eviction can drop such a descendant and walk up to nd, so nd is
        // pinned (one extra child) while it runs.  nd's ancestors each have
        // an interned child and stay.
        bm->nodes[size_t(nd)].children += 1;
        bm->evict_lru();
        bm->nodes[size_t(nd)].children -= 1;
      }
      bm->cache_block(nd, s.table[size_t(j)]);
      added += 1;
    } else {
      bm->touch(nd);
    }
    parent = nd;
  }
  return added;
}

int pa_bm_prefix_stats(const pa_block_manager* bm, int64_t* out) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (!out) return bm_fail(PA_ERR_NULL, "out is NULL");
  out[0] = bm->hits;
  out[1] = bm->misses;
  out[2] = bm->cached;
  out[3] = bm->capacity;
  return PA_OK;
}

}  // extern "C"
