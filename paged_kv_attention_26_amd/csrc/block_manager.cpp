// Host block manager of libpa (host memory only; no HIP calls).
//
// The paged allocator whose decisions the kernels consume as data, after the
// serving-stack page, section 2.3 (手写一个 Block Manager) and section 2.2
// (分页思想): fixed-size blocks with a reference count, a free list,
// allocation that reports exhaustion, copy on write of a shared block, fork
// by sharing every block, and a block table per sequence.
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
  pa_block_manager::Seq child = bm->seqs[size_t(seq)];
  for (int32_t b : child.table) bm->ref[size_t(b)] += 1;
  bm->seqs.push_back(std::move(child));
  return int32_t(bm->seqs.size() - 1);
}

int pa_bm_release(pa_block_manager* bm, int32_t seq) {
  if (!bm) return bm_fail(PA_ERR_NULL, "block manager is NULL");
  if (!bm->valid_seq(seq)) return bm_fail(PA_ERR_SHAPE, "unknown sequence %d", seq);
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

}  // extern "C"
