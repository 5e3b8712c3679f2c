// Host-side block allocator of the paged KV cache (declared in include/pkv.h).
//
// Blocks are handed out on demand from a free list; a block table per
// sequence maps logical block j to a physical block; a reference count per
// physical block says how many tables hold it.  A forked sequence shares its
// parent's blocks, and a write into a block whose count is above 1 first
// moves the writer to a private copy (copy-on-write); the copy itself is
// device work that the caller batches into pkv_copy_blocks.
//   KV-cache post, "PagedAttention: the KV cache in blocks" (allocate on
//   demand, free immediately, sharing with copy-on-write);
//   brunomaga post, "PagedAttention: memory management for the KV cache"
//   (PagedKVCache: the free list starts as 0 .. n-1, allocation takes its
//   last entry, freeing a sequence appends its table);
//   serving lesson, "Sharing (section 4.4)" and exercise 3 (reference counts;
//   the first writers copy, the last sharer writes in place).
#include "../../include/pkv.h"

#include <stdint.h>

#include <new>
#include <unordered_map>
#include <vector>

struct pkv_block_manager {
  struct Seq {
    std::vector<int32_t> table;
    int64_t length = 0;
  };
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::vector<int32_t> free_list;        // allocation takes the back
  std::vector<int32_t> refcount;
  std::unordered_map<int64_t, Seq> seqs;

  // Blocks an append of n tokens needs: new logical blocks, plus one copy
  // when the partly filled last block is shared.
  int64_t blocks_needed(const Seq& s, int64_t n) const {
    const int64_t have = int64_t(s.table.size());
    const int64_t want = (s.length + n + block_size - 1) / block_size;
    int64_t need = want > have ? want - have : 0;
    if (n > 0 && s.length % block_size != 0 && refcount[s.table[s.length / block_size]] > 1)
      need += 1;
    return need;
  }

  int32_t take() {
    const int32_t b = free_list.back();
    free_list.pop_back();
    refcount[b] = 1;
    return b;
  }
};

extern "C" {

pkv_block_manager_t* pkv_bm_create(int32_t num_blocks, int32_t block_size) {
  if (num_blocks <= 0 || block_size <= 0) return nullptr;
  pkv_block_manager_t* m = new (std::nothrow) pkv_block_manager_t();
  if (!m) return nullptr;
  try {
    m->num_blocks = num_blocks;
    m->block_size = block_size;
    m->free_list.resize(size_t(num_blocks));
    for (int32_t i = 0; i < num_blocks; ++i) m->free_list[size_t(i)] = i;
    m->refcount.assign(size_t(num_blocks), 0);
  } catch (...) {
    delete m;
    return nullptr;
  }
  return m;
}

void pkv_bm_destroy(pkv_block_manager_t* m) { delete m; }

pkv_status_t pkv_bm_add_seq(pkv_block_manager_t* m, int64_t seq_id) {
  if (!m || m->seqs.count(seq_id)) return PKV_ERR_INVALID_ARG;
  try {
    m->seqs.emplace(seq_id, pkv_block_manager::Seq());
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  return PKV_OK;
}

pkv_status_t pkv_bm_fork(pkv_block_manager_t* m, int64_t parent, int64_t child) {
  if (!m || parent == child || !m->seqs.count(parent) || m->seqs.count(child))
    return PKV_ERR_INVALID_ARG;
  try {
    pkv_block_manager::Seq s = m->seqs.at(parent);
    for (int32_t b : s.table) m->refcount[size_t(b)] += 1;
    m->seqs.emplace(child, std::move(s));
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  return PKV_OK;
}

pkv_status_t pkv_bm_free_seq(pkv_block_manager_t* m, int64_t seq_id) {
  if (!m) return PKV_ERR_INVALID_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_INVALID_ARG;
  for (int32_t b : it->second.table) {
    if (--m->refcount[size_t(b)] == 0) m->free_list.push_back(b);
  }
  m->seqs.erase(it);
  return PKV_OK;
}

pkv_status_t pkv_bm_append_slots(pkv_block_manager_t* m, int64_t seq_id, int32_t num_tokens,
                                 int32_t* copy_src, int32_t* copy_dst, int32_t max_copies,
                                 int32_t* num_copies) {
  if (!m || num_tokens < 0 || !num_copies) return PKV_ERR_INVALID_ARG;
  auto it = m->seqs.find(seq_id);
  if (it == m->seqs.end()) return PKV_ERR_INVALID_ARG;
  pkv_block_manager::Seq& s = it->second;
  *num_copies = 0;
  const int64_t need = m->blocks_needed(s, num_tokens);
  const bool copy = num_tokens > 0 && s.length % m->block_size != 0 &&
                    m->refcount[size_t(s.table[size_t(s.length / m->block_size)])] > 1;
  if (copy && (max_copies < 1 || !copy_src || !copy_dst)) return PKV_ERR_INVALID_ARG;
  if (need > int64_t(m->free_list.size())) return PKV_ERR_OUT_OF_BLOCKS;
  try {
    s.table.reserve(size_t((s.length + num_tokens + m->block_size - 1) / m->block_size));
  } catch (...) {
    return PKV_ERR_INVALID_ARG;
  }
  if (copy) {                                   // the shared, partly filled last block
    const size_t lb = size_t(s.length / m->block_size);
    const int32_t old = s.table[lb];
    const int32_t fresh = m->take();
    m->refcount[size_t(old)] -= 1;
    s.table[lb] = fresh;
    copy_src[0] = old;
    copy_dst[0] = fresh;
    *num_copies = 1;
  }
  const int64_t want = (s.length + num_tokens + m->block_size - 1) / m->block_size;
  while (int64_t(s.table.size()) < want) s.table.push_back(m->take());
  s.length += num_tokens;
  return PKV_OK;
}

int32_t pkv_bm_num_free(const pkv_block_manager_t* m) {
  return m ? int32_t(m->free_list.size()) : -1;
}

int32_t pkv_bm_refcount(const pkv_block_manager_t* m, int32_t block) {
  if (!m || block < 0 || block >= m->num_blocks) return -1;
  return m->refcount[size_t(block)];
}

int64_t pkv_bm_seq_len(const pkv_block_manager_t* m, int64_t seq_id) {
  if (!m) return -1;
  auto it = m->seqs.find(seq_id);
  return it == m->seqs.end() ? -1 : it->second.length;
}

int32_t pkv_bm_free_list(const pkv_block_manager_t* m, int32_t* out, int32_t max_entries) {
  if (!m) return -1;
  const int32_t n = int32_t(m->free_list.size());
  if (out)
    for (int32_t i = 0; i < n && i < max_entries; ++i) out[i] = m->free_list[size_t(i)];
  return n;
}

pkv_status_t pkv_bm_block_tables(const pkv_block_manager_t* m, const int64_t* seq_ids,
                                 int32_t num_seqs, int32_t* block_tables,
                                 int32_t max_blocks_per_seq, int32_t* context_lens) {
  if (!m || num_seqs < 0 || max_blocks_per_seq <= 0) return PKV_ERR_INVALID_ARG;
  if (num_seqs == 0) return PKV_OK;
  if (!seq_ids || !block_tables || !context_lens) return PKV_ERR_INVALID_ARG;
  for (int32_t i = 0; i < num_seqs; ++i) {
    auto it = m->seqs.find(seq_ids[i]);
    if (it == m->seqs.end() || int64_t(it->second.table.size()) > max_blocks_per_seq ||
        it->second.length > INT32_MAX)
      return PKV_ERR_INVALID_ARG;
  }
  for (int32_t i = 0; i < num_seqs; ++i) {
    const pkv_block_manager::Seq& s = m->seqs.find(seq_ids[i])->second;
    int32_t* row = block_tables + size_t(i) * size_t(max_blocks_per_seq);
    for (int32_t j = 0; j < max_blocks_per_seq; ++j)
      row[j] = size_t(j) < s.table.size() ? s.table[size_t(j)] : -1;
    context_lens[i] = int32_t(s.length);
  }
  return PKV_OK;
}

}  // extern "C"
