// block_manager.cpp - host-side KV block manager (C ABI in include/pa_block_manager.h).
//
// Pages cited (title, site): [AB] "什么是分页注意力（PagedAttention）？" aiboss88.com;
// [CY] "深入解析 PagedAttention：vLLM 显存优化的核心魔法" cygnushan.xyz; [ASP]
// "PagedAttention" awesome-system-papers; [RK] "什么是 LLM 中的分页注意力(Paged
// Attention)?它是如何工作的?" news.rkmt.cn.
//
// Plain host bookkeeping: a FIFO free list of physical blocks, a reference count per
// block, and per sequence its block table and length.  Every operation checks
// everything first and changes state only when it cannot fail any more.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <deque>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa_block_manager.h"

// the error text lives in pa_api.cpp (one per thread)
extern "C" void pa_set_last_error_internal(const char* text);

namespace {

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  pa_set_last_error_internal(buf);
  return st;
}

struct Sequence {
  std::vector<int32_t> blocks;  // logical block j -> physical block ([RK] 块表)
  int32_t len = 0;              // tokens
};

}  // namespace

struct pa_block_manager {
  int64_t num_blocks;
  int32_t block_size;
  int32_t max_blocks;
  std::deque<int32_t> free_list;  // handed out from the front, returned to the back
  std::vector<int32_t> refs;      // per physical block
  std::unordered_map<int32_t, Sequence> seqs;
  int32_t next_id = 0;

  const Sequence* find(int32_t id) const {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  Sequence* find(int32_t id) {
    auto it = seqs.find(id);
    return it == seqs.end() ? nullptr : &it->second;
  }
  void release(int32_t b) {
    if (--refs[b] == 0) free_list.push_back(b);
  }
};

extern "C" {

pa_status pa_bm_create(int64_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       const int32_t* free_order, pa_block_manager** out) {
  pa_set_last_error_internal("");
  if (!out) return fail(PA_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  if (num_blocks < 1 || num_blocks > INT32_MAX)
    return fail(PA_ERR_INVALID_ARG, "num_blocks %lld outside [1, 2^31)", (long long)num_blocks);
  if (block_size < 1) return fail(PA_ERR_INVALID_ARG, "block_size %d < 1", block_size);
  if (max_blocks_per_seq < 1) return fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq %d < 1", max_blocks_per_seq);
  std::vector<int32_t> order;
  try {
    order.resize((size_t)num_blocks);
    if (free_order) {
      std::vector<char> seen((size_t)num_blocks, 0);
      for (int64_t i = 0; i < num_blocks; ++i) {
        const int32_t b = free_order[i];
        if (b < 0 || b >= num_blocks || seen[(size_t)b])
          return fail(PA_ERR_INVALID_ARG, "free_order is not a permutation of 0 .. num_blocks-1");
        seen[(size_t)b] = 1;
        order[(size_t)i] = b;
      }
    } else {
      for (int64_t i = 0; i < num_blocks; ++i) order[(size_t)i] = (int32_t)i;
    }
    auto* bm = new pa_block_manager();
    bm->num_blocks = num_blocks;
    bm->block_size = block_size;
    bm->max_blocks = max_blocks_per_seq;
    bm->free_list.assign(order.begin(), order.end());
    bm->refs.assign((size_t)num_blocks, 0);
    *out = bm;
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "out of host memory");
  }
  return PA_OK;
}

void pa_bm_destroy(pa_block_manager* bm) { delete bm; }

pa_status pa_bm_add_sequence(pa_block_manager* bm, int32_t* seq_out) {
  pa_set_last_error_internal("");
  if (!bm || !seq_out) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  if (bm->next_id == INT32_MAX) return fail(PA_ERR_CAPACITY, "sequence ids exhausted");
  try {
    bm->seqs.emplace(bm->next_id, Sequence());
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "out of host memory");
  }
  *seq_out = bm->next_id++;
  return PA_OK;
}

pa_status pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child_out) {
  pa_set_last_error_internal("");
  if (!bm || !child_out) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  const Sequence* p = bm->find(parent);
  if (!p) return fail(PA_ERR_INVALID_ARG, "no sequence %d", parent);
  if (bm->next_id == INT32_MAX) return fail(PA_ERR_CAPACITY, "sequence ids exhausted");
  try {
    Sequence c = *p;  // same table, same length
    bm->seqs.emplace(bm->next_id, std::move(c));
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "out of host memory");
  }
  for (int32_t b : bm->seqs[bm->next_id].blocks) ++bm->refs[(size_t)b];
  *child_out = bm->next_id++;
  return PA_OK;
}

pa_status pa_bm_free_sequence(pa_block_manager* bm, int32_t seq) {
  pa_set_last_error_internal("");
  if (!bm) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  Sequence* s = bm->find(seq);
  if (!s) return fail(PA_ERR_INVALID_ARG, "no sequence %d", seq);
  for (int32_t b : s->blocks) bm->release(b);
  bm->seqs.erase(seq);
  return PA_OK;
}

pa_status pa_bm_append(pa_block_manager* bm, const int32_t* seqs, int32_t n,
                       int64_t* slot_mapping, int32_t* copy_src, int32_t* copy_dst,
                       int32_t* n_copies) {
  pa_set_last_error_internal("");
  if (!bm || !n_copies || (n > 0 && (!seqs || !slot_mapping || !copy_src || !copy_dst)))
    return fail(PA_ERR_INVALID_ARG, "NULL argument");
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "n %d < 0", n);
  *n_copies = 0;
  // check everything first: ids exist and are distinct; count the blocks needed
  int64_t need = 0;
  try {
    std::vector<int32_t> sorted(seqs, seqs + n);
    std::sort(sorted.begin(), sorted.end());
    for (int32_t i = 1; i < n; ++i)
      if (sorted[(size_t)i] == sorted[(size_t)i - 1])
        return fail(PA_ERR_INVALID_ARG, "sequence %d listed twice", sorted[(size_t)i]);
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "out of host memory");
  }
  // A shared, partly filled last block X listed by k of its holders takes min(k,
  // refs(X) - 1) copies: holders are served in the order given, each copy drops X's
  // count by one, and the last holder left alone on X writes into it in place.
  std::unordered_map<int32_t, int32_t> holders;
  try {
    for (int32_t i = 0; i < n; ++i) {
      const Sequence* s = bm->find(seqs[i]);
      if (!s) return fail(PA_ERR_INVALID_ARG, "no sequence %d", seqs[i]);
      const int32_t off = s->len % bm->block_size;
      if (off == 0) {  // the last block is full (or there is none): take a new one
        if ((int64_t)s->blocks.size() + 1 > bm->max_blocks)
          return fail(PA_ERR_CAPACITY, "sequence %d would need more than %d blocks", seqs[i], bm->max_blocks);
        ++need;
      } else if (bm->refs[(size_t)s->blocks.back()] > 1) {  // shared, partly filled: copy first
        ++holders[s->blocks.back()];
      }
    }
  } catch (...) {
    return fail(PA_ERR_INVALID_ARG, "out of host memory");
  }
  for (const auto& h : holders) need += std::min<int64_t>(h.second, bm->refs[(size_t)h.first] - 1);
  if (need > (int64_t)bm->free_list.size())
    return fail(PA_ERR_CAPACITY, "%lld free blocks needed, %zu free", (long long)need,
                bm->free_list.size());
  // commit
  int32_t nc = 0;
  for (int32_t i = 0; i < n; ++i) {
    Sequence& s = *bm->find(seqs[i]);
    const int32_t off = s.len % bm->block_size;
    if (off == 0) {
      const int32_t b = bm->free_list.front();
      bm->free_list.pop_front();
      bm->refs[(size_t)b] = 1;
      s.blocks.push_back(b);
    } else if (bm->refs[(size_t)s.blocks.back()] > 1) {
      const int32_t src = s.blocks.back();
      const int32_t b = bm->free_list.front();
      bm->free_list.pop_front();
      bm->refs[(size_t)b] = 1;
      --bm->refs[(size_t)src];  // still referenced by the others: never reaches 0 here
      s.blocks.back() = b;
      copy_src[nc] = src;
      copy_dst[nc] = b;
      ++nc;
    }
    slot_mapping[i] = (int64_t)s.blocks.back() * bm->block_size + off;
    ++s.len;
  }
  *n_copies = nc;
  return PA_OK;
}

pa_status pa_bm_length(const pa_block_manager* bm, int32_t seq, int32_t* len) {
  pa_set_last_error_internal("");
  if (!bm || !len) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  const Sequence* s = bm->find(seq);
  if (!s) return fail(PA_ERR_INVALID_ARG, "no sequence %d", seq);
  *len = s->len;
  return PA_OK;
}

pa_status pa_bm_export(const pa_block_manager* bm, const int32_t* seqs, int32_t n,
                       int32_t* block_tables, int32_t* seq_lens) {
  pa_set_last_error_internal("");
  if (!bm || (n > 0 && (!seqs || !block_tables || !seq_lens)))
    return fail(PA_ERR_INVALID_ARG, "NULL argument");
  if (n < 0) return fail(PA_ERR_INVALID_ARG, "n %d < 0", n);
  for (int32_t i = 0; i < n; ++i)
    if (!bm->find(seqs[i])) return fail(PA_ERR_INVALID_ARG, "no sequence %d", seqs[i]);
  for (int32_t i = 0; i < n; ++i) {
    const Sequence& s = *bm->find(seqs[i]);
    int32_t* row = block_tables + (int64_t)i * bm->max_blocks;
    // the used entries, then -1 to the end of the row (a copy and a fill, not a
    // per-entry branch: the table is rewritten for every step)
    const size_t used = s.blocks.size();
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + used, row + bm->max_blocks, -1);
    seq_lens[i] = s.len;
  }
  return PA_OK;
}

int64_t pa_bm_free_blocks(const pa_block_manager* bm) {
  return bm ? (int64_t)bm->free_list.size() : -1;
}

pa_status pa_bm_ref_count(const pa_block_manager* bm, int32_t block, int32_t* count) {
  pa_set_last_error_internal("");
  if (!bm || !count) return fail(PA_ERR_INVALID_ARG, "NULL argument");
  if (block < 0 || block >= bm->num_blocks) return fail(PA_ERR_INVALID_ARG, "block %d outside the pool", block);
  *count = bm->refs[(size_t)block];
  return PA_OK;
}

}  // extern "C"
