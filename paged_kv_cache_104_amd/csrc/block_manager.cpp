// Host block manager: free list, block tables, reference counts, fork and
// copy-on-write.  Rules (ithome article 10417389 sections 3-4; ultralytics
// glossary "How paging works" with its code example; optiverse blog "Block
// table and non-contiguous allocation"):
//   - blocks come from the head of the free list, and a sequence takes a new
//     block only when its last block is full;
//   - token pos of a sequence sits at slot table[pos / B] * B + pos % B;
//   - fork makes the child point at the parent's blocks (count + 1 each);
//   - a write into a shared, partly filled last block takes a new block, emits
//     (old, new) for the device copy and drops the old block's count by one;
//     full shared blocks stay shared;
//   - freeing a sequence drops one count per block; blocks at zero go to the
//     tail of the free list, in the sequence's logical order.
// Every operation checks first and then mutates, so failures change nothing.
#include <algorithm>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv_internal.h"

namespace {

struct Seq {
  std::vector<int32_t> blocks;
  int64_t len = 0;
};

}  // namespace

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;

  int32_t pop_free() {
    int32_t b = free_list.front();
    free_list.pop_front();
    ref[b] = 1;
    return b;
  }

  int64_t slot_of(const Seq& s, int64_t pos) const {
    return int64_t(s.blocks[pos / block_size]) * block_size + pos % block_size;
  }

  // Reserve the next token of s (the caller has checked a free block exists if needed).
  int64_t append_one(Seq& s, int64_t* cow_src, int64_t* cow_dst) {
    const int64_t pos = s.len;
    *cow_src = *cow_dst = -1;
    if (pos % block_size == 0) {
      s.blocks.push_back(pop_free());
    } else {
      const int32_t last = s.blocks.back();
      if (ref[last] > 1) {
        const int32_t fresh = pop_free();
        ref[last] -= 1;
        s.blocks.back() = fresh;
        *cow_src = last;
        *cow_dst = fresh;
      }
    }
    s.len = pos + 1;
    return slot_of(s, pos);
  }

  bool needs_block(const Seq& s) const {
    if (s.len % block_size == 0) return true;
    return ref[s.blocks.back()] > 1;
  }
};

using pkv::fail;

extern "C" {

pkv_bm* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                      int32_t free_count) {
  pkv::clear_error();
  if (num_blocks <= 0 || block_size <= 0) {
    fail(PKV_E_INVAL, "num_blocks and block_size must be positive");
    return nullptr;
  }
  pkv_bm* bm = new (std::nothrow) pkv_bm();
  if (!bm) {
    fail(PKV_E_NOMEM, "out of host memory");
    return nullptr;
  }
  bm->num_blocks = num_blocks;
  bm->block_size = block_size;
  bm->ref.assign(num_blocks, 0);
  if (!free_order) {
    for (int32_t b = 0; b < num_blocks; ++b) bm->free_list.push_back(b);
  } else {
    if (free_count < 0 || free_count > num_blocks) {
      delete bm;
      fail(PKV_E_INVAL, "free_count %d out of [0, %d]", free_count, num_blocks);
      return nullptr;
    }
    std::vector<char> seen(num_blocks, 0);
    for (int32_t i = 0; i < free_count; ++i) {
      const int32_t b = free_order[i];
      if (b < 0 || b >= num_blocks || seen[b]) {
        delete bm;
        fail(PKV_E_INVAL, "free_order[%d] = %d is out of range or repeated", i, b);
        return nullptr;
      }
      seen[b] = 1;
      bm->free_list.push_back(b);
    }
    // blocks not on the free list are held by someone else
    for (int32_t b = 0; b < num_blocks; ++b)
      if (!seen[b]) bm->ref[b] = 0;
  }
  return bm;
}

void pkv_bm_destroy(pkv_bm* bm) { delete bm; }

int pkv_bm_add_seq(pkv_bm* bm, int64_t seq, int64_t num_tokens) {
  if (!bm) return fail(PKV_E_INVAL, "NULL manager");
  if (num_tokens < 0) return fail(PKV_E_INVAL, "negative num_tokens");
  if (bm->seqs.count(seq)) return fail(PKV_E_INVAL, "sequence %lld exists", (long long)seq);
  const int64_t need = (num_tokens + bm->block_size - 1) / bm->block_size;
  if (need > int64_t(bm->free_list.size()))
    return fail(PKV_E_NOMEM, "add_seq needs %lld blocks, %zu free", (long long)need,
                bm->free_list.size());
  Seq s;
  s.blocks.reserve(need);
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->pop_free());
  s.len = num_tokens;
  bm->seqs.emplace(seq, std::move(s));
  return PKV_OK;
}

int pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return fail(PKV_E_INVAL, "NULL manager");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end()) return fail(PKV_E_INVAL, "unknown parent %lld", (long long)parent);
  if (bm->seqs.count(child)) return fail(PKV_E_INVAL, "child %lld exists", (long long)child);
  Seq s = it->second;
  for (int32_t b : s.blocks) bm->ref[b] += 1;
  bm->seqs.emplace(child, std::move(s));
  return PKV_OK;
}

int pkv_bm_append(pkv_bm* bm, int64_t seq, int64_t* slot, int64_t* cow_src, int64_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return fail(PKV_E_INVAL, "NULL argument");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence %lld", (long long)seq);
  if (bm->needs_block(it->second) && bm->free_list.empty())
    return fail(PKV_E_NOMEM, "append needs a block, none free");
  *slot = bm->append_one(it->second, cow_src, cow_dst);
  return PKV_OK;
}

int pkv_bm_append_batch(pkv_bm* bm, const int64_t* seqs, int32_t n, int64_t* slots,
                        int64_t* pairs, int32_t* num_pairs) {
  if (!bm || (n > 0 && (!seqs || !slots || !pairs)) || !num_pairs || n < 0)
    return fail(PKV_E_INVAL, "bad append_batch arguments");
  std::vector<Seq*> ptr(n);
  std::unordered_set<int64_t> uniq;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence %lld", (long long)seqs[i]);
    if (!uniq.insert(seqs[i]).second)
      return fail(PKV_E_INVAL, "sequence %lld repeated in a batch", (long long)seqs[i]);
    ptr[i] = &it->second;
  }
  // dry run: count blocks, following the counts that earlier copies in this batch drop
  std::unordered_map<int32_t, int32_t> dropped;
  int64_t need = 0;
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = *ptr[i];
    if (s.len % bm->block_size == 0) {
      ++need;
      continue;
    }
    const int32_t last = s.blocks.back();
    auto d = dropped.find(last);
    const int32_t drop = d == dropped.end() ? 0 : d->second;
    if (bm->ref[last] - drop > 1) {
      ++need;
      dropped[last] = drop + 1;
    }
  }
  if (need > int64_t(bm->free_list.size()))
    return fail(PKV_E_NOMEM, "append_batch needs %lld blocks, %zu free", (long long)need,
                bm->free_list.size());
  int32_t np = 0;
  for (int32_t i = 0; i < n; ++i) {
    int64_t src, dst;
    slots[i] = bm->append_one(*ptr[i], &src, &dst);
    if (src >= 0) {
      pairs[2 * np] = src;
      pairs[2 * np + 1] = dst;
      ++np;
    }
  }
  *num_pairs = np;
  return PKV_OK;
}

int pkv_bm_extend(pkv_bm* bm, int64_t seq, int64_t n, int64_t* slots, int64_t* cow_src,
                  int64_t* cow_dst) {
  if (!bm || n < 0 || (n > 0 && !slots) || !cow_src || !cow_dst)
    return fail(PKV_E_INVAL, "bad extend arguments");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence %lld", (long long)seq);
  Seq& s = it->second;
  const int64_t have = int64_t(s.blocks.size()) * bm->block_size - s.len;
  const int64_t rest = n > have ? n - have : 0;
  int64_t need = (rest + bm->block_size - 1) / bm->block_size;
  if (n > 0 && have > 0 && bm->ref[s.blocks.back()] > 1) ++need;
  if (need > int64_t(bm->free_list.size()))
    return fail(PKV_E_NOMEM, "extend needs %lld blocks, %zu free", (long long)need,
                bm->free_list.size());
  *cow_src = *cow_dst = -1;
  for (int64_t i = 0; i < n; ++i) {
    int64_t src, dst;
    slots[i] = bm->append_one(s, &src, &dst);
    if (src >= 0) {
      *cow_src = src;
      *cow_dst = dst;
    }
  }
  return PKV_OK;
}

int pkv_bm_free_seq(pkv_bm* bm, int64_t seq) {
  if (!bm) return fail(PKV_E_INVAL, "NULL manager");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence %lld", (long long)seq);
  for (int32_t b : it->second.blocks) {
    bm->ref[b] -= 1;
    if (bm->ref[b] == 0) bm->free_list.push_back(b);
  }
  bm->seqs.erase(it);
  return PKV_OK;
}

int pkv_bm_slots(pkv_bm* bm, int64_t seq, int64_t start_pos, int64_t n, int64_t* out) {
  if (!bm || n < 0 || (n > 0 && !out)) return fail(PKV_E_INVAL, "bad slots arguments");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence %lld", (long long)seq);
  const Seq& s = it->second;
  if (start_pos < 0 || start_pos + n > s.len)
    return fail(PKV_E_INVAL, "positions [%lld, %lld) outside the %lld tokens of the sequence",
                (long long)start_pos, (long long)(start_pos + n), (long long)s.len);
  for (int64_t i = 0; i < n; ++i) out[i] = bm->slot_of(s, start_pos + i);
  return PKV_OK;
}

int pkv_bm_block_tables(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* tables,
                        int32_t max_blocks, int32_t* context_lens) {
  if (!bm || n < 0 || max_blocks < 0 || (n > 0 && (!seqs || !tables || !context_lens)))
    return fail(PKV_E_INVAL, "bad block_tables arguments");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end()) return fail(PKV_E_INVAL, "unknown sequence %lld", (long long)seqs[i]);
    if (int64_t(it->second.blocks.size()) > max_blocks)
      return fail(PKV_E_INVAL, "sequence %lld holds %zu blocks > max_blocks %d",
                  (long long)seqs[i], it->second.blocks.size(), max_blocks);
    if (it->second.len > INT32_MAX) return fail(PKV_E_INVAL, "context too long for int32");
  }
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.find(seqs[i])->second;
    int32_t* row = tables + int64_t(i) * max_blocks;
    const int32_t nb = int32_t(s.blocks.size());
    std::copy(s.blocks.begin(), s.blocks.end(), row);
    std::fill(row + nb, row + max_blocks, -1);
    context_lens[i] = int32_t(s.len);
  }
  return PKV_OK;
}

int pkv_bm_stats(pkv_bm* bm, pkv_bm_stats_t* out) {
  if (!bm || !out) return fail(PKV_E_INVAL, "NULL argument");
  out->free_blocks = int32_t(bm->free_list.size());
  out->used_blocks = bm->num_blocks - out->free_blocks;
  out->tokens = out->slots_allocated = out->logical_blocks = out->physical_blocks = 0;
  for (const auto& kv : bm->seqs) {
    out->tokens += kv.second.len;
    out->logical_blocks += int64_t(kv.second.blocks.size());
  }
  out->slots_allocated = out->logical_blocks * bm->block_size;
  for (int32_t r : bm->ref) out->physical_blocks += r > 0;
  return PKV_OK;
}

int32_t pkv_bm_refcount(pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= bm->num_blocks) return -1;
  return bm->ref[block];
}

int64_t pkv_bm_seq_len(pkv_bm* bm, int64_t seq) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  return it == bm->seqs.end() ? -1 : it->second.len;
}

int32_t pkv_bm_free_list(pkv_bm* bm, int32_t* out, int32_t cap) {
  if (!bm) return -1;
  const int32_t n = int32_t(bm->free_list.size());
  for (int32_t i = 0; i < n && i < cap; ++i) out[i] = bm->free_list[i];
  return n;
}

}  // extern "C"
