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
//
// Prefix caching (optional; review of the vLLM paper, the paragraphs on prefix
// caching; glossary "Sharing blocks between sequences"): a full block is known
// by its own tokens and every token before it, and a request whose prompt
// starts with cached full blocks reuses them.  The keys live in a trie with
// one node per full block's token prefix (a node's identity is exactly that
// prefix, so no two prefixes collide); a node names the block that caches it,
// if any.  Lookups take the longest cached run of full blocks from the start.
// A cached block whose count falls to zero stays findable and becomes
// evictable; blocks come from the free list first, then from the evictable
// block released longest ago, which loses its key.  A released sequence's
// cached blocks join the evictable queue last block first; its uncached blocks
// return to the free list as above.  A block that fills takes its key unless
// another block already holds it.
//
// Swapping (review of the vLLM paper, the preemption paragraphs): a set of
// sequences moves its KV to a host pool with the device pool's block shape and
// back.  A shared block moves once and keeps its count; a set sharing a block
// with a sequence outside it is refused.  Distinct blocks are taken in order
// of first appearance (sequences as given, blocks in logical order), the
// receiving side's free list supplies the new blocks, and the giving side's
// blocks return to its free list in that order (device blocks without their
// prefix-cache keys).  The caller copies the returned pairs before any later
// write.  A swapped-out sequence can only be swapped in or released.
#include <algorithm>
#include <cstring>
#include <deque>
#include <list>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

#include "pkv_internal.h"

namespace {

// One full block's token prefix: its tokens (the key in the parent's map) under
// the node of the prefix before it.
struct Node {
  Node* parent = nullptr;
  std::string key;
  std::unordered_map<std::string, Node*> children;
  int32_t block = -1;   // the block caching this prefix, or -1
  int64_t users = 0;    // sequence paths through it, children, and its block
};

struct Seq {
  std::vector<int32_t> blocks;   // host blocks while swapped out
  int64_t len = 0;
  bool swapped = false;
  bool tracked = false;          // admitted with its tokens (prefix caching)
  std::vector<int32_t> tokens;   // tracked sequences only
  std::vector<Node*> path;       // trie node of each full block (tracked only)
};

}  // namespace

struct pkv_bm {
  int32_t num_blocks = 0;
  int32_t block_size = 0;
  std::deque<int32_t> free_list;
  std::vector<int32_t> ref;
  std::unordered_map<int64_t, Seq> seqs;

  // prefix caching
  bool caching = false;
  Node root;
  std::vector<Node*> node_of;                         // block -> node it caches
  std::list<int32_t> evictable;                       // released longest ago first
  std::vector<std::list<int32_t>::iterator> ev_pos;   // valid while ev_in[b]
  std::vector<char> ev_in;
  int64_t hit_tokens = 0, query_tokens = 0, cached_blocks = 0;

  // swapping
  std::deque<int32_t> host_free;
  std::vector<int32_t> host_ref;
  int64_t swapped_seqs = 0;

  ~pkv_bm() { drop_children(&root); }

  static void drop_children(Node* n) {
    for (auto& kv : n->children) {
      drop_children(kv.second);
      delete kv.second;
    }
    n->children.clear();
  }

  int64_t available() const { return int64_t(free_list.size()) + int64_t(evictable.size()); }

  void release(Node* n) {
    while (n != &root && --n->users == 0) {
      Node* p = n->parent;
      p->children.erase(n->key);
      delete n;
      n = p;
    }
  }

  Node* child_of(Node* p, const int32_t* toks) {
    std::string k(reinterpret_cast<const char*>(toks), sizeof(int32_t) * size_t(block_size));
    auto it = p->children.find(k);
    if (it != p->children.end()) return it->second;
    Node* c = new Node();
    c->parent = p;
    c->key = std::move(k);
    p->children.emplace(c->key, c);
    p->users += 1;
    return c;
  }

  Node* find_child(Node* p, const int32_t* toks) const {
    std::string k(reinterpret_cast<const char*>(toks), sizeof(int32_t) * size_t(block_size));
    auto it = p->children.find(k);
    return it == p->children.end() ? nullptr : it->second;
  }

  void uncache(int32_t b) {
    Node* n = node_of[b];
    n->block = -1;
    node_of[b] = nullptr;
    cached_blocks -= 1;
    release(n);
  }

  // A block for a new use: the free list's head, else the evictable block
  // released longest ago (which loses its key).  The caller has checked that
  // one is available.
  int32_t pop_free() {
    int32_t b;
    if (!free_list.empty()) {
      b = free_list.front();
      free_list.pop_front();
    } else {
      b = evictable.front();
      evictable.pop_front();
      ev_in[b] = 0;
      uncache(b);
    }
    ref[b] = 1;
    return b;
  }

  // Full block i of a tracked sequence: extend its trie path, and let the block
  // take the key if neither the key nor the block is taken.
  void register_block(Seq& s, int64_t i) {
    Node* p = i == 0 ? &root : s.path[i - 1];
    Node* n = child_of(p, s.tokens.data() + i * block_size);
    n->users += 1;
    s.path.push_back(n);
    const int32_t b = s.blocks[i];
    if (n->block < 0 && !node_of[b]) {
      n->block = b;
      node_of[b] = n;
      n->users += 1;
      cached_blocks += 1;
    }
  }

  void note_tokens(Seq& s, const int32_t* toks, int64_t n) {
    if (!s.tracked) return;
    s.tokens.insert(s.tokens.end(), toks, toks + n);
    const int64_t full = int64_t(s.tokens.size()) / block_size;
    for (int64_t i = int64_t(s.path.size()); i < full; ++i) register_block(s, i);
  }

  // cached blocks of the longest run of full blocks from the start of toks
  void lookup(const int32_t* toks, int64_t n, std::vector<int32_t>* hits) const {
    const Node* p = &root;
    for (int64_t i = 0; i < n / block_size; ++i) {
      const Node* c = find_child(const_cast<Node*>(p), toks + i * block_size);
      if (!c || c->block < 0) break;
      hits->push_back(c->block);
      p = c;
    }
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
  if (need > bm->available())
    return fail(PKV_E_NOMEM, "add_seq needs %lld blocks, %lld available", (long long)need,
                (long long)bm->available());
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
  if (it == bm->seqs.end() || it->second.swapped)
    return fail(PKV_E_INVAL, "unknown or swapped-out parent %lld", (long long)parent);
  if (bm->seqs.count(child)) return fail(PKV_E_INVAL, "child %lld exists", (long long)child);
  Seq s = it->second;
  for (int32_t b : s.blocks) bm->ref[b] += 1;
  for (Node* n : s.path) n->users += 1;
  bm->seqs.emplace(child, std::move(s));
  return PKV_OK;
}

int pkv_bm_append(pkv_bm* bm, int64_t seq, int64_t* slot, int64_t* cow_src, int64_t* cow_dst) {
  if (!bm || !slot || !cow_src || !cow_dst) return fail(PKV_E_INVAL, "NULL argument");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end() || it->second.swapped)
    return fail(PKV_E_INVAL, "unknown or swapped-out sequence %lld", (long long)seq);
  if (bm->needs_block(it->second) && bm->available() == 0)
    return fail(PKV_E_NOMEM, "append needs a block, none available");
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
    if (it == bm->seqs.end() || it->second.swapped)
      return fail(PKV_E_INVAL, "unknown or swapped-out sequence %lld", (long long)seqs[i]);
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
  if (need > bm->available())
    return fail(PKV_E_NOMEM, "append_batch needs %lld blocks, %lld available", (long long)need,
                (long long)bm->available());
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
  if (it == bm->seqs.end() || it->second.swapped)
    return fail(PKV_E_INVAL, "unknown or swapped-out sequence %lld", (long long)seq);
  Seq& s = it->second;
  const int64_t have = int64_t(s.blocks.size()) * bm->block_size - s.len;
  const int64_t rest = n > have ? n - have : 0;
  int64_t need = (rest + bm->block_size - 1) / bm->block_size;
  if (n > 0 && have > 0 && bm->ref[s.blocks.back()] > 1) ++need;
  if (need > bm->available())
    return fail(PKV_E_NOMEM, "extend needs %lld blocks, %lld available", (long long)need,
                (long long)bm->available());
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
  if (it->second.swapped) {                       // its blocks are host blocks
    for (int32_t h : it->second.blocks)
      if (--bm->host_ref[h] == 0) bm->host_free.push_back(h);
    for (Node* n : it->second.path) bm->release(n);
    bm->seqs.erase(it);
    bm->swapped_seqs -= 1;
    return PKV_OK;
  }
  std::vector<int32_t> zero;
  for (int32_t b : it->second.blocks) {
    bm->ref[b] -= 1;
    if (bm->ref[b] == 0) zero.push_back(b);
  }
  for (int32_t b : zero)
    if (!bm->caching || !bm->node_of[b]) bm->free_list.push_back(b);
  if (bm->caching) {
    for (auto r = zero.rbegin(); r != zero.rend(); ++r) {
      if (!bm->node_of[*r]) continue;
      bm->ev_pos[*r] = bm->evictable.insert(bm->evictable.end(), *r);
      bm->ev_in[*r] = 1;
    }
  }
  for (Node* n : it->second.path) bm->release(n);
  bm->seqs.erase(it);
  return PKV_OK;
}

int pkv_bm_slots(pkv_bm* bm, int64_t seq, int64_t start_pos, int64_t n, int64_t* out) {
  if (!bm || n < 0 || (n > 0 && !out)) return fail(PKV_E_INVAL, "bad slots arguments");
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end() || it->second.swapped)
    return fail(PKV_E_INVAL, "unknown or swapped-out sequence %lld", (long long)seq);
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
    if (it == bm->seqs.end() || it->second.swapped)
      return fail(PKV_E_INVAL, "unknown or swapped-out sequence %lld", (long long)seqs[i]);
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
    if (kv.second.swapped) continue;             // their tables hold host blocks
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

// ------------------------------------------------------------------ prefix caching

int pkv_bm_set_prefix_caching(pkv_bm* bm, int32_t enable) {
  if (!bm) return fail(PKV_E_INVAL, "NULL manager");
  if (!bm->seqs.empty()) return fail(PKV_E_INVAL, "prefix caching changes only with no sequences");
  if (enable && !bm->caching) {
    bm->node_of.assign(bm->num_blocks, nullptr);
    bm->ev_pos.assign(bm->num_blocks, bm->evictable.end());
    bm->ev_in.assign(bm->num_blocks, 0);
  } else if (!enable && bm->caching) {
    // evictable blocks go back to the free list in queue order, without keys
    for (int32_t b : bm->evictable) {
      bm->ev_in[b] = 0;
      bm->uncache(b);
      bm->free_list.push_back(b);
    }
    bm->evictable.clear();
  }
  bm->caching = enable != 0;
  return PKV_OK;
}

int pkv_bm_lookup(pkv_bm* bm, const int32_t* tokens, int64_t n, int64_t* cached_tokens) {
  if (!bm || n < 0 || (n > 0 && !tokens) || !cached_tokens)
    return fail(PKV_E_INVAL, "bad lookup arguments");
  std::vector<int32_t> hits;
  if (bm->caching) bm->lookup(tokens, n, &hits);
  *cached_tokens = int64_t(hits.size()) * bm->block_size;
  return PKV_OK;
}

int pkv_bm_add_seq_tokens(pkv_bm* bm, int64_t seq, const int32_t* tokens, int64_t n,
                          int64_t* cached_tokens) {
  if (!bm || n < 0 || (n > 0 && !tokens) || !cached_tokens)
    return fail(PKV_E_INVAL, "bad add_seq_tokens arguments");
  if (!bm->caching) return fail(PKV_E_INVAL, "prefix caching is off");
  if (bm->seqs.count(seq)) return fail(PKV_E_INVAL, "sequence %lld exists", (long long)seq);
  std::vector<int32_t> hits;
  bm->lookup(tokens, n, &hits);
  const int64_t need = (n + bm->block_size - 1) / bm->block_size - int64_t(hits.size());
  int64_t revived = 0;
  for (int32_t b : hits) revived += bm->ref[b] == 0;
  if (need > bm->available() - revived)
    return fail(PKV_E_NOMEM, "add_seq_tokens needs %lld blocks, %lld available", (long long)need,
                (long long)(bm->available() - revived));
  for (int32_t b : hits) {
    if (bm->ref[b] == 0) {
      bm->evictable.erase(bm->ev_pos[b]);
      bm->ev_in[b] = 0;
    }
    bm->ref[b] += 1;
  }
  Seq s;
  s.tracked = true;
  s.blocks = hits;
  s.blocks.reserve(hits.size() + need);
  for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->pop_free());
  s.len = n;
  Seq& live = bm->seqs.emplace(seq, std::move(s)).first->second;
  bm->note_tokens(live, tokens, n);
  bm->query_tokens += n;
  bm->hit_tokens += int64_t(hits.size()) * bm->block_size;
  *cached_tokens = int64_t(hits.size()) * bm->block_size;
  return PKV_OK;
}

int pkv_bm_append_batch_tokens(pkv_bm* bm, const int64_t* seqs, const int32_t* tokens, int32_t n,
                               int64_t* slots, int64_t* pairs, int32_t* num_pairs) {
  if (!bm || (n > 0 && !tokens)) return fail(PKV_E_INVAL, "bad append_batch_tokens arguments");
  if (!bm->caching) return fail(PKV_E_INVAL, "prefix caching is off");
  const int rc = pkv_bm_append_batch(bm, seqs, n, slots, pairs, num_pairs);
  if (rc) return rc;
  for (int32_t i = 0; i < n; ++i) bm->note_tokens(bm->seqs.find(seqs[i])->second, tokens + i, 1);
  return PKV_OK;
}

int pkv_bm_extend_tokens(pkv_bm* bm, int64_t seq, const int32_t* tokens, int64_t n,
                         int64_t* slots, int64_t* cow_src, int64_t* cow_dst) {
  if (!bm || n < 0 || (n > 0 && !tokens)) return fail(PKV_E_INVAL, "bad extend_tokens arguments");
  if (!bm->caching) return fail(PKV_E_INVAL, "prefix caching is off");
  const int rc = pkv_bm_extend(bm, seq, n, slots, cow_src, cow_dst);
  if (rc) return rc;
  bm->note_tokens(bm->seqs.find(seq)->second, tokens, n);
  return PKV_OK;
}

int pkv_bm_cache_stats(pkv_bm* bm, int64_t* out) {
  if (!bm || !out) return fail(PKV_E_INVAL, "NULL argument");
  out[0] = bm->cached_blocks;
  out[1] = int64_t(bm->evictable.size());
  out[2] = bm->hit_tokens;
  out[3] = bm->query_tokens;
  return PKV_OK;
}

// ------------------------------------------------------------------ swapping

int pkv_bm_set_host_pool(pkv_bm* bm, int32_t num_host_blocks) {
  if (!bm) return fail(PKV_E_INVAL, "NULL manager");
  if (num_host_blocks < 0) return fail(PKV_E_INVAL, "negative host pool");
  if (bm->swapped_seqs) return fail(PKV_E_INVAL, "sequences are swapped out");
  bm->host_free.clear();
  for (int32_t h = 0; h < num_host_blocks; ++h) bm->host_free.push_back(h);
  bm->host_ref.assign(num_host_blocks, 0);
  return PKV_OK;
}

namespace {

// Distinct blocks of a set of sequences in order of first appearance, provided
// every holder of each is in the set (counts[] = holders over all sequences).
int distinct_blocks(pkv_bm* bm, const int64_t* seqs, int32_t n, bool swapped,
                    const std::vector<int32_t>& counts, std::vector<Seq*>* ptr,
                    std::vector<int32_t>* order) {
  std::unordered_set<int64_t> uniq;
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (!uniq.insert(seqs[i]).second)
      return fail(PKV_E_INVAL, "sequence %lld repeated", (long long)seqs[i]);
    if (it == bm->seqs.end() || it->second.swapped != swapped)
      return fail(PKV_E_INVAL, "sequence %lld is unknown or %s", (long long)seqs[i],
                  swapped ? "resident" : "swapped out");
    ptr->push_back(&it->second);
  }
  std::unordered_map<int32_t, int32_t> seen;
  for (Seq* s : *ptr)
    for (int32_t b : s->blocks)
      if (seen[b]++ == 0) order->push_back(b);
  for (int32_t b : *order)
    if (seen[b] != counts[b])
      return fail(PKV_E_INVAL, "block %d is shared with a sequence outside the set", b);
  return PKV_OK;
}

}  // namespace

int pkv_bm_swap_out(pkv_bm* bm, const int64_t* seqs, int32_t n, int64_t* pairs, int32_t cap,
                    int32_t* num_pairs) {
  if (!bm || n < 0 || (n > 0 && !seqs) || !num_pairs || cap < 0 || (cap > 0 && !pairs))
    return fail(PKV_E_INVAL, "bad swap_out arguments");
  std::vector<Seq*> ptr;
  std::vector<int32_t> blocks;
  int rc = distinct_blocks(bm, seqs, n, false, bm->ref, &ptr, &blocks);
  if (rc) return rc;
  *num_pairs = int32_t(blocks.size());
  if (int64_t(blocks.size()) > cap) return fail(PKV_E_INVAL, "pairs buffer holds %d < %zu", cap, blocks.size());
  if (blocks.size() > bm->host_free.size())
    return fail(PKV_E_NOMEM, "swap_out needs %zu host blocks, %zu free", blocks.size(),
                bm->host_free.size());
  std::unordered_map<int32_t, int32_t> to;
  for (size_t i = 0; i < blocks.size(); ++i) {
    const int32_t b = blocks[i], h = bm->host_free.front();
    bm->host_free.pop_front();
    bm->host_ref[h] = bm->ref[b];
    to[b] = h;
    pairs[2 * i] = b;
    pairs[2 * i + 1] = h;
  }
  for (Seq* s : ptr) {
    for (int32_t& b : s->blocks) b = to[b];
    s->swapped = true;
  }
  bm->swapped_seqs += n;
  for (int32_t b : blocks) {
    bm->ref[b] = 0;
    if (bm->caching && bm->node_of[b]) bm->uncache(b);
    bm->free_list.push_back(b);
  }
  return PKV_OK;
}

int pkv_bm_swap_in(pkv_bm* bm, const int64_t* seqs, int32_t n, int64_t* pairs, int32_t cap,
                   int32_t* num_pairs) {
  if (!bm || n < 0 || (n > 0 && !seqs) || !num_pairs || cap < 0 || (cap > 0 && !pairs))
    return fail(PKV_E_INVAL, "bad swap_in arguments");
  std::vector<Seq*> ptr;
  std::vector<int32_t> hosts;
  int rc = distinct_blocks(bm, seqs, n, true, bm->host_ref, &ptr, &hosts);
  if (rc) return rc;
  *num_pairs = int32_t(hosts.size());
  if (int64_t(hosts.size()) > cap) return fail(PKV_E_INVAL, "pairs buffer holds %d < %zu", cap, hosts.size());
  if (int64_t(hosts.size()) > bm->available())
    return fail(PKV_E_NOMEM, "swap_in needs %zu blocks, %lld available", hosts.size(),
                (long long)bm->available());
  std::unordered_map<int32_t, int32_t> to;
  for (size_t i = 0; i < hosts.size(); ++i) {
    const int32_t h = hosts[i], d = bm->pop_free();
    bm->ref[d] = bm->host_ref[h];
    to[h] = d;
    pairs[2 * i] = h;
    pairs[2 * i + 1] = d;
  }
  for (Seq* s : ptr) {
    for (int32_t& b : s->blocks) b = to[b];
    s->swapped = false;
  }
  bm->swapped_seqs -= n;
  for (int32_t h : hosts) {
    bm->host_ref[h] = 0;
    bm->host_free.push_back(h);
  }
  return PKV_OK;
}

int pkv_bm_swap_stats(pkv_bm* bm, int64_t* out) {
  if (!bm || !out) return fail(PKV_E_INVAL, "NULL argument");
  out[0] = int64_t(bm->host_free.size());
  out[1] = int64_t(bm->host_ref.size());
  out[2] = bm->swapped_seqs;
  return PKV_OK;
}

int32_t pkv_bm_host_refcount(pkv_bm* bm, int32_t block) {
  if (!bm || block < 0 || block >= int32_t(bm->host_ref.size())) return -1;
  return bm->host_ref[block];
}

int32_t pkv_bm_host_free_list(pkv_bm* bm, int32_t* out, int32_t cap) {
  if (!bm) return -1;
  const int32_t n = int32_t(bm->host_free.size());
  for (int32_t i = 0; i < n && i < cap; ++i) out[i] = bm->host_free[i];
  return n;
}

int pkv_bm_seq_blocks(pkv_bm* bm, int64_t seq, int32_t* out, int32_t cap) {
  if (!bm) return -1;
  auto it = bm->seqs.find(seq);
  if (it == bm->seqs.end()) return -1;
  const int32_t n = int32_t(it->second.blocks.size());
  for (int32_t i = 0; i < n && i < cap; ++i) out[i] = it->second.blocks[i];
  return n;
}

int32_t pkv_bm_block_fills(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* blocks,
                           int32_t* fills, int32_t cap) {
  if (!bm || n < 0 || cap < 0 || (n > 0 && !seqs) || (cap > 0 && (!blocks || !fills)))
    return fail(PKV_E_INVAL, "bad block_fills arguments");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seqs[i]);
    if (it == bm->seqs.end() || it->second.swapped)
      return fail(PKV_E_INVAL, "unknown or swapped-out sequence %lld", (long long)seqs[i]);
  }
  // position of each block in the output, in order of first appearance
  std::unordered_map<int32_t, int32_t> at;
  std::vector<int32_t> order, fill;
  const int64_t B = bm->block_size;
  for (int32_t i = 0; i < n; ++i) {
    const Seq& s = bm->seqs.find(seqs[i])->second;
    for (size_t j = 0; j < s.blocks.size(); ++j) {
      // logical block j holds tokens [j * B, min(len, (j + 1) * B))
      const int32_t f = int32_t(std::max<int64_t>(0, std::min<int64_t>(B, s.len - int64_t(j) * B)));
      auto ins = at.emplace(s.blocks[j], int32_t(order.size()));
      if (ins.second) {
        order.push_back(s.blocks[j]);
        fill.push_back(f);
      } else {
        fill[ins.first->second] = std::max(fill[ins.first->second], f);
      }
    }
  }
  const int32_t m = int32_t(order.size());
  for (int32_t k = 0; k < m && k < cap; ++k) {
    blocks[k] = order[k];
    fills[k] = fill[k];
  }
  return m;
}

int32_t pkv_quest_blocks_of_slots(const int64_t* slots, int64_t n, int32_t block_size,
                                  int32_t* blocks, int32_t* fills, int32_t cap) {
  pkv::clear_error();
  if (n < 0 || block_size <= 0 || cap < 0 || (n > 0 && !slots) ||
      (cap > 0 && (!blocks || !fills)))
    return fail(PKV_E_INVAL, "bad blocks_of_slots arguments");
  // highest slot written in each block; a block's slots fill in order, so it gives the fill
  std::vector<std::pair<int64_t, int64_t>> hit;   // (block, slot)
  hit.reserve(size_t(n));
  for (int64_t i = 0; i < n; ++i)
    if (slots[i] >= 0) hit.emplace_back(slots[i] / block_size, slots[i]);
  std::sort(hit.begin(), hit.end());
  int32_t m = 0;
  for (size_t i = 0; i < hit.size(); ++i) {
    if (i + 1 < hit.size() && hit[i + 1].first == hit[i].first) continue;   // not the highest
    if (hit[i].first > INT32_MAX) return fail(PKV_E_INVAL, "slot %lld beyond int32 blocks",
                                              (long long)hit[i].second);
    if (m < cap) {
      blocks[m] = int32_t(hit[i].first);
      fills[m] = int32_t(hit[i].second % block_size) + 1;
    }
    ++m;
  }
  return m;
}

int32_t pkv_bm_evictable_list(pkv_bm* bm, int32_t* out, int32_t cap) {
  if (!bm) return -1;
  int32_t i = 0;
  for (int32_t b : bm->evictable) {
    if (i < cap) out[i] = b;
    ++i;
  }
  return i;
}

}  // extern "C"
