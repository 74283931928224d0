// Units of the shared-prefix decode: which sequences of a batch attend a run
// of shared leading blocks together.  Sequences forked from one prompt share the
// prompt's full blocks through their block tables (ithome article 10417389,
// section 4, "Physical block sharing"; glossary "PagedAttention", "Sharing
// blocks between sequences"): their keys and values are the same bytes, so
// the decode reads them once for all the sharers' queries.
//
// A group is a run of consecutive batch sequences (at most 32 / group size of
// them, the shared-prefix kernel's two 16-column query tiles) whose tables start with the
// same nb >= min_shared_blocks block ids; nb is also kept below every
// member's last block, so each member has tokens after the shared part.  A
// group becomes one unit {first member, nb * B shared tokens, members, reread};
// any other sequence is a unit of its own {seq, 0, 1, 0}.  reread is 1 when
// sequences outside the unit start with the unit's first block too (a prompt
// with more sharers than one unit holds): other units or sequences of the
// batch read the unit's shared blocks again, and the kernel then reads them
// with cached loads.
#include <algorithm>
#include <cstdint>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"
#include "pkv_internal.h"

using namespace pkv;

extern "C" int32_t pkv_prefix_rows(const int32_t* tables, const int32_t* lens, int32_t num_seqs,
                                   int32_t max_blocks, int32_t block_size, int32_t group,
                                   int32_t min_shared_blocks, int32_t* rows, int32_t* seq_rows) {
  clear_error();
  if (num_seqs < 0 || max_blocks < 0 || block_size <= 0 || group < 1 || group > 16)
    return fail(PKV_E_INVAL, "bad sizes (num_seqs %d, max_blocks %d, block_size %d, group %d)",
                num_seqs, max_blocks, block_size, group);
  if (num_seqs > 0 && (!tables || !lens || !rows || !seq_rows))
    return fail(PKV_E_INVAL, "NULL pointer");
  const int max_members = 32 / group;   // query columns of a unit (two 16-column tiles)
  const int min_nb = std::max(1, min_shared_blocks);
  // full blocks of sequence i before its last token: the most it can share
  auto shareable = [&](int i) {
    const int64_t n = lens[i] > 0 ? (int64_t(lens[i]) - 1) / block_size : 0;
    return int(std::min<int64_t>(n, max_blocks));
  };
  auto common = [&](int i, int j, int limit) {
    const int32_t* a = tables + int64_t(i) * max_blocks;
    const int32_t* b = tables + int64_t(j) * max_blocks;
    int k = 0;
    while (k < limit && a[k] == b[k] && a[k] >= 0) ++k;
    return k;
  };
  int nr = 0;
  auto put_unit = [&](int seq, int shared_tokens, int members) {
    int32_t* r = rows + int64_t(nr) * 4;
    r[0] = seq;
    r[1] = shared_tokens;
    r[2] = members;
    r[3] = 0;
    for (int m = 0; m < members; ++m) {
      int32_t* sr = seq_rows + int64_t(seq + m) * 4;
      sr[0] = nr;
      sr[1] = m;
      sr[2] = 0;
      sr[3] = 0;
    }
    ++nr;
  };
  // readers of each first block: sequences with a context whose table starts with it
  std::unordered_map<int32_t, int> first_readers;
  for (int i = 0; i < num_seqs && max_blocks > 0; ++i)
    if (lens[i] > 0 && tables[int64_t(i) * max_blocks] >= 0)
      ++first_readers[tables[int64_t(i) * max_blocks]];
  for (int i = 0; i < num_seqs;) {
    int nb = shareable(i);
    int n = 1;
    while (n < max_members && i + n < num_seqs) {
      const int c = common(i, i + n, std::min(nb, shareable(i + n)));
      if (c < min_nb) break;
      nb = c;
      ++n;
    }
    if (n >= 2 && nb >= min_nb) {
      put_unit(i, nb * block_size, n);
      rows[int64_t(nr - 1) * 4 + 3] = first_readers[tables[int64_t(i) * max_blocks]] > n;
      i += n;
    } else {
      put_unit(i, 0, 1);
      ++i;
    }
  }
  return nr;
}

// A batch order that puts sharers next to each other: sequences sorted by the
// block ids of their shareable blocks, compared as sequences (lexicographic,
// a shorter run of ids first when it is the other's start), equal ones in
// batch order.  Sequences with a common run of leading blocks then form one
// contiguous range, which pkv_prefix_rows can group.
extern "C" int32_t pkv_prefix_order(const int32_t* tables, const int32_t* lens, int32_t num_seqs,
                                    int32_t max_blocks, int32_t block_size, int32_t* order) {
  clear_error();
  if (num_seqs < 0 || max_blocks < 0 || block_size <= 0)
    return fail(PKV_E_INVAL, "bad sizes (num_seqs %d, max_blocks %d, block_size %d)", num_seqs,
                max_blocks, block_size);
  if (num_seqs > 0 && (!tables || !lens || !order)) return fail(PKV_E_INVAL, "NULL pointer");
  std::vector<int> n(num_seqs);
  for (int i = 0; i < num_seqs; ++i) {
    const int64_t full = lens[i] > 0 ? (int64_t(lens[i]) - 1) / block_size : 0;
    const int32_t* row = tables + int64_t(i) * max_blocks;
    int k = 0;
    while (k < std::min<int64_t>(full, max_blocks) && row[k] >= 0) ++k;
    n[i] = k;
    order[i] = i;
  }
  std::stable_sort(order, order + num_seqs, [&](int32_t a, int32_t b) {
    const int32_t* ra = tables + int64_t(a) * max_blocks;
    const int32_t* rb = tables + int64_t(b) * max_blocks;
    return std::lexicographical_compare(ra, ra + n[a], rb, rb + n[b]);
  });
  return PKV_OK;
}
