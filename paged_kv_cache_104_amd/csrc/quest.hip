// Query-aware block selection for decode (QUEST; tencent cloud article
// 2526001, section "QUEST: Query-Aware Sparsity for Efficient Long-Context LLM
// Inference"): every KV block keeps the channel-wise minimum and maximum of its
// keys; a query bounds its score with any key of a block by taking, channel by
// channel, the larger of its products with that minimum and maximum, summed;
// only the blocks with the K largest bounds are attended.
//
// Device design:
//  * Metadata pool [N][H][2][D] in the pool's own element type (row 0 the
//    minimum, row 1 the maximum of the block's valid keys).  The minimum or
//    maximum of values of a type is a value of that type, so the metadata is
//    exact; it is 2 rows per block of B rows, 2/B of the key pool.
//    quest_update_*_kernel recompute it for written blocks.
//  * quest_score_kernel: one bound per (sequence, KV head, block), the largest
//    over the KV head's query heads (grouped-query attention), into a
//    workspace row per (sequence, KV head).  Reads only metadata.
//  * quest_select_kernel: one workgroup per (sequence, KV head) (256 threads up
//    to 4096 blocks, 1024 up to 16384, 16 keys per thread); a 4-pass radix
//    select of the K-th largest bound (keys held in registers, histograms in
//    LDS), ties to the lower block index, then the chosen blocks compacted in
//    logical order into a per-(sequence, KV head) block table.  Its entries
//    are block * H + head: the (block, head) slab of the pools seen as
//    [N * H] one-head blocks.  The decode kernels then run unchanged on
//    S * H one-head "sequences" of g query heads each, whose q and out rows
//    are exactly the rows of the original [S][Hq][D] layout.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kQuestChunk = 64;        // blocks per scoring workgroup
constexpr int kScoreThreads = 256;
constexpr int kSelThreadsSmall = 256;  // selecting workgroup for contexts of <= 4096 blocks
constexpr int kSelThreads = 1024;      // ... and up to 16384 blocks
constexpr int kSelPerThread = 16;      // keys held by one selecting thread
constexpr int kQuestMaxBlocks = kSelThreads * kSelPerThread;
constexpr int kQuestMaxGroup = 16;

struct QuestArgs {
  const void* q;
  const void* meta;
  const int32_t* tables;
  const int32_t* lens;
  float* scores;          // [pairs][score_stride]
  int32_t* sel_tables;    // [pairs][out_stride]
  int32_t* sel_lens;      // [pairs]
  int32_t max_blocks;     // row stride of tables
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t num_blocks;
  int32_t block_size;
  int32_t max_ctx;
  int32_t budget;         // blocks kept per (sequence, KV head)
  int32_t score_stride;   // blocks of the longest context
  int32_t out_stride;     // min(max_blocks, budget)
  int32_t chunks;         // scoring workgroups per pair
};

__device__ __forceinline__ int quest_ctx(const QuestArgs& a, int s) {
  return max(0, min(a.lens[s], a.max_ctx));
}

// ------------------------------------------------------------------------ metadata

// (min, max) per channel of rows [0, count) of one (block, head) key slab.
template <int KV>
__device__ __forceinline__ void slab_minmax(const typename KvTraits<KV>::T* __restrict__ slab,
                                            typename KvTraits<KV>::T* __restrict__ meta,
                                            int count, int D) {
  typedef typename KvTraits<KV>::T T;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    T lo = slab[d], hi = lo;
    float flo = kv_to_f32<KV>(lo), fhi = flo;
    for (int r0 = 1; r0 < count; r0 += 8) {
      // eight rows' loads issued together, then compared in row order (a compare between
      // two loads made each load wait for the one before); rows past count repeat the
      // last one, which changes neither extreme
      T x[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = slab[int64_t(min(r0 + i, count - 1)) * D + d];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float f = kv_to_f32<KV>(x[i]);
        if (f < flo) { flo = f; lo = x[i]; }
        if (f > fhi) { fhi = f; hi = x[i]; }
      }
    }
    meta[d] = lo;
    meta[D + d] = hi;
  }
}

// fp8 keys: the codes are sign and magnitude, so their values order as the bytes
// c ^ 0x80 (c >= 0) and c ^ 0xFF (c < 0) do as unsigned numbers (-0 just below +0; the
// NaN codes 0x7F and 0xFF at the top and the bottom).  A thread owns four channels (one
// 32-bit word of a row) and every kQuestFp8RowGroups-th row of the slab; the minimum and
// maximum of each byte are taken on two 16-bit halves (even and odd bytes) with packed
// 16-bit integer min / max, the row groups are combined through LDS, and the order map,
// its own inverse up to the top bit's test, is undone before the store.  Two or three
// integer instructions per key, against a decode to fp32 and two float compares: the fp32
// path held the whole-pool update near 3 TB/s, bound by arithmetic.  A 128-thread
// workgroup.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t fp8_order(uint32_t u) {   // four codes at once
  const uint32_t neg = (u >> 7) & 0x01010101u;
  return u ^ ((neg << 7) - neg) ^ 0x80808080u;                 // 0xFF where negative, else 0x80
}
__device__ __forceinline__ uint32_t fp8_unorder(uint32_t k) {
  const uint32_t pos = (k >> 7) & 0x01010101u;                 // top bit set: a code >= 0
  return k ^ ((pos << 7) - pos) ^ 0xFFFFFFFFu;                 // 0x80 where it was >= 0, else 0xFF
}
__device__ __forceinline__ u16x2 as_u16x2(uint32_t x) { return __builtin_bit_cast(u16x2, x); }
__device__ __forceinline__ uint32_t as_u32(u16x2 x) { return __builtin_bit_cast(uint32_t, x); }

__device__ __forceinline__ void slab_minmax_fp8(const uint8_t* __restrict__ slab,
                                                uint8_t* __restrict__ meta, int count, int D) {
  constexpr int kThreads = 128;
  __shared__ uint32_t s_m[4][kThreads];    // min even, min odd, max even, max odd
  const int groups = D / 4, row_groups = kThreads / groups;
  const int cg = threadIdx.x % groups, rg = threadIdx.x / groups;
  uint32_t mn_e = 0x00ff00ffu, mn_o = 0x00ff00ffu, mx_e = 0, mx_o = 0;
  for (int r0 = rg; r0 < count; r0 += 4 * row_groups) {
    // four rows' words requested together; rows past count repeat the last one
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = *reinterpret_cast<const uint32_t*>(slab + int64_t(min(r0 + i * row_groups, count - 1)) * D + cg * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t k = fp8_order(w[i]);
      const uint32_t e = k & 0x00ff00ffu, o = (k >> 8) & 0x00ff00ffu;
      mn_e = as_u32(__builtin_elementwise_min(as_u16x2(mn_e), as_u16x2(e)));
      mn_o = as_u32(__builtin_elementwise_min(as_u16x2(mn_o), as_u16x2(o)));
      mx_e = as_u32(__builtin_elementwise_max(as_u16x2(mx_e), as_u16x2(e)));
      mx_o = as_u32(__builtin_elementwise_max(as_u16x2(mx_o), as_u16x2(o)));
    }
  }
  s_m[0][threadIdx.x] = mn_e;
  s_m[1][threadIdx.x] = mn_o;
  s_m[2][threadIdx.x] = mx_e;
  s_m[3][threadIdx.x] = mx_o;
  __syncthreads();
  if (rg == 0) {
    for (int g = 1; g < row_groups; ++g) {
      const int t = g * groups + cg;
      mn_e = as_u32(__builtin_elementwise_min(as_u16x2(mn_e), as_u16x2(s_m[0][t])));
      mn_o = as_u32(__builtin_elementwise_min(as_u16x2(mn_o), as_u16x2(s_m[1][t])));
      mx_e = as_u32(__builtin_elementwise_max(as_u16x2(mx_e), as_u16x2(s_m[2][t])));
      mx_o = as_u32(__builtin_elementwise_max(as_u16x2(mx_o), as_u16x2(s_m[3][t])));
    }
    *reinterpret_cast<uint32_t*>(meta + cg * 4) = fp8_unorder(mn_e | (mn_o << 8));
    *reinterpret_cast<uint32_t*>(meta + D + cg * 4) = fp8_unorder(mx_e | (mx_o << 8));
  }
}

template <int KV>
__device__ __forceinline__ void slab_update(const typename KvTraits<KV>::T* __restrict__ slab,
                                            typename KvTraits<KV>::T* __restrict__ meta,
                                            int count, int D) {
  if constexpr (KV == KV_FP8) slab_minmax_fp8(slab, meta, count, D);
  else slab_minmax<KV>(slab, meta, count, D);
}

// Entry i: block blocks[i] over its first counts[i] slots, for head blockIdx.y.
template <int KV>
__global__ __launch_bounds__(128) void quest_update_blocks_kernel(
    const typename KvTraits<KV>::T* __restrict__ k_pool, typename KvTraits<KV>::T* __restrict__ meta,
    const int32_t* __restrict__ blocks, const int32_t* __restrict__ counts, int N, int H, int B,
    int D) {
  const int b = blocks[blockIdx.x], cnt = counts[blockIdx.x], h = blockIdx.y;
  if (b < 0 || b >= N || cnt < 1 || cnt > B) return;
  const int64_t slab = int64_t(b) * H + h;
  slab_update<KV>(k_pool + slab * B * D, meta + slab * 2 * D, cnt, D);
}

// Row blockIdx.x: the block that holds its last token (context_lens - 1).
template <int KV>
__global__ __launch_bounds__(128) void quest_update_tails_kernel(
    const typename KvTraits<KV>::T* __restrict__ k_pool, typename KvTraits<KV>::T* __restrict__ meta,
    const int32_t* __restrict__ tables, int max_blocks, const int32_t* __restrict__ lens, int N,
    int H, int B, int D) {
  const int len = lens[blockIdx.x], h = blockIdx.y;
  if (len <= 0) return;
  const int j = (len - 1) / B;
  if (j >= max_blocks) return;
  const int b = tables[int64_t(blockIdx.x) * max_blocks + j];
  if (b < 0 || b >= N) return;
  const int64_t slab = int64_t(b) * H + h;
  slab_update<KV>(k_pool + slab * B * D, meta + slab * 2 * D, (len - 1) % B + 1, D);
}

// ------------------------------------------------------------------------ scores

// Eight consecutive stored values, kept packed until they are used.
template <int KV>
struct Raw8;
template <>
struct Raw8<KV_F32> { float4 a, b; };
template <>
struct Raw8<KV_BF16> { uint4 a; };
template <>
struct Raw8<KV_FP8> { uint2 a; };

template <int KV>
__device__ __forceinline__ Raw8<KV> load_raw8(const typename KvTraits<KV>::T* p);
template <>
__device__ __forceinline__ Raw8<KV_F32> load_raw8<KV_F32>(const float* p) {
  return Raw8<KV_F32>{reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]};
}
template <>
__device__ __forceinline__ Raw8<KV_BF16> load_raw8<KV_BF16>(const uint16_t* p) {
  return Raw8<KV_BF16>{*reinterpret_cast<const uint4*>(p)};
}
template <>
__device__ __forceinline__ Raw8<KV_FP8> load_raw8<KV_FP8>(const uint8_t* p) {
  return Raw8<KV_FP8>{*reinterpret_cast<const uint2*>(p)};
}

__device__ __forceinline__ void unpack8(const Raw8<KV_F32>& r, float (&f)[8]) {
  f[0] = r.a.x; f[1] = r.a.y; f[2] = r.a.z; f[3] = r.a.w;
  f[4] = r.b.x; f[5] = r.b.y; f[6] = r.b.z; f[7] = r.b.w;
}
__device__ __forceinline__ void unpack8(const Raw8<KV_BF16>& r, float (&f)[8]) {
  const uint32_t w[4] = {r.a.x, r.a.y, r.a.z, r.a.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_to_f32(w[i] >> 16);
  }
}
// fp8: the conversion instruction, two codes at a time (exact: every E4M3 value is an
// fp32 value).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void unpack8(const Raw8<KV_FP8>& r, float (&f)[8]) {
  const uint32_t w[2] = {r.a.x, r.a.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[i]), false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(w[i]), true);
    f[4 * i] = lo.x; f[4 * i + 1] = lo.y; f[4 * i + 2] = hi.x; f[4 * i + 3] = hi.y;
  }
}

// Sum over the LPB (8 or 16) lanes that share a block, aligned groups inside one row of 16
// lanes, with DPP lane moves instead of LDS permutes: swap neighbours, swap pairs, mirror
// each half row (sums of the two quads), and for 16 lanes mirror the row.  Every lane of the
// group ends with the same sum (each step adds two equal partial sums in either order).
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

template <int LPB>
__device__ __forceinline__ float group_sum(float u) {
  static_assert(LPB == 8 || LPB == 16, "a block's lanes are a half row or a row");
  u += dpp_move<0xb1>(u);    // quad_perm [1, 0, 3, 2]
  u += dpp_move<0x4e>(u);    // quad_perm [2, 3, 0, 1]
  u += dpp_move<0x141>(u);   // row_half_mirror
  if constexpr (LPB == 16) u += dpp_move<0x140>(u);   // row_mirror
  return u;
}

// Workgroup (pair, chunk): bounds of blocks [chunk * 64, chunk * 64 + 64) of
// the pair's context.  D / 8 lanes share a block, 8 channels each, so a
// block's minimum and maximum rows are read with coalesced 16-byte loads.
// Every table entry and then every metadata row of the chunk is requested
// before any arithmetic, so the workgroup waits for memory twice in all.  The
// group's queries sit in LDS as fp32.  Each lane sums its 8 channels per head,
// DPP moves over the block's lanes complete the bound, and the score is the
// largest bound over the group's heads.  Pairs whose context fits the budget
// are not scored (the selection keeps all their blocks).
template <int KV, typename QT, int D>
__global__ __launch_bounds__(kScoreThreads) void quest_score_kernel(QuestArgs a) {
  typedef typename KvTraits<KV>::T T;
  constexpr int LPB = D / 8;                 // lanes per block
  constexpr int BPP = kScoreThreads / LPB;   // blocks per pass
  constexpr int PASSES = kQuestChunk / BPP;
  __shared__ float q_s[kQuestMaxGroup][D];
  const int pair = blockIdx.x / a.chunks, chunk = blockIdx.x - pair * a.chunks;
  const int H = a.num_kv_heads, s = pair / H, kvh = pair - s * H;
  const int B = a.block_size;
  const int ctx = quest_ctx(a, s);
  const int nb = (ctx + B - 1) / B;
  if (nb <= a.budget) return;
  const int j0 = chunk * kQuestChunk;
  if (j0 >= nb) return;
  const int jend = min(nb, j0 + kQuestChunk);
  const int tid = threadIdx.x, sub = tid % LPB, slot = tid / LPB, d0 = sub * 8;
  const int g = a.group;
  const int32_t* trow = a.tables + int64_t(s) * a.max_blocks;
  int pb[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int j = j0 + slot + p * BPP;
    pb[p] = j < jend ? trow[j] : -1;
  }
  const T* meta = static_cast<const T*>(a.meta);
  // unconditional loads (an entry outside the pool reads block 0 and scores -inf),
  // so no branch separates the requests
  Raw8<KV> rmn[PASSES], rmx[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int b = (pb[p] >= 0 && pb[p] < a.num_blocks) ? pb[p] : 0;
    const T* m = meta + (int64_t(b) * H + kvh) * 2 * D + d0;
    rmn[p] = load_raw8<KV>(m);
    rmx[p] = load_raw8<KV>(m + D);
  }
  // q after the metadata requests (its wait covers both), 8 values per thread
  constexpr int QKV = std::is_same<QT, float>::value ? KV_F32 : KV_BF16;
  const QT* qrow = static_cast<const QT*>(a.q) + (int64_t(s) * a.num_q_heads + kvh * g) * D;
  for (int i = tid * 8; i < g * D; i += kScoreThreads * 8) {
    float f[8];
    unpack8(load_raw8<QKV>(qrow + i), f);
    *reinterpret_cast<float4*>(&q_s[i / D][i % D]) = make_float4(f[0], f[1], f[2], f[3]);
    *reinterpret_cast<float4*>(&q_s[i / D][i % D + 4]) = make_float4(f[4], f[5], f[6], f[7]);
  }
  __syncthreads();
  // every pass's block at once (a pass past the chunk's end scores block 0 and stores
  // nothing), heads outer: each head's query segment is read from LDS once
  float mn[PASSES][8], mx[PASSES][8], best[PASSES];
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    unpack8(rmn[p], mn[p]);
    unpack8(rmx[p], mx[p]);
    best[p] = -INFINITY;
  }
  for (int h = 0; h < g; ++h) {
    const float4 qa = *reinterpret_cast<const float4*>(&q_s[h][d0]);
    const float4 qb = *reinterpret_cast<const float4*>(&q_s[h][d0 + 4]);
    const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      float u = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) u = fmaf(qv[i], qv[i] >= 0.f ? mx[p][i] : mn[p][i], u);
      best[p] = fmaxf(best[p], group_sum<LPB>(u));
    }
  }
#pragma unroll
  for (int p = 0; p < PASSES; ++p) {
    const int j = j0 + slot + p * BPP;
    if (sub == 0 && j < jend)
      a.scores[int64_t(pair) * a.score_stride + j] =
          (pb[p] >= 0 && pb[p] < a.num_blocks) ? best[p] : -INFINITY;
  }
}

// ------------------------------------------------------------------------ selection

// float -> uint32 with the same order (larger float, larger key).
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the wave's 64 lanes with DPP moves (no LDS round
// trips): shifts by 1, 2, 4 and 8 lanes within each row of 16, then the last
// lane of row 0 into row 1 and of row 2 into row 3, then lane 31 into rows 2
// and 3.  Lanes a move does not reach add 0.
__device__ __forceinline__ int scan64_incl(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return v;
}

// Minimum / maximum over the wave, in every lane: the scan's moves with min / max
// (lanes a move does not reach take the identity), then lane 63's result.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
  int t = int(v);
  t = int(min(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(-1, t, 0x111, 0xf, 0xf, false))));
  t = int(min(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(-1, t, 0x112, 0xf, 0xf, false))));
  t = int(min(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(-1, t, 0x114, 0xf, 0xf, false))));
  t = int(min(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(-1, t, 0x118, 0xf, 0xf, false))));
  t = int(min(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(-1, t, 0x142, 0xa, 0xf, false))));
  t = int(min(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(-1, t, 0x143, 0xc, 0xf, false))));
  return uint32_t(__builtin_amdgcn_readlane(t, 63));
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  int t = int(v);
  t = int(max(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(0, t, 0x111, 0xf, 0xf, false))));
  t = int(max(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(0, t, 0x112, 0xf, 0xf, false))));
  t = int(max(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(0, t, 0x114, 0xf, 0xf, false))));
  t = int(max(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(0, t, 0x118, 0xf, 0xf, false))));
  t = int(max(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(0, t, 0x142, 0xa, 0xf, false))));
  t = int(max(uint32_t(t), uint32_t(__builtin_amdgcn_update_dpp(0, t, 0x143, 0xc, 0xf, false))));
  return uint32_t(__builtin_amdgcn_readlane(t, 63));
}

// Exclusive prefix sum of v over the workgroup's threads in thread order.
__device__ __forceinline__ int block_excl_scan(int v, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int incl = scan64_incl(v);
  if (lane == 63) wsum[wv] = incl;
  __syncthreads();
  int off = 0;
  for (int w = 0; w < wv; ++w) off += wsum[w];
  __syncthreads();
  return off + incl - v;
}

template <int NT>
__global__ __launch_bounds__(NT) void quest_select_kernel(QuestArgs a) {
  static_assert(NT >= 256 && NT % 64 == 0, "one thread per histogram bin at least");
  __shared__ int hist[256];
  __shared__ int wsum[NT / 64];
  __shared__ int sh_digit, sh_above;
  __shared__ uint32_t wlo[NT / 64], whi[NT / 64];
  const int pair = blockIdx.x;
  const int H = a.num_kv_heads, s = pair / H, kvh = pair - s * H;
  const int B = a.block_size;
  const int tid = threadIdx.x;
  const int ctx = quest_ctx(a, s);
  const int nb = (ctx + B - 1) / B;
  const int32_t* trow = a.tables + int64_t(s) * a.max_blocks;
  int32_t* orow = a.sel_tables + int64_t(pair) * a.out_stride;
  auto slab_id = [&](int pb) { return (pb >= 0 && pb < a.num_blocks) ? pb * H + kvh : -1; };
  if (nb <= a.budget) {
    for (int j = tid; j < nb; j += NT) orow[j] = slab_id(trow[j]);
    if (tid == 0) a.sel_lens[pair] = ctx;
    return;
  }
  const int nper = (nb + NT - 1) / NT;  // keys per thread (uniform)
  const int first = tid * nper;
  const float* srow = a.scores + int64_t(pair) * a.score_stride;
  // keys first + i for i < nper, with their table entries, all requested before
  // any is used: every load is unconditional (indices past the thread's share or
  // the context read the context's last block and are masked out)
  uint32_t key[kSelPerThread];
  int32_t ent[kSelPerThread];
  uint32_t vmask = 0;
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i) {
    const int j = min(first + min(i, nper - 1), nb - 1);
    key[i] = order_key(srow[j]);
    ent[i] = trow[j];
    if (i < nper && first + i < nb) vmask |= 1u << i;
  }
  // Bits above the highest one in which the smallest and largest key differ are
  // common to every key (one context's bounds are usually of one magnitude):
  // the radix passes start below them, so the first pass already spreads the
  // keys over many bins.
  uint32_t lo_k = 0xffffffffu, hi_k = 0;
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i)
    if ((vmask >> i) & 1u) {
      lo_k = min(lo_k, key[i]);
      hi_k = max(hi_k, key[i]);
    }
  lo_k = wave_min_u32(lo_k);
  hi_k = wave_max_u32(hi_k);
  if ((tid & 63) == 63) {
    wlo[tid >> 6] = lo_k;
    whi[tid >> 6] = hi_k;
  }
  __syncthreads();
  lo_k = wlo[0];
  hi_k = whi[0];
  for (int w = 1; w < NT / 64; ++w) {
    lo_k = min(lo_k, wlo[w]);
    hi_k = max(hi_k, whi[w]);
  }
  // K-th largest key: up to 8 bits per pass below the common bits, most significant first
  int bits = lo_k == hi_k ? 0 : 32 - __clz(lo_k ^ hi_k);   // bits that still differ
  uint32_t pmask = bits == 32 ? 0u : ~((1u << bits) - 1u);
  uint32_t prefix = hi_k & pmask;
  int k = a.budget;
  while (bits > 0) {
    const int shift = max(bits - 8, 0);
    const uint32_t dmask = (1u << (bits - shift)) - 1u;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSelPerThread; ++i) {
      if (i < nper) {
        // plain LDS atomics: lanes that hit one bin are serialised by the LDS, which
        // costs less than combining them in the wave first
        if (((vmask >> i) & 1u) && (key[i] & pmask) == prefix)
          atomicAdd(&hist[(key[i] >> shift) & dmask], 1);
      }
    }
    __syncthreads();
    if (tid < 64) {
      // lane l holds bins 4 (63 - l) .. 4 (63 - l) + 3, so a prefix sum over the
      // lanes counts the keys in this lane's bins and every higher bin
      const int base = 4 * (63 - tid);
      int h[4], tot = 0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        h[c] = hist[base + c];
        tot += h[c];
      }
      int above = scan64_incl(tot) - tot;  // keys in higher bins
#pragma unroll
      for (int c = 3; c >= 0; --c) {
        if (above < k && above + h[c] >= k) {
          sh_digit = base + c;
          sh_above = above;
        }
        above += h[c];
      }
    }
    __syncthreads();
    prefix |= uint32_t(sh_digit) << shift;
    pmask |= dmask << shift;
    k -= sh_above;
    bits = shift;
  }
  const uint32_t kth = prefix;  // keys above it are kept, and the first k equal to it
  int ceq = 0;
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i)
    if (((vmask >> i) & 1u) && key[i] == kth) ++ceq;
  int eq_rank = block_excl_scan(ceq, wsum);
  uint32_t sel = 0;
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i) {
    if (!((vmask >> i) & 1u)) continue;
    if (key[i] > kth) {
      sel |= 1u << i;
    } else if (key[i] == kth) {
      if (eq_rank < k) sel |= 1u << i;
      ++eq_rank;
    }
  }
  int pos = block_excl_scan(__popc(sel), wsum);
#pragma unroll
  for (int i = 0; i < kSelPerThread; ++i)
    if (((sel >> i) & 1u) && pos >= 0 && pos < a.budget) orow[pos++] = slab_id(ent[i]);
  // the thread holding the last block knows whether the partial block is kept
  const int last = nb - 1;
  if (last >= first && last < first + nper) {
    const bool kept = (sel >> (last - first)) & 1u;
    a.sel_lens[pair] = a.budget * B - (kept ? nb * B - ctx : 0);
  }
}

// ------------------------------------------------------------------------ host side

static size_t qalign(size_t n) { return (n + 255) & ~size_t(255); }
static bool qaligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct QuestLayout {
  int64_t pairs, score_stride, out_stride, chunks;
  int32_t max_ctx2;
  size_t tables_off, lens_off, dec_off, dec_bytes, total;
};

static int quest_layout(const pkv_cache_desc* c, int32_t num_seqs, int32_t num_q_heads,
                        int32_t max_blocks, int32_t max_ctx, int32_t partition_size,
                        int32_t budget, QuestLayout* L) {
  int rc = check_desc(c);
  if (rc) return rc;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks < 0 || max_ctx < 0 || partition_size < 0)
    return fail(PKV_E_INVAL, "negative size");
  if (num_q_heads % c->num_kv_heads)
    return fail(PKV_E_INVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                c->num_kv_heads);
  if (num_q_heads / c->num_kv_heads > kQuestMaxGroup)
    return fail(PKV_E_UNSUPPORTED, "group size %d > %d", num_q_heads / c->num_kv_heads,
                kQuestMaxGroup);
  if (budget < 1) return fail(PKV_E_INVAL, "budget_blocks %d < 1", budget);
  if (int64_t(max_blocks) * c->block_size < max_ctx)
    return fail(PKV_E_INVAL, "max_blocks_per_seq %d cannot hold max_context_len %d", max_blocks,
                max_ctx);
  if (int64_t(c->num_blocks) * c->num_kv_heads >= (int64_t(1) << 31))
    return fail(PKV_E_INVAL, "num_blocks * num_kv_heads does not fit 31 bits");
  L->pairs = int64_t(num_seqs) * c->num_kv_heads;
  L->score_stride = std::max<int64_t>(1, (int64_t(max_ctx) + c->block_size - 1) / c->block_size);
  if (L->score_stride > kQuestMaxBlocks)
    return fail(PKV_E_UNSUPPORTED, "contexts of more than %d blocks", kQuestMaxBlocks);
  L->out_stride = std::max<int64_t>(1, std::min<int64_t>(max_blocks, budget));
  L->chunks = (L->score_stride + kQuestChunk - 1) / kQuestChunk;
  if (L->pairs * L->score_stride >= (int64_t(1) << 31) || L->pairs * L->chunks >= (int64_t(1) << 31))
    return fail(PKV_E_INVAL, "batch too large for one call");
  L->max_ctx2 = int32_t(std::min<int64_t>(max_ctx, L->out_stride * c->block_size));
  const size_t scores = qalign(size_t(L->pairs) * L->score_stride * sizeof(float));
  L->tables_off = scores;
  L->lens_off = L->tables_off + qalign(size_t(L->pairs) * L->out_stride * sizeof(int32_t));
  L->dec_off = L->lens_off + qalign(size_t(L->pairs) * sizeof(int32_t));
  L->dec_bytes = pkv_decode_workspace_bytes(int32_t(std::max<int64_t>(1, L->pairs)),
                                            num_q_heads / c->num_kv_heads, c->head_dim,
                                            L->max_ctx2, partition_size);
  L->total = L->dec_off + L->dec_bytes;
  return PKV_OK;
}

template <typename K>
static int qlaunch(K kernel, dim3 grid, dim3 block, hipStream_t s, const char* what,
                   const QuestArgs& a) {
  kernel<<<grid, block, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

template <int D>
static int launch_score(const QuestArgs& a, int kv, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(int64_t(a.num_seqs) * a.num_kv_heads * a.chunks));
  const dim3 block(kScoreThreads);
  if (kv == PKV_F32) return qlaunch(quest_score_kernel<KV_F32, float, D>, grid, block, s, "score", a);
  if (kv == PKV_BF16)
    return qlaunch(quest_score_kernel<KV_BF16, uint16_t, D>, grid, block, s, "score", a);
  return qlaunch(quest_score_kernel<KV_FP8, uint16_t, D>, grid, block, s, "score", a);
}

// Validates, fills the arguments and launches scoring + selection.
static int quest_select_impl(const void* q, int32_t q_dtype, const void* meta,
                             const pkv_cache_desc* c, const int32_t* block_tables,
                             int32_t max_blocks, const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_q_heads, int32_t max_ctx, int32_t budget,
                             int32_t* sel_tables, int32_t* sel_lens, void* workspace,
                             size_t workspace_bytes, const QuestLayout& L, hipStream_t s) {
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16)
    return fail(PKV_E_INVAL, "q_dtype must be f32 or bf16");
  if ((c->kv_dtype == PKV_F32) != (q_dtype == PKV_F32))
    return fail(PKV_E_UNSUPPORTED, "q %s with a %s pool", dtype_name(q_dtype),
                dtype_name(c->kv_dtype));
  if (num_seqs == 0) return PKV_OK;
  if (!q || !meta || !block_tables || !context_lens || !sel_tables || !sel_lens || !workspace)
    return fail(PKV_E_INVAL, "NULL pointer");
  if (!qaligned16(q) || !qaligned16(meta) || !qaligned16(workspace))
    return fail(PKV_E_INVAL, "device pointers must be 16-byte aligned");
  if (workspace_bytes < L.tables_off)
    return fail(PKV_E_INVAL, "workspace of %zu bytes needed (got %zu)", L.tables_off,
                workspace_bytes);
  QuestArgs a;
  a.q = q;
  a.meta = meta;
  a.tables = block_tables;
  a.lens = context_lens;
  a.scores = static_cast<float*>(workspace);
  a.sel_tables = sel_tables;
  a.sel_lens = sel_lens;
  a.max_blocks = max_blocks;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = c->num_kv_heads;
  a.group = num_q_heads / c->num_kv_heads;
  a.num_blocks = c->num_blocks;
  a.block_size = c->block_size;
  a.max_ctx = max_ctx;
  a.budget = budget;
  a.score_stride = int32_t(L.score_stride);
  a.out_stride = int32_t(L.out_stride);
  a.chunks = int32_t(L.chunks);
  int rc = c->head_dim == 64 ? launch_score<64>(a, c->kv_dtype, s)
                             : launch_score<128>(a, c->kv_dtype, s);
  if (rc) return rc;
  const dim3 grid(static_cast<unsigned>(L.pairs));
  if (L.score_stride <= kSelThreadsSmall * kSelPerThread)
    return qlaunch(quest_select_kernel<kSelThreadsSmall>, grid, dim3(kSelThreadsSmall), s,
                   "select", a);
  return qlaunch(quest_select_kernel<kSelThreads>, grid, dim3(kSelThreads), s, "select", a);
}

template <int KV>
static int launch_update_blocks(const pkv_cache_desc* c, const void* k_pool, void* meta,
                                const int32_t* blocks, const int32_t* counts, int32_t n,
                                hipStream_t s) {
  typedef typename KvTraits<KV>::T T;
  quest_update_blocks_kernel<KV><<<dim3(n, c->num_kv_heads), dim3(128), 0, s>>>(
      static_cast<const T*>(k_pool), static_cast<T*>(meta), blocks, counts, c->num_blocks,
      c->num_kv_heads, c->block_size, c->head_dim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "quest update launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

template <int KV>
static int launch_update_tails(const pkv_cache_desc* c, const void* k_pool, void* meta,
                               const int32_t* tables, int32_t max_blocks, const int32_t* lens,
                               int32_t n, hipStream_t s) {
  typedef typename KvTraits<KV>::T T;
  quest_update_tails_kernel<KV><<<dim3(n, c->num_kv_heads), dim3(128), 0, s>>>(
      static_cast<const T*>(k_pool), static_cast<T*>(meta), tables, max_blocks, lens,
      c->num_blocks, c->num_kv_heads, c->block_size, c->head_dim);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "quest update launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_quest_meta_bytes(const pkv_cache_desc* c) {
  if (!c || check_desc(c)) return 0;
  return size_t(c->num_blocks) * c->num_kv_heads * 2 * c->head_dim * elem_bytes(c->kv_dtype);
}

extern "C" int pkv_quest_update_blocks(const void* k_pool, const pkv_cache_desc* c, void* meta,
                                       const int32_t* blocks, const int32_t* counts, int32_t n,
                                       void* stream) {
  clear_error();
  int rc = check_desc(c);
  if (rc) return rc;
  if (n < 0) return fail(PKV_E_INVAL, "negative count");
  if (n == 0) return PKV_OK;
  if (!k_pool || !meta || !blocks || !counts) return fail(PKV_E_INVAL, "NULL pointer");
  if (!qaligned16(k_pool) || !qaligned16(meta))
    return fail(PKV_E_INVAL, "device pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c->kv_dtype == PKV_F32) return launch_update_blocks<KV_F32>(c, k_pool, meta, blocks, counts, n, s);
  if (c->kv_dtype == PKV_BF16) return launch_update_blocks<KV_BF16>(c, k_pool, meta, blocks, counts, n, s);
  return launch_update_blocks<KV_FP8>(c, k_pool, meta, blocks, counts, n, s);
}

extern "C" int pkv_quest_update_tails(const void* k_pool, const pkv_cache_desc* c, void* meta,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      void* stream) {
  clear_error();
  int rc = check_desc(c);
  if (rc) return rc;
  if (num_seqs < 0 || max_blocks_per_seq < 0) return fail(PKV_E_INVAL, "negative size");
  if (num_seqs == 0 || max_blocks_per_seq == 0) return PKV_OK;
  if (!k_pool || !meta || !block_tables || !context_lens) return fail(PKV_E_INVAL, "NULL pointer");
  if (!qaligned16(k_pool) || !qaligned16(meta))
    return fail(PKV_E_INVAL, "device pointers must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (c->kv_dtype == PKV_F32)
    return launch_update_tails<KV_F32>(c, k_pool, meta, block_tables, max_blocks_per_seq,
                                       context_lens, num_seqs, s);
  if (c->kv_dtype == PKV_BF16)
    return launch_update_tails<KV_BF16>(c, k_pool, meta, block_tables, max_blocks_per_seq,
                                        context_lens, num_seqs, s);
  return launch_update_tails<KV_FP8>(c, k_pool, meta, block_tables, max_blocks_per_seq,
                                     context_lens, num_seqs, s);
}

extern "C" size_t pkv_quest_workspace_bytes(const pkv_cache_desc* c, int32_t num_seqs,
                                            int32_t num_q_heads, int32_t max_blocks_per_seq,
                                            int32_t max_context_len, int32_t partition_size,
                                            int32_t budget_blocks) {
  QuestLayout L;
  clear_error();
  if (quest_layout(c, std::max(num_seqs, 1), num_q_heads, max_blocks_per_seq, max_context_len,
                   partition_size, budget_blocks, &L))
    return 0;
  return L.total;
}

extern "C" int pkv_quest_select(const void* q, int32_t q_dtype, const void* meta,
                                const pkv_cache_desc* c, const int32_t* block_tables,
                                int32_t max_blocks_per_seq, const int32_t* context_lens,
                                int32_t num_seqs, int32_t num_q_heads, int32_t max_context_len,
                                int32_t budget_blocks, int32_t* sel_tables, int32_t* sel_lens,
                                void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  QuestLayout L;
  int rc = quest_layout(c, num_seqs, num_q_heads, max_blocks_per_seq, max_context_len, 0,
                        budget_blocks, &L);
  if (rc) return rc;
  return quest_select_impl(q, q_dtype, meta, c, block_tables, max_blocks_per_seq, context_lens,
                           num_seqs, num_q_heads, max_context_len, budget_blocks, sel_tables,
                           sel_lens, workspace, workspace_bytes, L,
                           static_cast<hipStream_t>(stream));
}

extern "C" int pkv_quest_decode(const void* q, int32_t q_dtype, const void* k_pool,
                                const void* v_pool, const void* meta, const pkv_cache_desc* c,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, float scale, void* out,
                                int32_t max_context_len, int32_t partition_size,
                                int32_t budget_blocks, void* workspace, size_t workspace_bytes,
                                void* stream, int32_t impl) {
  clear_error();
  QuestLayout L;
  int rc = quest_layout(c, num_seqs, num_q_heads, max_blocks_per_seq, max_context_len,
                        partition_size, budget_blocks, &L);
  if (rc) return rc;
  if (num_seqs == 0) return PKV_OK;
  if (!workspace || workspace_bytes < L.total)
    return fail(PKV_E_INVAL, "workspace of %zu bytes needed (got %zu)", L.total, workspace_bytes);
  if (!k_pool || !v_pool || !out) return fail(PKV_E_INVAL, "NULL pointer");
  char* ws = static_cast<char*>(workspace);
  int32_t* sel_tables = reinterpret_cast<int32_t*>(ws + L.tables_off);
  int32_t* sel_lens = reinterpret_cast<int32_t*>(ws + L.lens_off);
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = quest_select_impl(q, q_dtype, meta, c, block_tables, max_blocks_per_seq, context_lens,
                         num_seqs, num_q_heads, max_context_len, budget_blocks, sel_tables,
                         sel_lens, workspace, workspace_bytes, L, s);
  if (rc) return rc;
  // the pools as [N * H] one-head blocks; one "sequence" per (sequence, KV head)
  pkv_cache_desc slabs = *c;
  slabs.num_blocks = c->num_blocks * c->num_kv_heads;
  slabs.num_kv_heads = 1;
  return pkv_paged_attn_decode_ex(q, q_dtype, k_pool, v_pool, &slabs, sel_tables,
                                  int32_t(L.out_stride), sel_lens, int32_t(L.pairs),
                                  num_q_heads / c->num_kv_heads, scale, out, L.max_ctx2,
                                  partition_size, ws + L.dec_off, L.dec_bytes, stream, impl);
}
