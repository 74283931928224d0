// Paged decode attention: one new query per sequence attends over its cached
// keys and values, read block by block through the sequence's block table
// (ultralytics glossary "PagedAttention", section "How paging works";
// optiverse blog "paged-kv-cache", section "Block table and non-contiguous
// allocation").  The score matrix is never written out: scores are folded
// into a running max / running sum / running output as in FlashAttention-style
// tiled attention (glossary, "Related techniques").  Query heads share KV heads
// in contiguous groups (grouped-query attention, same section).
//
// Work split: one work item = (sequence, KV head, partition of the context).
// Partitions run in parallel; when a context has more than one, each writes
// (running max, running sum, normalised output) to the workspace and
// merge_partitions_kernel combines them.
//
// Two kernel families:
//  * decode_mfma_kernel (bf16 / fp8 pools): one wave64 per work item.  The
//    context is walked 32 tokens at a time; Q.K^T and P.V of the whole head
//    group are 16x16x32 bf16 MFMAs (group padded to 16 columns), with P
//    rounded to bf16.  Every lane issues 16-byte loads; the next 32 tokens are
//    loaded while the current ones are computed.
//  * decode_vector_kernel (any pool dtype): a plain, fp32-arithmetic kernel
//    with LDS staging; the f32 path and a cross-check of the MFMA kernel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <type_traits>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* ws_ml;         // [S][Hq][P][2]: running max (log2 units), running sum
  float* ws_acc;        // [S][Hq][P][D]: partition output, normalised
  int32_t max_blocks;   // row stride of block_tables
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;        // num_q_heads / num_kv_heads
  int32_t num_blocks;   // pool blocks (block ids outside [0, num_blocks) are skipped)
  int32_t max_ctx;      // contexts are cut at this host-known bound
  int32_t part_tokens;  // partition length (tokens); the whole context when 0
  int32_t max_parts;    // partitions per (sequence, KV head) in the grid
  float qk_scale_log2;  // scale * log2(e) * k_scale
  float v_scale;
};

// Grid position -> work item.  Consecutive workgroups go to different XCDs
// (round robin over 8); the remap keeps the partitions of one (sequence, KV
// head) on one XCD so their table rows and query share that XCD's L2.
__device__ __forceinline__ int remap_xcd(int bid, int nblocks) {
  const int per = nblocks / 8;
  if (bid >= per * 8) return bid;  // tail that does not fill all XCDs
  return (bid % 8) * per + bid / 8;
}

template <typename OutT>
__device__ __forceinline__ void store_out(OutT* p, float x);
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) { *p = f32_to_bf16(x); }

// ------------------------------------------------------------------------ vector kernel

constexpr int kVecThreads = 256;
constexpr int kVecChunk = 256;  // tokens per LDS chunk
constexpr int kMaxGroup = 16;

template <int KV, typename QT, int D, int BS>
__global__ __launch_bounds__(kVecThreads) void decode_vector_kernel(DecodeArgs a) {
  typedef typename KvTraits<KV>::T T;
  __shared__ float q_s[kMaxGroup][D];
  __shared__ float p_s[kMaxGroup][kVecChunk];
  __shared__ float acc_s[kMaxGroup][D];
  __shared__ float m_s[kMaxGroup], l_s[kMaxGroup], alpha_s[kMaxGroup];
  __shared__ int32_t blk_s[kVecChunk / BS + 1];

  const int wid = blockIdx.x;
  const int p = wid % a.max_parts;
  const int kvh = (wid / a.max_parts) % a.num_kv_heads;
  const int s = wid / (a.max_parts * a.num_kv_heads);
  const int tid = threadIdx.x;
  const int g = a.group;
  const int ctx = min(a.context_lens[s], a.max_ctx);
  const int t0 = a.part_tokens ? p * a.part_tokens : 0;
  const int t1 = a.part_tokens ? min(ctx, t0 + a.part_tokens) : ctx;
  const int nparts = a.part_tokens ? (ctx + a.part_tokens - 1) / a.part_tokens : 1;
  QT* out = static_cast<QT*>(a.out);
  if (t0 >= t1) {
    if (p == 0) {  // empty context: zeros
      for (int i = tid; i < g * D; i += kVecThreads)
        store_out(out + (int64_t(s) * a.num_q_heads + kvh * g + i / D) * D + i % D, 0.f);
    }
    return;
  }
  const QT* q = static_cast<const QT*>(a.q) + (int64_t(s) * a.num_q_heads + kvh * g) * D;
  for (int i = tid; i < g * D; i += kVecThreads) {
    float x;
    if constexpr (sizeof(QT) == 4) x = q[i]; else x = bf16_to_f32(q[i]);
    q_s[i / D][i % D] = x;
    acc_s[i / D][i % D] = 0.f;
  }
  if (tid < g) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  const T* kp = static_cast<const T*>(a.k_pool);
  const T* vp = static_cast<const T*>(a.v_pool);
  const int32_t* table = a.block_tables + int64_t(s) * a.max_blocks;
  const int64_t head_stride = int64_t(BS) * D;
  __syncthreads();

  for (int cs = t0; cs < t1; cs += kVecChunk) {
    const int n = min(kVecChunk, t1 - cs);
    // physical blocks of this chunk (cs is a multiple of BS)
    for (int i = tid; i < (n + BS - 1) / BS; i += kVecThreads) blk_s[i] = table[cs / BS + i];
    __syncthreads();
    // scores: thread i owns token cs + i for every head of the group
    if (tid < n) {
      const int pb = blk_s[tid / BS];
      float dots[kMaxGroup];
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h) dots[h] = 0.f;
      const bool ok = pb >= 0 && pb < a.num_blocks;
      if (ok) {
        const T* krow = kp + (int64_t(pb) * a.num_kv_heads + kvh) * head_stride +
                        int64_t((cs + tid) % BS) * D;
        for (int d = 0; d < D; ++d) {
          const float kv = kv_to_f32<KV>(krow[d]);
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h)
            if (h < g) dots[h] = fmaf(q_s[h][d], kv, dots[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
        if (h < g) p_s[h][tid] = ok ? dots[h] * a.qk_scale_log2 : -INFINITY;
    }
    __syncthreads();
    // running max and weights, one thread per head
    if (tid < g) {
      float mx = m_s[tid];
      for (int i = 0; i < n; ++i) mx = fmaxf(mx, p_s[tid][i]);
      const float alpha = mx == -INFINITY ? 1.f : exp2f(m_s[tid] - mx);
      float sum = 0.f;
      for (int i = 0; i < n; ++i) {
        const float w = mx == -INFINITY ? 0.f : exp2f(p_s[tid][i] - mx);
        p_s[tid][i] = w;
        sum += w;
      }
      l_s[tid] = l_s[tid] * alpha + sum;
      m_s[tid] = mx;
      alpha_s[tid] = alpha;
    }
    __syncthreads();
    // P.V: thread per (head, dimension)
    for (int idx = tid; idx < g * D; idx += kVecThreads) {
      const int h = idx / D, d = idx % D;
      float acc = acc_s[h][d] * alpha_s[h];
      for (int i = 0; i < n; ++i) {
        const float w = p_s[h][i];
        const int pb = blk_s[i / BS];
        if (w != 0.f && pb >= 0 && pb < a.num_blocks) {
          const T* vcol = vp + (int64_t(pb) * a.num_kv_heads + kvh) * head_stride +
                          int64_t(d) * BS + (cs + i) % BS;
          acc = fmaf(w, kv_to_f32<KV>(*vcol), acc);
        }
      }
      acc_s[h][d] = acc;
    }
    __syncthreads();
  }

  for (int idx = tid; idx < g * D; idx += kVecThreads) {
    const int h = idx / D, d = idx % D;
    const float l = l_s[h];
    const float o = l > 0.f ? acc_s[h][d] * (a.v_scale / l) : 0.f;
    const int64_t row = int64_t(s) * a.num_q_heads + kvh * g + h;
    if (nparts == 1) {
      store_out(out + row * D + d, o);
    } else {
      a.ws_acc[(row * a.max_parts + p) * D + d] = o;
      if (d == 0) {
        a.ws_ml[(row * a.max_parts + p) * 2] = m_s[h];
        a.ws_ml[(row * a.max_parts + p) * 2 + 1] = l;
      }
    }
  }
}

// ------------------------------------------------------------------------ MFMA kernel

// Per-lane registers of one 32-token step.
template <int KV, int D>
struct StepRegs {
  static constexpr int NK = KV == KV_FP8 ? D / 64 : D / 32;  // 16-byte K loads per tile
  uint4 ka[NK];   // K rows, tile a (MFMA A operand of Q.K^T)
  uint4 kb[NK];   // K rows, tile b
  typename std::conditional<KV == KV_FP8, uint2, uint4>::type v[D / 16];  // V^T, 8 tokens x 1 dim
};

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Two fp8 codes (low or high half of w) -> two bf16 (exact: every e4m3 value is a bf16).
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t,
                            __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(int(w), 1.0f, HI));
}

__device__ __forceinline__ uint4 fp8x8_to_bf16x8(uint2 w) {
  return make_uint4(fp8x2_to_bf16x2<false>(w.x), fp8x2_to_bf16x2<true>(w.x),
                    fp8x2_to_bf16x2<false>(w.y), fp8x2_to_bf16x2<true>(w.y));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef float float2_t __attribute__((ext_vector_type(2)));
  const float2_t f = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
}

// Start dimension of the 8 dimensions lane group r feeds into k-step i of Q.K^T.
// bf16: one 16-byte load per k-step, the 4 lane groups read 64 contiguous bytes.
// fp8: one 16-byte load covers two k-steps.
template <int KV>
__device__ __forceinline__ int qk_dim0(int i, int r) {
  if constexpr (KV == KV_FP8) return 64 * (i >> 1) + 16 * r + 8 * (i & 1);
  else return 32 * i + 8 * r;
}

// Lane-constant parts of the step addresses.  A step covers tokens tt .. tt+31
// (tt is a multiple of BS); lane (r, c) reads
//   K tile a: token ka_tok = 8*(c>>2) + (c&3), tile b: ka_tok + 4, dimensions qk_dim0(., r)
//   V^T:      tokens 8r .. 8r+7 of dimension 16*j + c
template <int KV, int D, int BS>
struct LaneMap {
  int ka_blk, kb_blk, v_blk;    // which of the step's 32/BS blocks
  int64_t ka_off, kb_off, v_off;  // element offset inside a (block, head) tile
  __device__ LaneMap(int r, int c) {
    const int ta = 8 * (c >> 2) + (c & 3), tb = ta + 4, tv = 8 * r;
    ka_blk = ta / BS;
    kb_blk = tb / BS;
    v_blk = tv / BS;
    ka_off = int64_t(ta % BS) * D + qk_dim0<KV>(0, r);
    kb_off = int64_t(tb % BS) * D + qk_dim0<KV>(0, r);
    v_off = int64_t(c) * BS + (tv % BS);
  }
};

template <int BS>
__device__ __forceinline__ int pick_block(const int (&pbs)[32 / BS], int which) {
  int pb = pbs[0];
#pragma unroll
  for (int b = 1; b < 32 / BS; ++b) pb = which == b ? pbs[b] : pb;
  return pb;
}

// A KV block that no other sequence shares is read once per decode: streaming
// (non-temporal) loads keep it from displacing useful lines.  Blocks shared by
// several sequences (forked samples) are read with ordinary loads so that the
// other readers can hit in L2 / the Infinity Cache.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

template <bool NT>
__device__ __forceinline__ uint4 ld16(const void* p) {
  u32x4_t v;
  if constexpr (NT) v = __builtin_nontemporal_load(static_cast<const u32x4_t*>(p));
  else v = *static_cast<const u32x4_t*>(p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <bool NT>
__device__ __forceinline__ uint2 ld8(const void* p) {
  u32x2_t v;
  if constexpr (NT) v = __builtin_nontemporal_load(static_cast<const u32x2_t*>(p));
  else v = *static_cast<const u32x2_t*>(p);
  return make_uint2(v.x, v.y);
}

// Issue the loads of one step.  Block ids outside the pool (and blocks past the
// context, whose tokens are masked later) read block 0 instead, so every load is
// in bounds and no lane branches.
template <int KV, int D, int BS, bool NT>
__device__ __forceinline__ void load_step(StepRegs<KV, D>& R, const typename KvTraits<KV>::T* kp,
                                          const typename KvTraits<KV>::T* vp,
                                          const int32_t* table, int nlb, int num_blocks,
                                          int64_t blk_stride, int tt, const LaneMap<KV, D, BS>& L) {
  constexpr int NB = 32 / BS;
  int pbs[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int lb = tt / BS + b;
    const int pb = lb < nlb ? table[lb] : 0;
    pbs[b] = (pb >= 0 && pb < num_blocks) ? pb : 0;
  }
  const auto* ka = kp + int64_t(pick_block<BS>(pbs, L.ka_blk)) * blk_stride + L.ka_off;
  const auto* kb = kp + int64_t(pick_block<BS>(pbs, L.kb_blk)) * blk_stride + L.kb_off;
  const auto* vb = vp + int64_t(pick_block<BS>(pbs, L.v_blk)) * blk_stride + L.v_off;
#pragma unroll
  for (int i = 0; i < StepRegs<KV, D>::NK; ++i) {
    // bf16: k-step i starts 32*i dimensions further; fp8: load i covers k-steps 2i, 2i+1
    const int di = KV == KV_FP8 ? 64 * i : 32 * i;
    R.ka[i] = ld16<NT>(ka + di);
    R.kb[i] = ld16<NT>(kb + di);
  }
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    const auto* col = vb + 16 * j * BS;
    if constexpr (KV == KV_FP8) R.v[j] = ld8<NT>(col);
    else R.v[j] = ld16<NT>(col);
  }
}

// Rescaling threshold (log2 units): the running reference max is only raised
// when a score exceeds it by more than this, so weights stay below 2^8.
constexpr float kRescaleLog2 = 8.0f;

template <int KV, int D>
__device__ __forceinline__ void compute_step(const StepRegs<KV, D>& R, const bf16x8_t (&qb)[D / 32],
                                             floatx4_t (&acc)[D / 16], floatx4_t& lsum, float& m,
                                             float sl2, int tt, int t1, int r) {
  // scores S^T[token][head] of the two 16-token tiles
  floatx4_t sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int i = 0; i < D / 32; ++i) {
    bf16x8_t ka, kb;
    if constexpr (KV == KV_FP8) {
      const uint4 wa = R.ka[i >> 1], wb = R.kb[i >> 1];
      ka = as_bf16x8((i & 1) ? fp8x8_to_bf16x8(make_uint2(wa.z, wa.w))
                             : fp8x8_to_bf16x8(make_uint2(wa.x, wa.y)));
      kb = as_bf16x8((i & 1) ? fp8x8_to_bf16x8(make_uint2(wb.z, wb.w))
                             : fp8x8_to_bf16x8(make_uint2(wb.x, wb.y)));
    } else {
      ka = as_bf16x8(R.ka[i]);
      kb = as_bf16x8(R.kb[i]);
    }
    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb[i], sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, qb[i], sb, 0, 0, 0);
  }
  // lane (r, c): x[e] = raw score of head c for token 8r + e of the step
  float x[8] = {sa[0], sa[1], sa[2], sa[3], sb[0], sb[1], sb[2], sb[3]};
  const bool tail = tt + 32 > t1;
  if (tail) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (tt + 8 * r + e >= t1) x[e] = -INFINITY;
  }
  float lmax = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) lmax = fmaxf(lmax, x[e]);
  // raise the reference max (and rescale what was summed so far) only when needed
  if (__builtin_amdgcn_ballot_w64(lmax * sl2 > m + kRescaleLog2)) {
    float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m, cmax * sl2);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[j] *= alpha;
    lsum *= alpha;
    m = m_new;
  }
  uint32_t pw[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2)
    pw[e / 2] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(x[e], sl2, -m)),
                            __builtin_amdgcn_exp2f(fmaf(x[e + 1], sl2, -m)));
  const bf16x8_t pb = as_bf16x8(make_uint4(pw[0], pw[1], pw[2], pw[3]));
  // invalid tokens have p = 0, but 0 * NaN is NaN: zero their V elements
  uint32_t vmask[4] = {~0u, ~0u, ~0u, ~0u};
  if (tail) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (tt + 8 * r + e >= t1) vmask[e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
  }
#pragma unroll
  for (int j = 0; j < D / 16; ++j) {
    uint4 vw;
    if constexpr (KV == KV_FP8) vw = fp8x8_to_bf16x8(R.v[j]);
    else vw = R.v[j];
    if (tail) {
      vw.x &= vmask[0];
      vw.y &= vmask[1];
      vw.z &= vmask[2];
      vw.w &= vmask[3];
    }
    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vw), pb, acc[j], 0, 0, 0);
  }
  // running sum of the same bf16 weights: a ones operand sums P^T over the 32 tokens
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
  lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ones), pb, lsum, 0, 0, 0);
}

// Software pipeline depth (32-token steps whose loads are in flight while one
// computes) and the waves per SIMD the register budget is sized for.  Measured
// on the 8B-like GQA layer: bf16 steps (16 KB) run best 3 deep at 1 wave/SIMD,
// fp8 steps (8 KB) 2 deep at 2 waves/SIMD.
template <int KV>
struct MfmaTuning {
  static constexpr int stages = KV == KV_FP8 ? 2 : 3;
  static constexpr int waves = KV == KV_FP8 ? 2 : 1;
};

template <int KV, int D, int BS, bool NT>
__global__ __launch_bounds__(64, MfmaTuning<KV>::waves) void decode_mfma_kernel(DecodeArgs a) {
  typedef typename KvTraits<KV>::T T;
  constexpr int NS = MfmaTuning<KV>::stages;
  const int lane = threadIdx.x;
  const int r = lane >> 4, c = lane & 15;
  const int wid = remap_xcd(blockIdx.x, gridDim.x);
  const int p = wid % a.max_parts;
  const int kvh = (wid / a.max_parts) % a.num_kv_heads;
  const int s = wid / (a.max_parts * a.num_kv_heads);
  const int g = a.group;
  const int ctx = min(a.context_lens[s], a.max_ctx);
  const int t0 = a.part_tokens ? p * a.part_tokens : 0;
  const int t1 = a.part_tokens ? min(ctx, t0 + a.part_tokens) : ctx;
  const int nparts = a.part_tokens ? (ctx + a.part_tokens - 1) / a.part_tokens : 1;
  uint16_t* out = static_cast<uint16_t*>(a.out);
  const int64_t row0 = int64_t(s) * a.num_q_heads + kvh * g;  // first q head of the group
  if (t0 >= t1) {
    if (p == 0 && c < g) {  // empty context: zeros
      for (int d = r; d < D; d += 4) out[(row0 + c) * D + d] = 0;
    }
    return;
  }
  const int32_t* table = a.block_tables + int64_t(s) * a.max_blocks;
  const int nlb = (ctx + BS - 1) / BS;
  const int64_t blk_stride = int64_t(a.num_kv_heads) * BS * D;
  const T* kp = static_cast<const T*>(a.k_pool) + int64_t(kvh) * BS * D;
  const T* vp = static_cast<const T*>(a.v_pool) + int64_t(kvh) * BS * D;
  const LaneMap<KV, D, BS> L(r, c);

  // start the first steps' loads before anything else
  StepRegs<KV, D> buf[NS];
#pragma unroll
  for (int i = 0; i < NS - 1; ++i)
    if (t0 + 32 * i < t1)
      load_step<KV, D, BS, NT>(buf[i], kp, vp, table, nlb, a.num_blocks, blk_stride, t0 + 32 * i,
                               L);

  // Q^T as the B operand of Q.K^T: column c = head c of the group (zero beyond the group)
  bf16x8_t qb[D / 32];
  {
    const uint16_t* q = static_cast<const uint16_t*>(a.q) + (row0 + min(c, g - 1)) * D;
#pragma unroll
    for (int i = 0; i < D / 32; ++i) {
      const uint4 w = *reinterpret_cast<const uint4*>(q + qk_dim0<KV>(i, r));
      qb[i] = as_bf16x8(c < g ? w : make_uint4(0, 0, 0, 0));
    }
  }
  floatx4_t acc[D / 16];
#pragma unroll
  for (int j = 0; j < D / 16; ++j) acc[j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
  floatx4_t lsum = {0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
  const float sl2 = a.qk_scale_log2;

  // ring of NS register buffers: step k computes from buf[k % NS] while the loads
  // of steps k+1 .. k+NS-1 are in flight
  int tt = t0;
  while (true) {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      const int tl = tt + 32 * (NS - 1);
      if (tl < t1)
        load_step<KV, D, BS, NT>(buf[(st + NS - 1) % NS], kp, vp, table, nlb, a.num_blocks,
                                 blk_stride, tl, L);
      compute_step<KV, D>(buf[st], qb, acc, lsum, m, sl2, tt, t1, r);
      tt += 32;
      if (tt >= t1) goto done;
    }
  }
done:

  if (c >= g) return;
  const float l = lsum[0];
  const float inv = a.v_scale / l;
  const int64_t row = row0 + c;
  if (nparts == 1) {
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const int d = 16 * j + 4 * r;
      uint2 w;
      w.x = pack_bf16x2(acc[j][0] * inv, acc[j][1] * inv);
      w.y = pack_bf16x2(acc[j][2] * inv, acc[j][3] * inv);
      *reinterpret_cast<uint2*>(out + row * D + d) = w;
    }
  } else {
    float* wacc = a.ws_acc + (row * a.max_parts + p) * D;
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
      const int d = 16 * j + 4 * r;
      *reinterpret_cast<float4*>(wacc + d) =
          make_float4(acc[j][0] * inv, acc[j][1] * inv, acc[j][2] * inv, acc[j][3] * inv);
    }
    if (r == 0) {
      a.ws_ml[(row * a.max_parts + p) * 2] = m;
      a.ws_ml[(row * a.max_parts + p) * 2 + 1] = l;
    }
  }
}

// ------------------------------------------------------------------------ partition merge

// out = sum_p w_p * o_p / sum_p w_p with w_p = l_p * 2^(m_p - max_p m_p): the
// same rescaling the running softmax applies between tiles.  One workgroup per
// (sequence, q head); its 256 threads split the partitions into 256/D groups.
constexpr int kMergeThreads = 256;

template <typename QT, int D>
__global__ __launch_bounds__(kMergeThreads) void merge_partitions_kernel(DecodeArgs a) {
  constexpr int PG = kMergeThreads / D;       // partition groups
  __shared__ float red[kMergeThreads];
  __shared__ float part_o[PG][D];
  __shared__ float part_l[PG];
  const int row = blockIdx.x;                 // s * Hq + h
  const int s = row / a.num_q_heads;
  const int ctx = min(a.context_lens[s], a.max_ctx);
  const int nparts = (ctx + a.part_tokens - 1) / a.part_tokens;
  if (nparts <= 1) return;                    // written directly by the decode kernel
  const int tid = threadIdx.x;
  const float* ml = a.ws_ml + int64_t(row) * a.max_parts * 2;
  float mx = -INFINITY;
  for (int p = tid; p < nparts; p += kMergeThreads) mx = fmaxf(mx, ml[2 * p]);
  red[tid] = mx;
  __syncthreads();
  for (int w = kMergeThreads / 2; w > 0; w >>= 1) {
    if (tid < w) red[tid] = fmaxf(red[tid], red[tid + w]);
    __syncthreads();
  }
  const float M = red[0];
  const int d = tid % D, pg = tid / D;
  const float* acc = a.ws_acc + int64_t(row) * a.max_parts * D + d;
  float L = 0.f, o = 0.f;
#pragma unroll 4
  for (int p = pg; p < nparts; p += PG) {
    const float w = ml[2 * p + 1] * exp2f(ml[2 * p] - M);
    L += w;
    o = fmaf(w, acc[int64_t(p) * D], o);
  }
  part_o[pg][d] = o;
  if (d == 0) part_l[pg] = L;
  __syncthreads();
  if (pg == 0) {
    float ot = 0.f, lt = 0.f;
#pragma unroll
    for (int g = 0; g < PG; ++g) {
      ot += part_o[g][d];
      lt += part_l[g];
    }
    store_out(static_cast<QT*>(a.out) + int64_t(row) * D + d, ot / lt);
  }
}

// ------------------------------------------------------------------------ host side

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int64_t parts_for(int32_t max_ctx, int32_t part) {
  if (part <= 0 || max_ctx <= 0) return 1;
  return (int64_t(max_ctx) + part - 1) / part;
}

template <typename K>
static int launch(K kernel, dim3 grid, dim3 block, hipStream_t s, const DecodeArgs& a,
                  const char* what) {
  kernel<<<grid, block, 0, s>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

template <int D, int BS>
static int dispatch_vector(const DecodeArgs& a, int kv, int qd, dim3 grid, hipStream_t s) {
  dim3 block(kVecThreads);
  if (kv == PKV_F32 && qd == PKV_F32)
    return launch(decode_vector_kernel<KV_F32, float, D, BS>, grid, block, s, a, "decode");
  if (kv == PKV_BF16 && qd == PKV_BF16)
    return launch(decode_vector_kernel<KV_BF16, uint16_t, D, BS>, grid, block, s, a, "decode");
  if (kv == PKV_FP8_E4M3 && qd == PKV_BF16)
    return launch(decode_vector_kernel<KV_FP8, uint16_t, D, BS>, grid, block, s, a, "decode");
  return fail(PKV_E_UNSUPPORTED, "q %s with a %s pool", dtype_name(qd), dtype_name(kv));
}

template <int D, int BS>
static int dispatch_mfma(const DecodeArgs& a, int kv, bool shared, dim3 grid, hipStream_t s) {
  dim3 block(64);
  if (kv == PKV_BF16)
    return shared ? launch(decode_mfma_kernel<KV_BF16, D, BS, false>, grid, block, s, a, "decode")
                  : launch(decode_mfma_kernel<KV_BF16, D, BS, true>, grid, block, s, a, "decode");
  if (kv == PKV_FP8_E4M3)
    return shared ? launch(decode_mfma_kernel<KV_FP8, D, BS, false>, grid, block, s, a, "decode")
                  : launch(decode_mfma_kernel<KV_FP8, D, BS, true>, grid, block, s, a, "decode");
  return fail(PKV_E_UNSUPPORTED, "the MFMA kernel needs a bf16 or fp8 pool");
}

template <int D>
static int dispatch_bs(const DecodeArgs& a, int bs, int kv, int qd, bool mfma, bool shared,
                       dim3 grid, hipStream_t s) {
  switch (bs) {
    case 8:
      return mfma ? dispatch_mfma<D, 8>(a, kv, shared, grid, s)
                  : dispatch_vector<D, 8>(a, kv, qd, grid, s);
    case 16:
      return mfma ? dispatch_mfma<D, 16>(a, kv, shared, grid, s)
                  : dispatch_vector<D, 16>(a, kv, qd, grid, s);
    case 32:
      return mfma ? dispatch_mfma<D, 32>(a, kv, shared, grid, s)
                  : dispatch_vector<D, 32>(a, kv, qd, grid, s);
  }
  return fail(PKV_E_UNSUPPORTED, "block_size %d", bs);
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_context_len,
                                             int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0) return 0;
  const int64_t P = parts_for(max_context_len, partition_size);
  if (P <= 1) return 0;
  const int64_t rows = int64_t(num_seqs) * num_q_heads * P;
  const size_t ml = size_t(rows) * 2 * sizeof(float);
  const size_t ml_padded = (ml + 255) & ~size_t(255);
  return ml_padded + size_t(rows) * head_dim * sizeof(float);
}

// Validate the arguments of a decode call and fill the kernel arguments.
static int prepare(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                   const pkv_cache_desc* c, const int32_t* block_tables,
                   int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                   int32_t num_q_heads, float scale, void* out, int32_t max_context_len,
                   int32_t partition_size, void* workspace, size_t workspace_bytes,
                   DecodeArgs* a, int64_t* parts) {
  int rc = check_desc(c);
  if (rc) return rc;
  if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq < 0 || max_context_len < 0)
    return fail(PKV_E_INVAL, "negative size");
  if (num_q_heads % c->num_kv_heads)
    return fail(PKV_E_INVAL, "num_q_heads %d is not a multiple of num_kv_heads %d", num_q_heads,
                c->num_kv_heads);
  const int group = num_q_heads / c->num_kv_heads;
  if (group > kMaxGroup) return fail(PKV_E_UNSUPPORTED, "group size %d > %d", group, kMaxGroup);
  if (!std::isfinite(scale)) return fail(PKV_E_INVAL, "scale is not finite");
  if (partition_size < 0 || (partition_size % c->block_size))
    return fail(PKV_E_INVAL, "partition_size %d is not a non-negative multiple of block_size %d",
                partition_size, c->block_size);
  if (int64_t(max_blocks_per_seq) * c->block_size < max_context_len)
    return fail(PKV_E_INVAL, "max_blocks_per_seq %d cannot hold max_context_len %d",
                max_blocks_per_seq, max_context_len);
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16)
    return fail(PKV_E_INVAL, "q_dtype must be f32 or bf16");
  if ((c->kv_dtype == PKV_F32) != (q_dtype == PKV_F32))
    return fail(PKV_E_UNSUPPORTED, "q %s with a %s pool", dtype_name(q_dtype),
                dtype_name(c->kv_dtype));
  const int64_t P = parts_for(max_context_len, partition_size);
  *parts = P;
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return fail(PKV_E_INVAL, "NULL pointer");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return fail(PKV_E_INVAL, "device pointers must be 16-byte aligned");
  const size_t need = pkv_decode_workspace_bytes(num_seqs, num_q_heads, c->head_dim,
                                                 max_context_len, partition_size);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return fail(PKV_E_INVAL, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  const int64_t items = int64_t(num_seqs) * c->num_kv_heads * P;
  if (items > 0x7fffffff) return fail(PKV_E_INVAL, "grid too large");
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->out = out;
  const int64_t rows = int64_t(num_seqs) * num_q_heads * P;
  a->ws_ml = need ? static_cast<float*>(workspace) : nullptr;
  a->ws_acc = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                              ((size_t(rows) * 2 * sizeof(float) + 255) &
                                               ~size_t(255)))
                   : nullptr;
  a->max_blocks = max_blocks_per_seq;
  a->num_seqs = num_seqs;
  a->num_q_heads = num_q_heads;
  a->num_kv_heads = c->num_kv_heads;
  a->group = group;
  a->num_blocks = c->num_blocks;
  a->max_ctx = max_context_len;
  a->part_tokens = P > 1 ? partition_size : 0;
  a->max_parts = int32_t(P);
  a->qk_scale_log2 = scale * kLog2e * (c->kv_dtype == PKV_FP8_E4M3 ? c->k_scale : 1.f);
  a->v_scale = c->kv_dtype == PKV_FP8_E4M3 ? c->v_scale : 1.f;
  return PKV_OK;
}

static int launch_partials(const DecodeArgs& a, const pkv_cache_desc* c, int32_t q_dtype,
                           int64_t P, int32_t impl, hipStream_t s) {
  const int family = impl & PKV_IMPL_FAMILY_MASK;
  const bool shared = (impl & PKV_IMPL_SHARED_BLOCKS) != 0;
  if (impl & ~(PKV_IMPL_FAMILY_MASK | PKV_IMPL_SHARED_BLOCKS))
    return fail(PKV_E_INVAL, "unknown impl flags 0x%x", impl);
  bool mfma;
  if (family == PKV_IMPL_AUTO) mfma = c->kv_dtype != PKV_F32;
  else if (family == PKV_IMPL_VECTOR) mfma = false;
  else if (family == PKV_IMPL_MFMA) {
    if (c->kv_dtype == PKV_F32) return fail(PKV_E_UNSUPPORTED, "no MFMA kernel for an f32 pool");
    mfma = true;
  } else {
    return fail(PKV_E_INVAL, "unknown kernel family %d", family);
  }
  const dim3 grid(static_cast<unsigned>(int64_t(a.num_seqs) * a.num_kv_heads * P));
  return c->head_dim == 64
             ? dispatch_bs<64>(a, c->block_size, c->kv_dtype, q_dtype, mfma, shared, grid, s)
             : dispatch_bs<128>(a, c->block_size, c->kv_dtype, q_dtype, mfma, shared, grid, s);
}

static int launch_merge(const DecodeArgs& a, int32_t head_dim, int32_t q_dtype, hipStream_t s) {
  const dim3 mgrid(static_cast<unsigned>(int64_t(a.num_seqs) * a.num_q_heads));
  if (head_dim == 64)
    return q_dtype == PKV_F32
               ? launch(merge_partitions_kernel<float, 64>, mgrid, dim3(kMergeThreads), s, a, "merge")
               : launch(merge_partitions_kernel<uint16_t, 64>, mgrid, dim3(kMergeThreads), s, a, "merge");
  return q_dtype == PKV_F32
             ? launch(merge_partitions_kernel<float, 128>, mgrid, dim3(kMergeThreads), s, a, "merge")
             : launch(merge_partitions_kernel<uint16_t, 128>, mgrid, dim3(kMergeThreads), s, a, "merge");
}

extern "C" int pkv_paged_attn_partials(const void* q, int32_t q_dtype, const void* k_pool,
                                       const void* v_pool, const pkv_cache_desc* c,
                                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_q_heads, float scale, void* out,
                                       int32_t max_context_len, int32_t partition_size,
                                       void* workspace, size_t workspace_bytes, void* stream,
                                       int32_t impl) {
  clear_error();
  DecodeArgs a;
  int64_t P = 1;
  int rc = prepare(q, q_dtype, k_pool, v_pool, c, block_tables, max_blocks_per_seq, context_lens,
                   num_seqs, num_q_heads, scale, out, max_context_len, partition_size, workspace,
                   workspace_bytes, &a, &P);
  if (rc || num_seqs == 0) return rc;
  return launch_partials(a, c, q_dtype, P, impl, static_cast<hipStream_t>(stream));
}

extern "C" int pkv_paged_attn_merge(int32_t q_dtype, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                    int32_t max_context_len, int32_t partition_size,
                                    const void* workspace, size_t workspace_bytes, void* out,
                                    void* stream) {
  clear_error();
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || partition_size < 0)
    return fail(PKV_E_INVAL, "negative size");
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_E_UNSUPPORTED, "head_dim %d not built (64, 128)", head_dim);
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16) return fail(PKV_E_INVAL, "bad q_dtype");
  const int64_t P = parts_for(max_context_len, partition_size);
  if (P <= 1 || num_seqs == 0) return PKV_OK;  // nothing was split
  const size_t need =
      pkv_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_context_len, partition_size);
  if (!workspace || workspace_bytes < need || !aligned16(workspace))
    return fail(PKV_E_INVAL, "workspace of %zu bytes needed (got %zu)", need, workspace_bytes);
  if (!context_lens || !out || !aligned16(out)) return fail(PKV_E_INVAL, "bad pointer");
  if (int64_t(num_seqs) * num_q_heads > 0x7fffffff) return fail(PKV_E_INVAL, "grid too large");
  DecodeArgs a = {};
  const int64_t rows = int64_t(num_seqs) * num_q_heads * P;
  a.context_lens = context_lens;
  a.out = out;
  a.ws_ml = static_cast<float*>(const_cast<void*>(workspace));
  a.ws_acc = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(workspace)) +
                                      ((size_t(rows) * 2 * sizeof(float) + 255) & ~size_t(255)));
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.max_ctx = max_context_len;
  a.part_tokens = partition_size;
  a.max_parts = int32_t(P);
  return launch_merge(a, head_dim, q_dtype, static_cast<hipStream_t>(stream));
}

extern "C" int pkv_paged_attn_decode_ex(const void* q, int32_t q_dtype, const void* k_pool,
                                        const void* v_pool, const pkv_cache_desc* c,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, float scale, void* out,
                                        int32_t max_context_len, int32_t partition_size,
                                        void* workspace, size_t workspace_bytes, void* stream,
                                        int32_t impl) {
  clear_error();
  DecodeArgs a;
  int64_t P = 1;
  int rc = prepare(q, q_dtype, k_pool, v_pool, c, block_tables, max_blocks_per_seq, context_lens,
                   num_seqs, num_q_heads, scale, out, max_context_len, partition_size, workspace,
                   workspace_bytes, &a, &P);
  if (rc || num_seqs == 0) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  rc = launch_partials(a, c, q_dtype, P, impl, s);
  if (rc || P <= 1) return rc;
  return launch_merge(a, c->head_dim, q_dtype, s);
}

extern "C" int pkv_paged_attn_decode(const void* q, int32_t q_dtype, const void* k_pool,
                                     const void* v_pool, const pkv_cache_desc* c,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_q_heads, float scale, void* out,
                                     int32_t max_context_len, int32_t partition_size,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return pkv_paged_attn_decode_ex(q, q_dtype, k_pool, v_pool, c, block_tables, max_blocks_per_seq,
                                  context_lens, num_seqs, num_q_heads, scale, out, max_context_len,
                                  partition_size, workspace, workspace_bytes, stream,
                                  PKV_IMPL_AUTO);
}
