// Paged decode attention: one new query per sequence attends over its cached
// keys and values, read block by block through the sequence's block table
// (ultralytics glossary "PagedAttention", section "How paging works";
// optiverse blog "paged-kv-cache", section "Block table and non-contiguous
// allocation").  The score matrix is never written out: scores are folded
// into a running max / running sum / running output as in FlashAttention-style
// tiled attention (glossary, "Related techniques").  Query heads share KV heads
// in contiguous groups (grouped-query attention, same section).
//
// Two kernel families:
//  * decode_mfma_kernel (bf16 / fp8 pools).  The contexts of all (sequence,
//    KV head) pairs are laid end to end as one stream of 32-token steps, cut
//    into equal contiguous ranges, one per persistent wave64 worker, so every
//    worker reads the same amount of KV whatever the context lengths.  Each
//    worker finds its own range from the context lengths (a wave-wide prefix
//    sum) and walks it with a ring of register buffers that keeps the next
//    steps' loads in flight across context boundaries; Q.K^T and P.V of the
//    whole head group are 16x16x32 bf16 MFMAs (group padded to 16 columns),
//    with P rounded to bf16.  Each piece of a context a worker covers
//    ("segment") ends with (running max, running sum, normalised output); a
//    context covered by one segment writes its output directly, the others
//    are combined by merge_kernel.
//  * decode_vector_kernel (any pool dtype): a plain, fp32-arithmetic kernel
//    with LDS staging, one workgroup per (sequence, KV head, partition of
//    partition_size tokens); the f32 path and a cross-check of the MFMA kernel.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>
#include <unordered_map>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxWorkers = 4096;     // persistent workers (wave64) at most
constexpr int kProtoPartitions = 0;   // workspace rows are (row, partition)
constexpr int kProtoSegments = 1;     // workspace rows are (segment, head of group)

struct DecodeArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  int32_t* hdr;         // [0] which kernel wrote the partial rows
  int2* recs;           // per (sequence, KV head) pair: {first worker, workers} (MFMA kernel)
  float* ws_ml;         // partial (running max in log2 units, running sum) rows
  float* ws_acc;        // partial normalised outputs, D floats per row
  int32_t max_blocks;   // row stride of block_tables
  int32_t num_seqs;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;        // num_q_heads / num_kv_heads
  int32_t num_blocks;   // pool blocks (block ids outside [0, num_blocks) are skipped)
  int32_t max_ctx;      // contexts are cut at this host-known bound
  int32_t part_tokens;  // vector kernel: partition length (0 = whole context);
                        // MFMA kernel: least tokens per worker while at least
                        // half the workers get steps (0 = balance only)
  int32_t max_parts;    // vector kernel: partitions of the longest context
  int32_t workers;      // MFMA kernel: persistent workers launched
  float qk_scale_log2;  // scale * log2(e) * k_scale
  float v_scale;
  // shared-prefix decode only
  const int4* rows;     // [num_rows] units {first sequence, shared tokens, members, 0}
  const int4* seq_rows; // [num_seqs] {unit, member index, 0, 0}
  int32_t num_rows;
  int32_t block_size;
};

// Partitions of a context of ctx tokens for the vector kernel: max(1, ctx / P),
// the last one taking the remainder; none for an empty context.
__host__ __device__ __forceinline__ int num_parts(int ctx, int part) {
  if (ctx <= 0) return 0;
  if (part <= 0) return 1;
  const int n = ctx / part;
  return n > 1 ? n : 1;
}

__device__ __forceinline__ int part_end(int p, int np, int ctx, int part) {
  return (part <= 0 || p == np - 1) ? ctx : (p + 1) * part;
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
// Query columns of a shared-prefix unit: two 16-column matrix-core tiles, so
// that up to 32 / group forked samples read their shared blocks once.
constexpr int kUnitCols = 32;

// Four consecutive pool elements as floats, with one 16-, 8- or 4-byte load (p is
// 4-element aligned; fp8 without its scale).
template <int KV>
__device__ __forceinline__ float4 load4_f32(const typename KvTraits<KV>::T* p) {
  if constexpr (KV == KV_F32) {
    return *reinterpret_cast<const float4*>(p);
  } else if constexpr (KV == KV_BF16) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(bf16_to_f32(u.x & 0xffffu), bf16_to_f32(u.x >> 16),
                       bf16_to_f32(u.y & 0xffffu), bf16_to_f32(u.y >> 16));
  } else {
    const uint32_t u = *reinterpret_cast<const uint32_t*>(p);
    return make_float4(e4m3_to_f32(u & 0xffu), e4m3_to_f32((u >> 8) & 0xffu),
                       e4m3_to_f32((u >> 16) & 0xffu), e4m3_to_f32(u >> 24));
  }
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

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
  if (wid == 0 && tid == 0) a.hdr[0] = kProtoPartitions;
  const int ctx = min(a.context_lens[s], a.max_ctx);
  const int nparts = num_parts(ctx, a.part_tokens);
  QT* out = static_cast<QT*>(a.out);
  if (p >= nparts) {
    if (p == 0) {  // empty context: zeros
      for (int i = tid; i < g * D; i += kVecThreads)
        store_out(out + (int64_t(s) * a.num_q_heads + kvh * g + i / D) * D + i % D, 0.f);
    }
    return;
  }
  const int t0 = p * a.part_tokens;
  const int t1 = part_end(p, nparts, ctx, a.part_tokens);
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
        for (int d = 0; d < D; d += 4) {
          const float4 kv = load4_f32<KV>(krow + d);
#pragma unroll
          for (int h = 0; h < kMaxGroup; ++h) {
            if (h < g) {
              dots[h] = fmaf(q_s[h][d], kv.x, dots[h]);
              dots[h] = fmaf(q_s[h][d + 1], kv.y, dots[h]);
              dots[h] = fmaf(q_s[h][d + 2], kv.z, dots[h]);
              dots[h] = fmaf(q_s[h][d + 3], kv.w, dots[h]);
            }
          }
        }
      }
#pragma unroll
      for (int h = 0; h < kMaxGroup; ++h)
        if (h < g) p_s[h][tid] = ok ? dots[h] * a.qk_scale_log2 : -INFINITY;
    }
    __syncthreads();
    // running max and weights: one wave per head, the chunk's tokens over its lanes
    {
      const int wv = tid >> 6, ln = tid & 63;
      for (int h = wv; h < g; h += kVecThreads / 64) {
        const float m0 = m_s[h];
        float lm = -INFINITY;
        for (int i = ln; i < n; i += 64) lm = fmaxf(lm, p_s[h][i]);
        const float mx = fmaxf(m0, wave_max_f(lm));
        const float alpha = mx == -INFINITY ? 1.f : exp2f(m0 - mx);
        float sum = 0.f;
        for (int i = ln; i < n; i += 64) {
          const float w = mx == -INFINITY ? 0.f : exp2f(p_s[h][i] - mx);
          p_s[h][i] = w;
          sum += w;
        }
        sum = wave_sum_f(sum);
        if (ln == 0) {
          l_s[h] = l_s[h] * alpha + sum;
          m_s[h] = mx;
          alpha_s[h] = alpha;
        }
      }
    }
    __syncthreads();
    // P.V: thread per (head, dimension), four tokens of the dimension's row per load
    // (cs and i are multiples of 4 and the block size is); a token with weight 0 (masked,
    // or past the chunk) adds nothing, whatever its slot holds
    for (int idx = tid; idx < g * D; idx += kVecThreads) {
      const int h = idx / D, d = idx % D;
      float acc = acc_s[h][d] * alpha_s[h];
      for (int i = 0; i < n; i += 4) {
        const int pb = blk_s[i / BS];
        if (pb >= 0 && pb < a.num_blocks) {
          const float4 v4 = load4_f32<KV>(vp + (int64_t(pb) * a.num_kv_heads + kvh) * head_stride +
                                          int64_t(d) * BS + (cs + i) % BS);
          const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float w = i + e < n ? p_s[h][i + e] : 0.f;
            acc = w != 0.f ? fmaf(w, vv[e], acc) : acc;
          }
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

// Per-lane registers of one 32-token step; NQ 16-column query tiles.
template <int KV, int D, int NQ>
struct StepRegs {
  static constexpr int NK = KV == KV_FP8 ? D / 64 : D / 32;  // 16-byte K loads per tile
  uint4 ka[NK];   // K rows, tile a (MFMA A operand of Q.K^T)
  uint4 kb[NK];   // K rows, tile b
  typename std::conditional<KV == KV_FP8, uint2, uint4>::type v[D / 16];  // V^T, 8 tokens x 1 dim
  uint4 q[NQ][D / 32];  // Q^T of the pair's columns, loaded with a pair's first step only
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

// Block `which` of the step's 32 / BS blocks (uniform values, a lane-dependent
// choice).  Each block id goes through readfirstlane (free: it is uniform)
// before the selects, so the compiler cannot fold the choice into an indexed
// load, which would put the array in scratch memory.
template <int BS>
__device__ __forceinline__ int pick_block(const int (&pbs)[32 / BS], int which) {
  int v[32 / BS];
#pragma unroll
  for (int b = 0; b < 32 / BS; ++b) v[b] = __builtin_amdgcn_readfirstlane(pbs[b]);
  if constexpr (32 / BS == 1) {
    return v[0];
  } else if constexpr (32 / BS == 2) {
    return (which & 1) ? v[1] : v[0];
  } else {
    static_assert(32 / BS == 4, "block sizes 8, 16, 32");
    const int lo = (which & 1) ? v[1] : v[0];
    const int hi = (which & 1) ? v[3] : v[2];
    return (which & 2) ? hi : lo;
  }
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

// Rescaling threshold (log2 units): the running reference max is only raised
// when a score exceeds it by more than this, so weights stay below 2^8.
constexpr float kRescaleLog2 = 8.0f;

template <int KV, int D, class Regs>
__device__ __forceinline__ void compute_step(const Regs& R, const uint4 (&qv)[D / 32],
                                             floatx4_t (&acc)[D / 16],
                                             floatx4_t& lsum, float& m, float sl2, int tt, int t1,
                                             int r, bool active) {
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
    sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, as_bf16x8(qv[i]), sa, 0, 0, 0);
    sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kb, as_bf16x8(qv[i]), sb, 0, 0, 0);
  }
  // lane (r, c): x[e] = score of head c for token 8r + e of the step, in log2
  // units (scaled first, so the running max below is the max of the scaled
  // scores whatever the sign of the scale)
  float x[8] = {sa[0] * sl2, sa[1] * sl2, sa[2] * sl2, sa[3] * sl2,
                sb[0] * sl2, sb[1] * sl2, sb[2] * sl2, sb[3] * sl2};
  const bool tail = tt + 32 > t1;
  if (tail) {
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (tt + 8 * r + e >= t1) x[e] = -INFINITY;
  }
  // a query column that does not attend these tokens (shared-prefix decode)
  if (!active) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = -INFINITY;
  }
  float lmax = x[0];
#pragma unroll
  for (int e = 1; e < 8; ++e) lmax = fmaxf(lmax, x[e]);
  // raise the reference max (and rescale what was summed so far) only when needed
  if (__builtin_amdgcn_ballot_w64(lmax > m + kRescaleLog2)) {
    float cmax = fmaxf(lmax, __shfl_xor(lmax, 16));
    cmax = fmaxf(cmax, __shfl_xor(cmax, 32));
    const float m_new = fmaxf(m, cmax);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[j] *= alpha;
    lsum *= alpha;
    m = m_new;
  }
  uint32_t pw[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2)
    pw[e / 2] = pack_bf16x2(__builtin_amdgcn_exp2f(x[e] - m), __builtin_amdgcn_exp2f(x[e + 1] - m));
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
// computes) and the waves per SIMD the register budget is sized for.  bf16: two
// steps (32 KB per wave, 32 MB over 1024 waves); three or four steps in flight
// ran 0.3% (8B-like layer) to 7% (one 32k context, the multi-query layer)
// slower, and two waves per SIMD with two steps each slower still.
#ifndef PKV_BF16_STAGES
#define PKV_BF16_STAGES 2
#endif
#ifndef PKV_BF16_WAVES
#define PKV_BF16_WAVES 1
#endif
#ifndef PKV_FP8_STAGES
#define PKV_FP8_STAGES 2
#endif
#ifndef PKV_FP8_WAVES
#define PKV_FP8_WAVES 2
#endif
// Two query tiles (the shared-prefix decode) need registers for a second set of
// scores, weights, accumulators and queries: fp8 then runs one wave per SIMD,
// with three steps in flight (four would spill registers).
template <int KV, int NQ>
struct MfmaTuning {
  static constexpr int stages =
      KV == KV_FP8 ? (NQ == 1 ? PKV_FP8_STAGES : 3) : PKV_BF16_STAGES;
  static constexpr int waves = KV == KV_FP8 ? (NQ == 1 ? PKV_FP8_WAVES : 1) : PKV_BF16_WAVES;
};

// Physical blocks of the step at tokens tt .. tt+31 of a context of t1 tokens
// whose table row is `table`.  The part of the step past the context (masked
// tokens) reads the context's last block again: the same lines the step
// already reads.  (Reading one fixed block there instead made every worker's
// last step of every context hit the same few DRAM pages at once.)  Ids
// outside the pool read block 0.
template <int BS>
__device__ __forceinline__ void step_blocks(int (&pbs)[32 / BS], const int32_t* __restrict__ table,
                                            int tt, int t1, int num_blocks) {
  const int last = (t1 + BS - 1) / BS - 1;
#pragma unroll
  for (int b = 0; b < 32 / BS; ++b) {
    // a block past the context's last one holds only masked tokens: it repeats the last
    // block, whose lines the same step loads anyway
    const int pb = table[min(tt / BS + b, last)];
    pbs[b] = (pb >= 0 && pb < num_blocks) ? pb : 0;
  }
}

// 16 bytes of the query through a buffer descriptor over the whole q tensor.
// An offset at or past the descriptor's size reads zeros without touching
// memory, which gives the padding columns of the head group a zero query
// with the same instruction (no branch).
__device__ __forceinline__ uint4 ld16_q(__amdgpu_buffer_rsrc_t rsrc, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, 0));
}

// Q^T of one (sequence, KV head) pair's head group, the B operand of Q.K^T:
// lane (r, c) holds the dimensions qk_dim0(i, r) .. +7 of query head c.  Only
// lanes of real heads read the query (the group is padded to 16 MFMA
// columns); the padding columns get a zero query, and their results are
// computed and never written.
template <int KV, int D>
__device__ __forceinline__ void load_query(uint4 (&qv)[D / 32], __amdgpu_buffer_rsrc_t qrsrc,
                                           uint32_t qoff, bool qlane, uint32_t qoob, int r) {
#pragma unroll
  for (int i = 0; i < D / 32; ++i)
    qv[i] = ld16_q(qrsrc, qlane ? qoff + 2u * uint32_t(qk_dim0<KV>(i, r)) : qoob);
}

// Issue the loads of one step: the pair's query tiles when the step is the
// first the worker computes of that pair, then K rows, then V^T columns.
template <int KV, int D, int BS, bool NT, int NQ>
__device__ __forceinline__ void issue_step(StepRegs<KV, D, NQ>& R,
                                           const typename KvTraits<KV>::T* kp,
                                           const typename KvTraits<KV>::T* vp,
                                           const int (&pbs)[32 / BS], int64_t blk_stride,
                                           const LaneMap<KV, D, BS>& L, bool with_q,
                                           __amdgpu_buffer_rsrc_t qrsrc,
                                           const uint32_t (&qoff)[NQ], const bool (&qlane)[NQ],
                                           uint32_t qoob, int r) {
  if (with_q) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) load_query<KV, D>(R.q[t], qrsrc, qoff[t], qlane[t], qoob, r);
  }
  const auto* ka = kp + int64_t(pick_block<BS>(pbs, L.ka_blk)) * blk_stride + L.ka_off;
  const auto* kb = kp + int64_t(pick_block<BS>(pbs, L.kb_blk)) * blk_stride + L.kb_off;
  const auto* vb = vp + int64_t(pick_block<BS>(pbs, L.v_blk)) * blk_stride + L.v_off;
#pragma unroll
  for (int i = 0; i < StepRegs<KV, D, NQ>::NK; ++i) {
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

// A position in the step stream: pair (unit s, KV head kvh), step x of the
// pair's n steps, P the pair's first step in the stream.  The stream orders
// pairs by unit, then KV head.  In the plain decode a unit is one sequence.
// In the shared-prefix decode a unit is a family of M consecutive sequences
// seq0 .. seq0 + M - 1 whose first T tokens sit in the same blocks: its steps
// are the shared span [0, T), read through seq0's table with every member's
// query columns active, then each member's own span [T, its context), read
// through its own table with only its columns active.  The current span
// (sub = -1 shared, else the member): table row seq, first token tb, tokens
// ctx, pair steps [x0, xe).
struct Cursor {
  int s, kvh, x, P, n;
  int seq, tb, ctx, x0, xe;
  int seq0, M, T, sub;
};

__device__ __forceinline__ int clamp_ctx(int len, int max_ctx) { return max(0, min(len, max_ctx)); }
__device__ __forceinline__ int ctx_steps(int ctx) { return (ctx + 31) >> 5; }

// Sequence whose context length a unit descriptor needs first (a valid index).
__device__ __forceinline__ int row_seq(const DecodeArgs& a, int4 d) {
  return (d.x >= 0 && d.x < a.num_seqs) ? d.x : 0;
}

// Unit of descriptor d {first sequence, shared tokens, members, reread} given
// the first sequence's context length len0: members cut to the kUnitCols query
// columns and to the batch, shared tokens to whole blocks of the first member's
// context.  An out-of-range first sequence gives a unit without members.
__device__ __forceinline__ void unit_of(const DecodeArgs& a, int4 d, int len0, int& seq0, int& M,
                                        int& T) {
  if (d.x < 0 || d.x >= a.num_seqs) {
    seq0 = 0;
    M = 0;
    T = 0;
    return;
  }
  seq0 = d.x;
  M = max(1, min(min(d.z, kUnitCols / a.group), a.num_seqs - d.x));
  T = min(max(0, d.y), clamp_ctx(len0, a.max_ctx)) & ~(a.block_size - 1);
}

// Unit d's fields and the steps of one of its KV heads: the shared span, then
// every member's own.  The members' lengths are requested eight at a time, all
// of a batch before any is used (a loop over M would wait for each load in
// turn); the first batch holds the first member's, which fixes the unit.
__device__ __forceinline__ int unit_load(const DecodeArgs& a, int4 d,
                                         const int32_t* __restrict__ lens, int& seq0, int& M,
                                         int& T) {
  constexpr int kBatch = 8;
  const int first = row_seq(a, d);
  int len[kBatch];
#pragma unroll
  for (int k = 0; k < kBatch; ++k) len[k] = lens[min(first + k, a.num_seqs - 1)];
  unit_of(a, d, len[0], seq0, M, T);
  int n = ctx_steps(T);
  for (int m0 = 0;;) {
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
      n += m0 + k < M ? ctx_steps(max(0, clamp_ctx(len[k], a.max_ctx) - T)) : 0;
    m0 += kBatch;
    if (m0 >= M) break;
#pragma unroll
    for (int k = 0; k < kBatch; ++k) len[k] = lens[min(first + m0 + k, a.num_seqs - 1)];
  }
  return n;
}

// Enter span cu.sub of the unit, whose first step is pair step cu.x0.
__device__ __forceinline__ void enter_span(Cursor& cu, const DecodeArgs& a,
                                           const int32_t* __restrict__ lens) {
  if (cu.sub < 0) {
    cu.seq = cu.seq0;
    cu.tb = 0;
    cu.ctx = cu.T;
  } else {
    cu.seq = cu.seq0 + cu.sub;
    cu.tb = cu.T;
    cu.ctx = max(0, clamp_ctx(lens[cu.seq], a.max_ctx) - cu.T);
  }
  cu.xe = cu.x0 + ctx_steps(cu.ctx);
}

// Move on to the span that holds pair step cu.x (the pair has that step):
// from the first span, or from the one after the current.
__device__ __forceinline__ void seek_span(Cursor& cu, const DecodeArgs& a,
                                          const int32_t* __restrict__ lens) {
  cu.sub = -1;
  cu.x0 = 0;
  enter_span(cu, a, lens);
  while (cu.x >= cu.xe) {
    cu.x0 = cu.xe;
    ++cu.sub;
    enter_span(cu, a, lens);
  }
}
__device__ __forceinline__ void next_span(Cursor& cu, const DecodeArgs& a,
                                          const int32_t* __restrict__ lens) {
  do {
    cu.x0 = cu.xe;
    ++cu.sub;
    enter_span(cu, a, lens);
  } while (cu.x >= cu.xe);
}

// The unit fields and the span of pair step cu.x, from the unit's descriptor
// and its members' lengths (len[m] of sequence d.x + m).
__device__ __forceinline__ void walk_unit(Cursor& cu, const DecodeArgs& a, int4 d,
                                          const int (&len)[kUnitCols]) {
  unit_of(a, d, len[0], cu.seq0, cu.M, cu.T);
  cu.sub = -1;
  cu.seq = cu.seq0;
  cu.tb = 0;
  cu.ctx = cu.T;
  cu.x0 = 0;
  cu.xe = ctx_steps(cu.T);
#pragma unroll
  for (int m = 0; m < kUnitCols; ++m) {
    if (m < cu.M && cu.x >= cu.xe) {
      cu.sub = m;
      cu.seq = cu.seq0 + m;
      cu.tb = cu.T;
      cu.ctx = max(0, clamp_ctx(len[m], a.max_ctx) - cu.T);
      cu.x0 = cu.xe;
      cu.xe += ctx_steps(cu.ctx);
    }
  }
}

// The cursor at step x of the pair of unit s, KV head kvh (fields s, kvh, x,
// P, n already set).
template <bool ROWS>
__device__ __forceinline__ void enter_unit(Cursor& cu, const DecodeArgs& a,
                                           const int4* __restrict__ rows,
                                           const int32_t* __restrict__ lens) {
  if constexpr (ROWS) {
    // the members' lengths requested together, then the spans walked in registers
    // (a walk span by span would wait for one length after another)
    const int4 d = rows[cu.s];
    const int first = row_seq(a, d);
    int len[kUnitCols];
#pragma unroll
    for (int m = 0; m < kUnitCols; ++m) len[m] = lens[min(first + m, a.num_seqs - 1)];
    walk_unit(cu, a, d, len);
  } else {
    cu.seq0 = cu.seq = cu.s;
    cu.M = 1;
    cu.T = 0;
    cu.sub = 0;
    cu.tb = 0;
    cu.x0 = 0;
    cu.ctx = clamp_ctx(lens[cu.s], a.max_ctx);
    cu.xe = cu.n;
  }
}

// Move to the next pair that has steps; the caller knows there is one.
template <bool ROWS>
__device__ __forceinline__ void next_pair(Cursor& cu, const DecodeArgs& a,
                                          const int4* __restrict__ rows,
                                          const int32_t* __restrict__ lens, int hkv,
                                          int max_ctx) {
  cu.P += cu.n;
  cu.x = 0;
  if (++cu.kvh < hkv) {
    if constexpr (ROWS) seek_span(cu, a, lens);
    return;
  }
  cu.kvh = 0;
  if constexpr (ROWS) {
    do {
      ++cu.s;
      cu.n = unit_load(a, rows[cu.s], lens, cu.seq0, cu.M, cu.T);
    } while (cu.n == 0);
    seek_span(cu, a, lens);
  } else {
    do {
      ++cu.s;
      cu.seq = cu.seq0 = cu.s;
      cu.ctx = clamp_ctx(lens[cu.s], max_ctx);
    } while (cu.ctx == 0);
    cu.n = ctx_steps(cu.ctx);
    cu.xe = cu.n;
  }
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int t = __shfl_up(v, o);
    if (lane >= o) v += t;
  }
  return v;
}

// Steps of unit (or sequence) i, for the scan in find_start.
template <bool ROWS>
__device__ __forceinline__ int unit_steps(const DecodeArgs& a, const int4* __restrict__ rows,
                                          const int32_t* __restrict__ lens, int i) {
  if constexpr (ROWS) {
    int seq0, M, T;
    return unit_load(a, rows[i], lens, seq0, M, T);
  } else {
    return ctx_steps(clamp_ctx(lens[i], a.max_ctx));
  }
}

// Every worker derives the split itself from the context lengths (the wave's
// results are made uniform so the cursor lives in scalar registers): the
// stream's length `total`, the steps per worker `q` (equal for all, at least
// part_tokens / 32) and the cursor at its own first step w * q.  False when
// worker w has no steps.
template <bool ROWS>
__device__ __forceinline__ bool find_start(const DecodeArgs& a, const int4* __restrict__ rows,
                                           const int32_t* __restrict__ lens, int w, int lane,
                                           int& total, int& q, Cursor& cu) {
  const int S = ROWS ? a.num_rows : a.num_seqs, hkv = a.num_kv_heads;
  int sum = 0;
  int v[4];   // steps of the units of the last chunk (all of them when S <= 256)
  int cx[4] = {0, 0, 0, 0};   // plain decode: their context lengths (cut to max_ctx)
  // Shared-prefix decode with at most 64 units: lane i's unit and its members'
  // lengths stay in registers, and the worker's cursor is read from the lane
  // that holds its unit instead of loading them again.
  int4 dk = make_int4(0, 0, 0, 0);
  int lk[kUnitCols];
  const bool few = ROWS && S <= 64;
  if (few) {
    dk = rows[min(lane, S - 1)];
    const int first = row_seq(a, dk);
#pragma unroll
    for (int m = 0; m < kUnitCols; ++m) lk[m] = lens[min(first + m, a.num_seqs - 1)];
    int seq0, M, T;
    unit_of(a, dk, lk[0], seq0, M, T);
    int n = ctx_steps(T);
#pragma unroll
    for (int m = 0; m < kUnitCols; ++m)
      n += m < M ? ctx_steps(max(0, clamp_ctx(lk[m], a.max_ctx) - T)) : 0;
    v[0] = lane < S ? n : 0;
    v[1] = v[2] = v[3] = 0;
    sum = v[0];
  }
  for (int s0 = 0; s0 < (few ? 0 : S); s0 += 256) {
    // every load of the chunk is requested before any is used
    if constexpr (ROWS) {
      int4 d[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) d[u] = rows[min(s0 + 64 * u + lane, S - 1)];  // unconditional
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        int seq0, M, T;
        const int n = unit_load(a, d[u], lens, seq0, M, T);
        v[u] = s0 + 64 * u + lane < S ? n : 0;
      }
    } else {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int s = s0 + 64 * u + lane;
        cx[u] = s < S ? clamp_ctx(lens[s], a.max_ctx) : 0;
        v[u] = ctx_steps(cx[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) sum += v[u];
  }
  total = __builtin_amdgcn_readfirstlane(wave_sum(sum)) * hkv;
  // Steps per worker: an even share, or more when partition_size asks for longer
  // pieces, but never so many that fewer than half the workers get steps (a short
  // stream over a few workers runs at their latency, not at the memory's rate).
  const int q_even = (total + a.workers - 1) / a.workers;
  const int q_half = (2 * total + a.workers - 1) / a.workers;
  q = max(q_even, min(max(1, a.part_tokens >> 5), q_half));
  if (int64_t(w) * q >= total) return false;
  const int target = w * q;
  int base = 0;  // steps of one KV head of the units before the chunk
  for (int s0 = 0; s0 < S; s0 += 64) {
    const int s = s0 + lane;
    // a batch of one chunk reuses the counts above (the selects keep v in registers)
    const int n = S <= 256 ? (s0 == 0 ? v[0] : s0 == 64 ? v[1] : s0 == 128 ? v[2] : v[3])
                           : s < S ? unit_steps<ROWS>(a, rows, lens, s) : 0;
    const int incl = wave_inclusive_scan(n, lane);
    const uint64_t hit = __ballot(hkv * (base + incl) > target);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      const int ns = __builtin_amdgcn_readfirstlane(__shfl(n, l));
      const int first = hkv * (base + __builtin_amdgcn_readfirstlane(__shfl(incl, l)) - ns);
      cu.s = s0 + l;
      cu.kvh = (target - first) / ns;
      cu.x = target - first - cu.kvh * ns;
      cu.n = ns;
      cu.P = first + cu.kvh * ns;
      if (!ROWS && S <= 256) {
        // the context length is in lane l's registers: no second load of it
        const int c = s0 == 0 ? cx[0] : s0 == 64 ? cx[1] : s0 == 128 ? cx[2] : cx[3];
        cu.seq0 = cu.seq = cu.s;
        cu.M = 1;
        cu.T = 0;
        cu.sub = 0;
        cu.tb = 0;
        cu.x0 = 0;
        cu.ctx = __builtin_amdgcn_readlane(c, l);
        cu.xe = cu.n;
      } else if (few) {
        const int4 d = make_int4(__builtin_amdgcn_readlane(dk.x, l),
                                 __builtin_amdgcn_readlane(dk.y, l),
                                 __builtin_amdgcn_readlane(dk.z, l),
                                 __builtin_amdgcn_readlane(dk.w, l));
        int len[kUnitCols];
#pragma unroll
        for (int m = 0; m < kUnitCols; ++m) len[m] = __builtin_amdgcn_readlane(lk[m], l);
        walk_unit(cu, a, d, len);
      } else {
        enter_unit<ROWS>(cu, a, rows, lens);
      }
      return true;
    }
    base += __builtin_amdgcn_readfirstlane(__shfl(incl, 63));
  }
  return false;
}

// A worker's outputs, staged in LDS while its loop runs and written to memory
// after it: a store in the loop waits for room behind the loads that keep the
// memory pipeline full, which cost about 3 us at every change of pair.  The
// staged items are the outputs of pairs that lie inside the worker's range
// (bf16 rows), the piece records of the pairs it starts, and the partial
// segment of the pair that began before its range.  A full buffer is written
// out where it fills.
template <int D, int COLS>
struct OutStage {
  static constexpr int kOutBytes = 8192;
  static constexpr int kMaxOut = kOutBytes / (D * 2);   // entries of a one-head group
  static constexpr int kMaxRecs = 64;
  uint2 out[kOutBytes / 8];
  int out_row[kMaxOut];            // first q row (s * Hq + kvh * g) of each entry
  int rec_pair[kMaxRecs];
  int2 rec[kMaxRecs];
  float seg[COLS * D];             // normalised rows of the slot-0 segment
  float seg_ml[COLS * 2];
};

template <int D, class Stage>
__device__ __forceinline__ void flush_outputs(const DecodeArgs& a, Stage& st, int& n_out,
                                              int lane) {
  if (n_out == 0) return;
  __syncthreads();
  const int cpe = a.group * D / 4;               // 8-byte chunks of one entry
  uint16_t* out = static_cast<uint16_t*>(a.out);
  for (int i = lane; i < n_out * cpe; i += 64) {
    const int e = i / cpe, k = i - e * cpe;
    *reinterpret_cast<uint2*>(out + int64_t(st.out_row[e]) * D + 4 * k) = st.out[e * cpe + k];
  }
  __syncthreads();
  n_out = 0;
}

template <class Stage>
__device__ __forceinline__ void flush_recs(const DecodeArgs& a, Stage& st, int& n_rec, int lane) {
  if (n_rec == 0) return;
  __syncthreads();
  for (int i = lane; i < n_rec; i += 64) a.recs[st.rec_pair[i]] = st.rec[i];
  __syncthreads();
  n_rec = 0;
}

// Columns of a pair with a query behind them, and the workspace rows per
// partial-segment slot: the head group (plain decode), or the head groups of
// the unit's M members side by side (shared-prefix decode, whose slots are
// kUnitCols rows apart).
template <bool ROWS>
__device__ __forceinline__ int pair_cols(const DecodeArgs& a, const Cursor& cu) {
  return ROWS ? cu.M * a.group : a.group;
}
template <bool ROWS>
__device__ __forceinline__ int slot_rows(const DecodeArgs& a) {
  return ROWS ? kUnitCols : a.group;
}

// Normalised output rows of the pair's columns, or its partial segment, at
// workspace row `row0` (column c at row0 + c).
template <int D>
__device__ __forceinline__ void store_piece(const DecodeArgs& a, int64_t row0, int ncols,
                                            const floatx4_t (&acc)[D / 16], float m, float l,
                                            float inv, int r, int c) {
  if (c >= ncols) return;
  const int64_t row = row0 + c;
  float* wacc = a.ws_acc + row * D;
#pragma unroll
  for (int j = 0; j < D / 16; ++j)
    *reinterpret_cast<float4*>(wacc + 16 * j + 4 * r) =
        make_float4(acc[j][0] * inv, acc[j][1] * inv, acc[j][2] * inv, acc[j][3] * inv);
  if (r == 0) {
    a.ws_ml[row * 2] = m;
    a.ws_ml[row * 2 + 1] = l;
  }
}

// End of a worker's share of a pair.  A pair that lies inside the worker's
// range [lo, lo + q) has its outputs staged (one head group per member);
// otherwise the share is a partial segment, for the worker's slot 0 (the pair
// began before the range, staged) or slot 1 (it goes on past the range: the
// end of the range, stored now).  The worker that holds a pair's first step
// also records {first worker, workers} of the pair for the merge.  A column
// that saw no token (a member whose span lies outside the segment) has sum 0:
// its partial row is stored as zeros.
template <int D, bool ROWS, int NQ, class Stage>
__device__ __forceinline__ void write_segment(const DecodeArgs& a, const Cursor& cu, int w, int q,
                                              const floatx4_t (&acc)[NQ][D / 16],
                                              const floatx4_t (&lsum)[NQ], const float (&m)[NQ],
                                              int r, int c, int lane, Stage& st, int& n_out,
                                              int& n_rec, int& seg0_cols) {
  const int g = a.group;
  const int ncols = pair_cols<ROWS>(a, cu), srows = slot_rows<ROWS>(a);
  const int lo = w * q;
  const bool head = cu.P >= lo;                  // the pair starts in this range
  const bool whole = head && cu.P + cu.n <= lo + q;
  if (head) {
    if (n_rec == Stage::kMaxRecs) flush_recs(a, st, n_rec, lane);
    if (lane == 0) {
      st.rec_pair[n_rec] = cu.s * a.num_kv_heads + cu.kvh;
      st.rec[n_rec] = make_int2(w, (cu.P + cu.n - 1) / q - w + 1);
    }
    ++n_rec;
  }
  if (whole) {
    const int ne = ROWS ? cu.M : 1;              // staged entries: one head group each
    if ((n_out + ne) * g > Stage::kMaxOut) flush_outputs<D>(a, st, n_out, lane);
    if (lane < ne) st.out_row[n_out + lane] = (cu.seq0 + lane) * a.num_q_heads + cu.kvh * g;
  }
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    const int col = 16 * t + c;                  // this lane's column of tile t
    const float l = lsum[t][0];
    const float inv = ROWS ? (l > 0.f ? a.v_scale / l : 0.f) : a.v_scale / l;
    if (whole) {
      if (col < ncols) {
        uint2* o = st.out + (n_out * g + col) * (D / 4);
#pragma unroll
        for (int j = 0; j < D / 16; ++j) {
          uint2 v;
          v.x = pack_bf16x2(acc[t][j][0] * inv, acc[t][j][1] * inv);
          v.y = pack_bf16x2(acc[t][j][2] * inv, acc[t][j][3] * inv);
          o[4 * j + r] = v;
        }
      }
    } else if (!head) {
      if (col < ncols) {
#pragma unroll
        for (int j = 0; j < D / 16; ++j)
          *reinterpret_cast<float4*>(st.seg + col * D + 16 * j + 4 * r) =
              make_float4(acc[t][j][0] * inv, acc[t][j][1] * inv, acc[t][j][2] * inv,
                          acc[t][j][3] * inv);
        if (r == 0) {
          st.seg_ml[2 * col] = m[t];
          st.seg_ml[2 * col + 1] = l;
        }
      }
    } else {
      store_piece<D>(a, int64_t(2 * w + 1) * srows, ncols, acc[t], m[t], l, inv, r, col);
    }
  }
  if (whole) n_out += ROWS ? cu.M : 1;
  else if (!head) seg0_cols = ncols;
}

// The staged outputs, records and slot-0 segment, after the loop.
template <int D, bool ROWS, class Stage>
__device__ __forceinline__ void flush_stage(const DecodeArgs& a, Stage& st, int w, int n_out,
                                            int n_rec, int seg0_cols, int lane) {
  flush_outputs<D>(a, st, n_out, lane);
  flush_recs(a, st, n_rec, lane);
  if (seg0_cols > 0) {
    __syncthreads();
    const int64_t row0 = int64_t(2 * w) * slot_rows<ROWS>(a);
    float4* wacc = reinterpret_cast<float4*>(a.ws_acc + row0 * D);
    const float4* src = reinterpret_cast<const float4*>(st.seg);
    for (int i = lane; i < seg0_cols * D / 4; i += 64) wacc[i] = src[i];
    float* wml = a.ws_ml + row0 * 2;
    for (int i = lane; i < 2 * seg0_cols; i += 64) wml[i] = st.seg_ml[i];
  }
}

// Persistent worker w: steps [w*q, min(total, (w+1)*q)) of the stream.  The
// load cursor runs NS-1 steps ahead of the compute cursor; every iteration
// issues exactly one step of loads (past the end of the range it repeats the
// last step), so the count of loads in flight is the same on every path.
// The query of a pair is loaded once, with the first step of the pair that the
// worker computes, into that step's ring slot (ahead of its K and V, so the
// wait for the step's data covers it); the compute cursor copies it from the
// slot when it reaches that step and keeps it for the pair's other steps.
// Loading it into registers of its own instead would leave the compiler
// unable to tell, at the copy, that the load is older than the step's data,
// and it would drain the whole load pipeline at every change of pair.
// Context lengths and block tables come in as separate restrict arguments:
// the kernel's stores cannot alias them, so their uniform loads stay scalar
// and never wait on the vector-load counter.
template <int KV, int D, int BS, bool NT, bool ROWS>
__global__ __launch_bounds__(64, (MfmaTuning<KV, ROWS ? 2 : 1>::waves)) void decode_mfma_kernel(
    DecodeArgs a, const int32_t* __restrict__ lens, const int32_t* __restrict__ tables,
    const int4* __restrict__ rows) {
  typedef typename KvTraits<KV>::T T;
  // query tiles of 16 columns: the head group, or a shared-prefix unit's kUnitCols columns
  constexpr int NQ = ROWS ? kUnitCols / 16 : 1;
  constexpr int NS = MfmaTuning<KV, NQ>::stages;
  constexpr int NB = 32 / BS;
  const int lane = threadIdx.x;
  const int r = lane >> 4, c = lane & 15;
  const int w = blockIdx.x;
  if (w == 0 && lane == 0) a.hdr[0] = kProtoSegments;
  int total, q;
  Cursor cu;                                       // compute cursor
  if (!find_start<ROWS>(a, rows, lens, w, lane, total, q, cu)) return;
  int rem = min(total - w * q, q);                 // steps left to compute
  const uint16_t* __restrict__ qbase = static_cast<const uint16_t*>(a.q);
  const int64_t head_stride = int64_t(BS) * D;
  const int64_t blk_stride = int64_t(a.num_kv_heads) * head_stride;
  const T* k_pool = static_cast<const T*>(a.k_pool);
  const T* v_pool = static_cast<const T*>(a.v_pool);
  const LaneMap<KV, D, BS> L(r, c);
  const float sl2 = a.qk_scale_log2;
  const int g = a.group, hkv = a.num_kv_heads, max_ctx = a.max_ctx;
  // q is [num_seqs][num_q_heads][D] bf16; its size fits 31 bits (checked on the host)
  const uint32_t qbytes = uint32_t(a.num_seqs) * uint32_t(a.num_q_heads) * uint32_t(D) * 2u;
  const __amdgpu_buffer_rsrc_t qrsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(qbase), 0, int(qbytes), 0x00020000);

  Cursor la = cu;                                  // load cursor
  int la_left = rem;                               // steps the load cursor still has to load
  int la_pbs[NB];
  step_blocks<BS>(la_pbs, tables + int64_t(la.seq) * a.max_blocks,
                  ROWS ? la.tb + 32 * (la.x - la.x0) : 32 * la.x, ROWS ? la.tb + la.ctx : la.ctx,
                  a.num_blocks);

  floatx4_t acc[NQ][D / 16];
  floatx4_t lsum[NQ];
  // a finite start: a shared-prefix column that sees no token keeps exp2(-inf - m) = 0
  constexpr float kMStart = ROWS ? -1e30f : -INFINITY;
  float m[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
#pragma unroll
    for (int j = 0; j < D / 16; ++j) acc[t][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    lsum[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    m[t] = kMStart;
  }
  StepRegs<KV, D, NQ> buf[NS];
  uint4 qc[NQ][D / 32];             // query of the compute cursor's pair
  __shared__ OutStage<D, ROWS ? kUnitCols : kMaxGroup> stage;
  int n_out = 0, n_rec = 0;         // staged outputs and records
  int seg0_cols = 0;                // columns of the staged slot-0 segment (0: none)
  bool la_first = true, cu_first = true;   // the next step is the worker's first

  // query column 16 t + c of a pair (tile t): head (16 t + c) % g of member (16 t + c) / g
  int cm[NQ], ch[NQ];
#pragma unroll
  for (int t = 0; t < NQ; ++t) {
    cm[t] = (16 * t + c) / g;
    ch[t] = 16 * t + c - cm[t] * g;
  }
  uint32_t qoff[NQ];
  bool qlane[NQ];
  // issue the load cursor's step into R, then move the cursor on
#define PKV_ISSUE(R)                                                                           \
  do {                                                                                         \
    for (int t = 0; t < NQ; ++t) {                                                             \
      qoff[t] = uint32_t(((la.seq0 + cm[t]) * a.num_q_heads + la.kvh * g + ch[t]) * D * 2);    \
      qlane[t] = 16 * t + c < pair_cols<ROWS>(a, la);                                          \
    }                                                                                          \
    issue_step<KV, D, BS, NT, NQ>(                                                             \
        R, k_pool + int64_t(la.kvh) * head_stride, v_pool + int64_t(la.kvh) * head_stride,     \
        la_pbs, blk_stride, L, la_first || la.x == 0, qrsrc, qoff, qlane, qbytes, r);          \
    la_first = false;                                                                          \
    if (la_left > 1) {                                                                         \
      --la_left;                                                                               \
      if (++la.x == la.n) next_pair<ROWS>(la, a, rows, lens, hkv, max_ctx);                    \
      else if (ROWS && la.x == la.xe) next_span(la, a, lens);                                  \
      step_blocks<BS>(la_pbs, tables + int64_t(la.seq) * a.max_blocks,                         \
                      ROWS ? la.tb + 32 * (la.x - la.x0) : 32 * la.x,                          \
                      ROWS ? la.tb + la.ctx : la.ctx, a.num_blocks);                           \
    } else {                                                                                   \
      /* the range is loaded: the round's remaining issues read block 0 */                     \
      for (int b = 0; b < NB; ++b) la_pbs[b] = 0;                                              \
    }                                                                                          \
  } while (0)

#pragma unroll
  for (int i = 0; i < NS - 1; ++i) PKV_ISSUE(buf[i]);
  // Rounds of NS steps, the loop's only exit at the bottom of a round: an exit
  // from inside the unrolled round would give the loop header a second
  // incoming path on which the round's fresh loads are pending, and the
  // compiler would then wait for them before reusing any of their registers.
  // Steps of the last round past the range are skipped, but their loads still
  // issue (one or two steps per worker).  They read block 0, the same for every
  // worker: streamed again from the worker's last step they cost 16-32 KB of
  // memory reads each, 30 MB per launch (10% of a multi-query layer's bytes).
  do {
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      PKV_ISSUE(buf[(st + NS - 1) % NS]);
      if (rem > 0) {
        if (cu_first || cu.x == 0) {
#pragma unroll
          for (int t = 0; t < NQ; ++t) {
#pragma unroll
            for (int i = 0; i < D / 32; ++i) qc[t][i] = buf[st].q[t][i];
          }
          cu_first = false;
        }
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
          // a tile past the pair's columns (a narrow unit) has nothing to compute
          if (t > 0 && 16 * t >= pair_cols<ROWS>(a, cu)) continue;
          compute_step<KV, D>(buf[st], qc[t], acc[t], lsum[t], m[t], sl2,
                              ROWS ? 32 * (cu.x - cu.x0) : 32 * cu.x, cu.ctx, r,
                              !ROWS || cu.sub < 0 || cm[t] == cu.sub);
        }
        --rem;
        if (++cu.x == cu.n || rem == 0) {
          write_segment<D, ROWS, NQ>(a, cu, w, q, acc, lsum, m, r, c, lane, stage, n_out, n_rec,
                                     seg0_cols);
          if (rem > 0) {
            next_pair<ROWS>(cu, a, rows, lens, hkv, max_ctx);
#pragma unroll
            for (int t = 0; t < NQ; ++t) {
#pragma unroll
              for (int j = 0; j < D / 16; ++j) acc[t][j] = floatx4_t{0.f, 0.f, 0.f, 0.f};
              lsum[t] = floatx4_t{0.f, 0.f, 0.f, 0.f};
              m[t] = kMStart;
            }
          }
        } else if (ROWS && cu.x == cu.xe) {
          next_span(cu, a, lens);
        }
      }
    }
  } while (rem > 0);
  flush_stage<D, ROWS>(a, stage, w, n_out, n_rec, seg0_cols, lane);
#undef PKV_ISSUE
}

// ------------------------------------------------------------------------ merge

// out = sum_k w_k * o_k / sum_k w_k with w_k = l_k * 2^(m_k - max_k m_k): the
// same rescaling the running softmax applies between tiles.  One workgroup per
// (sequence, KV head) pair merges the pieces of all the pair's query heads;
// the pieces are the vector kernel's partitions or the MFMA kernel's segments,
// whichever wrote the workspace last (its header says which).  Empty contexts
// get zeros here.
//
// A thread owns 4 consecutive output elements (a float4 of one head's row) of
// up to (16 x 128 / 4) / kMergeThreads such chunks; when the pair has fewer
// chunks than threads, the spare threads split the pieces into groups.  Each
// thread runs the merge as one online pass over its pieces, loading a
// piece's (max, sum) and its partial row together, so a workgroup waits for
// memory twice: for the context length and piece record, then for the pieces.
// The groups' partial results are combined through LDS.  Batches of few pairs
// (long contexts, many pieces each) get a workgroup per (pair, query head).
constexpr int kMergeThreads = 256;

template <typename QT, int D, int NT, bool ROWS, bool SPLIT>
__global__ __launch_bounds__(NT) void merge_kernel(DecodeArgs a) {
  constexpr int kMergeThreads = NT;
  __shared__ float4 part_o[kMergeThreads];
  __shared__ float part_m[kMergeThreads], part_l[kMergeThreads];
  const int g = a.group;
  // SPLIT: one workgroup per (pair, query head) instead of per pair
  const int hs = SPLIT ? int(blockIdx.x) % g : 0;
  const int pair = SPLIT ? int(blockIdx.x) / g : int(blockIdx.x);   // s * Hkv + kvh
  const int s = pair / a.num_kv_heads, kvh = pair - s * a.num_kv_heads;
  const int gw = SPLIT ? 1 : g;                      // query heads this workgroup merges
  const int nchunks = gw * D / 4;                    // float4 chunks of those rows
  const int tid = threadIdx.x;
  const int ctx = max(0, min(a.context_lens[s], a.max_ctx));
  QT* out = static_cast<QT*>(a.out) + (int64_t(s) * a.num_q_heads + int64_t(kvh) * g + hs) * D;
  if (ctx == 0) {
    for (int e = tid; e < gw * D; e += kMergeThreads) store_out(out + e, 0.f);
    return;
  }
  // piece k of head hg is row first(hg) + k * stride (+ fix for k > 0)
  int count = 0;
  int64_t first0 = 0, head_step = 0, stride = 0, fix = 0;
  if constexpr (ROWS) {
    // shared-prefix decode: the segments of the sequence's unit, in its member's columns
    // (kUnitCols-row slots); a sequence outside every unit is left alone
    const int4 sr = a.seq_rows[s];
    const int u = sr.x, mem = sr.y;
    if (u < 0 || u >= a.num_rows || mem < 0 || (mem + 1) * g > kUnitCols) return;
    const int2 rec = a.recs[int64_t(u) * a.num_kv_heads + kvh];
    const int u0 = min(max(rec.x, 0), kMaxWorkers - 1);
    count = min(rec.y, kMaxWorkers - u0);
    if (count <= 1) return;                          // written directly by the decode kernel
    first0 = int64_t(2 * u0 + 1) * kUnitCols + mem * g;
    head_step = 1;
    stride = 2 * kUnitCols;
    fix = -kUnitCols;
  } else {
    const int proto = a.hdr[0];
    const int2 rec = a.recs[pair];
    if (proto == kProtoSegments) {
      // segments of workers w0 .. w0+count-1: slot 1 of the first, slot 0 after
      count = rec.y;
      first0 = int64_t(2 * rec.x + 1) * g;
      head_step = 1;
      stride = 2 * int64_t(g);
      fix = -int64_t(g);
    } else {
      count = num_parts(ctx, a.part_tokens);
      first0 = (int64_t(s) * a.num_q_heads + int64_t(kvh) * g) * a.max_parts;
      head_step = a.max_parts;
      stride = 1;
    }
    if (count <= 1) return;                          // written directly by the decode kernel
  }
  first0 += hs * head_step;
  const int groups = nchunks >= kMergeThreads ? 1 : kMergeThreads / nchunks;
  const int pg = tid / min(nchunks, kMergeThreads);  // piece group of this thread
  const int c0 = tid - pg * min(nchunks, kMergeThreads);
  const float4* acc4 = reinterpret_cast<const float4*>(a.ws_acc);
  for (int ch = c0; ch < nchunks && pg < groups; ch += kMergeThreads) {
    const int hg = (4 * ch) / D, d4 = ch - hg * (D / 4);
    const int64_t first = first0 + hg * head_step;
    float M = -INFINITY, L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 4
    for (int k = pg; k < count; k += groups) {
      const int64_t pc = first + k * stride + (k ? fix : 0);
      const float2 ml = *reinterpret_cast<const float2*>(a.ws_ml + pc * 2);
      const float4 o = acc4[pc * (D / 4) + d4];
      const float Mn = fmaxf(M, ml.x);
      const float sc = exp2f(M - Mn);
      const float wk = ml.y * exp2f(ml.x - Mn);
      L = fmaf(L, sc, wk);
      O.x = fmaf(O.x, sc, wk * o.x);
      O.y = fmaf(O.y, sc, wk * o.y);
      O.z = fmaf(O.z, sc, wk * o.z);
      O.w = fmaf(O.w, sc, wk * o.w);
      M = Mn;
    }
    if (groups > 1) {
      part_o[tid] = O;
      part_m[tid] = M;
      part_l[tid] = L;
    } else {
      const float inv = 1.f / L;
      QT* o = out + int64_t(hg) * D + 4 * d4;
      store_out(o + 0, O.x * inv);
      store_out(o + 1, O.y * inv);
      store_out(o + 2, O.z * inv);
      store_out(o + 3, O.w * inv);
    }
  }
  if (groups == 1) return;
  __syncthreads();
  if (pg == 0 && c0 < nchunks) {
    // combine the groups of chunk c0 (group k's partial sits at thread k * nchunks + c0)
    float M = -INFINITY;
    for (int k = 0; k < groups && k < count; ++k) M = fmaxf(M, part_m[k * nchunks + c0]);
    float L = 0.f;
    float4 O = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < groups && k < count; ++k) {
      const int t = k * nchunks + c0;
      const float sc = exp2f(part_m[t] - M);
      const float4 o = part_o[t];
      L = fmaf(part_l[t], sc, L);
      O.x = fmaf(o.x, sc, O.x);
      O.y = fmaf(o.y, sc, O.y);
      O.z = fmaf(o.z, sc, O.z);
      O.w = fmaf(o.w, sc, O.w);
    }
    const float inv = 1.f / L;
    const int hg = (4 * c0) / D, d4 = c0 - hg * (D / 4);
    QT* o = out + int64_t(hg) * D + 4 * d4;
    store_out(o + 0, O.x * inv);
    store_out(o + 1, O.y * inv);
    store_out(o + 2, O.z * inv);
    store_out(o + 3, O.w * inv);
  }
}

// ------------------------------------------------------------------------ host side

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

static int64_t max_parts_for(int32_t max_ctx, int32_t part) {
  if (part <= 0 || max_ctx <= 0) return 1;
  return std::max<int64_t>(1, max_ctx / part);
}

static size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

// Workspace: header | per-pair records | partial rows ((max, sum) then D
// floats each).  Sized with num_q_heads (>= num_kv_heads) so the size does not
// depend on the pool; the partial rows cover both the vector kernel's
// partitions and the MFMA kernel's segments (two slots per worker, each
// holding a head group of at most 16 heads).
struct WsLayout {
  size_t recs_off, ml_off, acc_off, total;
  int64_t parts, rows, pairs;
};

static WsLayout ws_layout(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                          int32_t max_ctx, int32_t part) {
  WsLayout w;
  w.parts = max_parts_for(max_ctx, part);
  w.pairs = int64_t(num_seqs) * num_q_heads;
  w.recs_off = 256;
  w.ml_off = w.recs_off + align256(size_t(w.pairs) * sizeof(int2));
  const int64_t part_rows = w.parts > 1 ? w.pairs * w.parts : 0;
  const int64_t seg_rows = 2 * int64_t(kMaxWorkers) * std::min<int64_t>(num_q_heads, kMaxGroup);
  w.rows = std::max(part_rows, seg_rows);
  w.acc_off = w.ml_off + align256(size_t(w.rows) * 2 * sizeof(float));
  w.total = w.acc_off + size_t(w.rows) * head_dim * sizeof(float);
  return w;
}

// Shared-prefix decode workspace: header | records of the (unit, KV head) pairs |
// partial rows: the workers' two slots of kUnitCols rows each (for the workers
// the shared-prefix kernel runs on the current device).
static WsLayout ws_layout_rows(int32_t num_rows, int32_t num_kv_heads, int32_t head_dim,
                               int64_t workers) {
  WsLayout w;
  w.parts = 1;
  w.pairs = int64_t(num_rows) * num_kv_heads;
  w.recs_off = 256;
  w.ml_off = w.recs_off + align256(size_t(w.pairs) * sizeof(int2));
  w.rows = 2 * workers * kUnitCols;
  w.acc_off = w.ml_off + align256(size_t(w.rows) * 2 * sizeof(float));
  w.total = w.acc_off + size_t(w.rows) * head_dim * sizeof(float);
  return w;
}

template <typename K, typename... Extra>
static int launch(K kernel, dim3 grid, dim3 block, hipStream_t s, const DecodeArgs& a,
                  const char* what, Extra... extra) {
  kernel<<<grid, block, 0, s>>>(a, extra...);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "%s launch: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

// Events that the calling thread's next decode kernel records its start and end
// in (pkv_time_next_decode); that launch clears them.
static thread_local hipEvent_t t_time_start = nullptr, t_time_stop = nullptr;

// A decode kernel's launch: through hipExtLaunchKernel when timing events are
// set, so that the events hold the kernel's own start and end.
template <typename K, typename... Extra>
static int launch_decode(K kernel, dim3 grid, dim3 block, hipStream_t s, const DecodeArgs& a,
                         Extra... extra) {
  if (!t_time_start) return launch(kernel, grid, block, s, a, "decode", extra...);
  hipEvent_t t0 = t_time_start, t1 = t_time_stop;
  t_time_start = t_time_stop = nullptr;
  hipExtLaunchKernelGGL(kernel, grid, block, 0, s, t0, t1, 0, a, extra...);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "decode launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

// Workers that fit on the current device at once for a one-wave kernel.
template <typename K>
static int64_t resident_workers(K kernel) {
  static std::mutex mu;
  static std::unordered_map<uint64_t, int64_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1024;
  const uint64_t key = (uint64_t(reinterpret_cast<uintptr_t>(reinterpret_cast<const void*>(kernel)))
                        << 8) ^ uint64_t(dev);
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kernel),
                                                   64, 0) != hipSuccess ||
      cus <= 0 || per_cu <= 0) {
    (void)hipGetLastError();   // clear the failed query's error; fall back to a fixed count
    return 1024;
  }
  const int64_t n = int64_t(cus) * per_cu;
  cache[key] = n;
  return n;
}

template <int D, int BS>
static int dispatch_vector(const DecodeArgs& a, int kv, int qd, hipStream_t s) {
  const dim3 grid(static_cast<unsigned>(int64_t(a.num_seqs) * a.num_kv_heads * a.max_parts));
  const dim3 block(kVecThreads);
  if (kv == PKV_F32 && qd == PKV_F32)
    return launch_decode(decode_vector_kernel<KV_F32, float, D, BS>, grid, block, s, a);
  if (kv == PKV_BF16 && qd == PKV_BF16)
    return launch_decode(decode_vector_kernel<KV_BF16, uint16_t, D, BS>, grid, block, s, a);
  if (kv == PKV_FP8_E4M3 && qd == PKV_BF16)
    return launch_decode(decode_vector_kernel<KV_FP8, uint16_t, D, BS>, grid, block, s, a);
  return fail(PKV_E_UNSUPPORTED, "q %s with a %s pool", dtype_name(qd), dtype_name(kv));
}

template <int KV, int D, int BS, bool NT, bool ROWS>
static int launch_mfma(const DecodeArgs& a0, hipStream_t s) {
  auto kernel = decode_mfma_kernel<KV, D, BS, NT, ROWS>;
  DecodeArgs a = a0;
  // a preset count (the no-allocation entry point sized its scratch for it) is a cap
  const int64_t resident = std::min<int64_t>(kMaxWorkers, resident_workers(kernel));
  int64_t w = a0.workers > 0 ? std::min<int64_t>(a0.workers, resident) : resident;
  // Few long pairs: half the workers.  Each worker's share doubles, so the fixed cost of
  // finding its start and of the pieces it writes and the merge reads weighs half as much.
  // bf16, four or more workers' shares per pair: two workers per CU instead of four, whose
  // two steps of loads in flight still keep the memory busy (multi-query layers of 32 to 256
  // sequences 12% to 1.4% faster, GQA layers of 64 to 256 pairs up to 3%; with thousands of
  // pairs four workers per CU stay ahead by about 2%).  fp8 (two waves per SIMD), eight or
  // more shares per pair of a group of 16: one wave per SIMD (multi-query layers of 32 to 256
  // sequences 13% to 2% faster).  With smaller groups the pieces weigh less and fp8 loses
  // more from halving the loads in flight (group 4: up to 5% slower from 128 pairs on).
  const int64_t pairs = int64_t(a.num_seqs) * a.num_kv_heads;
  const bool few_pairs = KV == KV_BF16 ? pairs * 4 <= w : (a.group >= 16 && pairs * 8 <= w);
  if (!ROWS && few_pairs && w >= 2) w /= 2;
  a.workers = int32_t(w);
  // Only the workers that can get steps are launched.  With a partition size each share is
  // at least part_tokens / 32 steps (unless that would leave fewer than half the workers
  // busy), so at most max(ceil(steps / share), ceil(w / 2)) workers have any, where steps is
  // the most the contexts can hold.  The split itself is computed for all w workers, so the
  // result is the same; the workers left out would only have started, scanned the context
  // lengths and left (one 32k-token context in partitions of 512: 513 of 1024 launched).
  int64_t grid = w;
  if (!ROWS && a.part_tokens > 0) {
    const int64_t share = std::max(1, a.part_tokens >> 5);
    const int64_t steps =
        int64_t(a.num_seqs) * a.num_kv_heads * ((int64_t(a.max_ctx) + 31) / 32);
    grid = std::min<int64_t>(w, std::max<int64_t>((steps + share - 1) / share, (w + 1) / 2));
  }
  return launch_decode(kernel, dim3(static_cast<unsigned>(grid)), dim3(64), s, a,
                       a.context_lens, a.block_tables, a.rows);
}

// Persistent workers a plain (not shared-prefix) matrix-core decode launches.
template <int KV, int D, int BS>
static int64_t mfma_workers_of(bool shared) {
  return std::min<int64_t>(kMaxWorkers,
                           shared ? resident_workers(decode_mfma_kernel<KV, D, BS, false, false>)
                                  : resident_workers(decode_mfma_kernel<KV, D, BS, true, false>));
}

template <int D>
static int64_t mfma_workers_d(int kv, int bs, bool shared) {
  if (kv == PKV_FP8_E4M3)
    return bs == 8 ? mfma_workers_of<KV_FP8, D, 8>(shared)
           : bs == 16 ? mfma_workers_of<KV_FP8, D, 16>(shared)
                      : mfma_workers_of<KV_FP8, D, 32>(shared);
  return bs == 8 ? mfma_workers_of<KV_BF16, D, 8>(shared)
         : bs == 16 ? mfma_workers_of<KV_BF16, D, 16>(shared)
                    : mfma_workers_of<KV_BF16, D, 32>(shared);
}

// Persistent workers of the shared-prefix decode on the current device.
template <int D>
static int64_t rows_workers_d(int kv, int bs) {
  auto w = [](auto kernel) { return std::min<int64_t>(kMaxWorkers, resident_workers(kernel)); };
  if (kv == PKV_FP8_E4M3)
    return bs == 8    ? w(decode_mfma_kernel<KV_FP8, D, 8, true, true>)
           : bs == 16 ? w(decode_mfma_kernel<KV_FP8, D, 16, true, true>)
                      : w(decode_mfma_kernel<KV_FP8, D, 32, true, true>);
  return bs == 8    ? w(decode_mfma_kernel<KV_BF16, D, 8, true, true>)
         : bs == 16 ? w(decode_mfma_kernel<KV_BF16, D, 16, true, true>)
                    : w(decode_mfma_kernel<KV_BF16, D, 32, true, true>);
}

static int64_t rows_workers(const pkv_cache_desc* c) {
  return c->head_dim == 64 ? rows_workers_d<64>(c->kv_dtype, c->block_size)
                           : rows_workers_d<128>(c->kv_dtype, c->block_size);
}

// `shared`: blocks are read again within the launch (by other sequences of a
// plain decode, or by other units of a shared-prefix decode), so K and V are read
// with ordinary loads that leave them in the caches; otherwise they stream.  The
// choice is per launch: a load whose kind depended on the step would be merged by
// the compiler into one ordinary load for both cases.
template <int D, int BS>
static int dispatch_mfma(const DecodeArgs& a, int kv, bool shared, bool rows, hipStream_t s) {
  if (kv == PKV_BF16)
    return rows ? (shared ? launch_mfma<KV_BF16, D, BS, false, true>(a, s)
                          : launch_mfma<KV_BF16, D, BS, true, true>(a, s))
                : (shared ? launch_mfma<KV_BF16, D, BS, false, false>(a, s)
                          : launch_mfma<KV_BF16, D, BS, true, false>(a, s));
  if (kv == PKV_FP8_E4M3)
    return rows ? (shared ? launch_mfma<KV_FP8, D, BS, false, true>(a, s)
                          : launch_mfma<KV_FP8, D, BS, true, true>(a, s))
                : (shared ? launch_mfma<KV_FP8, D, BS, false, false>(a, s)
                          : launch_mfma<KV_FP8, D, BS, true, false>(a, s));
  return fail(PKV_E_UNSUPPORTED, "the MFMA kernel needs a bf16 or fp8 pool");
}

template <int D>
static int dispatch_bs(const DecodeArgs& a, int bs, int kv, int qd, bool mfma, bool shared,
                       bool rows, hipStream_t s) {
  switch (bs) {
    case 8:
      return mfma ? dispatch_mfma<D, 8>(a, kv, shared, rows, s)
                  : dispatch_vector<D, 8>(a, kv, qd, s);
    case 16:
      return mfma ? dispatch_mfma<D, 16>(a, kv, shared, rows, s)
                  : dispatch_vector<D, 16>(a, kv, qd, s);
    case 32:
      return mfma ? dispatch_mfma<D, 32>(a, kv, shared, rows, s)
                  : dispatch_vector<D, 32>(a, kv, qd, s);
  }
  return fail(PKV_E_UNSUPPORTED, "block_size %d", bs);
}

}  // namespace pkv

using namespace pkv;

extern "C" size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                             int32_t head_dim, int32_t max_context_len,
                                             int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len < 0 ||
      partition_size < 0)
    return 0;
  return ws_layout(num_seqs, num_q_heads, head_dim, max_context_len, partition_size).total;
}

// Validate the arguments of a decode call and fill the kernel arguments.
static int prepare(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                   const pkv_cache_desc* c, const int32_t* block_tables,
                   int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                   int32_t num_q_heads, float scale, void* out, int32_t max_context_len,
                   int32_t partition_size, void* workspace, size_t workspace_bytes,
                   DecodeArgs* a, WsLayout* lay, int32_t num_rows = -1,
                   const WsLayout* fixed = nullptr) {
  // num_rows >= 0: a shared-prefix decode, whose layout comes in `fixed`
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
  if (int64_t(std::max(num_seqs, num_rows)) * c->num_kv_heads *
              ((int64_t(max_context_len) + 31) / 32) >= (1 << 30) ||
      int64_t(num_seqs) * num_q_heads * c->head_dim * 4 >= (int64_t(1) << 31))
    return fail(PKV_E_INVAL, "batch too large for one call");
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16)
    return fail(PKV_E_INVAL, "q_dtype must be f32 or bf16");
  if ((c->kv_dtype == PKV_F32) != (q_dtype == PKV_F32))
    return fail(PKV_E_UNSUPPORTED, "q %s with a %s pool", dtype_name(q_dtype),
                dtype_name(c->kv_dtype));
  *lay = fixed ? *fixed
               : ws_layout(std::max(num_seqs, 1), num_q_heads, c->head_dim, max_context_len,
                           partition_size);
  if (num_seqs == 0) return PKV_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !context_lens || !out)
    return fail(PKV_E_INVAL, "NULL pointer");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(out))
    return fail(PKV_E_INVAL, "device pointers must be 16-byte aligned");
  if (!workspace || workspace_bytes < lay->total || !aligned16(workspace))
    return fail(PKV_E_INVAL, "workspace of %zu bytes needed (got %zu)", lay->total,
                workspace_bytes);
  if (lay->rows > 0x7fffffff || lay->pairs > 0x7fffffff)
    return fail(PKV_E_INVAL, "batch too large for one call");
  char* ws = static_cast<char*>(workspace);
  a->q = q;
  a->k_pool = k_pool;
  a->v_pool = v_pool;
  a->block_tables = block_tables;
  a->context_lens = context_lens;
  a->out = out;
  a->hdr = reinterpret_cast<int32_t*>(ws);
  a->recs = reinterpret_cast<int2*>(ws + lay->recs_off);
  a->ws_ml = reinterpret_cast<float*>(ws + lay->ml_off);
  a->ws_acc = reinterpret_cast<float*>(ws + lay->acc_off);
  a->max_blocks = max_blocks_per_seq;
  a->num_seqs = num_seqs;
  a->num_q_heads = num_q_heads;
  a->num_kv_heads = c->num_kv_heads;
  a->group = group;
  a->num_blocks = c->num_blocks;
  a->max_ctx = max_context_len;
  a->part_tokens = partition_size;
  a->max_parts = int32_t(lay->parts);
  a->workers = 0;
  a->qk_scale_log2 = scale * kLog2e * (c->kv_dtype == PKV_FP8_E4M3 ? c->k_scale : 1.f);
  a->v_scale = c->kv_dtype == PKV_FP8_E4M3 ? c->v_scale : 1.f;
  a->rows = nullptr;
  a->seq_rows = nullptr;
  a->num_rows = 0;
  a->block_size = c->block_size;
  return PKV_OK;
}

// Launches the per-partition / per-segment kernels; *merge tells whether the
// merge kernel has pieces to combine.
static int launch_partials(const DecodeArgs& a0, const pkv_cache_desc* c, int32_t q_dtype,
                           const WsLayout& lay, int32_t impl, hipStream_t s, bool* merge) {
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
  DecodeArgs a = a0;
  if (!mfma && lay.parts <= 1) a.part_tokens = 0;   // the vector kernel does not split
  *merge = mfma || lay.parts > 1;
  return c->head_dim == 64
             ? dispatch_bs<64>(a, c->block_size, c->kv_dtype, q_dtype, mfma, shared, false, s)
             : dispatch_bs<128>(a, c->block_size, c->kv_dtype, q_dtype, mfma, shared, false, s);
}

template <bool ROWS, bool SPLIT>
static int launch_merge_nt(const DecodeArgs& a, int32_t head_dim, int32_t q_dtype, hipStream_t s) {
  constexpr int NT = kMergeThreads;
  const dim3 mgrid(static_cast<unsigned>(int64_t(a.num_seqs) * a.num_kv_heads *
                                         (SPLIT ? a.group : 1)));
  const dim3 block(NT);
  if (ROWS)  // bf16 q / out only (the matrix-core kernel)
    return head_dim == 64
               ? launch(merge_kernel<uint16_t, 64, NT, true, SPLIT>, mgrid, block, s, a, "merge")
               : launch(merge_kernel<uint16_t, 128, NT, true, SPLIT>, mgrid, block, s, a, "merge");
  if (head_dim == 64)
    return q_dtype == PKV_F32
               ? launch(merge_kernel<float, 64, NT, false, SPLIT>, mgrid, block, s, a, "merge")
               : launch(merge_kernel<uint16_t, 64, NT, false, SPLIT>, mgrid, block, s, a, "merge");
  return q_dtype == PKV_F32
             ? launch(merge_kernel<float, 128, NT, false, SPLIT>, mgrid, block, s, a, "merge")
             : launch(merge_kernel<uint16_t, 128, NT, false, SPLIT>, mgrid, block, s, a, "merge");
}

// A batch of few (sequence, KV head) pairs has long contexts in many pieces each:
// a workgroup per (pair, query head) splits those pieces into more groups.
static int launch_merge(const DecodeArgs& a, int32_t head_dim, int32_t q_dtype, hipStream_t s,
                        bool rows = false) {
  const bool few = int64_t(a.num_seqs) * a.num_kv_heads < 256;
  if (rows)
    return few ? launch_merge_nt<true, true>(a, head_dim, q_dtype, s)
               : launch_merge_nt<true, false>(a, head_dim, q_dtype, s);
  return few ? launch_merge_nt<false, true>(a, head_dim, q_dtype, s)
             : launch_merge_nt<false, false>(a, head_dim, q_dtype, s);
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
  WsLayout lay;
  int rc = prepare(q, q_dtype, k_pool, v_pool, c, block_tables, max_blocks_per_seq, context_lens,
                   num_seqs, num_q_heads, scale, out, max_context_len, partition_size, workspace,
                   workspace_bytes, &a, &lay);
  if (rc || num_seqs == 0) return rc;
  bool merge = false;
  return launch_partials(a, c, q_dtype, lay, impl, static_cast<hipStream_t>(stream), &merge);
}

extern "C" int pkv_paged_attn_merge(int32_t q_dtype, const int32_t* context_lens,
                                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t max_context_len,
                                    int32_t partition_size, const void* workspace,
                                    size_t workspace_bytes, void* out, void* stream) {
  clear_error();
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_context_len < 0 ||
      partition_size < 0)
    return fail(PKV_E_INVAL, "negative size");
  if (num_q_heads % num_kv_heads || num_q_heads / num_kv_heads > kMaxGroup)
    return fail(PKV_E_INVAL, "num_q_heads %d is not a multiple (at most %d) of num_kv_heads %d",
                num_q_heads, kMaxGroup, num_kv_heads);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_E_UNSUPPORTED, "head_dim %d not built (64, 128)", head_dim);
  if (q_dtype != PKV_F32 && q_dtype != PKV_BF16) return fail(PKV_E_INVAL, "bad q_dtype");
  if (num_seqs == 0) return PKV_OK;
  const WsLayout lay = ws_layout(num_seqs, num_q_heads, head_dim, max_context_len, partition_size);
  if (!workspace || workspace_bytes < lay.total || !aligned16(workspace))
    return fail(PKV_E_INVAL, "workspace of %zu bytes needed (got %zu)", lay.total,
                workspace_bytes);
  if (!context_lens || !out || !aligned16(out)) return fail(PKV_E_INVAL, "bad pointer");
  if (int64_t(num_seqs) * num_q_heads > 0x7fffffff) return fail(PKV_E_INVAL, "grid too large");
  DecodeArgs a = {};
  char* ws = static_cast<char*>(const_cast<void*>(workspace));
  a.context_lens = context_lens;
  a.out = out;
  a.hdr = reinterpret_cast<int32_t*>(ws);
  a.recs = reinterpret_cast<int2*>(ws + lay.recs_off);
  a.ws_ml = reinterpret_cast<float*>(ws + lay.ml_off);
  a.ws_acc = reinterpret_cast<float*>(ws + lay.acc_off);
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.group = num_q_heads / num_kv_heads;
  a.max_ctx = max_context_len;
  a.part_tokens = lay.parts > 1 ? partition_size : 0;
  a.max_parts = int32_t(lay.parts);
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
  WsLayout lay;
  int rc = prepare(q, q_dtype, k_pool, v_pool, c, block_tables, max_blocks_per_seq, context_lens,
                   num_seqs, num_q_heads, scale, out, max_context_len, partition_size, workspace,
                   workspace_bytes, &a, &lay);
  if (rc || num_seqs == 0) return rc;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool merge = false;
  rc = launch_partials(a, c, q_dtype, lay, impl, s, &merge);
  if (rc || !merge) return rc;
  DecodeArgs m = a;
  if (lay.parts <= 1) m.part_tokens = 0;
  return launch_merge(m, c->head_dim, q_dtype, s);
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

extern "C" int pkv_time_next_decode(void* start_event, void* stop_event) {
  clear_error();
  if ((start_event == nullptr) != (stop_event == nullptr))
    return fail(PKV_E_INVAL, "give both events or neither");
  t_time_start = static_cast<hipEvent_t>(start_event);
  t_time_stop = static_cast<hipEvent_t>(stop_event);
  return PKV_OK;
}

extern "C" size_t pkv_rows_workspace_bytes(const pkv_cache_desc* c, int32_t num_rows) {
  if (check_desc(c) || num_rows < 0 || c->kv_dtype == PKV_F32) return 0;
  return ws_layout_rows(num_rows, c->num_kv_heads, c->head_dim, rows_workers(c)).total;
}

extern "C" int pkv_paged_attn_decode_rows(const void* q, int32_t q_dtype, const void* k_pool,
                                          const void* v_pool, const pkv_cache_desc* c,
                                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                                          const int32_t* context_lens, int32_t num_seqs,
                                          int32_t num_q_heads, float scale, void* out,
                                          int32_t max_context_len, int32_t partition_size,
                                          const int32_t* rows, int32_t num_rows,
                                          const int32_t* seq_rows, void* workspace,
                                          size_t workspace_bytes, void* stream, int32_t phases) {
  clear_error();
  if (num_rows < 0) return fail(PKV_E_INVAL, "negative num_rows");
  const bool cached = (phases & PKV_IMPL_SHARED_BLOCKS) != 0;
  phases &= ~PKV_IMPL_SHARED_BLOCKS;
  if (phases < 1 || phases > 3)
    return fail(PKV_E_INVAL, "phases must be 1, 2 or 3 (optionally with PKV_IMPL_SHARED_BLOCKS)");
  int rc = check_desc(c);
  if (rc) return rc;
  if (c->kv_dtype == PKV_F32)
    return fail(PKV_E_UNSUPPORTED, "the shared-prefix decode needs a bf16 or fp8 pool");
  const int64_t workers = rows_workers(c);
  const WsLayout rows_lay = ws_layout_rows(num_rows, c->num_kv_heads, c->head_dim, workers);
  DecodeArgs a;
  WsLayout lay;
  rc = prepare(q, q_dtype, k_pool, v_pool, c, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, scale, out, max_context_len, partition_size, workspace,
               workspace_bytes, &a, &lay, num_rows, &rows_lay);
  if (rc || num_seqs == 0) return rc;
  a.workers = int32_t(workers);
  if (!rows || !seq_rows || num_rows == 0) return fail(PKV_E_INVAL, "no rows");
  if ((reinterpret_cast<uintptr_t>(rows) | reinterpret_cast<uintptr_t>(seq_rows)) & 15u)
    return fail(PKV_E_INVAL, "rows and seq_rows must be 16-byte aligned");
  a.rows = reinterpret_cast<const int4*>(rows);
  a.seq_rows = reinterpret_cast<const int4*>(seq_rows);
  a.num_rows = num_rows;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (phases & 1) {
    rc = c->head_dim == 64
             ? dispatch_bs<64>(a, c->block_size, c->kv_dtype, q_dtype, true, cached, true, s)
             : dispatch_bs<128>(a, c->block_size, c->kv_dtype, q_dtype, true, cached, true, s);
    if (rc) return rc;
  }
  if (phases & 2) return launch_merge(a, c->head_dim, q_dtype, s, true);
  return PKV_OK;
}

// ------------------------------------------------------------------------ no-allocation variant
//
// pkv_paged_attn_decode without a workspace argument, for callers that cannot
// allocate device memory.  The partial rows, piece records and header live in
// `scratch`, a file-scope device array of kScratchBytes that each device holds
// for the life of the process.  Host code never passes the array's name to a
// kernel (in host code it is a stand-in, not a device address): the device
// address comes from hipGetSymbolAddress, once per device, and is kept.  The
// kernels write every scratch byte they later read, so nothing is cleared
// between calls; calls that overlap on one device (two streams) race on it.

constexpr size_t kScratchBytes = size_t(40) << 20;
constexpr int kScratchMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kScratchMaxDevices] = {};

// Device address of the current device's scratch in *out; PKV_OK, or the status and a
// message on failure.
static int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(PKV_E_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kScratchMaxDevices)
    return fail(PKV_E_UNSUPPORTED, "device %d beyond the %d the scratch table holds", dev,
                kScratchMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_E_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

// Scratch layout of one call: header | records of the (sequence, head) pairs | partial
// rows, sized for the kernel family and worker count that will run (the generic
// workspace is sized without them).
static WsLayout ws_layout_noalloc(int32_t num_seqs, int32_t num_q_heads, int32_t group,
                                  int32_t head_dim, int32_t max_ctx, int32_t part, bool mfma,
                                  int64_t workers) {
  WsLayout w;
  w.parts = max_parts_for(max_ctx, part);
  w.pairs = int64_t(num_seqs) * num_q_heads;
  w.recs_off = 256;
  w.ml_off = w.recs_off + align256(size_t(w.pairs) * sizeof(int2));
  w.rows = mfma ? 2 * workers * group : (w.parts > 1 ? w.pairs * w.parts : 0);
  w.acc_off = w.ml_off + align256(size_t(w.rows) * 2 * sizeof(float));
  w.total = w.acc_off + size_t(w.rows) * head_dim * sizeof(float);
  return w;
}

extern "C" size_t pkv_decode_scratch_bytes(void) { return kScratchBytes; }

extern "C" int pkv_paged_attn_decode_noalloc(const void* q, int32_t q_dtype, const void* k_pool,
                                             const void* v_pool, const pkv_cache_desc* c,
                                             const int32_t* block_tables,
                                             int32_t max_blocks_per_seq,
                                             const int32_t* context_lens, int32_t num_seqs,
                                             int32_t num_q_heads, float scale, void* out,
                                             int32_t max_context_len, int32_t partition_size,
                                             void* stream, int32_t impl) {
  clear_error();
  int rc = check_desc(c);
  if (rc) return rc;
  if (num_seqs < 0 || num_q_heads <= 0 || max_context_len < 0 || partition_size < 0)
    return fail(PKV_E_INVAL, "negative size");
  if (num_q_heads % c->num_kv_heads || num_q_heads / c->num_kv_heads > kMaxGroup)
    return fail(PKV_E_INVAL, "num_q_heads %d is not a multiple (at most %d) of num_kv_heads %d",
                num_q_heads, kMaxGroup, c->num_kv_heads);
  if (num_seqs == 0) return PKV_OK;
  const int family = impl & PKV_IMPL_FAMILY_MASK;
  const bool shared = (impl & PKV_IMPL_SHARED_BLOCKS) != 0;
  const bool mfma = family == PKV_IMPL_MFMA || (family == PKV_IMPL_AUTO && c->kv_dtype != PKV_F32);
  const int64_t workers =
      mfma && c->kv_dtype != PKV_F32
          ? (c->head_dim == 64 ? mfma_workers_d<64>(c->kv_dtype, c->block_size, shared)
                               : mfma_workers_d<128>(c->kv_dtype, c->block_size, shared))
          : 0;
  const WsLayout lay = ws_layout_noalloc(num_seqs, num_q_heads, num_q_heads / c->num_kv_heads,
                                         c->head_dim, max_context_len, partition_size, mfma,
                                         workers);
  if (lay.total > kScratchBytes)
    return fail(PKV_E_INVAL,
                "the batch needs %zu bytes of scratch, more than the %zu the no-allocation "
                "decode holds (use pkv_paged_attn_decode with a workspace)",
                lay.total, kScratchBytes);
  void* ws = nullptr;
  rc = scratch_ptr(&ws);
  if (rc) return rc;
  DecodeArgs a;
  WsLayout got;
  rc = prepare(q, q_dtype, k_pool, v_pool, c, block_tables, max_blocks_per_seq, context_lens,
               num_seqs, num_q_heads, scale, out, max_context_len, partition_size, ws,
               kScratchBytes, &a, &got, -1, &lay);
  if (rc) return rc;
  a.workers = int32_t(workers);
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool merge = false;
  rc = launch_partials(a, c, q_dtype, lay, impl, s, &merge);
  if (rc || !merge) return rc;
  DecodeArgs m = a;
  if (lay.parts <= 1) m.part_tokens = 0;
  return launch_merge(m, c->head_dim, q_dtype, s);
}
