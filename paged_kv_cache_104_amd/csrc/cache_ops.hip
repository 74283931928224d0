// Cache operations: the write of new tokens into their (block, slot) and the
// whole-block copy of copy-on-write.
//
// reshape_and_cache follows the ultralytics glossary ("How paging works"): the
// token at position pos of a sequence lives in row pos mod B of the block its
// table lists at entry pos div B, i.e. slot = table[pos / B] * B + pos % B.
// copy_blocks is the copy step of copy-on-write (ithome article 10417389,
// section 4): the writer's new block receives the whole shared block.
// swap_blocks moves whole blocks between the device pool and a host pool of
// the same block shape (review of the vLLM paper, the preemption paragraphs:
// swapping out to host memory and back).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <vector>

#include "device_common.h"
#include "pkv_internal.h"

namespace pkv {

// x / scale rounded to fp32 as an IEEE fp32 division rounds it, from inv = 1 / scale
// rounded to fp64 (on the host).  The fp64 product x * inv is within about 2^-52 (relative)
// of the exact quotient.  A quotient of two fp32 numbers is never exactly halfway between
// two fp32 numbers (its numerator would need 25 significant bits), and when it is not, it
// lies more than 2^-49 (relative) from every halfway point (x - m * scale, for a halfway
// point m of 25 significant bits, is a nonzero multiple of the smaller of the two terms'
// last-bit units); so the product rounds to the same fp32 value as the quotient.  (Quotients below the fp32 normal range, where the
// spacing is absolute, encode to a zero code either way; an overflow saturates either
// way.)  One multiply and two conversions, against a division sequence whose steps share
// one condition register and so run one division after another.
__device__ __forceinline__ float div_by_scale(float x, double inv) {
  return float(double(x) * inv);
}

// 8 consecutive dimensions of one (token, head) key row, from the input segment ks to
// the pool segment kd (fp8: divided by the key scale and encoded, as every cache write
// does; k_inv is 1 / k_scale in fp64).
template <int KV, typename In>
__device__ __forceinline__ void write_key_segment(const In* __restrict__ ks,
                                                  typename KvTraits<KV>::T* __restrict__ kd,
                                                  double k_inv) {
  if constexpr (KV == KV_BF16) {
    *reinterpret_cast<uint4*>(kd) = *reinterpret_cast<const uint4*>(ks);
  } else {
    float kf[8];
    if constexpr (sizeof(In) == 2) {
      const uint4 ku = *reinterpret_cast<const uint4*>(ks);
      const uint32_t kw[4] = {ku.x, ku.y, ku.z, ku.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        kf[2 * i] = bf16_to_f32(kw[i] & 0xffffu);
        kf[2 * i + 1] = bf16_to_f32(kw[i] >> 16);
      }
    } else {
      const float4 k0 = reinterpret_cast<const float4*>(ks)[0];
      const float4 k1 = reinterpret_cast<const float4*>(ks)[1];
      kf[0] = k0.x; kf[1] = k0.y; kf[2] = k0.z; kf[3] = k0.w;
      kf[4] = k1.x; kf[5] = k1.y; kf[6] = k1.z; kf[7] = k1.w;
    }
    if constexpr (KV == KV_FP8) {
      float q[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) q[i] = div_by_scale(kf[i], k_inv);
      *reinterpret_cast<uint2*>(kd) = make_uint2(e4m3_encode4(q[0], q[1], q[2], q[3]),
                                                 e4m3_encode4(q[4], q[5], q[6], q[7]));
    } else {
      reinterpret_cast<float4*>(kd)[0] = make_float4(kf[0], kf[1], kf[2], kf[3]);
      reinterpret_cast<float4*>(kd)[1] = make_float4(kf[4], kf[5], kf[6], kf[7]);
    }
  }
}

// One value element in the pool's storage format (fp8: divided by the value scale and
// encoded; v_inv is 1 / v_scale in fp64).
template <int KV, typename In>
__device__ __forceinline__ typename KvTraits<KV>::T encode_value(In x, double v_inv) {
  if constexpr (KV == KV_BF16) {
    return x;
  } else {
    float f;
    if constexpr (sizeof(In) == 2) f = bf16_to_f32(x); else f = x;
    if constexpr (KV == KV_FP8) return uint8_t(e4m3_encode(div_by_scale(f, v_inv)));
    else return f;
  }
}

// One token of k / v ([tokens][heads][D]) into slot `slot` of the pools, by one
// workgroup.  Keys: each thread moves 8 consecutive dimensions of one head, a
// contiguous row segment of the key tile.  Values: the token is one column of
// each dimension-major value tile, so each thread writes one element, with
// consecutive threads on consecutive dimensions: the lanes that write into one
// line do it in one instruction, which the memory pipeline merges into one
// write.  The value elements go out as non-temporal (streaming) stores.  A
// token's values touch every line of its tile with a few bytes each; written
// through the caches, such partial lines slowed the next decode's reads of
// those tiles (every context's last block is read right after its new token
// is written) by up to 10% on a 40-head layer.
template <int KV, typename In>
__device__ __forceinline__ void write_token(
    const In* __restrict__ k, const In* __restrict__ v, int64_t tok, int64_t slot,
    typename KvTraits<KV>::T* __restrict__ k_pool, typename KvTraits<KV>::T* __restrict__ v_pool,
    int num_kv_heads, int head_dim, int block_size, double k_inv, double v_inv) {
  typedef typename KvTraits<KV>::T T;
  const int64_t blk = slot / block_size;
  const int pos = int(slot - blk * block_size);
  const int n = num_kv_heads * head_dim;
  const int64_t head_stride = int64_t(block_size) * head_dim;
  const int64_t tile0 = blk * num_kv_heads * head_stride;
  // keys: 8 consecutive dimensions per thread, a contiguous row segment of the pool
  for (int ch = threadIdx.x; ch < n / 8; ch += blockDim.x) {
    const int h = (ch * 8) / head_dim;
    const int d0 = ch * 8 - h * head_dim;
    write_key_segment<KV, In>(k + tok * n + ch * 8,
                              k_pool + tile0 + h * head_stride + int64_t(pos) * head_dim + d0,
                              k_inv);
  }
  // values: one element per thread, consecutive threads on consecutive dimensions, so
  // the lanes that write one line of the dimension-major tile do it in one instruction;
  // eight elements' loads are requested before any is stored
  for (int e0 = threadIdx.x; e0 < n; e0 += 8 * blockDim.x) {
    In raw[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = e0 + i * int(blockDim.x);
      raw[i] = v[tok * n + min(e, n - 1)];
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int e = e0 + i * int(blockDim.x);
      if (e >= n) break;
      const int h = e / head_dim, d = e - h * head_dim;
      T* vd = v_pool + tile0 + h * head_stride + int64_t(d) * block_size + pos;
      __builtin_nontemporal_store(encode_value<KV, In>(raw[i], v_inv), vd);
    }
  }
}

template <int KV, typename In>
__global__ __launch_bounds__(128) void reshape_and_cache_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const int64_t* __restrict__ slots,
    typename KvTraits<KV>::T* __restrict__ k_pool, typename KvTraits<KV>::T* __restrict__ v_pool,
    int num_kv_heads, int head_dim, int block_size, int64_t num_slots, double k_inv,
    double v_inv) {
  const int64_t tok = blockIdx.x;
  const int64_t slot = slots[tok];
  if (slot < 0 || slot >= num_slots) return;             // skip (negative) / never write outside
  write_token<KV, In>(k, v, tok, slot, k_pool, v_pool, num_kv_heads, head_dim, block_size,
                      k_inv, v_inv);
}

// Writes of many tokens at once (a prompt's prefill): the value tile of a (block, head)
// is dimension-major, so one token writes one element in each of its D rows, a few bytes
// of every line; one store per element held such writes near 0.5 TB/s.  Here one
// workgroup takes B consecutive tokens.  Keys go out as contiguous row segments as above.
// For the values the call's tokens fall into runs: maximal sequences of consecutive
// tokens whose slots are consecutive within one block.  A run holds at most B tokens and
// belongs to the workgroup of the chunk its first token is in (it may reach into the next
// chunk), so every token is written once.  A run of B tokens fills its block: each thread
// owns one (head, dimension) row at a time, gathers that element of the run's tokens into
// registers and writes the row whole, with 16-byte stores (8 bytes for an fp8 pool of
// 8-token blocks).  Prompts laid end to end in one call are such runs in every block but
// the last of each prompt, wherever the prompts start in the call.  The tokens of shorter
// runs are stored one element at a time: through the caches when a neighbouring token
// shares its block, so that the parts of a line meet in L2, and streamed when it is alone
// in its block (a decode step's token, whose partial lines would otherwise sit dirty in L2
// when the decode reads that block).
// A call of few chunks (a large decode batch: single tokens, each alone in its block)
// splits each chunk's rows over several workgroups (blockIdx.y), up to kRunsTargetGroups
// workgroups in all and at least kRunsThreads value rows each; a prefill has enough chunks
// for one workgroup per chunk.
constexpr int kRunsThreads = 256;
constexpr int64_t kRunsMinTokens = 512;    // fewer: the per-token kernel (decode steps)
constexpr int64_t kRunsTargetGroups = 2048;

template <typename T>
__device__ __forceinline__ uint32_t storage_bits(T x) {
  if constexpr (sizeof(T) == 4) return __builtin_bit_cast(uint32_t, x);
  else return uint32_t(x);
}

// B input elements as one row of the dimension-major value tile, encoded and written
// with whole 16-byte (or 8-byte) stores; dst is the row's start (aligned: a row is B
// elements, 8 bytes at least).
template <int KV, typename In, int B>
__device__ __forceinline__ void store_value_row(typename KvTraits<KV>::T* __restrict__ dst,
                                                const In (&raw)[B], double v_inv) {
  constexpr int words = B * KvTraits<KV>::bytes / 4;
  uint32_t w[words];
  if constexpr (KV == KV_FP8) {
    float q[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      float f;
      if constexpr (sizeof(In) == 2) f = bf16_to_f32(raw[j]); else f = raw[j];
      q[j] = div_by_scale(f, v_inv);
    }
#pragma unroll
    for (int i = 0; i < words; ++i)
      w[i] = e4m3_encode4(q[4 * i], q[4 * i + 1], q[4 * i + 2], q[4 * i + 3]);
  } else {
    constexpr int per_word = 4 / KvTraits<KV>::bytes;
#pragma unroll
    for (int i = 0; i < words; ++i) {
      uint32_t u = 0;
#pragma unroll
      for (int b = 0; b < per_word; ++b)
        u |= storage_bits(encode_value<KV, In>(raw[i * per_word + b], v_inv))
             << (8 * KvTraits<KV>::bytes * b);
      w[i] = u;
    }
  }
  if constexpr (words % 4 == 0) {
#pragma unroll
    for (int i = 0; i < words / 4; ++i)
      reinterpret_cast<uint4*>(dst)[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
  } else {
    static_assert(words == 2, "rows of 8 bytes or a multiple of 16");
    *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
  }
}

template <int KV, typename In, int B>
__global__ __launch_bounds__(kRunsThreads) void reshape_and_cache_runs_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const int64_t* __restrict__ slots,
    typename KvTraits<KV>::T* __restrict__ k_pool, typename KvTraits<KV>::T* __restrict__ v_pool,
    int num_kv_heads, int head_dim, int64_t num_tokens, int64_t num_slots, double k_inv,
    double v_inv) {
  typedef typename KvTraits<KV>::T T;
  static_assert(2 * B <= 64 && 2 * B + 1 <= kRunsThreads,
                "the window fits the workgroup, its bit masks one wavefront");
  // the window: tokens i0 - 1 .. i0 + 2B - 1 at index t = token - i0 + 1
  __shared__ int64_t s_blk[2 * B + 1];   // block of the token, or -1: skipped / outside the call
  __shared__ int s_off[2 * B + 1];
  __shared__ int s_part[2 * B];          // token i0 + j is in a shorter run this chunk owns
  __shared__ int s_whole;                // first token (minus i0) of the run of B tokens, or -1
  __shared__ uint64_t s_mask[2];         // bit j: s_part[j]; of those, stored streamed
  const int64_t i0 = int64_t(blockIdx.x) * B;
  const int n_tok = int(min<int64_t>(B, num_tokens - i0));
  const int H = num_kv_heads, D = head_dim, n = H * D;
  const int tid = threadIdx.x;
  if (tid < 2 * B + 1) {
    const int64_t tok = i0 - 1 + tid;
    int64_t blk = -1;
    int off = 0;
    if (tok >= 0 && tok < num_tokens) {
      const int64_t sl = slots[tok];
      if (sl >= 0 && sl < num_slots) {
        blk = sl / B;
        off = int(sl - blk * B);
      }
    }
    s_blk[tid] = blk;
    s_off[tid] = off;
  }
  if (tid < 2 * B) s_part[tid] = 0;
  if (tid == 0) s_whole = -1;
  __syncthreads();
  if (tid < B) {
    // does a run start at token i0 + tid, and how long is it
    const int t = tid + 1;
    const int64_t blk = s_blk[t];
    if (blk >= 0 && !(s_blk[t - 1] == blk && s_off[t - 1] + 1 == s_off[t])) {
      int len = 1;
      while (len < B && s_blk[t + len] == blk && s_off[t + len] == s_off[t] + len) ++len;
      if (len == B) s_whole = tid;   // at most one: a second would start B tokens later
      else
        for (int j = tid; j < tid + len; ++j) s_part[j] = 1;
    }
  }
  __syncthreads();
  if (tid < 64) {
    // the first wavefront gathers the shorter runs' tokens into two bit masks
    const int t = tid + 1;
    const bool part = tid < 2 * B && s_part[tid] != 0;
    const bool alone = part && s_blk[t - 1] != s_blk[t] && s_blk[min(t + 1, 2 * B)] != s_blk[t];
    const uint64_t pm = __ballot(part), am = __ballot(alone);
    if (tid == 0) {
      s_mask[0] = pm;
      s_mask[1] = am;
    }
  }
  __syncthreads();
  // this workgroup's share of the chunk's rows (blockIdx.y of gridDim.y): key segments
  // [k_lo, k_hi) of every token and value rows [v_lo, v_hi)
  const int parts = gridDim.y, part = blockIdx.y;
  const int segs = n / 8, k_lo = segs * part / parts, k_hi = segs * (part + 1) / parts;
  const int v_lo = n * part / parts, v_hi = n * (part + 1) / parts;
  // keys: every token of the chunk
  for (int e = tid; e < n_tok * (k_hi - k_lo); e += kRunsThreads) {
    const int j = e / (k_hi - k_lo), ch = k_lo + (e - j * (k_hi - k_lo));
    const int64_t blk = s_blk[j + 1];
    if (blk < 0) continue;
    const int h = (ch * 8) / D, d0 = ch * 8 - h * D;
    write_key_segment<KV, In>(k + (i0 + j) * n + ch * 8,
                              k_pool + (blk * H + h) * int64_t(B) * D + int64_t(s_off[j + 1]) * D + d0,
                              k_inv);
  }
  // values: row e = h * D + d of the value tiles, at element e * B of the (block, 0) tile
  // (the tiles of one block's heads follow one another).  All of a pass's loads are issued
  // before its encodes: an encode between two loads would make each load wait for the one
  // before it (65 536 tokens into an fp8 pool, with a longer integer encode than the one
  // now: 221 against 142 us).
  const int whole = s_whole;
  const uint64_t part_mask = s_mask[0], alone_mask = s_mask[1];
  if (whole >= 0) {
    const int64_t s0 = i0 + whole;
    T* const tile = v_pool + s_blk[whole + 1] * n * int64_t(B);
    for (int e = v_lo + tid; e < v_hi; e += kRunsThreads) {
      In raw[B];
#pragma unroll
      for (int j = 0; j < B; ++j) raw[j] = v[(s0 + j) * n + e];
      store_value_row<KV, In, B>(tile + int64_t(e) * B, raw, v_inv);
    }
  }
#pragma unroll 1
  for (int half = 0; half < 2; ++half) {
    const uint32_t pm = uint32_t(part_mask >> (half * B)), am = uint32_t(alone_mask >> (half * B));
    if (pm == 0) continue;
    const int j0 = half * B;
    for (int e = v_lo + tid; e < v_hi; e += kRunsThreads) {
      In raw[B];
#pragma unroll
      for (int j = 0; j < B; ++j) raw[j] = (pm >> j) & 1u ? v[(i0 + j0 + j) * n + e] : In(0);
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (!((pm >> j) & 1u)) continue;
        const int t = j0 + j + 1;
        T* dst = v_pool + s_blk[t] * n * int64_t(B) + int64_t(e) * B + s_off[t];
        const T x = encode_value<KV, In>(raw[j], v_inv);
        if ((am >> j) & 1u) __builtin_nontemporal_store(x, dst);
        else *dst = x;
      }
    }
  }
}

// The decode step's append for up to kAppendMax tokens, with the host's slots and
// positions passed by value in the kernel arguments (no upload): token i of
// the chunk is row `first + i` of the batch; besides its K / V it sets the
// device block table entry that holds it and the row's context length, which
// is all an append changes in them (a new block, or the copy that replaced a
// shared last block).
constexpr int kAppendMax = 256;
struct AppendChunk {
  int64_t slot[kAppendMax];
  int32_t pos[kAppendMax];
};

template <int KV, typename In>
__global__ __launch_bounds__(128) void append_tokens_kernel(
    const In* __restrict__ k, const In* __restrict__ v, AppendChunk chunk, int32_t first,
    typename KvTraits<KV>::T* __restrict__ k_pool, typename KvTraits<KV>::T* __restrict__ v_pool,
    int32_t* __restrict__ tables, int32_t max_blocks, int32_t* __restrict__ lens,
    int num_kv_heads, int head_dim, int block_size, int64_t num_slots, double k_inv,
    double v_inv) {
  const int i = blockIdx.x;
  const int64_t slot = chunk.slot[i];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t row = int64_t(first) + i;
  write_token<KV, In>(k, v, row, slot, k_pool, v_pool, num_kv_heads, head_dim, block_size,
                      k_inv, v_inv);
  if (threadIdx.x == 0) {
    const int32_t pos = chunk.pos[i];
    tables[row * max_blocks + pos / block_size] = int32_t(slot / block_size);
    lens[row] = pos + 1;
  }
}

// One workgroup per (pair, pool): 16-byte copies of a whole block.
__global__ __launch_bounds__(256) void copy_blocks_kernel(uint8_t* __restrict__ k_pool,
                                                          uint8_t* __restrict__ v_pool,
                                                          const int64_t* __restrict__ pairs,
                                                          int64_t block_bytes, int64_t num_blocks) {
  const int64_t src = pairs[2 * int64_t(blockIdx.x)];
  const int64_t dst = pairs[2 * int64_t(blockIdx.x) + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  uint8_t* pool = blockIdx.y == 0 ? k_pool : v_pool;
  const uint4* s = reinterpret_cast<const uint4*>(pool + src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>(pool + dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

// One workgroup per (pair, pool), 16-byte copies of a whole block from one pool
// to another; either may be pinned host memory, which the GPU reads and writes
// across the host link.  Many blocks in flight at once keep the link busy with
// one launch, whatever the block size.
__global__ __launch_bounds__(256) void swap_blocks_kernel(
    const uint8_t* __restrict__ src_k, const uint8_t* __restrict__ src_v, uint8_t* __restrict__ dst_k,
    uint8_t* __restrict__ dst_v, const int64_t* __restrict__ pairs, int64_t block_bytes,
    int64_t src_blocks, int64_t dst_blocks) {
  const int64_t src = pairs[2 * int64_t(blockIdx.x)];
  const int64_t dst = pairs[2 * int64_t(blockIdx.x) + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const uint4* s = reinterpret_cast<const uint4*>((blockIdx.y == 0 ? src_k : src_v) + src * block_bytes);
  uint4* d = reinterpret_cast<uint4*>((blockIdx.y == 0 ? dst_k : dst_v) + dst * block_bytes);
  const int64_t n = block_bytes / 16;
  for (int64_t i = threadIdx.x; i < n; i += blockDim.x) d[i] = s[i];
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// 1 / scale rounded to fp64, the factor the device's division by a scale multiplies by.
static double inv_scale(float scale) { return 1.0 / double(scale); }

template <int KV, typename In>
static int launch_runs(const In* k, const In* v, const int64_t* slots,
                       typename KvTraits<KV>::T* k_pool, typename KvTraits<KV>::T* v_pool,
                       const pkv_cache_desc* c, int64_t num_tokens, int64_t num_slots,
                       hipStream_t s) {
  const int64_t chunks = (num_tokens + c->block_size - 1) / c->block_size;
  if (chunks > 0x7fffffff) return fail(PKV_E_INVAL, "too many tokens for one call");
  const int H = c->num_kv_heads, D = c->head_dim;
  const int64_t parts = std::max<int64_t>(
      1, std::min<int64_t>((kRunsTargetGroups + chunks - 1) / chunks, int64_t(H) * D / kRunsThreads));
  const dim3 grid(static_cast<unsigned>(chunks), static_cast<unsigned>(parts)), block(kRunsThreads);
  const double ks = inv_scale(KV == KV_FP8 ? c->k_scale : 1.f),
               vs = inv_scale(KV == KV_FP8 ? c->v_scale : 1.f);
  switch (c->block_size) {
    case 8:
      reshape_and_cache_runs_kernel<KV, In, 8><<<grid, block, 0, s>>>(
          k, v, slots, k_pool, v_pool, H, D, num_tokens, num_slots, ks, vs);
      return PKV_OK;
    case 16:
      reshape_and_cache_runs_kernel<KV, In, 16><<<grid, block, 0, s>>>(
          k, v, slots, k_pool, v_pool, H, D, num_tokens, num_slots, ks, vs);
      return PKV_OK;
    case 32:
      reshape_and_cache_runs_kernel<KV, In, 32><<<grid, block, 0, s>>>(
          k, v, slots, k_pool, v_pool, H, D, num_tokens, num_slots, ks, vs);
      return PKV_OK;
  }
  return fail(PKV_E_UNSUPPORTED, "block_size %d", c->block_size);
}

}  // namespace pkv

using namespace pkv;

extern "C" int pkv_reshape_and_cache(const void* k, const void* v, int32_t in_dtype,
                                     const int64_t* slot_mapping, int64_t num_tokens,
                                     void* k_pool, void* v_pool, const pkv_cache_desc* c,
                                     void* stream) {
  clear_error();
  int rc = check_desc(c);
  if (rc) return rc;
  if (num_tokens < 0) return fail(PKV_E_INVAL, "negative num_tokens");
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_pool || !v_pool) return fail(PKV_E_INVAL, "NULL pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool) ||
      !aligned16(slot_mapping))
    return fail(PKV_E_INVAL, "device pointers must be 16-byte aligned");
  if (num_tokens > 0x7fffffff) return fail(PKV_E_INVAL, "too many tokens for one call");
  const bool ok = (c->kv_dtype == PKV_F32 && in_dtype == PKV_F32) ||
                  (c->kv_dtype == PKV_BF16 && in_dtype == PKV_BF16) ||
                  (c->kv_dtype == PKV_FP8_E4M3 && (in_dtype == PKV_BF16 || in_dtype == PKV_F32));
  if (!ok)
    return fail(PKV_E_UNSUPPORTED, "%s input into a %s pool", dtype_name(in_dtype),
                dtype_name(c->kv_dtype));
  const int64_t num_slots = int64_t(c->num_blocks) * c->block_size;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int H = c->num_kv_heads, D = c->head_dim, B = c->block_size;
  if (num_tokens >= kRunsMinTokens) {
    int rc;
    if (c->kv_dtype == PKV_F32)
      rc = launch_runs<KV_F32>(static_cast<const float*>(k), static_cast<const float*>(v),
                               slot_mapping, static_cast<float*>(k_pool),
                               static_cast<float*>(v_pool), c, num_tokens, num_slots, s);
    else if (c->kv_dtype == PKV_BF16)
      rc = launch_runs<KV_BF16>(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                                slot_mapping, static_cast<uint16_t*>(k_pool),
                                static_cast<uint16_t*>(v_pool), c, num_tokens, num_slots, s);
    else if (in_dtype == PKV_BF16)
      rc = launch_runs<KV_FP8>(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                               slot_mapping, static_cast<uint8_t*>(k_pool),
                               static_cast<uint8_t*>(v_pool), c, num_tokens, num_slots, s);
    else
      rc = launch_runs<KV_FP8>(static_cast<const float*>(k), static_cast<const float*>(v),
                               slot_mapping, static_cast<uint8_t*>(k_pool),
                               static_cast<uint8_t*>(v_pool), c, num_tokens, num_slots, s);
    if (rc) return rc;
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
      return fail(PKV_E_HIP, "reshape_and_cache launch: %s", hipGetErrorString(e));
    return PKV_OK;
  }
  const dim3 grid(static_cast<unsigned>(num_tokens)), block(128);
  if (c->kv_dtype == PKV_F32) {
    reshape_and_cache_kernel<KV_F32, float><<<grid, block, 0, s>>>(
        static_cast<const float*>(k), static_cast<const float*>(v), slot_mapping,
        static_cast<float*>(k_pool), static_cast<float*>(v_pool), H, D, B, num_slots, 1.0, 1.0);
  } else if (c->kv_dtype == PKV_BF16) {
    reshape_and_cache_kernel<KV_BF16, uint16_t><<<grid, block, 0, s>>>(
        static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), slot_mapping,
        static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), H, D, B, num_slots, 1.0,
        1.0);
  } else if (in_dtype == PKV_BF16) {
    reshape_and_cache_kernel<KV_FP8, uint16_t><<<grid, block, 0, s>>>(
        static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), slot_mapping,
        static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), H, D, B, num_slots,
        inv_scale(c->k_scale), inv_scale(c->v_scale));
  } else {
    reshape_and_cache_kernel<KV_FP8, float><<<grid, block, 0, s>>>(
        static_cast<const float*>(k), static_cast<const float*>(v), slot_mapping,
        static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), H, D, B, num_slots,
        inv_scale(c->k_scale), inv_scale(c->v_scale));
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "reshape_and_cache launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" int pkv_append_tokens(const void* k, const void* v, int32_t in_dtype,
                                 const int64_t* host_slots, const int32_t* host_positions,
                                 int32_t num_tokens, void* k_pool, void* v_pool,
                                 const pkv_cache_desc* c, int32_t* block_tables,
                                 int32_t max_blocks_per_seq, int32_t* context_lens,
                                 void* stream) {
  clear_error();
  int rc = check_desc(c);
  if (rc) return rc;
  if (num_tokens < 0 || max_blocks_per_seq <= 0) return fail(PKV_E_INVAL, "bad sizes");
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !host_slots || !host_positions || !k_pool || !v_pool || !block_tables ||
      !context_lens)
    return fail(PKV_E_INVAL, "NULL pointer");
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_pool) || !aligned16(v_pool))
    return fail(PKV_E_INVAL, "device pointers must be 16-byte aligned");
  const bool ok = (c->kv_dtype == PKV_F32 && in_dtype == PKV_F32) ||
                  (c->kv_dtype == PKV_BF16 && in_dtype == PKV_BF16) ||
                  (c->kv_dtype == PKV_FP8_E4M3 && (in_dtype == PKV_BF16 || in_dtype == PKV_F32));
  if (!ok)
    return fail(PKV_E_UNSUPPORTED, "%s input into a %s pool", dtype_name(in_dtype),
                dtype_name(c->kv_dtype));
  const int B = c->block_size;
  const int64_t num_slots = int64_t(c->num_blocks) * B;
  for (int32_t i = 0; i < num_tokens; ++i) {
    const int64_t sl = host_slots[i];
    const int32_t pos = host_positions[i];
    if (sl < 0) continue;
    if (sl >= num_slots) return fail(PKV_E_INVAL, "slot %lld of token %d outside the pool", (long long)sl, i);
    if (pos < 0 || pos / B >= max_blocks_per_seq || pos % B != sl % B)
      return fail(PKV_E_INVAL, "position %d of token %d does not match slot %lld", pos, i,
                  (long long)sl);
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int H = c->num_kv_heads, D = c->head_dim;
  for (int32_t first = 0; first < num_tokens; first += kAppendMax) {
    const int32_t n = std::min<int32_t>(kAppendMax, num_tokens - first);
    AppendChunk chunk;
    for (int32_t i = 0; i < n; ++i) {
      chunk.slot[i] = host_slots[first + i];
      chunk.pos[i] = host_positions[first + i];
    }
    const dim3 grid(static_cast<unsigned>(n)), block(128);
    if (c->kv_dtype == PKV_F32) {
      append_tokens_kernel<KV_F32, float><<<grid, block, 0, st>>>(
          static_cast<const float*>(k), static_cast<const float*>(v), chunk, first,
          static_cast<float*>(k_pool), static_cast<float*>(v_pool), block_tables,
          max_blocks_per_seq, context_lens, H, D, B, num_slots, 1.0, 1.0);
    } else if (c->kv_dtype == PKV_BF16) {
      append_tokens_kernel<KV_BF16, uint16_t><<<grid, block, 0, st>>>(
          static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), chunk, first,
          static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), block_tables,
          max_blocks_per_seq, context_lens, H, D, B, num_slots, 1.0, 1.0);
    } else if (in_dtype == PKV_BF16) {
      append_tokens_kernel<KV_FP8, uint16_t><<<grid, block, 0, st>>>(
          static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), chunk, first,
          static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), block_tables,
          max_blocks_per_seq, context_lens, H, D, B, num_slots, inv_scale(c->k_scale), inv_scale(c->v_scale));
    } else {
      append_tokens_kernel<KV_FP8, float><<<grid, block, 0, st>>>(
          static_cast<const float*>(k), static_cast<const float*>(v), chunk, first,
          static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), block_tables,
          max_blocks_per_seq, context_lens, H, D, B, num_slots, inv_scale(c->k_scale), inv_scale(c->v_scale));
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return fail(PKV_E_HIP, "append_tokens launch: %s", hipGetErrorString(e));
  }
  return PKV_OK;
}

extern "C" int pkv_copy_blocks(void* k_pool, void* v_pool, const int64_t* src_dst_pairs,
                               int64_t num_pairs, const pkv_cache_desc* c, void* stream) {
  clear_error();
  int rc = check_desc(c);
  if (rc) return rc;
  if (num_pairs < 0) return fail(PKV_E_INVAL, "negative num_pairs");
  if (num_pairs == 0) return PKV_OK;
  if (!k_pool || !v_pool || !src_dst_pairs) return fail(PKV_E_INVAL, "NULL pointer");
  if (!aligned16(k_pool) || !aligned16(v_pool))
    return fail(PKV_E_INVAL, "pools must be 16-byte aligned");
  if (num_pairs > 0x7fffffff) return fail(PKV_E_INVAL, "too many pairs for one call");
  const int64_t block_bytes =
      int64_t(c->num_kv_heads) * c->block_size * c->head_dim * elem_bytes(c->kv_dtype);
  const dim3 grid(static_cast<unsigned>(num_pairs), 2), block(256);
  copy_blocks_kernel<<<grid, block, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<uint8_t*>(k_pool), static_cast<uint8_t*>(v_pool), src_dst_pairs, block_bytes,
      c->num_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "copy_blocks launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" int32_t pkv_memory_kind(const void* p) {
  if (!p) return 0;
  hipPointerAttribute_t at;
  if (hipPointerGetAttributes(&at, p) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  if (at.type == hipMemoryTypeDevice) return 2;
  if (at.type == hipMemoryTypeHost && at.devicePointer == p) return 1;
  return 0;
}

static int64_t block_bytes_of(const pkv_cache_desc* c) {
  return int64_t(c->num_kv_heads) * c->block_size * c->head_dim * elem_bytes(c->kv_dtype);
}

static int check_swap(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                      int64_t num_pairs, int32_t src_num_blocks, int32_t dst_num_blocks,
                      const pkv_cache_desc* c) {
  int rc = check_desc(c);
  if (rc) return rc;
  if (num_pairs < 0 || src_num_blocks < 0 || dst_num_blocks < 0)
    return fail(PKV_E_INVAL, "negative size");
  if (num_pairs > 0x7fffffff) return fail(PKV_E_INVAL, "too many pairs for one call");
  if (num_pairs && (!src_k || !src_v || !dst_k || !dst_v)) return fail(PKV_E_INVAL, "NULL pool");
  if (num_pairs && (!aligned16(src_k) || !aligned16(src_v) || !aligned16(dst_k) || !aligned16(dst_v)))
    return fail(PKV_E_INVAL, "pools must be 16-byte aligned");
  if (num_pairs) {
    // every pool must be device memory or pinned host memory that the GPU sees at the
    // same address: pageable host memory is refused here, never touched by a kernel
    const void* pools[4] = {src_k, src_v, dst_k, dst_v};
    for (const void* p : pools)
      if (pkv_memory_kind(p) == 0)
        return fail(PKV_E_INVAL, "pool %p is neither device nor mapped pinned host memory", p);
  }
  return PKV_OK;
}

extern "C" int pkv_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                               const int64_t* src_dst_pairs, int64_t num_pairs,
                               int32_t src_num_blocks, int32_t dst_num_blocks,
                               const pkv_cache_desc* c, void* stream) {
  clear_error();
  int rc = check_swap(src_k, src_v, dst_k, dst_v, num_pairs, src_num_blocks, dst_num_blocks, c);
  if (rc || num_pairs == 0) return rc;
  if (!src_dst_pairs) return fail(PKV_E_INVAL, "NULL pairs");
  const dim3 grid(static_cast<unsigned>(num_pairs), 2), block(256);
  swap_blocks_kernel<<<grid, block, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint8_t*>(src_k), static_cast<const uint8_t*>(src_v),
      static_cast<uint8_t*>(dst_k), static_cast<uint8_t*>(dst_v), src_dst_pairs,
      block_bytes_of(c), src_num_blocks, dst_num_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_E_HIP, "swap_blocks launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

extern "C" int pkv_swap_blocks_dma(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                                   const int64_t* src_dst_pairs, int64_t num_pairs,
                                   int32_t src_num_blocks, int32_t dst_num_blocks,
                                   const pkv_cache_desc* c, void* stream) {
  clear_error();
  int rc = check_swap(src_k, src_v, dst_k, dst_v, num_pairs, src_num_blocks, dst_num_blocks, c);
  if (rc || num_pairs == 0) return rc;
  if (!src_dst_pairs) return fail(PKV_E_INVAL, "NULL pairs");
  // the pairs are on the host here: check them all before the first copy
  std::vector<char> seen(size_t(dst_num_blocks), 0);
  for (int64_t i = 0; i < num_pairs; ++i) {
    const int64_t sb = src_dst_pairs[2 * i], db = src_dst_pairs[2 * i + 1];
    if (sb < 0 || sb >= src_num_blocks || db < 0 || db >= dst_num_blocks)
      return fail(PKV_E_INVAL, "pair %lld (%lld, %lld) out of range", (long long)i, (long long)sb,
                  (long long)db);
    if (seen[size_t(db)]++) return fail(PKV_E_INVAL, "destination %lld repeated", (long long)db);
  }
  const int64_t bb = block_bytes_of(c);
  hipStream_t st = static_cast<hipStream_t>(stream);
  // one transfer per run of pairs that are consecutive on both sides
  for (int64_t i = 0; i < num_pairs;) {
    int64_t j = i + 1;
    while (j < num_pairs && src_dst_pairs[2 * j] == src_dst_pairs[2 * i] + (j - i) &&
           src_dst_pairs[2 * j + 1] == src_dst_pairs[2 * i + 1] + (j - i))
      ++j;
    const int64_t sb = src_dst_pairs[2 * i], db = src_dst_pairs[2 * i + 1], bytes = (j - i) * bb;
    hipError_t e = hipMemcpyAsync(static_cast<uint8_t*>(dst_k) + db * bb,
                                  static_cast<const uint8_t*>(src_k) + sb * bb, size_t(bytes),
                                  hipMemcpyDefault, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(static_cast<uint8_t*>(dst_v) + db * bb,
                         static_cast<const uint8_t*>(src_v) + sb * bb, size_t(bytes),
                         hipMemcpyDefault, st);
    if (e != hipSuccess) return fail(PKV_E_HIP, "swap copy: %s", hipGetErrorString(e));
    i = j;
  }
  return PKV_OK;
}
