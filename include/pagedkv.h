/*
 * pagedkv.h -- C ABI of the paged-KV decode library for AMD MI355X (gfx950).
 *
 * The operations follow the pages that describe PagedAttention:
 *  - the KV cache lives in fixed-size physical blocks of B tokens held in one
 *    pool shared by all requests, reached through a per-request block table
 *    (ithome article 10417389, section 3 "PagedAttention"; ultralytics glossary
 *    "PagedAttention", section "How paging works"; optiverse-tech blog
 *    "paged-kv-cache", section "Block table and non-contiguous allocation");
 *  - a new token's key/value is written to pool[table[pos / B], pos % B]
 *    (glossary code example);
 *  - the attention kernel reads keys and values back block by block through
 *    the table (glossary, "How paging works"; optiverse, same section);
 *  - shared blocks are reference counted and copied on write (ithome,
 *    section 4, "Physical block sharing" and "Copy-on-Write").
 *
 * Conventions for every device call
 *  - All device pointers are caller-owned (torch tensors on ROCm in the Python
 *    binding).  The library allocates no device memory and keeps no pointer
 *    after a call returns.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null stream)
 *    and return PKV_OK or a negative pkv_status.  Arguments are validated on
 *    the host before anything is launched; on error nothing is launched and
 *    pkv_last_error() describes the failure.
 *  - Device data is trusted only as far as memory safety: block ids and slots
 *    outside the pool are skipped by the kernels (never read or written), but
 *    the result for such entries is unspecified.
 *  - Device pointers must be 16-byte aligned.
 *
 * Pool layout (one layer), num_blocks = N, num_kv_heads = H, block_size = B,
 * head_dim = D, element type = kv_dtype:
 *    key pool   [N][H][B][D]   a token's key for one head is a contiguous row
 *    value pool [N][H][D][B]   within a block, values are dimension-major
 * The value layout puts the B tokens of one dimension next to each other so
 * that the P.V product of the decode kernel reads its matrix-core operand with
 * one 16-byte load per lane.
 *
 * fp8 (PKV_FP8_E4M3) is OCP FP8 E4M3FN.  A stored code c of a pool with scale
 * s stands for e4m3(c) * s; reshape_and_cache encodes x as
 * round_nearest_even_saturating(fp32(x) / fp32(s)) (NaN -> 0x7F, sign kept).
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_E_INVAL = -1,        /* bad argument or shape */
  PKV_E_NOMEM = -2,        /* block manager: not enough free blocks (state unchanged) */
  PKV_E_UNSUPPORTED = -3,  /* valid but not built: dtype / head_dim / block_size combination */
  PKV_E_HIP = -4           /* a HIP runtime call failed */
} pkv_status;

typedef enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_FP8_E4M3 = 2 } pkv_dtype;

/* One layer's K and V pools (layouts above). */
typedef struct {
  int32_t num_blocks;
  int32_t num_kv_heads;
  int32_t block_size;     /* 8, 16 or 32 */
  int32_t head_dim;       /* 64 or 128 */
  int32_t kv_dtype;       /* pkv_dtype */
  float k_scale;          /* fp8 only; must be 1.0f for f32 / bf16 pools */
  float v_scale;
} pkv_cache_desc;

/* ------------------------------------------------------------------ device calls */

/*
 * reshape_and_cache -- write new tokens' keys and values into their slots.
 * Ultralytics glossary, "How paging works": position pos of a sequence is row
 * pos mod B of the block that its table lists at entry pos div B.
 *
 *   k, v          device [num_tokens][H][D] of in_dtype (f32 for an f32 pool;
 *                 bf16 for a bf16 pool; bf16 or f32 for an fp8 pool, encoded
 *                 with the pool's k_scale / v_scale)
 *   slot_mapping  device int64 [num_tokens]; slot = block * B + position;
 *                 a negative slot skips the token
 *   k_pool/v_pool device pools described by *c
 * Slots of one call must be distinct (two writes to one slot race).
 * Bytes of the pools outside the written slots are unchanged.  A call of 512
 * tokens or more runs a kernel that writes whole rows of the value tile
 * wherever B consecutive tokens fill a block in order, wherever in the call
 * they stand (a prefill's prompts may be laid end to end at any lengths), and
 * single elements elsewhere (a large decode batch's tokens); fewer tokens go
 * through a kernel of one workgroup per token.  The pools end the same either
 * way.
 */
int pkv_reshape_and_cache(const void* k, const void* v, int32_t in_dtype,
                          const int64_t* slot_mapping, int64_t num_tokens,
                          void* k_pool, void* v_pool, const pkv_cache_desc* c,
                          void* stream);

/*
 * copy_blocks -- the copy of copy-on-write (ithome, section 4): for every
 * (src, dst) pair, block dst of both pools becomes a bit copy of block src
 * (all heads, all B positions).
 *   src_dst_pairs device int64 [num_pairs][2]
 * Pairs must have src != dst, distinct dst, and no dst that is also a src, so
 * their order does not matter (the Python binding checks this on the host;
 * the library cannot see device data).  num_pairs == 0 launches nothing.
 */
int pkv_copy_blocks(void* k_pool, void* v_pool, const int64_t* src_dst_pairs,
                    int64_t num_pairs, const pkv_cache_desc* c, void* stream);

/*
 * append_tokens -- the decode step's cache write for a batch whose block tables
 * and context lengths stay on the device between steps.  Token i (batch row i)
 * is written like pkv_reshape_and_cache writes it to slot host_slots[i], and
 * the row's table entry and length are brought up to date:
 *   block_tables[i][host_positions[i] / B] = host_slots[i] / B
 *   context_lens[i] = host_positions[i] + 1
 * which is everything an append changes in them (a new block when the last was
 * full, or the copy that replaced a shared, partly filled last block -- the
 * block manager's slot for position pos is table[pos / B] * B + pos % B).
 *   k, v           device [num_tokens][Hkv][D] of in_dtype
 *   host_slots     host int64 [num_tokens]: the block manager's slots; < 0 skips
 *                  the token (its table row is left alone)
 *   host_positions host int32 [num_tokens]: each token's position in its sequence
 *   block_tables, context_lens  device int32 [rows][max_blocks_per_seq], [rows]
 * The host arrays travel in the kernel arguments (256 tokens per launch), so
 * nothing is uploaded.  PKV_E_INVAL, before any launch, for a slot outside the
 * pool or a position that does not match its slot (pos % B != slot % B, or
 * pos / B >= max_blocks_per_seq).
 */
int pkv_append_tokens(const void* k, const void* v, int32_t in_dtype,
                      const int64_t* host_slots, const int32_t* host_positions,
                      int32_t num_tokens, void* k_pool, void* v_pool, const pkv_cache_desc* c,
                      int32_t* block_tables, int32_t max_blocks_per_seq, int32_t* context_lens,
                      void* stream);

/*
 * swap_blocks -- move whole blocks (K and V) between two pools of the same block
 * shape (c's heads, block size, head_dim and dtype): the device pool and a host
 * pool, in either direction (review of the vLLM paper, the preemption
 * paragraphs: swapping KV out to host memory and back).  For each pair (src,
 * dst) block dst of dst_k / dst_v becomes block src of src_k / src_v.
 *   src_*, dst_*     pools: device memory, or pinned host memory allocated with
 *                    hipHostMalloc (torch's pin_memory), caller-owned, 16-byte
 *                    aligned; src_num_blocks / dst_num_blocks are their sizes
 *   src_dst_pairs    pkv_swap_blocks: device int64 [num_pairs][2]; ids out of
 *                    range are skipped; destinations must be distinct (the
 *                    caller's duty, as for pkv_copy_blocks).
 *                    pkv_swap_blocks_dma: host int64 [num_pairs][2], checked on
 *                    the host (PKV_E_INVAL before any copy).
 * pkv_swap_blocks runs one kernel that copies every block with the GPU's own
 * loads and stores across the host link.  pkv_swap_blocks_dma issues one
 * copy-engine transfer per run of pairs that are consecutive on both sides (K
 * and V apart) -- the per-block transfer whose cost for small blocks the page
 * points out.  Both are asynchronous on `stream`.
 */
/* What kind of memory p points into, as the swap calls see it: 2 device memory,
 * 1 pinned host memory mapped for the GPU at the same address, 0 anything else
 * (pageable host memory, unknown pointers, NULL) -- which they refuse. */
int32_t pkv_memory_kind(const void* p);
int pkv_swap_blocks(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                    const int64_t* src_dst_pairs, int64_t num_pairs, int32_t src_num_blocks,
                    int32_t dst_num_blocks, const pkv_cache_desc* c, void* stream);
int pkv_swap_blocks_dma(const void* src_k, const void* src_v, void* dst_k, void* dst_v,
                        const int64_t* src_dst_pairs, int64_t num_pairs, int32_t src_num_blocks,
                        int32_t dst_num_blocks, const pkv_cache_desc* c, void* stream);

/*
 * Bytes of device workspace a decode call needs (0 only for an empty batch or
 * invalid sizes): a header, one record per (sequence, head) and the
 * (max, sum, output) rows of split contexts -- the matrix-core kernel's two
 * slots per persistent worker (at most 4096 workers, 16 heads per group) or
 * the vector kernel's partitions, whichever is larger.  A workspace serves one
 * call at a time; calls on different streams need their own.  It needs no
 * initialisation: every call writes what it later reads.
 */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                  int32_t max_context_len, int32_t partition_size);

/*
 * paged_attn_decode -- one new query per sequence attends over its cached
 * context through its block table (glossary "How paging works"; optiverse
 * "Block table and non-contiguous allocation"); query heads share KV heads in
 * contiguous groups of num_q_heads / num_kv_heads (grouped-query attention,
 * glossary "Related techniques").
 *
 *   q             device [num_seqs][num_q_heads][D] of q_dtype (f32 with an
 *                 f32 pool, bf16 with bf16 / fp8 pools)
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq]; entries past
 *                 ceil(ctx / B) are never read
 *   context_lens  device int32 [num_seqs]; tokens 0..ctx-1, including the one
 *                 being decoded (written by reshape_and_cache beforehand);
 *                 ctx == 0 gives zeros
 *   scale         softmax scale applied to q.k (e.g. 1/sqrt(D))
 *   out           device [num_seqs][num_q_heads][D] of q_dtype
 *   max_context_len  host-side upper bound of context_lens (sizes the grid
 *                 without reading device data); larger contexts are cut at it
 *   partition_size   0 or a multiple of B.  Vector kernel: 0 = one pass over
 *                 each context, else a context of ctx tokens is split into
 *                 max(1, ctx / P) partitions of P tokens, the last one also
 *                 taking the remainder, run in parallel and merged.  MFMA
 *                 kernel: the batch's steps are shared out evenly over the
 *                 persistent workers (as many as fit on the device, half as
 *                 many for a batch of few long (sequence, head) pairs; only
 *                 those that can get steps are launched), each taking at
 *                 least P tokens (0 = no
 *                 lower bound) as long as that leaves at least half the
 *                 workers some steps; contexts that cross a worker boundary
 *                 are merged.
 *   workspace     device buffer of >= pkv_decode_workspace_bytes(...) bytes
 * The result does not depend on the split beyond rounding; for given context
 * lengths and partition_size it depends only on the logical order of each
 * context, not on where blocks sit in the pool or on what unused slots hold.
 */
int pkv_paged_attn_decode(const void* q, int32_t q_dtype,
                          const void* k_pool, const void* v_pool, const pkv_cache_desc* c,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t num_seqs,
                          int32_t num_q_heads, float scale, void* out,
                          int32_t max_context_len, int32_t partition_size,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Decode kernel families (low byte of `impl`), for tests and benchmarks that pin one,
 * and hints (high bits). */
typedef enum {
  PKV_IMPL_AUTO = 0,     /* matrix-core kernel where built, else the vector kernel */
  PKV_IMPL_VECTOR = 1,   /* plain vector-ALU kernel: every dtype, fp32 arithmetic */
  PKV_IMPL_MFMA = 2,     /* bf16 / fp8 pools: QK^T and P.V on MFMA, group size <= 16 */
  PKV_IMPL_FAMILY_MASK = 0xff,
  /* Hint: some blocks are shared by several sequences of the batch (forked
   * samples, beam search).  The MFMA kernel then reads K/V with ordinary
   * cached loads so the other readers hit in L2 / Infinity Cache; without the
   * hint it streams them (non-temporal loads), which is faster when every
   * block is read once.  The cached loads allocate lines in the last-level
   * cache: when it holds dirty lines of earlier work (a large write just
   * before the decode) they pay for writing those back and can be slower than
   * streaming even with sharing.  The result is the same either way. */
  PKV_IMPL_SHARED_BLOCKS = 0x100
} pkv_decode_impl;

/* pkv_paged_attn_decode with an explicit kernel family and hints (PKV_E_UNSUPPORTED if the
 * family is not built for the pool's dtype). */
int pkv_paged_attn_decode_ex(const void* q, int32_t q_dtype,
                             const void* k_pool, const void* v_pool, const pkv_cache_desc* c,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t num_seqs,
                             int32_t num_q_heads, float scale, void* out,
                             int32_t max_context_len, int32_t partition_size,
                             void* workspace, size_t workspace_bytes, void* stream,
                             int32_t impl);

/*
 * The two phases of pkv_paged_attn_decode, for callers that time or schedule
 * them apart.
 *
 * pkv_paged_attn_partials -- same arguments as pkv_paged_attn_decode_ex.
 *   A context computed in one piece gets its output written to `out`; the
 *   others leave, per piece and q head, the running max (log2 units), running
 *   sum and normalised partial output in `workspace` for pkv_paged_attn_merge.
 *   The vector kernel's pieces are the partitions of partition_size tokens;
 *   the MFMA kernel's pieces are the parts of a context that fall to different
 *   persistent workers (each worker takes an equal share of all 32-token steps
 *   of the batch, and at least partition_size tokens when that is non-zero and
 *   leaves at least half the workers some steps).
 * pkv_paged_attn_merge -- combines the pieces of every context that has more
 *   than one, out = sum_p w_p o_p / sum_p w_p with w_p = l_p * 2^(m_p - max m)
 *   (the rescaling of the running softmax, FlashAttention-style tiling,
 *   glossary "Related techniques"), and writes zeros for empty contexts.
 *   Arguments must match the partials call; the workspace header says which
 *   kernel family wrote the pieces.
 */
int pkv_paged_attn_partials(const void* q, int32_t q_dtype,
                            const void* k_pool, const void* v_pool, const pkv_cache_desc* c,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_q_heads, float scale, void* out,
                            int32_t max_context_len, int32_t partition_size,
                            void* workspace, size_t workspace_bytes, void* stream,
                            int32_t impl);
int pkv_paged_attn_merge(int32_t q_dtype, const int32_t* context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t max_context_len, int32_t partition_size, const void* workspace,
                         size_t workspace_bytes, void* out, void* stream);

/* Timing hook for benchmarks: the calling thread's next decode-kernel launch
 * (the first phase of any decode entry point on this thread) records its own
 * start and end in these events, through hipExtLaunchKernel, so that their
 * elapsed time is the kernel's alone, without the idle time that separate
 * event records leave around it.  Both events are the caller's hipEvent_t,
 * created with timing enabled; (NULL, NULL) cancels.  Returns PKV_OK, or
 * PKV_E_INVAL when only one event is given. */
int pkv_time_next_decode(void* start_event, void* stop_event);

/*
 * paged_attn_decode_noalloc -- pkv_paged_attn_decode without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  The call allocates
 * nothing (no hipMalloc, no library allocation); the partial results and piece
 * records live in a static device array of pkv_decode_scratch_bytes() bytes
 * (40 MiB) that every device the library runs on holds until the process ends.
 *
 * Arguments, layouts and results as pkv_paged_attn_decode_ex (impl as there;
 * the same kernels run, so the output is the same bit for bit).  The scratch
 * a batch needs is the piece rows of the kernel that runs: two head groups of
 * (head_dim + 2) floats per persistent worker for the matrix-core kernel (for
 * instance 4.3 MB with 1024 workers at 4 query heads per KV head and
 * head_dim 128), or one row per (sequence, query head, partition) for the
 * vector kernel with partitions, plus 8 bytes per (sequence, query head).  A
 * batch needing more returns PKV_E_INVAL (use the workspace entry point); the
 * other errors are pkv_paged_attn_decode_ex's.  Every call on a device shares
 * that device's array and overwrites it: calls that overlap on one device (on
 * two streams, or from two threads) race and must be serialised by the caller.
 */
size_t pkv_decode_scratch_bytes(void);
int pkv_paged_attn_decode_noalloc(const void* q, int32_t q_dtype, const void* k_pool,
                                  const void* v_pool, const pkv_cache_desc* c,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t num_seqs,
                                  int32_t num_q_heads, float scale, void* out,
                                  int32_t max_context_len, int32_t partition_size, void* stream,
                                  int32_t impl);

/* ------------------------------------------------------------------ shared-prefix decode
 *
 * Sequences forked from one prompt point their block tables at the same
 * physical blocks for the prompt (ithome, section 4, "Physical block
 * sharing"; glossary "Sharing blocks between sequences").  The keys and
 * values of those blocks are the same bytes for every sharer, so the decode
 * can read them once and score all the sharers' queries against them: the
 * matrix-core kernel has 32 query columns (two 16-column tiles), of which a
 * head group uses num_q_heads / num_kv_heads.  The result is the same attention as
 * pkv_paged_attn_decode gives (softmax over each sequence's whole context),
 * up to rounding: a member's running softmax goes on from the shared tokens
 * to its own, and a unit split between workers is merged as a split context
 * is.
 *
 * Units: the decode runs over units instead of sequences.  Unit u is int32
 * [4] {seq0, shared_tokens, members, reread}: the `members` consecutive
 * sequences seq0 .. seq0 + members - 1 (at most 32 / group) hold the same
 * block ids over their first shared_tokens tokens (a multiple of block_size,
 * at most every member's context length).  The kernel reads those tokens
 * once, through seq0's table, scoring every member's queries, then each
 * member's remaining tokens through its own table.  reread = 1 marks a unit
 * whose shared blocks other units or sequences of the batch read too (a prompt
 * with more sharers than one unit holds); the kernel does not read the field,
 * it tells the caller to pass PKV_IMPL_SHARED_BLOCKS (below).  seq_rows[s] =
 * {unit, member index within the unit, 0, 0}.  A unit {s, 0, 1, 0} is a plain
 * sequence.
 */

/* Build the units for a batch on the host: runs of consecutive sequences (at
 * most 32 / group) whose tables start with the same >= min_shared_blocks
 * block ids share those blocks, kept below each member's last block.  A
 * unit's reread is 1 when sequences outside it start with its first block
 * too (a prompt with more sharers than one unit holds).
 *   tables   host int32 [num_seqs][max_blocks] (the batch's block tables)
 *   lens     host int32 [num_seqs] context lengths
 *   rows     host int32 [num_seqs][4] out (units); seq_rows host int32 [num_seqs][4] out
 * Returns the number of units (1 .. num_seqs; 0 for an empty batch) or a
 * negative pkv_status. */
int32_t pkv_prefix_rows(const int32_t* tables, const int32_t* lens, int32_t num_seqs,
                        int32_t max_blocks, int32_t block_size, int32_t group,
                        int32_t min_shared_blocks, int32_t* rows, int32_t* seq_rows);

/* A batch order that makes sharers consecutive, for batches whose sharers are
 * interleaved: order[k] = the batch index of the sequence that goes k-th.
 * Sequences are sorted by the block ids of their full blocks before their last
 * token, compared lexicographically (equal ones keep their batch order), so
 * every run of shared leading blocks is one contiguous range.  Reordering the
 * batch (q rows, tables, lengths, and reading the outputs back in that order)
 * is the caller's.
 *   tables, lens as pkv_prefix_rows; order host int32 [num_seqs] out
 * Returns PKV_OK or a negative pkv_status. */
int32_t pkv_prefix_order(const int32_t* tables, const int32_t* lens, int32_t num_seqs,
                         int32_t max_blocks, int32_t block_size, int32_t* order);

/* Workspace bytes of pkv_paged_attn_decode_rows for num_rows units (0 on
 * invalid arguments): a header, one record per (unit, KV head) and the
 * persistent workers' partial-segment slots (two of 32 rows each). */
size_t pkv_rows_workspace_bytes(const pkv_cache_desc* c, int32_t num_rows);

/* Decode attention over units (see above); arguments as pkv_paged_attn_decode,
 * plus rows / seq_rows (device int32 [num_rows][4] / [num_seqs][4], 16-byte
 * aligned, e.g. uploaded from pkv_prefix_rows) and phases: 1 the decode
 * kernel, 2 the merge, 3 both (1 then 2 on the same workspace and stream),
 * optionally or-ed with PKV_IMPL_SHARED_BLOCKS: read K and V with ordinary
 * loads instead of streaming them, which can pay when some unit has reread = 1
 * (its shared blocks are read again by other units of the launch and then hit
 * in the Infinity Cache) if the cache holds no dirty lines of earlier work,
 * and costs a few percent when no unit has it, much more after a large write
 * (see PKV_IMPL_SHARED_BLOCKS).  The result is the same either way.
 * bf16 or fp8 pools only (PKV_E_UNSUPPORTED for f32).  Unit fields are
 * trusted only as far as memory safety: out-of-range sequences and members
 * are cut, shared tokens are cut to whole blocks of seq0's context, and a
 * sequence whose seq_rows entry is out of range gets no output.  Outputs of
 * sequences whose units break the rules above are undefined. */
int pkv_paged_attn_decode_rows(const void* q, int32_t q_dtype,
                               const void* k_pool, const void* v_pool, const pkv_cache_desc* c,
                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                               const int32_t* context_lens, int32_t num_seqs,
                               int32_t num_q_heads, float scale, void* out,
                               int32_t max_context_len, int32_t partition_size,
                               const int32_t* rows, int32_t num_rows, const int32_t* seq_rows,
                               void* workspace, size_t workspace_bytes, void* stream,
                               int32_t phases);

/* ------------------------------------------------------------------ query-aware block selection
 *
 * QUEST (tencent cloud article 2526001, section "QUEST: Query-Aware Sparsity
 * for Efficient Long-Context LLM Inference"): each KV block carries the
 * channel-wise minimum and maximum of its keys; for a query q the bound
 * U = sum_d max(q_d * min_d, q_d * max_d) is never below q.k for any key k of
 * the block, and only the blocks with the budget_blocks largest bounds are
 * attended.  Readings where the page is silent:
 *  - the minimum / maximum run over the block's valid slots (the last block
 *    of a context may be partly filled);
 *  - the budget is in blocks; a context of no more blocks is attended whole
 *    (bit for bit as pkv_paged_attn_decode_ex with the same partition_size);
 *  - with grouped-query attention a (sequence, KV head) makes one choice for
 *    its query heads, ranking blocks by the largest bound over those heads;
 *  - equal bounds rank the lower logical block first; the chosen blocks are
 *    attended in logical order, the softmax running over their tokens only.
 * The bounds are summed in fp32 (unscaled q and stored key values); blocks
 * whose bounds differ by less than that rounding may rank either way.
 *
 * Metadata: device [num_blocks][num_kv_heads][2][head_dim] of the pool's
 * kv_dtype, pkv_quest_meta_bytes(c) bytes; row 0 the minimum, row 1 the
 * maximum (stored codes, exact: min / max of values of a type are values of
 * it).  For an fp8 pool a channel holding both zeros stores -0 as its minimum
 * and +0 as its maximum, and a NaN key becomes its channel's maximum (code
 * 0x7F) or minimum (0xFF).  The caller keeps it current after writing keys: a
 * block's entry covers its first `count` slots as of the last update.
 */
size_t pkv_quest_meta_bytes(const pkv_cache_desc* c);

/* Recompute the metadata of blocks[i] over its first counts[i] slots, all heads.
 * blocks, counts: device int32 [n].  Entries with a block outside the pool or a
 * count outside [1, block_size] are skipped.  blocks must be distinct. */
int pkv_quest_update_blocks(const void* k_pool, const pkv_cache_desc* c, void* meta,
                            const int32_t* blocks, const int32_t* counts, int32_t n,
                            void* stream);

/* Blocks touched by a cache write to host slots[0 .. n) (negative slots skipped), for
 * pkv_quest_update_blocks: the distinct blocks slot / block_size in ascending order, each
 * with the fill its highest written slot implies (slot % block_size + 1; a block's slots
 * fill in order).  Writes min(count, cap) entries to blocks / fills (host int32) and
 * returns the count, or a negative pkv_status (PKV_E_INVAL on bad arguments). */
int32_t pkv_quest_blocks_of_slots(const int64_t* slots, int64_t n, int32_t block_size,
                                  int32_t* blocks, int32_t* fills, int32_t cap);

/* The decode step's update, from device-resident tables: for every row, the block
 * holding its last token (context_lens - 1) over its first (context_lens - 1) % B + 1
 * slots.  Rows that share that block must agree on its fill (they do whenever the
 * shared block was copied on write before another row appended to it). */
int pkv_quest_update_tails(const void* k_pool, const pkv_cache_desc* c, void* meta,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* context_lens, int32_t num_seqs, void* stream);

/* Workspace bytes of pkv_quest_decode (0 on invalid sizes; the message says why); it
 * also serves pkv_quest_select.  Contexts may hold at most 16384 blocks. */
size_t pkv_quest_workspace_bytes(const pkv_cache_desc* c, int32_t num_seqs,
                                 int32_t num_q_heads, int32_t max_blocks_per_seq,
                                 int32_t max_context_len, int32_t partition_size,
                                 int32_t budget_blocks);

/*
 * The selection alone.  For pair p = s * num_kv_heads + kvh:
 *   sel_tables  device int32 [num_seqs * num_kv_heads][min(max_blocks_per_seq,
 *               budget_blocks)]: the chosen blocks in logical order, each as
 *               block * num_kv_heads + kvh (-1 for a table entry outside the pool)
 *   sel_lens    device int32 [num_seqs * num_kv_heads]: tokens of the chosen blocks
 * Other arguments as pkv_paged_attn_decode (max_context_len cuts contexts alike).
 */
int pkv_quest_select(const void* q, int32_t q_dtype, const void* meta, const pkv_cache_desc* c,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                     int32_t max_context_len, int32_t budget_blocks, int32_t* sel_tables,
                     int32_t* sel_lens, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention over the QUEST-chosen blocks: pkv_quest_select into the
 * workspace, then the decode kernels of pkv_paged_attn_decode_ex (family and
 * hints from `impl`) over one-head "sequences" (sequence, KV head), whose
 * tables address the pools as [num_blocks * num_kv_heads] one-head blocks.
 * Arguments as pkv_paged_attn_decode_ex plus `meta` and budget_blocks >= 1.
 */
int pkv_quest_decode(const void* q, int32_t q_dtype, const void* k_pool, const void* v_pool,
                     const void* meta, const pkv_cache_desc* c, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t num_seqs,
                     int32_t num_q_heads, float scale, void* out, int32_t max_context_len,
                     int32_t partition_size, int32_t budget_blocks, void* workspace,
                     size_t workspace_bytes, void* stream, int32_t impl);

/* ------------------------------------------------------------------ measurement aid
 *
 * read_probe -- a plain HBM read of num_tiles tiles of tile_bytes bytes each:
 * the rate a bare read stream reaches on the device, the reference beside the
 * decode kernel's KV-read rate (the decode reads the pools block by block
 * through the tables: ithome article, section 3; glossary, "How paging works").
 *
 *   buf          device, buf_bytes bytes, 16-byte aligned; only read
 *   tile_bytes   power of two >= 16 (4096 = one bf16 (block, KV head) tile of the
 *                key pool at B = 16, D = 128)
 *   tile_ids     device int64 [num_tiles]: tile i is read at byte offset
 *                tile_ids[i] * tile_bytes (ids outside the buffer read tile 0);
 *                NULL reads tiles 0 .. num_tiles - 1 in order (a sequential
 *                stream; then num_tiles * tile_bytes <= buf_bytes)
 *   sink         device uint32 [workgroups * 64], 16-byte aligned: one word per
 *                lane, the XOR of what it read (keeps the loads live)
 *   workgroups   one-wave (64-lane) workgroups of the launch; the tiles, in
 *                list order, are cut into equal contiguous shares, one per wave
 *                (1024 puts one wave on every SIMD of a 256-CU device)
 * The tiles must add up to whole 1 KB rows (one load instruction of a wave),
 * and tiles read through ids must hold at least 1 KB.  Not part of the paged
 * path.  Errors: PKV_E_INVAL for a NULL or misaligned pointer, a tile size
 * that is no power of two, tiles that break those rules, or a sequential read
 * past the buffer; PKV_E_HIP if the launch fails.
 */
int pkv_read_probe(const void* buf, size_t buf_bytes, int64_t tile_bytes, const int64_t* tile_ids,
                   int64_t num_tiles, uint32_t* sink, int32_t workgroups, void* stream);

/* Message of the last failure on the calling thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

/* ------------------------------------------------------------------ host block manager
 *
 * Refcounted block allocator (ithome sections 3-4; glossary "How paging works"
 * and "Sharing blocks between sequences"; optiverse "Block table ...").
 *  - Blocks are taken from the head of the free list (glossary code example,
 *    free_blocks.pop(0)), a new one only when the last block is full.
 *  - fork shares every block of the parent (count + 1).
 *  - append to a sequence whose last block is shared and partly filled takes a
 *    new block, reports the (old, new) pair to copy, and drops the old block's
 *    count; full shared blocks stay shared.
 *  - free_seq drops one count per block; blocks reaching 0 are appended to the
 *    tail of the free list in the sequence's logical order.
 *  - Every operation is all-or-nothing: PKV_E_NOMEM / PKV_E_INVAL leave the
 *    state unchanged.
 * Not thread-safe: one owner thread per manager.
 */
typedef struct pkv_bm pkv_bm;

typedef struct {
  int32_t free_blocks, used_blocks;
  int64_t tokens, slots_allocated, logical_blocks, physical_blocks;
} pkv_bm_stats_t;

/* free_order: the initial free list, head first (distinct ids in [0, num_blocks);
 * blocks not listed are held elsewhere); NULL = 0..num_blocks-1.  NULL on error. */
pkv_bm* pkv_bm_create(int32_t num_blocks, int32_t block_size, const int32_t* free_order,
                      int32_t free_count);
void pkv_bm_destroy(pkv_bm* bm);
/* admit seq holding num_tokens tokens: ceil(num_tokens / B) blocks */
int pkv_bm_add_seq(pkv_bm* bm, int64_t seq, int64_t num_tokens);
int pkv_bm_fork(pkv_bm* bm, int64_t parent, int64_t child);
/* slot of the next token; *cow_src / *cow_dst = the copy pair or -1 */
int pkv_bm_append(pkv_bm* bm, int64_t seq, int64_t* slot, int64_t* cow_src, int64_t* cow_dst);
/* one token for each of n distinct sequences, in the order given (pass ascending ids);
 * slots[n]; pairs[2 * n] receives *num_pairs (src, dst) pairs */
int pkv_bm_append_batch(pkv_bm* bm, const int64_t* seqs, int32_t n, int64_t* slots,
                        int64_t* pairs, int32_t* num_pairs);
/* n tokens for one sequence: slots[n]; at most one copy pair (the first token) */
int pkv_bm_extend(pkv_bm* bm, int64_t seq, int64_t n, int64_t* slots, int64_t* cow_src,
                  int64_t* cow_dst);
int pkv_bm_free_seq(pkv_bm* bm, int64_t seq);
/* slots of positions start .. start+n-1 (all < the sequence's length) */
int pkv_bm_slots(pkv_bm* bm, int64_t seq, int64_t start_pos, int64_t n, int64_t* out);
/* tables [n][max_blocks] (padding -1) and context lengths [n] of the listed sequences */
int pkv_bm_block_tables(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* tables,
                        int32_t max_blocks, int32_t* context_lens);
int pkv_bm_stats(pkv_bm* bm, pkv_bm_stats_t* out);
/* reference count of a block (-1 if out of range) */
int32_t pkv_bm_refcount(pkv_bm* bm, int32_t block);
/* number of tokens of seq (-1 if unknown) */
int64_t pkv_bm_seq_len(pkv_bm* bm, int64_t seq);
/* copy the free list (head first) into out[cap]; returns its length */
int32_t pkv_bm_free_list(pkv_bm* bm, int32_t* out, int32_t cap);

/* ------------------------------------------------------------------ prefix caching
 *
 * Full blocks found again by their tokens and every token before them (review of
 * the vLLM paper, the paragraphs on prefix caching; glossary "Sharing blocks
 * between sequences"), so a request whose prompt starts with full blocks an
 * earlier request computed reuses them (multi-turn dialogue, shared system
 * prompts).
 *  - Keys are exact token prefixes (a trie, no hashing: two prefixes never
 *    collide).  Only full blocks have keys; a lookup takes the longest run of
 *    cached full blocks from the start of the prompt.
 *  - A cached block whose count falls to zero keeps its key and becomes
 *    evictable; a lookup that finds it revives it.  Blocks come from the free
 *    list first, then from the evictable block released longest ago, which
 *    loses its key.  A released sequence's cached blocks join the evictable
 *    queue last block first (a prefix outlives the blocks that extend it); its
 *    uncached blocks return to the free list's tail in logical order.
 *  - A block that fills takes its key unless another block already holds it.
 *  - Only sequences admitted with their tokens (pkv_bm_add_seq_tokens) take
 *    part; sequences admitted by count never hit and never register.  Forks
 *    inherit their parent's tokens.
 * Token ids are int32 host arrays owned by the caller.
 *
 * pkv_bm_set_prefix_caching -- turn caching on (1) or off (0); only while the
 *   manager holds no sequence (PKV_E_INVAL otherwise).  Off returns the
 *   evictable blocks to the free list in queue order.
 * pkv_bm_lookup -- tokens a prompt would find cached (a multiple of B), no change.
 * pkv_bm_add_seq_tokens -- admit a sequence with its n tokens; *cached_tokens
 *   receives how many leading tokens were found cached (their KV is already in
 *   the pool; the caller writes tokens [*cached_tokens, n) only).
 *   All-or-nothing; PKV_E_NOMEM counts cached blocks it would revive.
 * pkv_bm_append_batch_tokens / pkv_bm_extend_tokens -- pkv_bm_append_batch /
 *   pkv_bm_extend with the new tokens' ids, so blocks they fill get keys.
 * pkv_bm_cache_stats -- out[0] cached blocks, out[1] evictable blocks,
 *   out[2] prompt tokens found cached, out[3] prompt tokens looked up.
 * pkv_bm_evictable_list -- the evictable queue, released longest ago first
 *   (returns its length; copies at most cap entries).
 */
int pkv_bm_set_prefix_caching(pkv_bm* bm, int32_t enable);
int pkv_bm_lookup(pkv_bm* bm, const int32_t* tokens, int64_t n, int64_t* cached_tokens);
int pkv_bm_add_seq_tokens(pkv_bm* bm, int64_t seq, const int32_t* tokens, int64_t n,
                          int64_t* cached_tokens);
int pkv_bm_append_batch_tokens(pkv_bm* bm, const int64_t* seqs, const int32_t* tokens, int32_t n,
                               int64_t* slots, int64_t* pairs, int32_t* num_pairs);
int pkv_bm_extend_tokens(pkv_bm* bm, int64_t seq, const int32_t* tokens, int64_t n,
                         int64_t* slots, int64_t* cow_src, int64_t* cow_dst);
int pkv_bm_cache_stats(pkv_bm* bm, int64_t* out);
int32_t pkv_bm_evictable_list(pkv_bm* bm, int32_t* out, int32_t cap);

/* ------------------------------------------------------------------ swapping
 *
 * Preemption by swapping (review of the vLLM paper, the preemption paragraphs):
 * a set of sequences not needed for now moves its KV to a host pool, freeing
 * device blocks, and moves back when there is room.  The host pool has the
 * device pool's block shape (the caller allocates it in pinned host memory;
 * pkv_swap_blocks moves the data).
 *  - A set moves together; every block one of its sequences holds must be held
 *    only by sequences of the set (forked samples move together), so a shared
 *    block moves once and keeps its count.  Otherwise PKV_E_INVAL.
 *  - Distinct blocks are taken in order of first appearance (sequences in the
 *    order given, blocks in logical order).  The receiving pool's free list
 *    (head) supplies new blocks; the giving pool's blocks return to the tail of
 *    its free list in that order.  Device blocks leave without their
 *    prefix-cache keys; blocks that come back carry none.
 *  - The returned (src, dst) pairs -- device->host for swap-out, host->device
 *    for swap-in -- must be copied before any later write reuses a block.
 *  - A swapped-out sequence can only be swapped in or released (releasing
 *    returns its host blocks); other calls on it give PKV_E_INVAL.
 *  - All-or-nothing: PKV_E_NOMEM when the receiving pool lacks blocks.
 *
 * pkv_bm_set_host_pool -- (re)create a host pool of num_host_blocks blocks,
 *   free list 0..n-1; PKV_E_INVAL while a sequence is swapped out.
 * pkv_bm_swap_out / pkv_bm_swap_in -- pairs: caller array of cap int64 pairs;
 *   *num_pairs receives the number of pairs (also when cap is too small, which
 *   gives PKV_E_INVAL with nothing changed).
 * pkv_bm_swap_stats -- out[0] free host blocks, out[1] host blocks, out[2]
 *   swapped-out sequences.
 * pkv_bm_host_refcount / pkv_bm_host_free_list -- host-side counts and free list.
 * pkv_bm_seq_blocks -- a sequence's blocks (host blocks while swapped out);
 *   returns the count (copies at most cap) or -1 for an unknown sequence.
 */
int pkv_bm_set_host_pool(pkv_bm* bm, int32_t num_host_blocks);
int pkv_bm_swap_out(pkv_bm* bm, const int64_t* seqs, int32_t n, int64_t* pairs, int32_t cap,
                    int32_t* num_pairs);
int pkv_bm_swap_in(pkv_bm* bm, const int64_t* seqs, int32_t n, int64_t* pairs, int32_t cap,
                   int32_t* num_pairs);
int pkv_bm_swap_stats(pkv_bm* bm, int64_t* out);
int32_t pkv_bm_host_refcount(pkv_bm* bm, int32_t block);
int32_t pkv_bm_host_free_list(pkv_bm* bm, int32_t* out, int32_t cap);
int pkv_bm_seq_blocks(pkv_bm* bm, int64_t seq, int32_t* out, int32_t cap);

/* The distinct device blocks of sequences seqs[0 .. n) (none swapped out), in order of
 * first appearance, each with its filled slots: logical block j of a sequence of len
 * tokens holds min(B, len - j * B) of them, and a block shared by several sequences
 * takes the largest such count.  This is what the QUEST metadata of those blocks must
 * cover (pkv_quest_update_blocks).  Writes min(count, cap) entries to blocks / fills and
 * returns the count; a negative pkv_status on error (unknown or swapped-out sequence). */
int32_t pkv_bm_block_fills(pkv_bm* bm, const int64_t* seqs, int32_t n, int32_t* blocks,
                           int32_t* fills, int32_t cap);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
