/*
 * pa.h -- C ABI of libpa, a paged-attention library for AMD MI355X (gfx950).
 *
 * The method: each sequence's K/V cache lives in fixed-size physical blocks
 * drawn from one pre-allocated pool; a per-sequence block table maps logical
 * block floor(pos / B) to a physical block id, and the token sits at offset
 * pos mod B inside it.  Attention for a query is softmax(q K^T * scale) V
 * over the sequence's keys, gathered through the table.  Passages defining
 * it: "High-Throughput Local LLM Infrastructure: Architecting a Distributed
 * Go API Gateway for vLLM & PagedAttention Clusters", section "1.2
 * PagedAttention Mechanics & Virtual Page Tables" (pool, block table, index
 * and offset equations, kernels taking the block table as a lookup
 * argument); "03 -- PagedAttention & the vLLM V1 Architecture", section "The
 * attention kernel side"; "Inside vLLM: Anatomy of a High-Throughput LLM
 * Inference System (2025)", section "Physical Block Mapping and Kernel
 * Invocation".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or retains memory, holds no mutable
 *    global state and is re-entrant -- except pa_decode_noalloc, whose
 *    workspace is a static device array (see its comment).
 *  - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *    Work is enqueued on it and the call returns once it is enqueued, so
 *    stream order gives slot mapping -> cache write -> attention.
 *  - No entry point synchronises the stream, allocates device memory or
 *    memsets on its own (PA_CHECK=1 below aside), so a step -- cache write
 *    and attention, with output and workspace allocated beforehand -- can
 *    be captured in a HIP graph and replayed.
 *  - The return value is a pa_status, known synchronously.  Argument
 *    checks (null pointers, sizes, head counts, dtype, workspace size) are
 *    made before anything is enqueued.  A failed launch returns PA_ERR_HIP.
 *  - Metadata that lives on the device (block tables, seq_lens, slots,
 *    query_start_loc) cannot be checked without a copy.  Kernels stay
 *    memory-safe on any values (indices are clamped or skipped), but
 *    out-of-contract values give unspecified results.  With the environment
 *    variable PA_CHECK=1 the library copies that metadata to the host,
 *    validates it (ranges, seq_len >= 1, seq_len <= max_blocks_per_seq * B,
 *    q_len <= seq_len, no duplicate slot), synchronises the stream and
 *    returns PA_ERR_INDEX on a violation.
 *
 * Layouts (one attention layer; e = element size)
 * -----------------------------------------------
 *   k_cache       [num_blocks, H_kv, B, D]   token rows, head_dim contiguous
 *   v_cache       [num_blocks, H_kv, D, B]   head_dim rows, B tokens contiguous
 *   query, out    [T, H_q, D]                packed rows (T = tokens this step)
 *   key, value    [T, H_kv, D]               this step's new K/V
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]
 *   seq_lens      int32 [num_seqs]   tokens per sequence INCLUDING this step's
 *   query_start_loc int32 [num_seqs + 1]; rows of sequence s are
 *                 [qsl[s], qsl[s+1]), at positions seq_len - q_len .. seq_len-1
 *   slot_mapping  int64 [T]; slot = block_id * B + offset; < 0 = skip
 *  Query head h reads KV head h / (H_q / H_kv).  A query at position P sees
 *  keys 0..P.  `out` has the dtype of `query`.
 *
 * Supported: dtype PA_F32 or PA_BF16; head_dim 64 or 128; block_size a
 * power of two from 1 to 64; H_q % H_kv == 0 with 1 <= H_q / H_kv <= 16;
 * kv_split_tokens 0 (auto) or a positive multiple of 64.
 *
 * Where this ABI departs from the plainest reading of the pages
 * -------------------------------------------------------------
 * The pages fix no intra-block layout and no argument list; the one a
 * caller would first expect is K and V both token-major, [NB, H_kv, B, D],
 * and the three calls with only the arguments the method names.  Here:
 *  - v_cache is head_dim-major, [NB, H_kv, D, B].  A lane then loads 8
 *    consecutive tokens of one head_dim column as one 16-byte load, which is
 *    the B operand of the P.V matrix instruction as it stands.  K stays
 *    token-major.  A caller holding token-major V pools must transpose each
 *    block once (torch: v.transpose(2, 3).contiguous()) or fill the pool
 *    through pa_reshape_and_cache, which writes this layout.  Passing a
 *    token-major V pool is NOT detected by the library (its size is the
 *    same) and gives wrong attention; the Python binding refuses it by
 *    shape whenever B != D.
 *  - pa_decode and pa_chunked_prefill take two more arguments:
 *    block_refcounts (a cache hint, may be NULL) and kv_split_tokens
 *    (0 = balanced; the workspace queries take it too, and the value must
 *    match).
 *  - dtype is passed as int32_t and the stream as void* (a hipStream_t), so
 *    this header needs no HIP header.
 *  - Added entry points: pa_compute_slot_mapping (the slot step on the
 *    device), pa_version, the e4m3 cache calls, pa_decode_shared_prefix,
 *    the whole-block copies, and pa_decode_append / pa_decode_fp8_append /
 *    pa_decode_shared_prefix_append (slot computation, cache write and
 *    decode of one step in one call).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,        /* a required pointer is NULL                    */
  PA_ERR_SHAPE = -2,       /* a size or count is out of range / inconsistent */
  PA_ERR_DTYPE = -3,       /* unknown dtype                                  */
  PA_ERR_UNSUPPORTED = -4, /* valid but not implemented (head_dim, B, G)     */
  PA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required        */
  PA_ERR_INDEX = -6,       /* PA_CHECK=1 found bad device metadata           */
  PA_ERR_HIP = -7,         /* a HIP runtime call or a launch failed          */
  PA_ERR_SCRATCH = -8      /* pa_decode_noalloc: needs more than its scratch */
} pa_status;

/* Human-readable name of a pa_status value (static string, never NULL). */
const char* pa_status_string(int status);

/* Library version as major * 10000 + minor * 100 + patch. */
int pa_version(void);

/*
 * pa_compute_slot_mapping -- slot of every query token.
 * Defined by the index and offset equations (logical block = floor(pos/B),
 * offset = pos mod B) in "High-Throughput Local LLM Infrastructure ...",
 * section "1.2 PagedAttention Mechanics & Virtual Page Tables".
 *   slot_mapping[qsl[s] + j] = block_tables[s][pos / B] * B + pos % B,
 *   pos = seq_lens[s] - q_len_s + j.
 * query_start_loc may be NULL: one query token per sequence (decode), and
 * then num_tokens must equal num_seqs.  Tokens whose position is negative or
 * beyond the table get slot -1.
 */
int pa_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t num_seqs,
                            int32_t num_tokens, int32_t block_size,
                            void* stream);

/*
 * pa_reshape_and_cache -- write this step's K/V into their cache slots.
 * The write of newly computed K/V into the physical blocks a sequence was
 * assigned: "High-Throughput Local LLM Infrastructure ...", section "2.1
 * PagedAttention Memory Allocation Life-Cycle", step 4.
 *   k_cache[slot / B][h][slot % B][:] = key[t][h][:]
 *   v_cache[slot / B][h][:][slot % B] = value[t][h][:]
 * for every token t with 0 <= slot < num_blocks * B.  Values are copied bit
 * for bit.  Two tokens with one slot race (forbidden; PA_CHECK reports it).
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache,
                         void* v_cache, const int64_t* slot_mapping,
                         int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size,
                         int32_t num_blocks, int32_t dtype, void* stream);

/*
 * Workspace for pa_decode: partial results (running max, sum and
 * unnormalised output) of the pieces a row's keys are cut into, plus a small
 * header.  kv_split_tokens: 0 lets the library balance the work over the
 * GPU (every resident wave streams an equal share of all keys); a positive
 * multiple of 64 cuts every sequence into fixed splits of that many keys
 * instead.  Pass the same value to pa_decode.  Returns 0 for invalid
 * arguments.
 */
size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_seq_len,
                                 int32_t block_size, int32_t kv_split_tokens);

/*
 * pa_decode -- one query token per sequence against its paged K/V.
 * Attention definition: "03 -- PagedAttention & the vLLM V1 Architecture",
 * section "The attention kernel side"; gather: "Inside vLLM ...", section
 * "Physical Block Mapping and Kernel Invocation".
 *   out[s][h] = softmax_t(scale * query[s][h] . K_s[t][h/G]) . V_s[t][h/G],
 *   t = 0 .. seq_lens[s]-1, K_s/V_s gathered through block_tables[s].
 * block_refcounts (may be NULL) is int32 [num_blocks]: how many block tables
 * hold each physical block, the reference count of the block manager
 * ("High-Throughput Local LLM Infrastructure ...", section "1.2", reference
 * counting and copy-on-write).  It is a cache hint only: blocks with a count
 * above 1 (shared prefixes) are read through the caches so that every
 * sharer hits them; all other blocks are streamed with non-temporal loads.
 * NULL treats every block as private.  Results do not depend on it.
 * scale must be finite and > 0 (1/sqrt(head_dim) in the pages); other
 * values return PA_ERR_SHAPE.
 * max_seq_len must be >= every seq_len.  Keys of one row may be cut into
 * pieces (see pa_decode_workspace_bytes); their partial results are merged
 * exactly (log-sum-exp) in a second pass.
 */
int pa_decode(void* out, const void* query, const void* k_cache,
              const void* v_cache, const int32_t* block_tables,
              int32_t max_blocks_per_seq, const int32_t* block_refcounts,
              const int32_t* seq_lens,
              int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
              int32_t num_blocks, float scale, int32_t dtype,
              int32_t kv_split_tokens, void* workspace,
              size_t workspace_bytes, void* stream);

/*
 * pa_decode_append -- one decode step's slot computation, cache write and
 * attention in one call: the same results, bit for bit, as
 * pa_compute_slot_mapping (query_start_loc NULL), pa_reshape_and_cache with
 * those slots and pa_decode on the same arguments.  Slot computation: "High-
 * Throughput Local LLM Infrastructure ...", section "1.2 PagedAttention
 * Mechanics & Virtual Page Tables" (block index and offset of a logical
 * position); cache write: same page, section "2.1 PagedAttention Memory
 * Allocation Life-Cycle", step 4.
 * key, value: [num_seqs, num_kv_heads, head_dim] in dtype, the new token of
 * every sequence, written at position seq_lens[s] - 1 (slot
 * block_tables[s][(seq_lens[s]-1) / block_size] * block_size +
 * (seq_lens[s]-1) % block_size) of k_cache / v_cache, which the call
 * modifies; nothing is written for a sequence whose table entry there lies
 * outside [0, num_blocks) (a negative or out-of-range slot in
 * pa_reshape_and_cache).  The attention then includes that token.  On the
 * balanced decode (bf16, block_size >= 8, kv_split_tokens 0, up to 4096
 * sequences) everything happens in the attention launch: the wave that
 * reads a sequence's last key step takes the new token's K/V from key /
 * value and writes its slot once its work is done.  Other shapes write the
 * new tokens in a launch of their own before the attention.
 * Workspace as for pa_decode (pa_decode_workspace_bytes).  Two sequences
 * whose new tokens share a slot are undefined (PA_ERR_INDEX under
 * PA_CHECK); key or value NULL with num_seqs > 0 is PA_ERR_NULL.
 */
int pa_decode_append(void* out, const void* query, const void* key,
                     const void* value, void* k_cache, void* v_cache,
                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                     const int32_t* block_refcounts, const int32_t* seq_lens,
                     int32_t num_seqs, int32_t max_seq_len,
                     int32_t num_q_heads, int32_t num_kv_heads,
                     int32_t head_dim, int32_t block_size, int32_t num_blocks,
                     float scale, int32_t dtype, int32_t kv_split_tokens,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Workspace for pa_chunked_prefill: fp32 partials for the query-chunk rows
 * (num_tokens * num_q_heads rows) and an int32 piece count per such row,
 * fp32 pieces for the balanced decode of single-token rows
 * (num_seqs * num_q_heads rows) and a small header.
 * kv_split_tokens: 0 lets the library spread the chunk rows' keys evenly
 * over the GPU (each workgroup takes an equal run of 32-key steps of all
 * row tiles, so a tile may be cut into a few pieces); a positive multiple
 * of 64 fixes that run to kv_split_tokens keys instead (and, for fp32 or
 * small-block caches, the split size of the vector-ALU path, 2048 keys when
 * 0).  Pass the same value to pa_chunked_prefill.  Returns 0 for invalid
 * arguments.
 */
size_t pa_chunked_prefill_workspace_bytes(int32_t num_seqs, int32_t num_tokens,
                                          int32_t num_q_heads,
                                          int32_t head_dim,
                                          int32_t max_seq_len,
                                          int32_t block_size,
                                          int32_t kv_split_tokens);

/*
 * pa_chunked_prefill -- packed query chunks (and single decode rows) of
 * several sequences against their paged context, causally.  Chunked prefill
 * co-schedules prompt chunks with decode tokens ("Tech Radar: vLLM v1
 * Production Engine Architecture ...", section "3. Dynamic Chunked
 * Prefill"); the attention each row computes is the one of pa_decode with
 * the row's own causal limit: row j of sequence s sits at position
 * P = seq_lens[s] - q_len_s + j and sees keys 0..P.  Sequences with
 * q_len == 1 are decode rows and may be mixed in freely.
 * max_query_len must be >= every q_len and num_tokens == qsl[num_seqs].
 * block_refcounts and scale: as for pa_decode.  On the bf16 path at most
 * 2048 sequences per call, and K / V pools under 2^40 bytes each
 * (PA_ERR_UNSUPPORTED otherwise).
 */
int pa_chunked_prefill(void* out, const void* query, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables,
                       int32_t max_blocks_per_seq,
                       const int32_t* block_refcounts,
                       const int32_t* seq_lens,
                       const int32_t* query_start_loc, int32_t num_seqs,
                       int32_t num_tokens, int32_t max_seq_len,
                       int32_t max_query_len, int32_t num_q_heads,
                       int32_t num_kv_heads, int32_t head_dim,
                       int32_t block_size, int32_t num_blocks, float scale,
                       int32_t dtype, int32_t kv_split_tokens,
                       void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Whole-block copies.  Copy-on-write copies a shared block into a fresh one
 * before a sequence writes into it ("03 -- PagedAttention & the vLLM V1
 * Architecture", section "The block table walkthrough"; "High-Throughput
 * Local LLM Infrastructure ...", section "Reference Counting &
 * Copy-on-Write (CoW)"); preemption by swapping moves a sequence's blocks to
 * pinned host memory and back ("03 -- ...", section "Preemption &
 * eviction"; "Inside vLLM ...", section "Preemption Mechanics: Swapping vs.
 * Recomputation").
 *
 * A pool is num_blocks blocks of block_bytes bytes, block b at
 * pool + b * block_bytes: a K or V pool (block_bytes = num_kv_heads *
 * block_size * head_dim * element size) or the scale array of an fp8 cache
 * (block_bytes = 4 * num_kv_heads).  block_bytes must be a positive
 * multiple of 4.  block_mapping is a device int64 array [num_pairs, 2] of
 * (src, dst) block ids; block dst of the destination pool becomes a bit
 * copy of block src of the source pool.  Destinations must be distinct, and
 * for pa_copy_blocks no destination may also be a source of the same call
 * (PA_ERR_INDEX under PA_CHECK=1, with ids out of range; without it such
 * pairs are undefined, and out-of-range pairs are skipped).
 * ---------------------------------------------------------------------- */

/* pa_copy_blocks -- copies inside one device pool (copy-on-write). */
int pa_copy_blocks(void* pool, const int64_t* block_mapping,
                   int32_t num_pairs, int64_t block_bytes,
                   int32_t num_blocks, void* stream);

/*
 * pa_swap_blocks -- copies from one pool into another; either may be pinned
 * host memory (hipHostMalloc or a pinned torch tensor: the swap space) or
 * device memory.  Pageable host memory returns PA_ERR_UNSUPPORTED before
 * anything is launched.  dst_pool == src_pool returns PA_ERR_SHAPE (use
 * pa_copy_blocks).
 */
int pa_swap_blocks(void* dst_pool, const void* src_pool,
                   const int64_t* block_mapping, int32_t num_pairs,
                   int64_t block_bytes, int32_t dst_num_blocks,
                   int32_t src_num_blocks, void* stream);

/* ------------------------------------------------------------------------
 * FP8 (e4m3) KV cache.  The cache may hold K and V as 8-bit floats, one
 * byte per element, quantised per block ("Tech Radar: vLLM v1 Production
 * Engine Architecture ...", section "Hopper TMA Warp Specialization & FP8
 * Kernel Integration", item "FP8 Block-Quantized Caching"; "High-Throughput
 * Local LLM Infrastructure ...", FAQ "Q5").
 *
 * Format: OCP e4m3 (no infinities; 0x7F/0xFF are NaN; largest finite 448).
 * Pools: uint8, K [num_blocks, num_kv_heads, block_size, head_dim] and
 * V [num_blocks, num_kv_heads, head_dim, block_size], as the bf16 pools.
 * Scales: k_scales and v_scales are float32 [num_blocks, num_kv_heads], one
 * per (physical block, KV head), owned and set by the caller (for example
 * when a block is allocated); the library only reads them.  The scales of
 * every block a call touches must be finite and > 0 (checked under
 * PA_CHECK=1, PA_ERR_INDEX otherwise).  Element x stored with scale s is
 * code(x) = e4m3 of clamp(x / s, -448, 448) (float32 division, correctly
 * rounded; round to nearest, ties to even); it stands for value(code) * s.
 * block_size must be 16, 32 or 64 (PA_ERR_UNSUPPORTED otherwise).
 * ---------------------------------------------------------------------- */

/*
 * pa_reshape_and_cache_fp8 -- as pa_reshape_and_cache, with bf16 key/value
 * [num_tokens, num_kv_heads, head_dim] quantised into the e4m3 pools with
 * the scales of each slot's (block, KV head).  Negative slots are skipped;
 * two tokens aiming at one slot is undefined (PA_ERR_INDEX under PA_CHECK).
 */
int pa_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                             void* v_cache, const float* k_scales,
                             const float* v_scales,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int32_t num_blocks,
                             void* stream);

/* Workspace for pa_decode_fp8 (the balanced decode's pieces and header);
 * 0 for invalid arguments. */
size_t pa_decode_fp8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                     int32_t head_dim, int32_t max_seq_len,
                                     int32_t block_size);

/*
 * pa_decode_fp8 -- pa_decode against e4m3 pools: bf16 query [num_seqs,
 * num_q_heads, head_dim] and bf16 out; attention over the dequantised
 * values value(code) * scale.  Always the balanced decode (no fixed split);
 * at most 4096 sequences per call.  Other arguments as for pa_decode.
 */
int pa_decode_fp8(void* out, const void* query, const void* k_cache,
                  const void* v_cache, const float* k_scales,
                  const float* v_scales, const int32_t* block_tables,
                  int32_t max_blocks_per_seq, const int32_t* block_refcounts,
                  const int32_t* seq_lens, int32_t num_seqs,
                  int32_t max_seq_len, int32_t num_q_heads,
                  int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                  int32_t num_blocks, float scale, void* workspace,
                  size_t workspace_bytes, void* stream);

/*
 * pa_decode_fp8_append -- pa_decode_append over e4m3 pools: bf16 key/value
 * [num_seqs, num_kv_heads, head_dim] quantised with the scales of the new
 * token's (block, KV head) exactly as pa_reshape_and_cache_fp8 does, then
 * pa_decode_fp8; always inside the attention launch.  Same results, bit for
 * bit, as those calls in sequence.  Arguments and limits otherwise as for
 * pa_decode_fp8 (workspace: pa_decode_fp8_workspace_bytes).
 */
int pa_decode_fp8_append(void* out, const void* query, const void* key,
                         const void* value, void* k_cache, void* v_cache,
                         const float* k_scales, const float* v_scales,
                         const int32_t* block_tables,
                         int32_t max_blocks_per_seq,
                         const int32_t* block_refcounts,
                         const int32_t* seq_lens, int32_t num_seqs,
                         int32_t max_seq_len, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, float scale,
                         void* workspace, size_t workspace_bytes,
                         void* stream);

/*
 * Workspace for pa_chunked_prefill_fp8: that of pa_chunked_prefill plus the
 * bf16 staging pools of the query-chunk sequences (chunk_context_blocks
 * blocks, K and V) and their staging tables.  0 for invalid arguments.
 */
size_t pa_chunked_prefill_fp8_workspace_bytes(int32_t num_seqs, int32_t num_tokens,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t max_seq_len,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              int64_t chunk_context_blocks);

/*
 * pa_chunked_prefill_fp8 -- pa_chunked_prefill against e4m3 pools (the
 * serving configuration that pairs an fp8 KV cache with chunked prefill:
 * "Tech Radar ...", section "5.2 Production Python 3.12+ Dynamic Chunked
 * Prefill Controller", the serving config; the cache format as for
 * pa_decode_fp8).  bf16 query [num_tokens, num_q_heads, head_dim] and out;
 * every row computes the attention pa_chunked_prefill defines over the
 * dequantised values value(code) * scale.
 * Work: the blocks of every sequence with more than one query row are first
 * staged in the workspace as bf16 (value(code) * scale rounded to nearest
 * even, one rounding more than the e4m3 decode makes) and the bf16 chunk
 * kernel runs on them; single-token rows run the e4m3 balanced decode on the
 * pools themselves.
 * chunk_context_blocks: room in the staging pools, at least the sum over
 * sequences with q_len > 1 of ceil(seq_len / block_size) (the batch builder
 * knows it); >= 1 when max_query_len > 1, else PA_ERR_SHAPE.  A batch that
 * needs more is PA_ERR_INDEX under PA_CHECK=1; without it, the blocks past
 * the room are not staged and those rows are undefined (every access stays
 * inside the pools).  block_size 16, 32 or 64; at most 2048 sequences;
 * each bf16 staging pool (chunk_context_blocks blocks) under 2^40 bytes
 * (PA_ERR_UNSUPPORTED otherwise).
 * Other arguments, errors and the workspace ownership as for
 * pa_chunked_prefill and pa_decode_fp8.
 */
int pa_chunked_prefill_fp8(void* out, const void* query, const void* k_cache,
                           const void* v_cache, const float* k_scales, const float* v_scales,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* block_refcounts, const int32_t* seq_lens,
                           const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                           int32_t max_seq_len, int32_t max_query_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int64_t chunk_context_blocks, float scale,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Workspace for pa_decode_shared_prefix; 0 for invalid arguments (also
 * when prefix_blocks * block_size > max_seq_len). */
size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t head_dim, int32_t max_seq_len,
                                               int32_t block_size, int32_t prefix_blocks);

/*
 * pa_decode_shared_prefix -- pa_decode (k_scales = v_scales = NULL: bf16
 * pools) or pa_decode_fp8 (both scale arrays given: e4m3 pools) for a batch
 * whose block tables all begin with the same prefix_blocks physical blocks,
 * the prefix sharing of "Inside vLLM ...", section "Zero-Copy Branching and
 * Parallel Sampling" (prefix caching) and of "03 -- PagedAttention & the
 * vLLM V1 Architecture", section "The insight: KV cache is virtual memory"
 * (pages shared between sequences).  The result is the attention pa_decode
 * defines; only the order of the work differs: the prefix keys of each KV
 * head are read once per group of sequences instead of once per sequence
 * (G = num_q_heads / num_kv_heads; a group is floor(32 / G) sequences on
 * bf16 pools, whose query rows fill two 16-row matrix tiles, and floor(16 /
 * G) on e4m3 pools, one tile), and each row's prefix part and own part are
 * combined exactly
 * (log-sum-exp) in the merge pass.  Only whole 32-key steps (64 for e4m3)
 * of the prefix are read this way; the rest of its blocks are read with
 * each sequence.
 *
 * Contract: block_tables[s][b] == block_tables[0][b] for b < prefix_blocks
 * and seq_lens[s] >= prefix_blocks * block_size for every s (checked, with
 * PA_ERR_INDEX, under PA_CHECK=1; otherwise results for a batch that breaks
 * it are undefined, but every access stays in bounds).  query and out: bf16
 * [num_seqs, num_q_heads, head_dim].  block_size >= 8 (>= 16 for e4m3);
 * when the prefix holds at least one whole step, num_seqs +
 * ceil(num_seqs / group) <= 4096, else PA_ERR_UNSUPPORTED.  A prefix shorter
 * than one step (prefix_blocks == 0 included) runs pa_decode's (e4m3:
 * pa_decode_fp8's) path with that call's limits.
 * Other arguments, errors and the workspace ownership as for pa_decode and
 * pa_decode_fp8.
 */
int pa_decode_shared_prefix(void* out, const void* query, const void* k_cache,
                            const void* v_cache, const float* k_scales,
                            const float* v_scales, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* block_refcounts,
                            const int32_t* seq_lens, int32_t num_seqs,
                            int32_t max_seq_len, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t prefix_blocks, float scale,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_shared_prefix_append -- pa_decode_shared_prefix with the step's
 * slot computation and cache write in the same call, as pa_decode_append
 * adds them to pa_decode (passages cited there): key, value [num_seqs,
 * num_kv_heads, head_dim] (bf16) are each sequence's new token, written at
 * position seq_lens[s] - 1 (quantised as pa_reshape_and_cache_fp8 does when
 * the scales are given) and attended to.  The same results, bit for bit, as
 * pa_compute_slot_mapping + pa_reshape_and_cache[_fp8] +
 * pa_decode_shared_prefix.  Every sequence must hold more than the prefix
 * (seq_lens[s] > prefix_blocks * block_size), so that no new token lands in
 * a shared block (PA_ERR_INDEX under PA_CHECK; undefined otherwise).
 * Workspace: pa_decode_shared_prefix_workspace_bytes.  Arguments and limits
 * otherwise as for pa_decode_shared_prefix.
 */
int pa_decode_shared_prefix_append(void* out, const void* query,
                                   const void* key, const void* value,
                                   void* k_cache, void* v_cache,
                                   const float* k_scales,
                                   const float* v_scales,
                                   const int32_t* block_tables,
                                   int32_t max_blocks_per_seq,
                                   const int32_t* block_refcounts,
                                   const int32_t* seq_lens, int32_t num_seqs,
                                   int32_t max_seq_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim,
                                   int32_t block_size, int32_t num_blocks,
                                   int32_t prefix_blocks, float scale,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ------------------------------------------------------------------------
 * For callers that cannot allocate device memory (code under stream
 * capture, tight serving loops, hosts that forbid hipMalloc).
 *
 * pa_decode_noalloc -- pa_decode without a workspace argument: the
 * workspace is a static device array of PA_NOALLOC_SCRATCH_BYTES (160 MiB,
 * enough for the Llama-3-70B-layer decode batch of 128 sequences of up to
 * 8,192 tokens, 64 query heads, which needs 145 MB) that the library holds on
 * each GPU it runs on until the process ends.  The call allocates and frees
 * nothing (no hipMalloc, no allocating library call); the caller still
 * passes every input and the output.  Its first call on a device looks up
 * that device's copy of the array (with the device current).
 * A batch whose workspace (pa_decode_workspace_bytes with the same
 * arguments) exceeds the scratch returns PA_ERR_SCRATCH before anything is
 * enqueued.  Every call on one GPU shares that GPU's scratch: calls that may
 * overlap on one GPU (different streams, or different host threads without
 * ordering) race and give undefined results; calls in one stream are
 * ordered.  The scratch keeps the last call's contents, which no call reads
 * (pa_decode's workspace needs no initialisation).  Arguments, results and
 * other errors: as for pa_decode.
 * ---------------------------------------------------------------------- */
#define PA_NOALLOC_SCRATCH_BYTES (160u * 1024u * 1024u)

int pa_decode_noalloc(void* out, const void* query, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* block_refcounts,
                      const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, float scale,
                      int32_t dtype, int32_t kv_split_tokens, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
