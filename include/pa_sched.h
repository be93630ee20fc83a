/*
 * pa_sched.h -- host batch builder of libpa: chunked-prefill scheduling with
 * prefix reuse, producing the block tables, sequence lengths, query offsets
 * and slot mapping that pa_reshape_and_cache / pa_chunked_prefill take.
 *
 * What it computes, from the pages:
 *   - the step's token budget: every active decode stream gets its token
 *     first, N_decode = |R_decode|; prompt chunks share
 *     C_avail = max(0, T_budget - N_decode), and a prompt with U_p tokens
 *     left gets c_p = min(U_p, C_chunk, C_avail) ("Tech Radar: vLLM v1
 *     Production Engine Architecture ...", section "The Dynamic Chunked
 *     Prefill Scheduler Formulation", equations 1-3);
 *   - the step order: running requests first (one that cannot get KV blocks
 *     is preempted), then waiting requests admitted in arrival order while
 *     budget is left, after a prefix-cache lookup, stopping at the first one
 *     that cannot be allocated ("03 -- PagedAttention & the vLLM V1
 *     Architecture", section "The scheduler's schedule() step");
 *   - prefix reuse: each full block is keyed by a hash of its tokens chained
 *     to the previous block's key; leading full blocks whose keys are cached
 *     are shared (reference count + 1) and not prefilled again ("Inside
 *     vLLM ...", section "Zero-Copy Branching and Parallel Sampling");
 *   - preemption by recomputation ("03 -- ...", section "Preemption &
 *     eviction"), or, with a swap space (pa_sched_enable_swap), by swapping:
 *     the request's blocks are copied to host blocks and released, and later
 *     copied back into fresh device blocks; the request then continues
 *     without recomputing ("03 -- ...", same section; "Inside vLLM ...",
 *     section "Preemption Mechanics: Swapping vs. Recomputation").
 *
 * Readings where the pages are silent: C_avail is consumed in order (running
 * prompt chunks, then admissions); decode tokens are always scheduled; the
 * batch is packed decodes, running prompt chunks, admissions; a cache hit
 * covers at most (tokens - 1) / block_size full blocks; freed blocks go to
 * the back of a FIFO free list and keep their key until handed out again; a
 * full block's key is registered when the step computing its last token is
 * scheduled (unless taken); keys are 64-bit FNV-1a over the parent key (8
 * bytes, little-endian) and the block's tokens (4 bytes each, little-endian),
 * the first parent being the FNV offset basis; the preempted request is the
 * one that cannot allocate, its prompt becomes all its tokens, and a step
 * that preempted admits nobody; a request ends when a step computed all its
 * tokens and it has generated max_new_tokens.  With a swap space: a
 * preempted request is swapped out when the swap space has a block for each
 * of its blocks, else recomputed; host blocks come from a FIFO free list;
 * swapped-out requests come back in order, in a step that preempted nobody,
 * after the running requests and before admissions, each while budget is
 * left and the device has blocks for all its tokens plus the step's (a
 * decode token takes one unit of budget), and are scheduled in that step;
 * nobody is admitted while a request is swapped out.
 *
 * All memory here is host memory.  The builder is a plain object owned by the
 * caller (create/destroy); it is not thread-safe.  Nothing here touches the
 * GPU.  Status codes are those of pa.h.
 */
#ifndef PA_SCHED_H_
#define PA_SCHED_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_sched pa_sched;

/*
 * A builder over a pool of num_blocks blocks of block_size tokens.
 * free_order (host int32 [num_blocks], a permutation of 0..num_blocks-1, or
 * NULL for 0, 1, ...) is the initial free list.  token_budget and
 * chunk_tokens are T_budget and C_chunk.  NULL on invalid arguments.
 */
pa_sched* pa_sched_create(int32_t num_blocks, int32_t block_size,
                          int32_t token_budget, int32_t chunk_tokens,
                          const int32_t* free_order);

void pa_sched_destroy(pa_sched* s);

/* Queue a request (prompt: host int32 [prompt_len], prompt_len >= 1,
 * max_new_tokens >= 1, req_id unused so far). */
int pa_sched_add_request(pa_sched* s, int64_t req_id, const int32_t* prompt,
                         int32_t prompt_len, int32_t max_new_tokens);

/*
 * Schedule one step and keep the batch inside the builder.  Outputs its
 * sizes: sequences, query tokens, the longest block table and the number of
 * requests preempted in this step.
 */
int pa_sched_step(pa_sched* s, int32_t* num_seqs, int32_t* num_tokens,
                  int32_t* max_blocks, int32_t* num_preempted);

/*
 * Copy the last step's batch into caller buffers sized from pa_sched_step:
 * req_ids int64 [num_seqs]; seq_lens int32 [num_seqs] (cached tokens after
 * the step); query_start_loc int32 [num_seqs + 1]; block_tables int32
 * [num_seqs, max_blocks_per_seq] (row-major, padded with pad_block);
 * slot_mapping int64 [num_tokens]; preempted int64 [num_preempted] (may be
 * NULL when there are none).  PA_ERR_SHAPE if max_blocks_per_seq is below
 * the batch's longest table.
 */
int pa_sched_get_batch(const pa_sched* s, int64_t* req_ids, int32_t* seq_lens,
                       int32_t* query_start_loc, int32_t* block_tables,
                       int32_t max_blocks_per_seq, int32_t pad_block,
                       int64_t* slot_mapping, int64_t* preempted);

/*
 * After the step ran: n (req_id, token) pairs of sampled tokens.  Every
 * request of the last batch whose tokens are now all computed either ends
 * (max_new_tokens generated; its blocks are released) or takes its sampled
 * token, which must be among the pairs (PA_ERR_INDEX otherwise).
 */
int pa_sched_update(pa_sched* s, const int64_t* req_ids, const int32_t* tokens,
                    int32_t n);

/* Reference count of every block (int32 [num_blocks]): the block_refcounts
 * hint of pa_decode / pa_chunked_prefill. */
int pa_sched_block_refcounts(const pa_sched* s, int32_t* out, int32_t num_blocks);

/*
 * Give the builder a swap space of num_host_blocks host blocks (ids 0 ..
 * num_host_blocks - 1, same block size as the device pool), which makes
 * swapping the preemption mode whenever the space can take the request.
 * Call once, before the first request (PA_ERR_INDEX otherwise).
 */
int pa_sched_enable_swap(pa_sched* s, int32_t num_host_blocks);

/*
 * The copies the last step needs, to be run before its cache write and
 * attention, swap-outs first: swap_out int64 [num_swap_out, 2] (device
 * block, host block) pairs, swap_in int64 [num_swap_in, 2] (host block,
 * device block) pairs -- the block_mapping arguments of pa_swap_blocks --
 * and the ids of the requests swapped out (int64 [num_swapped_out]; they are
 * also among pa_sched_get_batch's preempted ids).  Call with NULL arrays to
 * get the counts first.
 */
int pa_sched_get_swaps(const pa_sched* s, int32_t* num_swap_out, int32_t* num_swap_in,
                       int64_t* swap_out, int64_t* swap_in, int64_t* swapped_out_ids,
                       int32_t* num_swapped_out);

/* Requests waiting, running and finished so far. */
int pa_sched_counts(const pa_sched* s, int32_t* waiting, int32_t* running,
                    int32_t* finished);

#ifdef __cplusplus
}
#endif

#endif /* PA_SCHED_H_ */
