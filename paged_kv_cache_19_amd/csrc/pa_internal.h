// Internal launch interface between the C ABI (pa_api.cpp) and the HIP
// kernels (pa_kernels.hip).  Not installed; not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// Everything one attention launch needs.  Pointers are device pointers;
// element pointers are raw bits (bf16 as uint16_t, fp32 as float).
struct AttnArgs {
  const void* q;            // [T, Hq, D]
  const void* k_cache;      // [NB, Hkv, B, D]
  const void* v_cache;      // [NB, Hkv, D, B]
  const int32_t* block_tables;
  const int32_t* block_refcounts;  // nullptr: every block private (cache hint only)
  const int32_t* seq_lens;
  const int32_t* query_start_loc;  // nullptr: one row per sequence
  void* out;                // [T, Hq, D]
  float* part_o;            // [T * Hq, max_splits, D]   fixed-split / chunk partials
  float* part_ml;           // [T * Hq, max_splits, 2]   (max in log2 units, sum)
  float* sk_part_o;         // [num_seqs * Hq, sk_slots, D] balanced-decode pieces
  float* sk_part_ml;        // [num_seqs * Hq, sk_slots, 2]
  int32_t max_blocks;
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim;
  int32_t block_size, log2_block, num_blocks;
  int32_t split_tokens, max_splits, max_query_len;
  int32_t sk_slots;         // pieces per row in sk_part_*
  int32_t* row_pieces;      // [T * Hq] chunk rows: pieces of part_o the row's keys were cut into
  int32_t chunk_steps;      // chunk kernel: 32-key steps per workgroup range (minimum when auto)
  int32_t chunk_auto;       // 1: ranges sized to spread all steps over the resident workgroups
  float scale_log2;         // scale * log2(e)
  int32_t bf16;             // 1: bf16 elements, 0: fp32 (q, out and, unless kv_fp8, the cache)
  int32_t kv_fp8;           // 1: e4m3 cache with per-(block, KV head) scales, bf16 q/out
  const float* k_scales;    // [NB, Hkv] (kv_fp8 only)
  const float* v_scales;    // [NB, Hkv]
  // Shared-prefix decode (balanced decode only; 0: off).  Keys [0,
  // prefix_keys) of every sequence are the blocks table row 0 starts with;
  // they are read once per group of prefix_group sequences (one 16-row MFMA
  // tile of query rows), and each sequence's own items cover the keys after
  // them.  Every row is then left as pieces: the prefix pieces in the last
  // prefix_slots of its sk_slots.
  int32_t prefix_keys;
  int32_t prefix_group;
  int32_t prefix_slots;
  // Appending decode (pa_decode_append, pa_decode_fp8_append): the new
  // token of every sequence, key and value rows [num_seqs, Hkv, D] (the
  // pool dtype; bf16 for an e4m3 pool), attended to and written at
  // position seq_len - 1.  nullptr: nothing is written.
  const void* new_k;
  const void* new_v;
};

// 16-row MFMA tiles of query rows per shared-prefix item: a group holds
// floor(16 * tiles / G) sequences, and each of the item's K/V loads serves
// all of their rows.  The fp8 item keeps one tile (two would not fit its
// registers next to the widened codes).
__host__ __device__ constexpr int prefix_tiles(bool fp8) { return fp8 ? 1 : 2; }

// Work-list entries for the prefixes: one per group of sequences.
__host__ __device__ inline int prefix_items(int num_seqs, int group) {
  return group > 0 ? (num_seqs + group - 1) / group : 0;
}

// Balanced decode: every resident wave streams at least this many 32-key
// steps, which bounds the pieces one row can be cut into.
constexpr int kMinStepsPerWave = 8;
// Work-list cost of starting a piece (query rows, block-table window, ring
// fill), in steps: each (sequence, KV head) item costs its steps plus this,
// so waves whose share crosses more items get fewer steps.
constexpr int kPieceCostSteps = 3;

hipError_t launch_slot_mapping(int64_t* slots, const int32_t* bt, int32_t max_blocks,
                               const int32_t* seq_lens, const int32_t* qsl,
                               int32_t num_seqs, int32_t num_tokens, int32_t block_size,
                               hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slots,
                                    int32_t num_tokens, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t elem_bytes,
                                    hipStream_t stream);

// Copy whole blocks of block_bytes bytes (a multiple of 4): block dst of
// ``dst`` becomes block src of ``src`` for each (src, dst) pair.  Both pools
// are device-accessible addresses.
hipError_t launch_copy_blocks(void* dst, const void* src, const int64_t* mapping,
                              int32_t num_pairs, int64_t block_bytes, int64_t src_num_blocks,
                              int64_t dst_num_blocks, hipStream_t stream);

// Cache write into e4m3 pools (bf16 K/V in), quantised with the scale of
// each slot's (block, KV head).
hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                        void* v_cache, const float* k_scales,
                                        const float* v_scales, const int64_t* slots,
                                        int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        hipStream_t stream);

// The appending decode's cache writes on their own (a.new_k / a.new_v, one
// new token per sequence at position seq_len - 1; a.kv_fp8 selects the
// quantising write), for the attention paths that do not fuse them.
hipError_t launch_append_tokens(const AttnArgs& a, hipStream_t stream);

// Split-K attention pass (writes final rows for single-split rows and
// partials otherwise), then the log-sum-exp merge pass when needed.
// ``has_chunks``: rows of multi-token sequences go to the persistent chunk
// kernel and single-token rows to the balanced decode (whose ``header`` is
// workspace as for launch_decode_streamk).
hipError_t launch_attention(const AttnArgs& a, bool has_chunks, void* header,
                            hipStream_t stream);

// Largest batch the persistent chunk kernel takes (its per-sequence item
// prefix sums live in LDS).
constexpr int kMaxChunkSeqs = 2048;
// Largest batch whose chunk units and decode rows share one launch (both
// kinds of prefix sums sit next to the chunk kernel's LDS ring).
constexpr int kMaxMixSeqs = 1024;

// Balanced ("stream-K") decode over a fixed set of resident waves, then the
// merge of the pieces (bf16 or, with a.kv_fp8, e4m3 cache).  ``header`` is workspace for the step prefix sums
// (16 + 4 * (num_seqs + 1) bytes); a.max_splits is the piece capacity per row.
hipError_t launch_decode_streamk(const AttnArgs& a, void* header, hipStream_t stream);

// Query chunks and single-token rows over an e4m3 cache.  ``dec`` describes
// the call on the e4m3 pools (kv_fp8 = 1, the caller's tables); ``chunk`` is
// the same call on the bf16 staging pools (k_cache / v_cache: room for
// cap_blocks blocks in the bf16 layouts; block_tables: [num_seqs,
// max_blocks] int32 staging tables, written here; kv_fp8 = 0).  The blocks
// of every multi-token sequence are staged as bf16, the chunk kernel runs
// on the staging pools, the balanced e4m3 decode on the single-token rows,
// then the merge of cut chunk rows.  ``offsets`` is int32 [num_seqs + 1]
// workspace.
hipError_t launch_chunked_fp8(const AttnArgs& dec, const AttnArgs& chunk, void* header,
                              int64_t cap_blocks, int32_t* offsets, hipStream_t stream);

// True when the MFMA kernels serve this shape (bf16, B >= 8, D in {64,128}).
bool mfma_path(const AttnArgs& a);

}  // namespace pa
