// C ABI of libpa: argument validation, split planning, optional metadata
// checks (PA_CHECK=1) and dispatch to the HIP kernels.  See include/pa.h.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

constexpr int kDefaultSplitTokens = 512;        // decode rows on the fixed-split path
constexpr int kDefaultChunkSplitTokens = 2048;  // query-chunk rows on the vector-ALU path
// Chunk kernel (MFMA path): a workgroup range is at least this many 32-key
// steps, and long enough that no row tile is cut into more than
// kChunkPieces pieces.
constexpr int kMinChunkSteps = 16;
constexpr int kChunkPieces = 4;
// The balanced decode keeps every sequence's step prefix sum in LDS.
constexpr int kMaxBalancedSeqs = 4096;
// Largest K or V pool the chunk kernel takes (block offsets in 256-byte
// units in one dword).
constexpr int64_t kMaxChunkPoolBytes = (int64_t)1 << 40;
constexpr size_t kAlign = 256;

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int log2i(int x) { return __builtin_ctz((unsigned)x); }

bool check_enabled() {
  const char* v = getenv("PA_CHECK");
  return v && v[0] && strcmp(v, "0") != 0;
}

// Keys one split covers on the fixed-split paths: 0 selects the default,
// otherwise a positive multiple of 64.
int split_tokens_for(int requested, bool chunks) {
  if (requested == 0) return chunks ? kDefaultChunkSplitTokens : kDefaultSplitTokens;
  if (requested < 0 || requested % 64 != 0) return -1;
  return requested;
}

int check_common(int num_q_heads, int num_kv_heads, int head_dim, int block_size, int dtype) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0)
    return PA_ERR_SHAPE;
  if (num_q_heads % num_kv_heads != 0) return PA_ERR_SHAPE;
  if (num_q_heads / num_kv_heads > 16) return PA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!is_pow2(block_size) || block_size > 64) return PA_ERR_UNSUPPORTED;
  return PA_OK;
}

struct WorkspacePlan {
  int split_tokens = 0;   // fixed-split / chunk path: keys per split
  int max_splits = 0;     // fixed-split / chunk path: partial slots per row
  int max_pieces = 0;     // balanced decode: partial slots per row (0: unused)
  int chunk_steps = 0;    // chunk kernel: steps per workgroup range (minimum when auto)
  int chunk_auto = 0;
  size_t a_o = 0, a_ml = 0;  // region A: [T*Hq, max_splits] partials (o, then (m, l))
  size_t rp = 0;             // chunk rows: [T*Hq] piece counts
  size_t b_o = 0, b_ml = 0;  // region B: [S*Hq, max_pieces] balanced-decode pieces
  size_t header = 0;         // balanced-decode header
  size_t total = 0;
};

// Workspace layout: region A (fixed-split and query-chunk partials, one row
// per query token and head; then, for pa_chunked_prefill, the piece count of
// each row) | region B (balanced-decode pieces, one row per
// sequence and head) | header (step total, wave count, per-sequence step
// prefix sums).  pa_decode's two paths share one region (rows = sequences),
// so its size is the larger of the two slot counts.
// Partial slots a row's shared-prefix entry can need: its prefix_keys
// (<= max_seq_len) cut like any other item of the balanced decode.
int prefix_piece_slots(int prefix_keys) {
  const int steps = (prefix_keys + 31) / 32;
  return (steps + pa::kPieceCostSteps + pa::kMinStepsPerWave - 1) / pa::kMinStepsPerWave + 1;
}

// With prefix_keys > 0 (pa_decode_shared_prefix) every row also holds its
// prefix entry's pieces and the header the prefix entries' sums (at most one
// entry per sequence).
bool plan_workspace(int num_tokens, int num_seqs, int num_q_heads, int head_dim, int max_seq_len,
                    int block_size, int kv_split_tokens, bool chunk_entry, WorkspacePlan* p,
                    int prefix_keys = 0) {
  if (num_tokens < 0 || num_seqs < 0 || num_q_heads <= 0 || head_dim <= 0 ||
      max_seq_len <= 0 || !is_pow2(block_size) || block_size > 64)
    return false;
  const int st = split_tokens_for(kv_split_tokens, chunk_entry);
  if (st <= 0) return false;
  p->split_tokens = st;
  p->max_splits = (max_seq_len + st - 1) / st;
  const int steps = (max_seq_len + 31) / 32;
  p->max_pieces = (steps + pa::kPieceCostSteps + pa::kMinStepsPerWave - 1) / pa::kMinStepsPerWave + 1;
  const size_t ob = (size_t)head_dim * sizeof(float), mlb = 2 * sizeof(float);
  if (chunk_entry) {
    // The chunk kernel cuts each row tile's steps into at most
    // ceil(steps / chunk_steps) + 1 pieces; the vector-ALU path into
    // max_splits fixed splits.  Region A holds the larger count.
    p->chunk_auto = kv_split_tokens == 0;
    p->chunk_steps = p->chunk_auto
                         ? std::max(kMinChunkSteps, (steps + kChunkPieces - 2) / (kChunkPieces - 1))
                         : st / 32;
    p->max_splits = std::max(p->max_splits, (steps + p->chunk_steps - 1) / p->chunk_steps + 1);
    const size_t ra = (size_t)num_tokens * num_q_heads * p->max_splits;
    p->rp = align_up((size_t)num_tokens * num_q_heads * sizeof(int32_t));
    const size_t rb = (size_t)num_seqs * num_q_heads * p->max_pieces;
    p->a_o = align_up(ra * ob);
    p->a_ml = align_up(ra * mlb);
    p->b_o = align_up(rb * ob);
    p->b_ml = align_up(rb * mlb);
  } else {
    if (kv_split_tokens != 0) p->max_pieces = 0;
    if (prefix_keys > 0) p->max_pieces += prefix_piece_slots(prefix_keys);
    const int slots = p->max_splits > p->max_pieces ? p->max_splits : p->max_pieces;
    const size_t r = (size_t)num_seqs * num_q_heads * slots;
    p->a_o = align_up(r * ob);
    p->a_ml = align_up(r * mlb);
  }
  const size_t entries = (size_t)num_seqs * (prefix_keys > 0 ? 2 : 1);
  p->header = align_up(16 + (entries + 1) * 4);
  p->total = p->a_o + p->a_ml + p->rp + p->b_o + p->b_ml + p->header;
  return true;
}

// Host-side validation of device metadata (PA_CHECK=1).  Synchronous.
int validate_metadata(const int32_t* d_bt, int max_blocks, const int32_t* d_lens,
                      const int32_t* d_qsl, int num_seqs, int num_tokens, int max_seq_len,
                      int max_query_len, int block_size, int num_blocks, hipStream_t st) {
  std::vector<int32_t> bt((size_t)num_seqs * max_blocks), lens(num_seqs), qsl(num_seqs + 1);
  if (hipMemcpyAsync(bt.data(), d_bt, bt.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(lens.data(), d_lens, lens.size() * 4, hipMemcpyDeviceToHost, st) !=
          hipSuccess)
    return PA_ERR_HIP;
  if (d_qsl) {
    if (hipMemcpyAsync(qsl.data(), d_qsl, qsl.size() * 4, hipMemcpyDeviceToHost, st) !=
        hipSuccess)
      return PA_ERR_HIP;
  } else {
    for (int s = 0; s <= num_seqs; ++s) qsl[s] = s;
  }
  if (hipStreamSynchronize(st) != hipSuccess) return PA_ERR_HIP;
  if (qsl[0] != 0 || qsl[num_seqs] != num_tokens) return PA_ERR_INDEX;
  for (int s = 0; s < num_seqs; ++s) {
    const int L = lens[s];
    const int qn = qsl[s + 1] - qsl[s];
    if (qn < 0 || qn > max_query_len) return PA_ERR_INDEX;
    if (L < 1 || L > max_seq_len || (int64_t)L > (int64_t)max_blocks * block_size)
      return PA_ERR_INDEX;
    if (qn > L) return PA_ERR_INDEX;
    const int nb = (L + block_size - 1) / block_size;
    for (int b = 0; b < nb; ++b) {
      const int id = bt[(size_t)s * max_blocks + b];
      if (id < 0 || id >= num_blocks) return PA_ERR_INDEX;
    }
  }
  return PA_OK;
}

int validate_slots(const int64_t* d_slots, int num_tokens, int64_t num_slots, hipStream_t st) {
  std::vector<int64_t> slots(num_tokens);
  if (num_tokens == 0) return PA_OK;
  if (hipMemcpyAsync(slots.data(), d_slots, slots.size() * 8, hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return PA_ERR_HIP;
  std::vector<int64_t> valid;
  for (int64_t s : slots) {
    if (s >= num_slots) return PA_ERR_INDEX;
    if (s >= 0) valid.push_back(s);
  }
  std::sort(valid.begin(), valid.end());
  for (size_t i = 1; i < valid.size(); ++i)
    if (valid[i] == valid[i - 1]) return PA_ERR_INDEX;
  return PA_OK;
}

// PA_CHECK for the fp8 cache: the K and V scales of every listed block must
// be finite and > 0.
int validate_scales(const float* d_ks, const float* d_vs, int num_blocks, int num_kv_heads,
                    const std::vector<int64_t>& blocks, hipStream_t st) {
  if (blocks.empty()) return PA_OK;
  if (!d_ks || !d_vs) return PA_ERR_NULL;
  const size_t n = (size_t)num_blocks * num_kv_heads;
  std::vector<float> ks(n), vs(n);
  if (hipMemcpyAsync(ks.data(), d_ks, n * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(vs.data(), d_vs, n * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return PA_ERR_HIP;
  for (int64_t b : blocks) {
    for (int h = 0; h < num_kv_heads; ++h) {
      const float k = ks[(size_t)b * num_kv_heads + h], v = vs[(size_t)b * num_kv_heads + h];
      if (!isfinite(k) || !(k > 0.f) || !isfinite(v) || !(v > 0.f)) return PA_ERR_INDEX;
    }
  }
  return PA_OK;
}

// PA_CHECK for a shared prefix: every table starts with row 0's first
// prefix_blocks entries and every sequence holds at least the prefix (past
// it with `past`: an appending call's new token must not land in a shared
// block).
int validate_prefix(const int32_t* d_bt, int max_blocks, const int32_t* d_lens, int num_seqs,
                    int prefix_blocks, int block_size, hipStream_t st, bool past = false) {
  if (prefix_blocks > max_blocks) return PA_ERR_INDEX;
  std::vector<int32_t> bt((size_t)num_seqs * max_blocks), lens(num_seqs);
  if (hipMemcpyAsync(bt.data(), d_bt, bt.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(lens.data(), d_lens, lens.size() * 4, hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return PA_ERR_HIP;
  for (int s = 0; s < num_seqs; ++s) {
    if ((int64_t)lens[s] < (int64_t)prefix_blocks * block_size + (past ? 1 : 0)) return PA_ERR_INDEX;
    for (int b = 0; b < prefix_blocks; ++b)
      if (bt[(size_t)s * max_blocks + b] != bt[b]) return PA_ERR_INDEX;
  }
  return PA_OK;
}

// PA_CHECK for the appending decode: the slots of the new tokens (position
// seq_len - 1 of each table) are distinct.
int validate_append_slots(const int32_t* d_bt, int max_blocks, const int32_t* d_lens,
                          int num_seqs, int block_size, hipStream_t st) {
  std::vector<int32_t> bt((size_t)num_seqs * max_blocks), lens(num_seqs);
  if (hipMemcpyAsync(bt.data(), d_bt, bt.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(lens.data(), d_lens, lens.size() * 4, hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return PA_ERR_HIP;
  std::vector<int64_t> slots;
  for (int s = 0; s < num_seqs; ++s) {
    const int pos = lens[s] - 1;
    if (pos < 0 || pos / block_size >= max_blocks) continue;
    const int id = bt[(size_t)s * max_blocks + pos / block_size];
    slots.push_back((int64_t)id * block_size + pos % block_size);
  }
  std::sort(slots.begin(), slots.end());
  for (size_t i = 1; i < slots.size(); ++i)
    if (slots[i] == slots[i - 1]) return PA_ERR_INDEX;
  return PA_OK;
}

// Blocks the tables of a (validated) batch hold.
int table_blocks_used(const int32_t* d_bt, int max_blocks, const int32_t* d_lens, int num_seqs,
                      int block_size, hipStream_t st, std::vector<int64_t>* out) {
  std::vector<int32_t> bt((size_t)num_seqs * max_blocks), lens(num_seqs);
  if (hipMemcpyAsync(bt.data(), d_bt, bt.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(lens.data(), d_lens, lens.size() * 4, hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return PA_ERR_HIP;
  for (int s = 0; s < num_seqs; ++s) {
    const int nb = (lens[s] + block_size - 1) / block_size;
    for (int b = 0; b < nb; ++b) out->push_back(bt[(size_t)s * max_blocks + b]);
  }
  return PA_OK;
}

// fp8 cache arguments of the attention entry points (kv_fp8 = 0: none).
struct Fp8Kv {
  int kv_fp8 = 0;
  const float* k_scales = nullptr;
  const float* v_scales = nullptr;
};

int attention_common(void* out, const void* query, const void* k_cache, const void* v_cache,
                     const int32_t* block_tables, int max_blocks, const int32_t* refcounts,
                     const int32_t* seq_lens,
                     const int32_t* qsl, int num_seqs, int num_tokens, int max_seq_len,
                     int max_query_len, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int num_blocks, float scale, int dtype, int kv_split_tokens,
                     void* workspace, size_t workspace_bytes, void* stream,
                     const Fp8Kv& f8 = Fp8Kv(), int prefix_blocks = 0,
                     bool append = false, const void* new_k = nullptr,
                     const void* new_v = nullptr) {
  int rc = check_common(num_q_heads, num_kv_heads, head_dim, block_size, dtype);
  if (rc != PA_OK) return rc;
  if (num_seqs < 0 || num_tokens < 0 || max_blocks <= 0 || num_blocks <= 0 ||
      max_seq_len <= 0 || max_query_len <= 0 || !isfinite(scale) || !(scale > 0.f))
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !seq_lens) return PA_ERR_NULL;
  if (f8.kv_fp8 && (!f8.k_scales || !f8.v_scales)) return PA_ERR_NULL;
  if (append && (!new_k || !new_v)) return PA_ERR_NULL;
  if ((int64_t)num_seqs * num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  WorkspacePlan plan;
  const bool chunk_entry = qsl != nullptr;
  // Shared prefix: the whole key steps (32 keys, 64 for fp8) of the first
  // prefix_blocks blocks; the rest of them are read with each sequence.
  const int pstep = f8.kv_fp8 ? 64 : 32;
  const int prefix_keys =
      prefix_blocks > 0 ? (int)((int64_t)prefix_blocks * block_size / pstep * pstep) : 0;
  if (!plan_workspace(num_tokens, num_seqs, num_q_heads, head_dim, max_seq_len, block_size,
                      kv_split_tokens, chunk_entry, &plan, prefix_keys))
    return PA_ERR_SHAPE;
  if (plan.max_splits > 65535) return PA_ERR_UNSUPPORTED;
  if (!workspace) return PA_ERR_WORKSPACE;
  if (workspace_bytes < plan.total) return PA_ERR_WORKSPACE;
  pa::AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.bf16 = dtype == PA_BF16;
  a.head_dim = head_dim;
  a.block_size = block_size;
  const bool mfma = pa::mfma_path(a);
  const int G = num_q_heads / num_kv_heads;
  if (mfma && chunk_entry && num_seqs > pa::kMaxChunkSeqs) return PA_ERR_UNSUPPORTED;
  // The chunk kernel holds a block's offset in the pool as one dword of
  // 256-byte units.
  if (mfma && chunk_entry &&
      (int64_t)num_blocks * num_kv_heads * block_size * head_dim * 2 >= kMaxChunkPoolBytes)
    return PA_ERR_UNSUPPORTED;
  const int64_t tiles_y = mfma ? ((int64_t)G + 15) / 16 : max_query_len;
  if (tiles_y > 65535 || (int64_t)num_tokens > 65535 * 64) return PA_ERR_UNSUPPORTED;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    rc = validate_metadata(block_tables, max_blocks, seq_lens, qsl, num_seqs, num_tokens,
                           max_seq_len, max_query_len, block_size, num_blocks, st);
    if (rc != PA_OK) return rc;
    if (prefix_blocks > 0) {
      rc = validate_prefix(block_tables, max_blocks, seq_lens, num_seqs, prefix_blocks,
                           block_size, st, new_k != nullptr);
      if (rc != PA_OK) return rc;
    }
    if (new_k) {
      rc = validate_append_slots(block_tables, max_blocks, seq_lens, num_seqs, block_size, st);
      if (rc != PA_OK) return rc;
    }
    if (f8.kv_fp8) {
      std::vector<int64_t> used;
      rc = table_blocks_used(block_tables, max_blocks, seq_lens, num_seqs, block_size, st, &used);
      if (rc == PA_OK)
        rc = validate_scales(f8.k_scales, f8.v_scales, num_blocks, num_kv_heads, used, st);
      if (rc != PA_OK) return rc;
    }
  }
  char* ws = static_cast<char*>(workspace);
  a.q = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.block_refcounts = refcounts;
  a.seq_lens = seq_lens;
  a.query_start_loc = qsl;
  a.out = out;
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + plan.a_o);
  a.max_blocks = max_blocks;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.log2_block = log2i(block_size);
  a.num_blocks = num_blocks;
  a.split_tokens = plan.split_tokens;
  a.max_splits = plan.max_splits;
  a.max_query_len = max_query_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.kv_fp8 = f8.kv_fp8;
  a.k_scales = f8.k_scales;
  a.v_scales = f8.v_scales;
  a.new_k = new_k;
  a.new_v = new_v;
  // Piece counts per row: written by the MFMA chunk kernel only (the
  // vector-ALU path's merge derives its split count from split_tokens).
  a.row_pieces = plan.rp && mfma ? reinterpret_cast<int32_t*>(ws + plan.a_o + plan.a_ml) : nullptr;
  a.chunk_steps = plan.chunk_steps;
  a.chunk_auto = plan.chunk_auto;
  ws += plan.rp;  // region B and the header follow the piece counts
  void* header = ws + plan.a_o + plan.a_ml + plan.b_o + plan.b_ml;
  hipError_t err;
  if (chunk_entry) {
    a.sk_part_o = reinterpret_cast<float*>(ws + plan.a_o + plan.a_ml);
    a.sk_part_ml = reinterpret_cast<float*>(ws + plan.a_o + plan.a_ml + plan.b_o);
    a.sk_slots = plan.max_pieces;
    err = pa::launch_attention(a, true, header, st);
  } else if (plan.max_pieces > 0 && mfma && num_seqs <= kMaxBalancedSeqs) {
    a.sk_part_o = a.part_o;   // pa_decode: one region, rows = sequences
    a.sk_part_ml = a.part_ml;
    a.sk_slots = plan.max_pieces;
    if (prefix_keys > 0) {
      a.prefix_keys = prefix_keys;
      // sequences whose G query rows fill the prefix item's row tiles
      a.prefix_group = 16 * pa::prefix_tiles(f8.kv_fp8 != 0) / G;
      a.prefix_slots = prefix_piece_slots(prefix_keys);
    }
    err = pa::launch_decode_streamk(a, header, st);
  } else {
    if (a.kv_fp8) return PA_ERR_UNSUPPORTED;  // the fp8 cache has the balanced decode only
    // paths that do not fuse the appending decode's writes get them first
    err = new_k ? pa::launch_append_tokens(a, st) : hipSuccess;
    if (err == hipSuccess) err = pa::launch_attention(a, false, nullptr, st);
  }
  return err == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// Workspace of pa_chunked_prefill_fp8: the bf16 chunked-prefill plan, then
// the staging offsets (int32 [S + 1]), the staging tables (int32 [S,
// max_blocks]) and the bf16 staging pools (K then V, cap blocks each).
struct Fp8ChunkPlan {
  WorkspacePlan base;
  size_t off = 0, tables = 0, pool_k = 0, pool_v = 0, total = 0;
};

bool plan_chunked_fp8(int num_seqs, int num_tokens, int num_q_heads, int num_kv_heads,
                      int head_dim, int max_seq_len, int max_blocks, int block_size,
                      int64_t cap_blocks, Fp8ChunkPlan* p) {
  if (num_kv_heads <= 0 || max_blocks <= 0 || cap_blocks < 0) return false;
  if (!plan_workspace(num_tokens, num_seqs, num_q_heads, head_dim, max_seq_len, block_size, 0,
                      true, &p->base))
    return false;
  const size_t pool = (size_t)cap_blocks * num_kv_heads * block_size * head_dim * 2;
  p->off = p->base.total;
  p->tables = p->off + align_up((size_t)(num_seqs + 1) * 4);
  p->pool_k = p->tables + align_up((size_t)num_seqs * max_blocks * 4);
  p->pool_v = p->pool_k + align_up(pool);
  p->total = p->pool_v + align_up(pool);
  return true;
}

// PA_CHECK: the staging pool holds every block of the multi-token sequences.
int validate_stage_capacity(const int32_t* d_lens, const int32_t* d_qsl, int num_seqs,
                            int block_size, int max_blocks, int64_t cap, hipStream_t st) {
  std::vector<int32_t> lens(num_seqs), qsl(num_seqs + 1);
  if (hipMemcpyAsync(lens.data(), d_lens, lens.size() * 4, hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipMemcpyAsync(qsl.data(), d_qsl, qsl.size() * 4, hipMemcpyDeviceToHost, st) !=
          hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return PA_ERR_HIP;
  int64_t need = 0;
  for (int s = 0; s < num_seqs; ++s)
    if (qsl[s + 1] - qsl[s] > 1)
      need += std::min((std::max(lens[s], 0) + block_size - 1) / block_size, max_blocks);
  return need <= cap ? PA_OK : PA_ERR_INDEX;
}

// pa_decode_shared_prefix, with (append) or without the new tokens' write.
int shared_prefix_common(void* out, const void* query, const void* key, const void* value,
                         const void* k_cache, const void* v_cache, const float* k_scales,
                         const float* v_scales, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* block_refcounts,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, int32_t prefix_blocks,
                         float scale, void* workspace, size_t workspace_bytes, void* stream,
                         bool append) {
  if (prefix_blocks < 0 || (k_scales == nullptr) != (v_scales == nullptr)) return PA_ERR_SHAPE;
  const bool fp8 = k_scales != nullptr;
  if (block_size > 0 && block_size < (fp8 ? 16 : 8)) return PA_ERR_UNSUPPORTED;
  if ((int64_t)prefix_blocks * block_size > max_seq_len ||
      prefix_blocks > max_blocks_per_seq)
    return PA_ERR_SHAPE;
  // Without a whole prefix step there is no prefix entry: pa_decode's (or
  // pa_decode_fp8's) limits apply, including the bf16 fixed-split fallback.
  const int pstep = fp8 ? 64 : 32;
  const int64_t prefix_keys = block_size > 0 ? (int64_t)prefix_blocks * block_size / pstep * pstep : 0;
  if (prefix_keys > 0 && num_q_heads > 0 && num_kv_heads > 0 &&
      num_q_heads % num_kv_heads == 0 && num_q_heads / num_kv_heads <= 16) {
    const int spg = 16 * pa::prefix_tiles(fp8) / (num_q_heads / num_kv_heads);
    if ((int64_t)num_seqs + (num_seqs + spg - 1) / spg > kMaxBalancedSeqs)
      return PA_ERR_UNSUPPORTED;
  }
  Fp8Kv f8;
  f8.kv_fp8 = fp8 ? 1 : 0;
  f8.k_scales = k_scales;
  f8.v_scales = v_scales;
  return attention_common(out, query, k_cache, v_cache, block_tables, max_blocks_per_seq,
                          block_refcounts, seq_lens, nullptr, num_seqs, num_seqs, max_seq_len, 1,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                          PA_BF16, 0, workspace, workspace_bytes, stream, f8, prefix_blocks,
                          append, key, value);
}

}  // namespace

extern "C" {

const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: a size or count is out of range";
    case PA_ERR_DTYPE: return "PA_ERR_DTYPE: unknown dtype";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: shape not implemented";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_INDEX: return "PA_ERR_INDEX: device metadata out of range (PA_CHECK)";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime or launch failure";
    case PA_ERR_SCRATCH:
      return "PA_ERR_SCRATCH: the batch needs more workspace than pa_decode_noalloc's static "
             "scratch (PA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown pa_status";
  }
}

int pa_version(void) { return 100; }

int pa_compute_slot_mapping(int64_t* slot_mapping, const int32_t* block_tables,
                            int32_t max_blocks_per_seq, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t num_seqs,
                            int32_t num_tokens, int32_t block_size, void* stream) {
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq <= 0) return PA_ERR_SHAPE;
  if (!is_pow2(block_size) || block_size > 64) return PA_ERR_UNSUPPORTED;
  if (!query_start_loc && num_tokens != num_seqs) return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!slot_mapping || !block_tables || !seq_lens) return PA_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    // Table entries are checked against no pool size here (slots only).
    int rc = validate_metadata(block_tables, max_blocks_per_seq, seq_lens, query_start_loc,
                               num_seqs, num_tokens, 1 << 30, 1 << 30, block_size,
                               1 << 30, st);
    if (rc != PA_OK) return rc;
  }
  return pa::launch_slot_mapping(slot_mapping, block_tables, max_blocks_per_seq, seq_lens,
                                 query_start_loc, num_seqs, num_tokens, block_size,
                                 st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                         int32_t head_dim, int32_t block_size, int32_t num_blocks,
                         int32_t dtype, void* stream) {
  if (dtype != PA_F32 && dtype != PA_BF16) return PA_ERR_DTYPE;
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!is_pow2(block_size) || block_size > 64) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping) return PA_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    int rc = validate_slots(slot_mapping, num_tokens, (int64_t)num_blocks * block_size, st);
    if (rc != PA_OK) return rc;
  }
  return pa::launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, num_tokens,
                                      num_kv_heads, head_dim, block_size, num_blocks,
                                      dtype == PA_BF16 ? 2 : 4, st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

size_t pa_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                 int32_t max_seq_len, int32_t block_size,
                                 int32_t kv_split_tokens) {
  WorkspacePlan p;
  if (!plan_workspace(num_seqs, num_seqs, num_q_heads, head_dim, max_seq_len, block_size,
                      kv_split_tokens, false, &p))
    return 0;
  return p.total;
}

int pa_decode(void* out, const void* query, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, int32_t max_blocks_per_seq,
              const int32_t* block_refcounts, const int32_t* seq_lens,
              int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads, int32_t num_kv_heads,
              int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
              int32_t dtype, int32_t kv_split_tokens, void* workspace, size_t workspace_bytes,
              void* stream) {
  return attention_common(out, query, k_cache, v_cache, block_tables, max_blocks_per_seq,
                          block_refcounts, seq_lens, nullptr, num_seqs, num_seqs, max_seq_len, 1, num_q_heads,
                          num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                          kv_split_tokens, workspace, workspace_bytes, stream);
}

int pa_decode_append(void* out, const void* query, const void* key, const void* value,
                     void* k_cache, void* v_cache, const int32_t* block_tables,
                     int32_t max_blocks_per_seq, const int32_t* block_refcounts,
                     const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                     int32_t block_size, int32_t num_blocks, float scale, int32_t dtype,
                     int32_t kv_split_tokens, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return attention_common(out, query, k_cache, v_cache, block_tables, max_blocks_per_seq,
                          block_refcounts, seq_lens, nullptr, num_seqs, num_seqs, max_seq_len, 1,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                          dtype, kv_split_tokens, workspace, workspace_bytes, stream, Fp8Kv(), 0,
                          true, key, value);
}

size_t pa_chunked_prefill_workspace_bytes(int32_t num_seqs, int32_t num_tokens,
                                          int32_t num_q_heads, int32_t head_dim,
                                          int32_t max_seq_len, int32_t block_size,
                                          int32_t kv_split_tokens) {
  WorkspacePlan p;
  if (!plan_workspace(num_tokens, num_seqs, num_q_heads, head_dim, max_seq_len, block_size,
                      kv_split_tokens, true, &p))
    return 0;
  return p.total;
}

int pa_chunked_prefill(void* out, const void* query, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, int32_t max_blocks_per_seq,
                       const int32_t* block_refcounts, const int32_t* seq_lens,
                       const int32_t* query_start_loc,
                       int32_t num_seqs, int32_t num_tokens, int32_t max_seq_len,
                       int32_t max_query_len, int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                       int32_t dtype, int32_t kv_split_tokens, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (num_seqs > 0 && num_tokens > 0 && !query_start_loc) return PA_ERR_NULL;
  return attention_common(out, query, k_cache, v_cache, block_tables, max_blocks_per_seq,
                          block_refcounts, seq_lens, query_start_loc, num_seqs, num_tokens,
                          max_seq_len,
                          max_query_len, num_q_heads, num_kv_heads, head_dim, block_size,
                          num_blocks, scale, dtype, kv_split_tokens, workspace,
                          workspace_bytes, stream);
}

}  // extern "C"

namespace {

// Device-accessible address of a pool: device memory as is, pinned host
// memory through its mapped device pointer.  Pageable host memory (or any
// pointer HIP does not know) is refused.
int device_address(const void* p, const void** out) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // do not leave the error for the next call
    return PA_ERR_UNSUPPORTED;
  }
  if (attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged) {
    *out = p;
    return PA_OK;
  }
  if (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) {
    const char* host = static_cast<const char*>(attr.hostPointer ? attr.hostPointer : p);
    *out = static_cast<const char*>(attr.devicePointer) + (static_cast<const char*>(p) - host);
    return PA_OK;
  }
  return PA_ERR_UNSUPPORTED;
}

// PA_CHECK for block mappings: ids in range, destinations distinct, and
// within one pool no destination is also a source.
int validate_mapping(const int64_t* d_map, int num_pairs, int64_t src_nb, int64_t dst_nb,
                     bool same_pool, hipStream_t st) {
  std::vector<int64_t> m(2 * (size_t)num_pairs);
  if (hipMemcpyAsync(m.data(), d_map, m.size() * 8, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return PA_ERR_HIP;
  std::vector<int64_t> dsts, srcs;
  for (int p = 0; p < num_pairs; ++p) {
    const int64_t s = m[2 * (size_t)p], d = m[2 * (size_t)p + 1];
    if (s < 0 || s >= src_nb || d < 0 || d >= dst_nb) return PA_ERR_INDEX;
    srcs.push_back(s);
    dsts.push_back(d);
  }
  std::sort(dsts.begin(), dsts.end());
  for (size_t i = 1; i < dsts.size(); ++i)
    if (dsts[i] == dsts[i - 1]) return PA_ERR_INDEX;
  if (same_pool)
    for (int64_t s : srcs)
      if (std::binary_search(dsts.begin(), dsts.end(), s)) return PA_ERR_INDEX;
  return PA_OK;
}

int copy_common(void* dst, const void* src, const int64_t* mapping, int32_t num_pairs,
                int64_t block_bytes, int32_t dst_num_blocks, int32_t src_num_blocks,
                bool same_pool, void* stream) {
  if (num_pairs < 0 || block_bytes <= 0 || block_bytes % 4 != 0 || dst_num_blocks <= 0 ||
      src_num_blocks <= 0)
    return PA_ERR_SHAPE;
  if (num_pairs == 0) return PA_OK;
  if (!dst || !src || !mapping) return PA_ERR_NULL;
  const void* dd = nullptr;
  const void* sd = nullptr;
  int rc = device_address(dst, &dd);
  if (rc == PA_OK) rc = device_address(src, &sd);
  if (rc != PA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    rc = validate_mapping(mapping, num_pairs, src_num_blocks, dst_num_blocks, same_pool, st);
    if (rc != PA_OK) return rc;
  }
  return pa::launch_copy_blocks(const_cast<void*>(dd), sd, mapping, num_pairs, block_bytes,
                                src_num_blocks, dst_num_blocks, st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int pa_copy_blocks(void* pool, const int64_t* block_mapping, int32_t num_pairs,
                   int64_t block_bytes, int32_t num_blocks, void* stream) {
  return copy_common(pool, pool, block_mapping, num_pairs, block_bytes, num_blocks, num_blocks,
                     true, stream);
}

int pa_swap_blocks(void* dst_pool, const void* src_pool, const int64_t* block_mapping,
                   int32_t num_pairs, int64_t block_bytes, int32_t dst_num_blocks,
                   int32_t src_num_blocks, void* stream) {
  if (dst_pool == src_pool && dst_pool != nullptr) return PA_ERR_SHAPE;  // use pa_copy_blocks
  return copy_common(dst_pool, src_pool, block_mapping, num_pairs, block_bytes, dst_num_blocks,
                     src_num_blocks, false, stream);
}

int pa_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                             const float* k_scales, const float* v_scales,
                             const int64_t* slot_mapping, int32_t num_tokens,
                             int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                             int32_t num_blocks, void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || num_blocks <= 0) return PA_ERR_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (!is_pow2(block_size) || block_size < 16 || block_size > 64) return PA_ERR_UNSUPPORTED;
  if (num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
  if (num_tokens == 0) return PA_OK;
  if (!key || !value || !k_cache || !v_cache || !k_scales || !v_scales || !slot_mapping)
    return PA_ERR_NULL;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    int rc = validate_slots(slot_mapping, num_tokens, num_slots, st);
    if (rc != PA_OK) return rc;
    std::vector<int64_t> slots(num_tokens), blocks;
    if (hipMemcpyAsync(slots.data(), slot_mapping, slots.size() * 8, hipMemcpyDeviceToHost, st) !=
            hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess)
      return PA_ERR_HIP;
    for (int64_t s : slots)
      if (s >= 0) blocks.push_back(s / block_size);
    rc = validate_scales(k_scales, v_scales, num_blocks, num_kv_heads, blocks, st);
    if (rc != PA_OK) return rc;
  }
  return pa::launch_reshape_and_cache_fp8(key, value, k_cache, v_cache, k_scales, v_scales,
                                          slot_mapping, num_tokens, num_kv_heads, head_dim,
                                          block_size, num_blocks, st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

size_t pa_decode_fp8_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                     int32_t max_seq_len, int32_t block_size) {
  if (block_size < 16) return 0;
  return pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len, block_size, 0);
}

size_t pa_decode_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                               int32_t head_dim, int32_t max_seq_len,
                                               int32_t block_size, int32_t prefix_blocks) {
  if (prefix_blocks < 0 || block_size < 8) return 0;
  WorkspacePlan p;
  if ((int64_t)prefix_blocks * block_size > max_seq_len) return 0;
  const int64_t pk = (int64_t)prefix_blocks * block_size / 32 * 32;
  if (!plan_workspace(num_seqs, num_seqs, num_q_heads, head_dim, max_seq_len, block_size, 0,
                      false, &p, (int)pk))
    return 0;
  return p.total;
}

int pa_decode_shared_prefix(void* out, const void* query, const void* k_cache,
                            const void* v_cache, const float* k_scales, const float* v_scales,
                            const int32_t* block_tables, int32_t max_blocks_per_seq,
                            const int32_t* block_refcounts, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                            int32_t num_blocks, int32_t prefix_blocks, float scale,
                            void* workspace, size_t workspace_bytes, void* stream) {
  return shared_prefix_common(out, query, nullptr, nullptr, k_cache, v_cache, k_scales, v_scales,
                              block_tables, max_blocks_per_seq, block_refcounts, seq_lens,
                              num_seqs, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                              block_size, num_blocks, prefix_blocks, scale, workspace,
                              workspace_bytes, stream, false);
}

int pa_decode_shared_prefix_append(void* out, const void* query, const void* key,
                                   const void* value, void* k_cache, void* v_cache,
                                   const float* k_scales, const float* v_scales,
                                   const int32_t* block_tables, int32_t max_blocks_per_seq,
                                   const int32_t* block_refcounts, const int32_t* seq_lens,
                                   int32_t num_seqs, int32_t max_seq_len, int32_t num_q_heads,
                                   int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                   int32_t num_blocks, int32_t prefix_blocks, float scale,
                                   void* workspace, size_t workspace_bytes, void* stream) {
  return shared_prefix_common(out, query, key, value, k_cache, v_cache, k_scales, v_scales,
                              block_tables, max_blocks_per_seq, block_refcounts, seq_lens,
                              num_seqs, max_seq_len, num_q_heads, num_kv_heads, head_dim,
                              block_size, num_blocks, prefix_blocks, scale, workspace,
                              workspace_bytes, stream, true);
}

int pa_decode_fp8(void* out, const void* query, const void* k_cache, const void* v_cache,
                  const float* k_scales, const float* v_scales, const int32_t* block_tables,
                  int32_t max_blocks_per_seq, const int32_t* block_refcounts,
                  const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                  int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                  int32_t block_size, int32_t num_blocks, float scale, void* workspace,
                  size_t workspace_bytes, void* stream) {
  // The fp8 decode runs on the balanced kernel only (block_size >= 16: a
  // lane's 16 consecutive keys share one block and so one scale).
  if (block_size > 0 && block_size < 16) return PA_ERR_UNSUPPORTED;
  if (num_seqs > kMaxBalancedSeqs) return PA_ERR_UNSUPPORTED;
  Fp8Kv f8;
  f8.kv_fp8 = 1;
  f8.k_scales = k_scales;
  f8.v_scales = v_scales;
  return attention_common(out, query, k_cache, v_cache, block_tables, max_blocks_per_seq,
                          block_refcounts, seq_lens, nullptr, num_seqs, num_seqs, max_seq_len, 1,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                          PA_BF16, 0, workspace, workspace_bytes, stream, f8);
}

int pa_decode_fp8_append(void* out, const void* query, const void* key, const void* value,
                         void* k_cache, void* v_cache, const float* k_scales,
                         const float* v_scales, const int32_t* block_tables,
                         int32_t max_blocks_per_seq, const int32_t* block_refcounts,
                         const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         int32_t block_size, int32_t num_blocks, float scale, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (block_size > 0 && block_size < 16) return PA_ERR_UNSUPPORTED;
  if (num_seqs > kMaxBalancedSeqs) return PA_ERR_UNSUPPORTED;
  Fp8Kv f8;
  f8.kv_fp8 = 1;
  f8.k_scales = k_scales;
  f8.v_scales = v_scales;
  return attention_common(out, query, k_cache, v_cache, block_tables, max_blocks_per_seq,
                          block_refcounts, seq_lens, nullptr, num_seqs, num_seqs, max_seq_len, 1,
                          num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, scale,
                          PA_BF16, 0, workspace, workspace_bytes, stream, f8, 0, true, key,
                          value);
}

size_t pa_chunked_prefill_fp8_workspace_bytes(int32_t num_seqs, int32_t num_tokens,
                                              int32_t num_q_heads, int32_t num_kv_heads,
                                              int32_t head_dim, int32_t max_seq_len,
                                              int32_t max_blocks_per_seq, int32_t block_size,
                                              int64_t chunk_context_blocks) {
  if (block_size < 16) return 0;
  Fp8ChunkPlan p;
  if (!plan_chunked_fp8(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                        max_blocks_per_seq, block_size, chunk_context_blocks, &p))
    return 0;
  return p.total;
}

int pa_chunked_prefill_fp8(void* out, const void* query, const void* k_cache,
                           const void* v_cache, const float* k_scales, const float* v_scales,
                           const int32_t* block_tables, int32_t max_blocks_per_seq,
                           const int32_t* block_refcounts, const int32_t* seq_lens,
                           const int32_t* query_start_loc, int32_t num_seqs, int32_t num_tokens,
                           int32_t max_seq_len, int32_t max_query_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int64_t chunk_context_blocks, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int rc = check_common(num_q_heads, num_kv_heads, head_dim, block_size, PA_BF16);
  if (rc != PA_OK) return rc;
  if (block_size < 16) return PA_ERR_UNSUPPORTED;
  if (num_seqs < 0 || num_tokens < 0 || max_blocks_per_seq <= 0 || num_blocks <= 0 ||
      max_seq_len <= 0 || max_query_len <= 0 || chunk_context_blocks < 0 || !isfinite(scale) ||
      !(scale > 0.f))
    return PA_ERR_SHAPE;
  if (num_seqs == 0 || num_tokens == 0) return PA_OK;
  if (!out || !query || !k_cache || !v_cache || !k_scales || !v_scales || !block_tables ||
      !seq_lens || !query_start_loc)
    return PA_ERR_NULL;
  if (num_seqs > pa::kMaxChunkSeqs) return PA_ERR_UNSUPPORTED;
  if ((int64_t)num_seqs * num_kv_heads > 65535 || (int64_t)num_tokens > 65535 * 64)
    return PA_ERR_UNSUPPORTED;
  if (chunk_context_blocks > INT32_MAX) return PA_ERR_UNSUPPORTED;
  // the chunk kernel reads the bf16 staging pools (one dword of 256-byte
  // units per block offset)
  if (chunk_context_blocks * num_kv_heads * block_size * head_dim * 2 >= kMaxChunkPoolBytes)
    return PA_ERR_UNSUPPORTED;
  // query chunks need a staging pool of at least one block (every staging
  // table entry is clamped into it)
  if (max_query_len > 1 && chunk_context_blocks < 1) return PA_ERR_SHAPE;
  Fp8ChunkPlan plan;
  if (!plan_chunked_fp8(num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, max_seq_len,
                        max_blocks_per_seq, block_size, chunk_context_blocks, &plan))
    return PA_ERR_SHAPE;
  if (plan.base.max_splits > 65535) return PA_ERR_UNSUPPORTED;
  if (!workspace) return PA_ERR_WORKSPACE;
  if (workspace_bytes < plan.total) return PA_ERR_WORKSPACE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (check_enabled()) {
    rc = validate_metadata(block_tables, max_blocks_per_seq, seq_lens, query_start_loc, num_seqs,
                           num_tokens, max_seq_len, max_query_len, block_size, num_blocks, st);
    if (rc != PA_OK) return rc;
    std::vector<int64_t> used;
    rc = table_blocks_used(block_tables, max_blocks_per_seq, seq_lens, num_seqs, block_size, st,
                           &used);
    if (rc == PA_OK)
      rc = validate_scales(k_scales, v_scales, num_blocks, num_kv_heads, used, st);
    if (rc == PA_OK)
      rc = validate_stage_capacity(seq_lens, query_start_loc, num_seqs, block_size,
                                   max_blocks_per_seq, chunk_context_blocks, st);
    if (rc != PA_OK) return rc;
  }
  const WorkspacePlan& wp = plan.base;
  char* ws = static_cast<char*>(workspace);
  pa::AttnArgs a;
  memset(&a, 0, sizeof(a));
  a.bf16 = 1;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.q = query;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.block_refcounts = block_refcounts;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  a.out = out;
  a.part_o = reinterpret_cast<float*>(ws);
  a.part_ml = reinterpret_cast<float*>(ws + wp.a_o);
  a.row_pieces = reinterpret_cast<int32_t*>(ws + wp.a_o + wp.a_ml);
  char* wb = ws + wp.rp;  // region B and the header follow the piece counts
  a.sk_part_o = reinterpret_cast<float*>(wb + wp.a_o + wp.a_ml);
  a.sk_part_ml = reinterpret_cast<float*>(wb + wp.a_o + wp.a_ml + wp.b_o);
  a.sk_slots = wp.max_pieces;
  void* header = wb + wp.a_o + wp.a_ml + wp.b_o + wp.b_ml;
  a.max_blocks = max_blocks_per_seq;
  a.num_seqs = num_seqs;
  a.num_tokens = num_tokens;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.log2_block = log2i(block_size);
  a.num_blocks = num_blocks;
  a.split_tokens = wp.split_tokens;
  a.max_splits = wp.max_splits;
  a.max_query_len = max_query_len;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.chunk_steps = wp.chunk_steps;
  a.chunk_auto = wp.chunk_auto;
  a.kv_fp8 = 1;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  // the same call on the bf16 staging pools, for the chunk kernel
  pa::AttnArgs c = a;
  c.kv_fp8 = 0;
  c.k_scales = nullptr;
  c.v_scales = nullptr;
  c.block_refcounts = nullptr;  // staging blocks are private
  c.k_cache = ws + plan.pool_k;
  c.v_cache = ws + plan.pool_v;
  c.block_tables = reinterpret_cast<const int32_t*>(ws + plan.tables);
  c.num_blocks = (int32_t)std::max<int64_t>(chunk_context_blocks, 1);
  return pa::launch_chunked_fp8(a, c, header, chunk_context_blocks,
                                reinterpret_cast<int32_t*>(ws + plan.off), st) == hipSuccess
             ? PA_OK
             : PA_ERR_HIP;
}

}  // extern "C"
