// HIP kernels of libpa for gfx950 (CDNA4, wave64).
//
// The method these kernels implement: a sequence's K/V lives in fixed-size
// physical blocks named by its block table; logical block floor(pos / B),
// offset pos mod B ("High-Throughput Local LLM Infrastructure ...", section
// "1.2 PagedAttention Mechanics & Virtual Page Tables", index and offset
// equations).  Attention looks up the table, fetches each block's K and V
// tiles and computes softmax(q K^T * scale) V over them ("03 --
// PagedAttention & the vLLM V1 Architecture", section "The attention kernel
// side").
//
// Kernels
//   slot_mapping_kernel          slot of every query token (index equations)
//   reshape_and_cache_kernel     bit copy of new K/V into their slots
//   reshape_and_cache_fp8_kernel the same into e4m3 pools (per-block scales)
//   copy_blocks_kernel           whole-block copies (copy-on-write, swap)
//   decode_streamk_kernel<D, FP8, PREFIX>
//                                balanced split-K decode (bf16 or e4m3
//                                cache); QK^T and PV on
//                                v_mfma_f32_16x16x32_bf16, online softmax in
//                                fp32 with cross-lane max/sum; with PREFIX,
//                                a shared prefix read once per group of
//                                sequences
//   merge_streamk_kernel         log-sum-exp merge of its pieces
//   prefill_kernel<D>            causal query chunks on
//                                v_mfma_f32_32x32x16_bf16, K/V staged in LDS
//   chunk_mix_kernel<D>          the query chunks and the single-token rows
//                                of one call in one persistent launch, the
//                                CUs split between the two kinds of work
//   chunk_mix_fp8_kernel<D>      the same over an e4m3 cache (chunk units on
//                                bf16-staged blocks)
//   stage_offsets_kernel, stage_fp8_kernel<D>
//                                the staging of those blocks
//   attn_mfma_kernel<D>          fixed-split bf16 decode
//   attn_valu_kernel<ES, D>      fp32 (and small-block bf16) split-K attention
//                                on the vector ALUs
//   merge_kernel<ES, D>          exact log-sum-exp merge of split partials
//
// Cache layout: K [NB, Hkv, B, D] (token rows), V [NB, Hkv, D, B] (each
// head_dim row holds the block's tokens).  The V layout lets one 16-byte
// load fetch 8 consecutive tokens of one head_dim column, which is exactly
// what the PV MFMA's B operand holds per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <type_traits>

#include "pa_internal.h"

namespace pa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int clampi(int x, int lo, int hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt immediate that waits until at most n vector-memory operations of
// this wave are outstanding (vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt
// left at their "no wait" maxima).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}

// Streaming load: the line is not expected to be read again soon.
__device__ __forceinline__ bf16x8 load_bf16x8_nt(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
}

template <int ES>
__device__ __forceinline__ float load_elem(const void* base, int64_t idx) {
  if constexpr (ES == 2) {
    uint32_t bits = static_cast<const uint16_t*>(base)[idx];
    return __uint_as_float(bits << 16);
  } else {
    return static_cast<const float*>(base)[idx];
  }
}

template <int ES>
__device__ __forceinline__ void store_elem(void* base, int64_t idx, float v) {
  if constexpr (ES == 2) {
    static_cast<uint16_t*>(base)[idx] = f32_to_bf16_bits(v);
  } else {
    static_cast<float*>(base)[idx] = v;
  }
}

// Rows [r0, r0 + qn) of sequence s, clamped so that any metadata value keeps
// every access inside the q/out arrays.
__device__ __forceinline__ void seq_rows(const int32_t* qsl, int s, int T, int& r0, int& qn) {
  if (qsl) {
    r0 = clampi(qsl[s], 0, T);
    qn = clampi(qsl[s + 1] - r0, 0, T - r0);
  } else {
    r0 = s < T ? s : T;
    qn = s < T ? 1 : 0;
  }
}

// Number of cached keys the table of a sequence of length L can address.
__device__ __forceinline__ int table_blocks(int L, int lg, int max_blocks) {
  int B = 1 << lg;
  return min((max(L, 0) + B - 1) >> lg, max_blocks);
}

// ---------------------------------------------------------------------------
// Slot mapping: slot = table[pos / B] * B + pos % B for the query positions.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void slot_mapping_kernel(
    int64_t* __restrict__ slots, const int32_t* __restrict__ bt, int max_blocks,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ qsl, int T, int lg) {
  const int s = blockIdx.x;
  int r0, qn;
  seq_rows(qsl, s, T, r0, qn);
  const int L = seq_lens[s];
  const int B = 1 << lg;
  for (int j = threadIdx.x; j < qn; j += blockDim.x) {
    const int pos = L - qn + j;
    int64_t slot = -1;
    if (pos >= 0 && (pos >> lg) < max_blocks) {
      const int64_t id = bt[(int64_t)s * max_blocks + (pos >> lg)];
      slot = id * B + (pos & (B - 1));
    }
    slots[r0 + j] = slot;
  }
}

// ---------------------------------------------------------------------------
// reshape_and_cache: one workgroup moves 16 tokens of one KV head.  K rows are
// copied as 16-byte vectors (head_dim contiguous on both sides); V is written
// column-wise with lanes running over tokens so that tokens bound for
// consecutive offsets of one block land in consecutive bytes.
// ---------------------------------------------------------------------------
template <int ES, int D>
__global__ __launch_bounds__(16 * D * ES / 16) void reshape_and_cache_kernel(
    const void* __restrict__ key, const void* __restrict__ value, void* __restrict__ k_cache,
    void* __restrict__ v_cache, const int64_t* __restrict__ slots, int ntok, int H, int lg,
    int64_t num_slots) {
  typedef typename std::conditional<ES == 2, uint16_t, uint32_t>::type E;
  constexpr int VEC = 16 / ES;  // elements per 16-byte vector
  constexpr int NV = D / VEC;   // vectors per head row
  const int B = 1 << lg;
  const int h = blockIdx.y;
  const int t0 = blockIdx.x * 16;
  const int tid = threadIdx.x;
  {
    const int t = t0 + tid / NV;
    const int vec = tid % NV;
    if (t < ntok) {
      const int64_t slot = slots[t];
      if (slot >= 0 && slot < num_slots) {
        const int64_t blk = slot >> lg;
        const int off = (int)(slot & (B - 1));
        const u32x4* src = reinterpret_cast<const u32x4*>(
                               static_cast<const E*>(key) + ((int64_t)t * H + h) * D) + vec;
        u32x4* dst = reinterpret_cast<u32x4*>(
                         static_cast<E*>(k_cache) + ((blk * H + h) * B + off) * D) + vec;
        *dst = *src;
      }
    }
  }
  {
    const int t = t0 + (tid & 15);
    const int vec = tid >> 4;
    if (t < ntok) {
      const int64_t slot = slots[t];
      if (slot >= 0 && slot < num_slots) {
        const int64_t blk = slot >> lg;
        const int off = (int)(slot & (B - 1));
        const u32x4 raw = *(reinterpret_cast<const u32x4*>(
                                static_cast<const E*>(value) + ((int64_t)t * H + h) * D) + vec);
        E vals[VEC];
        __builtin_memcpy(vals, &raw, 16);
        E* dst = static_cast<E*>(v_cache) + ((blk * H + h) * D + vec * VEC) * B + off;
#pragma unroll
        for (int e = 0; e < VEC; ++e) dst[(int64_t)e * B] = vals[e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Whole-block copies between two pools (or inside one): copy-on-write and
// swapping to / from pinned host memory.  Grid: x = chunks of one block,
// y = mapping pairs (grid-stride); 16-byte accesses when the block size and
// both pools allow, 4-byte ones otherwise.  Pairs naming a block outside a
// pool are skipped.
// ---------------------------------------------------------------------------
template <typename V>
__global__ __launch_bounds__(256) void copy_blocks_kernel(
    uint8_t* __restrict__ dst, const uint8_t* __restrict__ src,
    const int64_t* __restrict__ mapping, int num_pairs, int64_t block_bytes, int64_t src_nb,
    int64_t dst_nb) {
  const int64_t n = block_bytes / (int64_t)sizeof(V);
  for (int p = blockIdx.y; p < num_pairs; p += gridDim.y) {
    const int64_t sb = mapping[2 * (int64_t)p];
    const int64_t db = mapping[2 * (int64_t)p + 1];
    if (sb < 0 || sb >= src_nb || db < 0 || db >= dst_nb) continue;
    const V* s = reinterpret_cast<const V*>(src + sb * block_bytes);
    V* d = reinterpret_cast<V*>(dst + db * block_bytes);
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
      d[i] = s[i];
  }
}

// ---------------------------------------------------------------------------
// reshape_and_cache into an fp8 (e4m3) cache.  Each element x of a bf16 K/V
// row becomes the e4m3 code of clamp(x / s, -448, 448), rounded to nearest
// even, with s the scale of the (block, KV head) the slot lies in; the
// division is the correctly rounded float32 one.  One thread converts 8
// elements of one token: 16 tokens of one KV head per workgroup.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t quant4_e4m3(float a, float b, float c, float d) {
  uint32_t r = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, r, true);
}

__device__ __forceinline__ float sat_e4m3(float y) { return fminf(fmaxf(y, -448.f), 448.f); }

template <int D>
__global__ __launch_bounds__(2 * D) void reshape_and_cache_fp8_kernel(
    const uint16_t* __restrict__ key, const uint16_t* __restrict__ value,
    uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
    const float* __restrict__ k_scales, const float* __restrict__ v_scales,
    const int64_t* __restrict__ slots, int ntok, int H, int lg, int64_t num_slots) {
  constexpr int NG = D / 8;  // 8-element groups per head row
  const int B = 1 << lg;
  const int h = blockIdx.y;
  const int t = blockIdx.x * 16 + threadIdx.x / NG;
  const int g = threadIdx.x % NG;
  if (t >= ntok) return;
  const int64_t slot = slots[t];
  if (slot < 0 || slot >= num_slots) return;
  const int64_t blk = slot >> lg;
  const int off = (int)(slot & (B - 1));
  const int64_t src = ((int64_t)t * H + h) * D + 8 * g;
  {
    const float ks = k_scales[blk * H + h];
    const u32x4 raw = *reinterpret_cast<const u32x4*>(key + src);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(raw[e] << 16);
      x[2 * e + 1] = __uint_as_float(raw[e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sat_e4m3(__fdiv_rn(x[e], ks));
    uint2 q;
    q.x = quant4_e4m3(x[0], x[1], x[2], x[3]);
    q.y = quant4_e4m3(x[4], x[5], x[6], x[7]);
    *reinterpret_cast<uint2*>(k_cache + ((blk * H + h) * B + off) * D + 8 * g) = q;
  }
  {
    const float vs = v_scales[blk * H + h];
    const u32x4 raw = *reinterpret_cast<const u32x4*>(value + src);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = __uint_as_float(raw[e] << 16);
      x[2 * e + 1] = __uint_as_float(raw[e] & 0xFFFF0000u);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = sat_e4m3(__fdiv_rn(x[e], vs));
    const uint32_t lo = quant4_e4m3(x[0], x[1], x[2], x[3]);
    const uint32_t hi = quant4_e4m3(x[4], x[5], x[6], x[7]);
    uint8_t* dst = v_cache + ((blk * H + h) * D + 8 * g) * B + off;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      dst[(int64_t)e * B] = (lo >> (8 * e)) & 0xFF;
      dst[(int64_t)(e + 4) * B] = (hi >> (8 * e)) & 0xFF;
    }
  }
}

// ---------------------------------------------------------------------------
// Appending decode: the new token of sequence s (row t of new_k / new_v) goes
// to position L - 1 of its table, slot table[s][(L-1) / B] * B + (L-1) mod B,
// the slot slot_mapping_kernel gives that position.  The bits written are
// those of reshape_and_cache_kernel (a copy) or, for an e4m3 pool, of
// reshape_and_cache_fp8_kernel (the same division, clamp and RNE
// conversion, element by element).  Nothing is written where the table
// cannot address the position or names a block outside the pool, as with a
// negative or out-of-range slot there.  One wave, D / 64 elements per lane.
// Nothing waits for the stores: the attention of the same call takes the
// token from its rows, and later calls are ordered by the stream.
// ---------------------------------------------------------------------------
template <int ES, int D, bool FP8>
__device__ __forceinline__ void append_token(const AttnArgs& a, int s, int kvh, int L, int t) {
  constexpr int PER = D / 64;  // elements per lane
  static_assert(PER == 1 || PER == 2, "head_dim 64 or 128");
  const int lane = threadIdx.x & 63;
  const int lg = a.log2_block;
  const int pos = L - 1;
  if (pos < 0 || (pos >> lg) >= a.max_blocks) return;
  const int id = a.block_tables[(int64_t)s * a.max_blocks + (pos >> lg)];
  if (id < 0 || id >= a.num_blocks) return;
  const int B = 1 << lg;
  const int off = pos & (B - 1);
  const int64_t hb = (int64_t)id * a.num_kv_heads + kvh;  // (block, KV head)
  const int64_t src = ((int64_t)t * a.num_kv_heads + kvh) * D + PER * lane;
  const int64_t kdst = (hb * B + off) * D + PER * lane;   // K row of the slot
  const int64_t vdst = (hb * D + PER * lane) * B + off;   // V column entries, stride B
  if constexpr (FP8) {
    const uint16_t* nk = static_cast<const uint16_t*>(a.new_k) + src;
    const uint16_t* nv = static_cast<const uint16_t*>(a.new_v) + src;
    const float ks = a.k_scales[hb], vs = a.v_scales[hb];
    float xk[2] = {0.f, 0.f}, xv[2] = {0.f, 0.f};
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      xk[e] = sat_e4m3(__fdiv_rn(__uint_as_float((uint32_t)nk[e] << 16), ks));
      xv[e] = sat_e4m3(__fdiv_rn(__uint_as_float((uint32_t)nv[e] << 16), vs));
    }
    const uint32_t ck = __builtin_amdgcn_cvt_pk_fp8_f32(xk[0], xk[1], 0, false);
    const uint32_t cv = __builtin_amdgcn_cvt_pk_fp8_f32(xv[0], xv[1], 0, false);
    uint8_t* kc = static_cast<uint8_t*>(const_cast<void*>(a.k_cache));
    uint8_t* vc = static_cast<uint8_t*>(const_cast<void*>(a.v_cache));
    if constexpr (PER == 2) *reinterpret_cast<uint16_t*>(kc + kdst) = (uint16_t)(ck & 0xFFFF);
    else kc[kdst] = (uint8_t)(ck & 0xFF);
#pragma unroll
    for (int e = 0; e < PER; ++e) vc[vdst + (int64_t)e * B] = (uint8_t)((cv >> (8 * e)) & 0xFF);
  } else {
    typedef typename std::conditional<ES == 2, uint16_t, uint32_t>::type E;
    const E* nk = static_cast<const E*>(a.new_k) + src;
    const E* nv = static_cast<const E*>(a.new_v) + src;
    E* kc = static_cast<E*>(const_cast<void*>(a.k_cache));
    E* vc = static_cast<E*>(const_cast<void*>(a.v_cache));
#pragma unroll
    for (int e = 0; e < PER; ++e) {
      kc[kdst + e] = nk[e];
      vc[vdst + (int64_t)e * B] = nv[e];
    }
  }
}

// The appending decode's writes on their own, before an attention path that
// does not fuse them (fixed splits, the vector-ALU kernel): one wave per
// (sequence, KV head).
template <int ES, int D, bool FP8>
__global__ __launch_bounds__(64) void append_tokens_kernel(AttnArgs a) {
  const int s = blockIdx.x, kvh = blockIdx.y;
  append_token<ES, D, FP8>(a, s, kvh, a.seq_lens[s], s);
}

// ---------------------------------------------------------------------------
// bf16 attention on MFMA.
//
// One wave serves one (sequence, KV head, row-tile group, context split).
// Query rows of a sequence are enumerated row = j * G + g (token j of the
// chunk, head g of the group); a wave holds R tiles of 16 rows.  Keys are
// walked in chunks of 32 tokens.
//
// QK^T uses the 16x16x32 MFMA with A = K (16 token rows x 32 head_dim) and
// B = Q^T (32 head_dim x 16 query rows), two MFMAs per chunk ("a" and "b").
// MFMA row i of "a" is token 8*(i/4) + i%4 of the chunk and row i of "b" is
// that token + 4, so the accumulator layout (lane l holds rows 4*(l/16)+r,
// column l%16) leaves lane l with tokens 8*(l/16) .. 8*(l/16)+7 of query
// row l%16: exactly the A operand of the PV MFMA (16 query rows x 32
// tokens).  The PV B operand (32 tokens x 16 head_dim columns) is then one
// 16-byte load per lane from the [D, B] V layout.  No LDS round trip.
// ---------------------------------------------------------------------------
// Cross-lane all-reduce over lanes l ^ 16 and l ^ 32 (the four lanes that
// hold one query row in the MFMA accumulator layout), on the VALU
// permlane-swap instructions of gfx950.  Each swap returns, in every lane,
// the lane's own value and its partner's value (in some order), so a
// symmetric combine of the pair is the butterfly step.
__device__ __forceinline__ float xl_max(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1]));
}

__device__ __forceinline__ float xl_sum(float v) {
  auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// One step (32 keys) of K and V fragments in MFMA operand layout.
template <int D>
struct KVFrag {
  bf16x8 ka[D / 32], kb[D / 32], v[D / 16];
};

// An appending decode's new token as the bf16 decode's fragments hold it:
// in the step whose first key is c it is token u = (L - 1) - c.  Its K row
// sits in the "a" (u % 8 < 4) or "b" fragments of the lanes with
// l % 16 == i (the row of MFMA "a"/"b" that is token u), dims 8 * (l / 16)
// + 32 * kk; its V entries in element u % 8 of the V fragments of the lanes
// with l / 16 == u / 8 (head_dim l % 16 + 16 * n).  Each lane holds its own
// share, loaded from the call's key / value rows.
template <int D>
struct NewToken {
  int c;              // first key of the step holding the token (-1: none)
  bool ka, kb;        // this lane's "a" / "b" K fragments hold the token
  int vd;             // dword of the V fragments holding element u % 8
  uint32_t vmask;     // its bits of the token in this lane (0: none)
  u32x4 k[D / 32];    // the lane's K dims of the token
  uint32_t v[D / 16]; // the lane's V entries, in place within dword vd
};

// The same token with its K row and V column (D bf16 each, head_dim order)
// in LDS instead, for kernels whose registers are full (the shared-prefix
// decode).
struct NewTokenL {
  int c;                // as NewToken
  bool ka, kb, v_sel;   // this lane's K fragments / a V element hold it
  int vd, sh;           // dword and bit offset of its V element
  const uint16_t* row;  // LDS: K row [D], then V column [D]
};

// Rescaling of the running output is skipped while a chunk's maximum stays
// within this many powers of two of the running maximum: the exponentials
// are then at most 2^8 and the final o / l is unchanged.
constexpr float kLazyRescaleLog2 = 8.f;
// The chunk kernel's form of it: a lane's 16 probabilities of one step may
// sum to at most 2^8 before the rows are rescaled (each is then <= 2^8).
constexpr float kLazyRescaleSum = 256.f;

// Keeps the (rarely taken) rescale branch a branch: without it the compiler
// turns the block into selects and multiplies the whole accumulator on
// every step.
__device__ __forceinline__ void rare_branch() { __asm__ volatile(""); }

// Query rows of one wave (R tiles of 16) and their online-softmax state.
template <int D, int R>
struct RowState {
  bf16x8 qf[R][D / 32];
  int klim[R];
  float m[R], l[R];
  f32x4 o[R][D / 16];
};

// One sequence / KV head as the kernels address it.
struct SeqView {
  int s, kvh, L, r0, qn, nblk, kcap;
};

__device__ __forceinline__ SeqView seq_view(const AttnArgs& a, int s, int kvh, int L, int r0, int qn) {
  SeqView v;
  v.s = s;
  v.kvh = kvh;
  v.L = L;
  v.r0 = r0;
  v.qn = qn;
  v.nblk = table_blocks(L, a.log2_block, a.max_blocks);
  v.kcap = v.nblk << a.log2_block;
  return v;
}

// Load the query rows row0 .. row0 + 16R - 1 of a sequence (row = j * G + g
// for chunk token j and group head g) into B-operand fragments, and reset
// the softmax state.  Rows past the sequence are zero and see no keys.
//
// With FP8DIMS the head_dim order inside the operands is the one of the fp8
// path: slice kk, lane group j4, element e holds dim (D/4)*j4 + 8*kk + e
// (any order gives the same dot product as long as K uses it too).
template <int D, int R, bool FP8DIMS = false>
__device__ __forceinline__ void load_rows(const AttnArgs& a, const SeqView& v, int row0,
                                          RowState<D, R>& st) {
  constexpr int KK = D / 32;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15;
  const int j4 = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int nrows = v.qn * G;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int row = row0 + 16 * t + i;
    st.klim[t] = 0;
    if (row < nrows) {
      const int j = row / G;
      const int g = row - j * G;
      st.klim[t] = min(v.L - v.qn + j + 1, v.kcap);
      const uint16_t* qp = q + ((int64_t)(v.r0 + j) * a.num_q_heads + v.kvh * G + g) * D +
                           (FP8DIMS ? (D / 4) * j4 : 8 * j4);
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) st.qf[t][kk] = load_bf16x8(qp + (FP8DIMS ? 8 : 32) * kk);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) st.qf[t][kk] = bf16x8{};
    }
    st.m[t] = neg_inf();
    st.l[t] = 0.f;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) st.o[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
}

// Keys held by the sequence's leading shared blocks (reference count above
// 1), rounded down to whole 32-key steps; looks at the first 64 blocks.
// Shared blocks always form a prefix of a table: forks copy a table prefix
// and copy-on-write replaces only a sequence's last block.  Used only to
// choose the cache policy, never for arithmetic.
__device__ __forceinline__ int leading_shared_keys(const AttnArgs& a, const SeqView& v) {
  if (a.block_refcounts == nullptr) return 0;
  const int lane = threadIdx.x & 63;
  int id = a.block_tables[(int64_t)v.s * a.max_blocks + min(lane, a.max_blocks - 1)];
  id = clampi(id, 0, a.num_blocks - 1);
  const bool shared = lane < v.nblk && a.block_refcounts[id] > 1;
  const uint64_t m = __builtin_amdgcn_ballot_w64(shared);
  const int n = (~m == 0) ? 64 : __builtin_ctzll(~m);
  return min(n << a.log2_block, v.kcap) & ~31;
}

// Stream keys [k_begin, k_end) of one sequence / KV head through the row
// tiles, 32 keys per step with the next step's K/V loads in flight.
//   kv_wave: one past the last key any row of the wave sees (keys from here
//            on may be unwritten slots: their V is zeroed);
//   kv_min:  keys below it are visible to every row (no mask needed).
//
// QK^T uses the 16x16x32 MFMA with A = K (16 token rows x 32 head_dim) and
// B = Q^T (32 head_dim x 16 query rows), two MFMAs per step ("a" and "b").
// MFMA row i of "a" is token 8*(i/4) + i%4 of the step and row i of "b" is
// that token + 4, so the accumulator layout (lane l holds rows 4*(l/16)+r,
// column l%16) leaves lane l with tokens 8*(l/16) .. 8*(l/16)+7 of query
// row l%16: exactly the A operand of the PV MFMA (16 query rows x 32
// tokens).  The PV B operand (32 tokens x 16 head_dim columns) is then one
// 16-byte load per lane from the [D, B] V layout.  No LDS round trip.
//
// Block ids come from a window of 64 logical blocks held one per lane; a
// step never straddles two windows (a window is 64*B keys, a multiple of
// 32), and the next window is loaded one window ahead.
//
// Cache policy: with STREAM every K/V load is non-temporal (private blocks
// are read once per call); without it loads go through the caches (shared
// prefix blocks, and query chunks whose K/V several waves re-read).
// PATCH: 0 none, 1 the new token from registers (nt), 2 from LDS (ntl).
template <int D, int R, bool STREAM, int NSETS = 2, int PATCH = 0>
__device__ __forceinline__ void attend(const AttnArgs& a, const SeqView& v, int kv_wave, int kv_min,
                                       int k_begin, int k_end, RowState<D, R>& st,
                                       const NewToken<D>* nt = nullptr,
                                       const NewTokenL* ntl = nullptr) {
  constexpr int KK = D / 32;
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15;
  const int j4 = lane >> 4;
  const int lg = a.log2_block;
  const int B = 1 << lg;
  const int64_t trow = (int64_t)v.s * a.max_blocks;
  auto window = [&](int b0) {
    const int x = a.block_tables[trow + min(b0 + lane, a.max_blocks - 1)];
    return clampi(x, 0, a.num_blocks - 1);
  };
  int blk0 = k_begin >> lg;
  int wid = window(blk0);
  int wid_next = window(blk0 + 64);
  auto block_id = [&](int pos) { return __shfl(wid, min(pos >> lg, v.nblk - 1) - blk0); };

  const int64_t blk_stride = (int64_t)a.num_kv_heads * B * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)v.kvh * B * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + (int64_t)v.kvh * D * B;
  const int tok_a = 8 * (i >> 2) + (i & 3);
  const float sl2 = a.scale_log2;

  auto load = [&](KVFrag<D>& f, int c) {
    if ((c >> lg) - blk0 >= 64) {  // wave-uniform: enter the next window
      blk0 += 64;
      wid = wid_next;
      wid_next = window(blk0 + 64);
    }
    const int pa_ = c + tok_a;
    const int pb_ = pa_ + 4;
    const int pv_ = c + 8 * j4;
    const uint16_t* ka = kbase + block_id(pa_) * blk_stride + (pa_ & (B - 1)) * D + 8 * j4;
    const uint16_t* kb = kbase + block_id(pb_) * blk_stride + (pb_ & (B - 1)) * D + 8 * j4;
    const uint16_t* vp = vbase + block_id(pv_) * blk_stride + (int64_t)i * B + (pv_ & (B - 1));
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      f.ka[kk] = STREAM ? load_bf16x8_nt(ka + 32 * kk) : load_bf16x8(ka + 32 * kk);
      f.kb[kk] = STREAM ? load_bf16x8_nt(kb + 32 * kk) : load_bf16x8(kb + 32 * kk);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n)
      f.v[n] = STREAM ? load_bf16x8_nt(vp + (int64_t)16 * n * B) : load_bf16x8(vp + (int64_t)16 * n * B);
  };

  auto compute = [&](KVFrag<D>& f, int c) {
    const int pv_ = c + 8 * j4;
    if constexpr (PATCH == 2) {
      // as below, from LDS
      if (c == ntl->c) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 x = *reinterpret_cast<const bf16x8*>(ntl->row + 8 * j4 + 32 * kk);
          f.ka[kk] = ntl->ka ? x : f.ka[kk];
          f.kb[kk] = ntl->kb ? x : f.kb[kk];
        }
        const uint32_t vmask = ntl->v_sel ? 0xFFFFu << ntl->sh : 0u;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint32_t val = (uint32_t)ntl->row[D + i + 16 * n] << ntl->sh;
          u32x4 x = __builtin_bit_cast(u32x4, f.v[n]);
#pragma unroll
          for (int d = 0; d < 4; ++d)
            x[d] = d == ntl->vd ? ((x[d] & ~vmask) | (val & vmask)) : x[d];
          f.v[n] = __builtin_bit_cast(bf16x8, x);
        }
      }
    }
    if constexpr (PATCH == 1) {
      // the step holding an appending call's new token: its K/V come from
      // the call's key / value rows, not from the slot (written later)
      if (c == nt->c) {
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          const bf16x8 x = __builtin_bit_cast(bf16x8, nt->k[kk]);
          f.ka[kk] = nt->ka ? x : f.ka[kk];
          f.kb[kk] = nt->kb ? x : f.kb[kk];
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          u32x4 x = __builtin_bit_cast(u32x4, f.v[n]);
#pragma unroll
          for (int d = 0; d < 4; ++d)
            x[d] = d == nt->vd ? ((x[d] & ~nt->vmask) | nt->v[n]) : x[d];
          f.v[n] = __builtin_bit_cast(bf16x8, x);
        }
      }
    }
    if (c + 32 > kv_wave) {
      // Keys past the last visible one may be unwritten slots: zero their V
      // so that 0-weight * garbage cannot produce NaN.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (pv_ + e >= kv_wave) {
#pragma unroll
          for (int n = 0; n < NT; ++n) f.v[n][e] = static_cast<__bf16>(0.f);
        }
      }
    }
    const bool need_mask = c + 32 > kv_min;
#pragma unroll
    for (int t = 0; t < R; ++t) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.ka[kk], st.qf[t][kk], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.kb[kk], st.qf[t][kk], sb, 0, 0, 0);
      }
      float sv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = sa[r] * sl2;
        sv[4 + r] = sb[r] * sl2;
      }
      if (need_mask) {
#pragma unroll
        for (int e = 0; e < 8; ++e) sv[e] = (pv_ + e < st.klim[t]) ? sv[e] : neg_inf();
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[e]);
      mx = xl_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx > st.m[t] + kLazyRescaleLog2) != 0) {
        rare_branch();
        const float mnew = fmaxf(st.m[t], mx);
        const float alpha = fast_exp2(st.m[t] - ((mnew == neg_inf()) ? 0.f : mnew));
        st.l[t] *= alpha;
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * j4 + r);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) st.o[t][n][r] *= ar[r];
        st.m[t] = mnew;
      }
      const float muse = (st.m[t] == neg_inf()) ? 0.f : st.m[t];
      float ps = 0.f;
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float p = fast_exp2(sv[e] - muse);
        ps += p;
        pf[e] = static_cast<__bf16>(p);
      }
      st.l[t] += xl_sum(ps);
#pragma unroll
      for (int n = 0; n < NT; ++n)
        st.o[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, f.v[n], st.o[t][n], 0, 0, 0);
    }
  };

  // A ring of NSETS fragment sets: the loads of step i + NSETS - 1 are
  // issued before step i is computed, so NSETS - 1 steps are in flight while
  // the wave computes.  Steps past the end are not loaded (a wave-uniform
  // test; the waits are the compiler's, on the registers each step reads).
  const int n = (k_end - k_begin + 31) >> 5;
  KVFrag<D> f[NSETS];
#pragma unroll
  for (int p = 0; p < NSETS - 1; ++p)
    if (p < n) load(f[p], k_begin + 32 * p);
  for (int i0 = 0; i0 < n; i0 += NSETS) {
#pragma unroll
    for (int j = 0; j < NSETS; ++j) {
      const int i = i0 + j;
      if (i >= n) break;
      if (i + NSETS - 1 < n) load(f[(j + NSETS - 1) % NSETS], k_begin + 32 * (i + NSETS - 1));
      compute(f[j], k_begin + 32 * i);
    }
  }
}

// ---------------------------------------------------------------------------
// Decode over an fp8 (e4m3) cache: 64 keys per step.
//
// Every e4m3 value is exactly a bf16 value, so K and V codes are widened to
// bf16 in registers and the bf16 MFMA does the products; the per-(block,
// KV head) scales are applied to the scores (K) and to the probabilities
// before the PV product (V), never to the 448-range codes themselves.
//
// QK^T: four MFMAs per head_dim slice ("a".."d", x = 0..3); MFMA x row i is
// token 16*(i/4) + 4x + i%4 of the step, so lane l ends up holding the
// scores of tokens 16*(l/16) + 0..15 (register 4x + r = token 4x + r of the
// lane's group of 16) for query row l%16.  A lane's K operand is one token
// row's D/4 consecutive bytes, dims (D/4)*(l/16) + 8*kk + e for slice kk
// (the query uses the same order).  PV: the lane's 16 probabilities are the
// A operand of two MFMAs (tokens 16*(l/16) + 0..7 and + 8..15); the B
// operand is one 16-byte load of 16 consecutive tokens of one head_dim
// column from the [D, B] V layout (B >= 16, so the group of 16 tokens sits
// in one block and so has one K and one V scale).
// ---------------------------------------------------------------------------
template <int D>
struct KVFrag8 {
  u32x4 k[4][D / 64];  // x = 0..3: the lane's D/4 bytes of one token row
  u32x4 v[D / 16];     // 16 tokens of head_dim column 16*n + l%16
  float ks, vs;        // scales of the block of the lane's 16 tokens
};

// An appending e4m3 decode's new token as attend_fp8's fragments hold it:
// token u of its 64-key step sits in K fragment x = (u / 4) % 4 of the
// lanes with l % 16 == 4 * (u / 16) + u % 4 (bytes (D/4) * (l/16) + ...),
// and in byte u % 4 of dword (u % 16) / 4 of the V fragments of the lanes
// with l / 16 == u / 16.  Its codes, those the cache write gives it, wait
// in LDS (K row, then V column, D bytes each, head_dim order): held in
// registers across the step loop they would not fit beside the ring.
struct NewToken8 {
  int c;                 // first key of the step holding the token (-1: none)
  int kx;                // K fragment holding it
  int vd, sh;            // dword and bit offset of its V byte
  bool k_sel, v_sel;     // this lane holds its K bytes / a V byte of it
  const uint8_t* codes;  // LDS: K codes [D], then V codes [D]
};

// Eight e4m3 codes (two dwords, lowest byte first) as bf16, exactly: gfx950
// converts a pair of fp8 codes straight to a pair of bf16 (with a unit
// scale the result is the code's value; every e4m3 value is a bf16 value).
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// The policy is a template parameter: as a run-time argument the two loads
// of the same address get merged before inlining, which drops the
// non-temporal hint.
template <bool STREAM>
__device__ __forceinline__ u32x4 load_u32x4(const uint8_t* p) {
  const u32x4* q = reinterpret_cast<const u32x4*>(p);
  if constexpr (STREAM) return __builtin_nontemporal_load(q);
  else return *q;
}

// Fragment sets of the balanced-decode rings (steps in flight + 1); with
// more than two sets the kernel runs one wave per SIMD (up to 512 registers).
constexpr int kDecodeSets = 3;
constexpr int kFp8Sets = 3;

template <int D, bool STREAM, int R = 1, int NSETS = kFp8Sets, bool PATCH = false>
__device__ __forceinline__ void attend_fp8(const AttnArgs& a, const SeqView& v, int kv_wave,
                                           int kv_min, int k_begin, int k_end,
                                           RowState<D, R>& st,
                                           const NewToken8* nt = nullptr) {
  constexpr int KK = D / 32;
  constexpr int KP = D / 64;
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15;
  const int j4 = lane >> 4;
  const int lg = a.log2_block;
  const int B = 1 << lg;
  const int Hkv = a.num_kv_heads;
  const int64_t trow = (int64_t)v.s * a.max_blocks;
  auto window = [&](int b0) {
    const int x = a.block_tables[trow + min(b0 + lane, a.max_blocks - 1)];
    return clampi(x, 0, a.num_blocks - 1);
  };
  int blk0 = k_begin >> lg;
  int wid = window(blk0);
  int wid_next = window(blk0 + 64);
  auto block_id = [&](int pos) { return __shfl(wid, min(pos >> lg, v.nblk - 1) - blk0); };

  const int64_t blk_stride = (int64_t)Hkv * B * D;  // bytes
  const uint8_t* kbase = static_cast<const uint8_t*>(a.k_cache) + (int64_t)v.kvh * B * D + (D / 4) * j4;
  const uint8_t* vbase = static_cast<const uint8_t*>(a.v_cache) + (int64_t)v.kvh * D * B + (int64_t)i * B;
  const int tok_k = 16 * (i >> 2) + (i & 3);
  const float sl2 = a.scale_log2;

  auto load = [&](KVFrag8<D>& f, int c) {
    if ((c >> lg) - blk0 >= 64) {  // wave-uniform: enter the next window
      blk0 += 64;
      wid = wid_next;
      wid_next = window(blk0 + 64);
    }
    // The scales go out first: loads complete in issue order, so the
    // step's scores wait for its K loads only, not for its V loads too.
    const int pv = c + 16 * j4;
    const int bv = block_id(pv);
    f.ks = a.k_scales[(int64_t)bv * Hkv + v.kvh];
    f.vs = a.v_scales[(int64_t)bv * Hkv + v.kvh];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int pos = c + tok_k + 4 * x;
      const uint8_t* kp = kbase + block_id(pos) * blk_stride + (int64_t)(pos & (B - 1)) * D;
#pragma unroll
      for (int p = 0; p < KP; ++p) f.k[x][p] = load_u32x4<STREAM>(kp + 16 * p);
    }
    const uint8_t* vp = vbase + bv * blk_stride + (pv & (B - 1));
#pragma unroll
    for (int n = 0; n < NT; ++n) f.v[n] = load_u32x4<STREAM>(vp + (int64_t)16 * n * B);
  };

  // mask: the step holds keys at or past kv_min (scores masked to -inf)
  // or kv_wave (V codes zeroed: they may be unwritten NaN slots).  Only the
  // last step of a piece can; the tests sit behind a wave-uniform branch.
  auto compute = [&](KVFrag8<D>& f, int c, bool mask) {
    const int pv = c + 16 * j4;
    if constexpr (PATCH) {
      // the step holding an appending call's new token: its codes come from
      // LDS, not from the slot (written after the share)
      if (c == nt->c) {
        u32x4 kc[KP];
#pragma unroll
        for (int p = 0; p < KP; ++p)
          kc[p] = *reinterpret_cast<const u32x4*>(nt->codes + (D / 4) * j4 + 16 * p);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int p = 0; p < KP; ++p) f.k[x][p] = nt->k_sel && x == nt->kx ? kc[p] : f.k[x][p];
        const uint32_t vmask = nt->v_sel ? 0xFFu << nt->sh : 0u;
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const uint32_t code = (uint32_t)nt->codes[D + i + 16 * n] << nt->sh;
#pragma unroll
          for (int d = 0; d < 4; ++d)
            f.v[n][d] = d == nt->vd ? ((f.v[n][d] & ~vmask) | (code & vmask)) : f.v[n][d];
        }
      }
    }
    if (mask) {
      rare_branch();
      // zero the V bytes of keys >= kv_wave (16 keys per lane, 4 per dword)
      const int nv = clampi(kv_wave - pv, 0, 16);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int n_in = clampi(nv - 4 * w, 0, 4);
        const uint32_t keep = n_in >= 4 ? 0xFFFFFFFFu : ((1u << (8 * n_in)) - 1u);
#pragma unroll
        for (int n = 0; n < NT; ++n) f.v[n][w] &= keep;
      }
    }
    // R row tiles share the widened K and V of the step.
    f32x4 s4[R][4];
#pragma unroll
    for (int t = 0; t < R; ++t)
#pragma unroll
      for (int x = 0; x < 4; ++x) s4[t][x] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
#pragma unroll
      for (int x = 0; x < 4; ++x) {
        const u32x4 w = f.k[x][kk >> 1];
        const bf16x8 kf = e4m3x8_to_bf16(w[2 * (kk & 1)], w[2 * (kk & 1) + 1]);
#pragma unroll
        for (int t = 0; t < R; ++t)
          s4[t][x] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, st.qf[t][kk], s4[t][x], 0, 0, 0);
      }
    }
    const float kscale = f.ks * sl2;
    bf16x8 pf[R][2];
#pragma unroll
    for (int t = 0; t < R; ++t) {
      float sv[16];
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int r = 0; r < 4; ++r) sv[4 * x + r] = s4[t][x][r] * kscale;
      if (mask) {
        rare_branch();
        const int lim = st.klim[t] - pv;
#pragma unroll
        for (int e = 0; e < 16; ++e) sv[e] = (e < lim) ? sv[e] : neg_inf();
      }
      float mx = sv[0];
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, sv[e]);
      mx = xl_max(mx);
      if (__builtin_amdgcn_ballot_w64(mx > st.m[t] + kLazyRescaleLog2) != 0) {
        rare_branch();
        const float mnew = fmaxf(st.m[t], mx);
        const float alpha = fast_exp2(st.m[t] - ((mnew == neg_inf()) ? 0.f : mnew));
        st.l[t] *= alpha;
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * j4 + r);
#pragma unroll
        for (int n = 0; n < NT; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) st.o[t][n][r] *= ar[r];
        st.m[t] = mnew;
      }
      const float muse = (st.m[t] == neg_inf()) ? 0.f : st.m[t];
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = fast_exp2(sv[e] - muse);
        ps += p;
        pf[t][e >> 3][e & 7] = static_cast<__bf16>(p * f.vs);
      }
      st.l[t] += xl_sum(ps);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) {
#pragma unroll
      for (int h2 = 0; h2 < 2; ++h2) {
        const bf16x8 vf = e4m3x8_to_bf16(f.v[n][2 * h2], f.v[n][2 * h2 + 1]);
#pragma unroll
        for (int t = 0; t < R; ++t)
          st.o[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[t][h2], vf, st.o[t][n], 0, 0, 0);
      }
    }
  };

  // Steps below k_safe need no mask; at most one step (the last) does.
  // A ring of NSETS fragment sets: the loads of step i + NSETS - 1 are
  // issued before step i is computed, so NSETS - 1 steps are in flight
  // while the wave computes; steps past the end are not loaded.
  const int k_safe = max(k_begin, min(k_end, (min(kv_min, kv_wave) - k_begin) / 64 * 64 + k_begin));
  const int n = (k_end - k_begin + 63) >> 6;
  KVFrag8<D> f[NSETS];
#pragma unroll
  for (int p = 0; p < NSETS - 1; ++p)
    if (p < n) load(f[p], k_begin + 64 * p);
  for (int i0 = 0; i0 < n; i0 += NSETS) {
#pragma unroll
    for (int j = 0; j < NSETS; ++j) {
      const int i = i0 + j;
      if (i >= n) break;
      if (i + NSETS - 1 < n) load(f[(j + NSETS - 1) % NSETS], k_begin + 64 * (i + NSETS - 1));
      const int c = k_begin + 64 * i;
      compute(f[j], c, c + 64 > k_safe);
    }
  }
}

// Where a wave's partial (o, m, l) rows go: ``slots`` partials per row,
// row index = row_base + head when row_base >= 0, else the output row.
struct PartialDst {
  float* o;
  float* ml;
  int slots;
  int64_t row_base;
};

// Write the wave's rows: normalised output when ``whole`` (this piece saw
// every key of the row), else the piece's (o, m, l) into partial slot
// ``slot`` of the row.  Lane l holds rows 4*(l/16)+r, columns 16*n + l%16.
//
// With ``split_tokens`` > 0 (fixed splits) the decision is made per row: a
// row whose keys fit in one split is final, rows that see no key of this
// split (k_begin) are skipped.
template <int D, int R>
__device__ __forceinline__ void write_rows(const AttnArgs& a, const SeqView& v, int row0,
                                           const RowState<D, R>& st, bool whole, int slot,
                                           const PartialDst& pd, int split_tokens = 0,
                                           int k_begin = 0) {
  constexpr int NT = D / 16;
  const int lane = threadIdx.x & 63;
  const int i = lane & 15;
  const int j4 = lane >> 4;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int nrows = v.qn * G;
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int t = 0; t < R; ++t) {
    float lr[4], mr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lr[r] = __shfl(st.l[t], 4 * j4 + r);
      mr[r] = __shfl(st.m[t], 4 * j4 + r);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 16 * t + 4 * j4 + r;
      if (row >= nrows) continue;
      const int j = row / G;
      const int g = row - j * G;
      const int64_t orow = (int64_t)(v.r0 + j) * a.num_q_heads + v.kvh * G + g;
      bool final_row = whole;
      if (split_tokens > 0) {
        const int kl = min(v.L - v.qn + j + 1, v.kcap);
        if (kl <= k_begin) continue;
        final_row = min((kl + split_tokens - 1) / split_tokens, pd.slots) == 1;
      }
      if (final_row) {
        const float inv = 1.f / lr[r];
#pragma unroll
        for (int n = 0; n < NT; ++n) out[orow * D + 16 * n + i] = f32_to_bf16_bits(st.o[t][n][r] * inv);
      } else {
        if (slot >= pd.slots) continue;  // out-of-contract lengths: stay in bounds
        const int64_t prow = pd.row_base >= 0 ? pd.row_base + v.kvh * G + g : orow;
        const int64_t pidx = prow * pd.slots + slot;
        float* po = pd.o + pidx * D;
#pragma unroll
        for (int n = 0; n < NT; ++n) po[16 * n + i] = st.o[t][n][r];
        if (i == 0) {
          pd.ml[2 * pidx] = mr[r];
          pd.ml[2 * pidx + 1] = lr[r];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Fixed-split bf16 decode: one wave per (sequence x KV head, 16-row tile of
// the G query heads, split of split_tokens keys).  pa_decode runs it when a
// split size is given (kv_split_tokens > 0).
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attn_mfma_kernel(AttnArgs a) {
  constexpr int R = 1;
  // Grid: x = (sequence, KV head) fastest, z = split.  Workgroups are dealt
  // to the 8 XCDs round-robin by linear id, so this gives every XCD the same
  // mix of sequences and splits (with the split fastest, XCD k would get
  // split k of every sequence and the long-context tail would pile up on a
  // few XCDs).
  const int s = blockIdx.x / a.num_kv_heads;
  const int kvh = blockIdx.x - s * a.num_kv_heads;
  const int tg = blockIdx.y;
  const int split = blockIdx.z;
  const int L = a.seq_lens[s];
  int r0, qn;
  seq_rows(a.query_start_loc, s, a.num_tokens, r0, qn);
  const int G = a.num_q_heads / a.num_kv_heads;
  const int nrows = qn * G;
  const int row0 = tg * 16 * R;
  if (row0 >= nrows) return;
  const SeqView v = seq_view(a, s, kvh, L, r0, qn);
  // Rows are ordered by query position: the first row has the smallest key
  // limit and the last row the largest.
  const int row_last = min(row0 + 16 * R, nrows) - 1;
  const int kv_wave = min(L - qn + row_last / G + 1, v.kcap);
  const int kv_min = min(L - qn + row0 / G + 1, v.kcap);
  const int k_begin = split * a.split_tokens;
  if (k_begin >= kv_wave) return;
  const int k_end = min(k_begin + a.split_tokens, kv_wave);
  RowState<D, R> st;
  load_rows<D, R>(a, v, row0, st);
  // A decode wave is the only reader of its K/V: stream it, except the
  // leading shared blocks.
  const int k_sh = k_begin < (64 << a.log2_block) ? leading_shared_keys(a, v) : 0;
  if (k_sh > k_begin) attend<D, R, false>(a, v, kv_wave, kv_min, k_begin, min(k_sh, k_end), st);
  if (k_end > max(k_begin, k_sh))
    attend<D, R, true>(a, v, kv_wave, kv_min, max(k_begin, k_sh), k_end, st);
  // A row whose keys span more than one split leaves a partial in slot
  // ``split`` for the merge pass; the others are final here.
  write_rows<D, R>(a, v, row0, st, false, split, PartialDst{a.part_o, a.part_ml, a.max_splits, -1},
                   a.split_tokens, k_begin);
}

// ---------------------------------------------------------------------------
// Balanced ("stream-K") bf16 decode.  The work is the list of 32-key steps
// of every (sequence, KV head), sequence-major; a fixed number of resident
// waves each take one contiguous, equal share of that list (at least
// kMinStepsPerWave steps), so all waves stream the same number of bytes and
// finish together.  A share may start or end inside a sequence; such pieces
// leave (o, m, l) partials that the merge pass combines.  Every wave
// rebuilds the per-sequence step prefix sums in LDS from seq_lens; wave 0
// also stores them (with the step total and wave count) in the workspace
// header for the merge pass.
// ---------------------------------------------------------------------------
struct StreamKHeader {
  int64_t total_steps;
  int64_t waves;
  // followed by int32 prefix[num_seqs + 1]
};

__device__ __forceinline__ int64_t wave_of_step(int64_t g, int64_t waves, int64_t total) {
  return ((g + 1) * waves - 1) / total;
}

// FP8: the cache is e4m3 with per-(block, KV head) scales and a step is 64
// keys (the bf16 cache steps 32 keys at a time).
// Decode steps (per KV head) of every sequence's single-token rows in
// P[s + 1] and the lengths in Ls[s], by nthreads threads; the caller
// synchronises before the scan.
//
// Shared-prefix decode (a.prefix_keys > 0): entries S .. S + ng - 1 are the
// prefix items, one per group of a.prefix_group sequences, and a sequence's
// own item covers its keys after the prefix.
template <bool FP8>
__device__ __forceinline__ void decode_prefix_fill(const AttnArgs& a, int* P, int* Ls, int tid,
                                                   int nthreads) {
  constexpr int STEP = FP8 ? 64 : 32;
  constexpr int LSTEP = FP8 ? 6 : 5;
  const int lg = a.log2_block;
  const int S = a.num_seqs;
  const int pk = a.prefix_keys;  // a multiple of STEP (checked by the host)
  const int ng = prefix_items(S, a.prefix_group);
  for (int s = tid; s < S + ng; s += nthreads) {
    if (s >= S) {  // a prefix item
      P[s + 1] = (pk >> LSTEP) + kPieceCostSteps;
      Ls[s] = pk;
      continue;
    }
    const int L = a.seq_lens[s];
    int r0, qn;
    seq_rows(a.query_start_loc, s, a.num_tokens, r0, qn);
    const int kl = min(L, table_blocks(L, lg, a.max_blocks) << lg);
    // Only single-token rows are decode work (query chunks have their own kernel).
    // An item's cost is its steps plus kPieceCostSteps for starting a piece.
    P[s + 1] = (qn == 1 && kl > pk) ? ((kl - pk + STEP - 1) >> LSTEP) + kPieceCostSteps : 0;
    Ls[s] = L;
  }
}

// In-place prefix sums of P[1..S] (P[0] = 0) by the 64 lanes of one wave.
__device__ __forceinline__ void decode_prefix_scan(int* P, int S, int lane) {
  const int k = (S + 63) >> 6;
  const int lo = min(lane * k, S);
  const int hi = min(lo + k, S);
  int run = 0;
  for (int s = lo; s < hi; ++s) {
    run += P[s + 1];
    P[s + 1] = run;
  }
  int incl = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d);
    if (lane >= d) incl += y;
  }
  const int off = incl - run;
  for (int s = lo; s < hi; ++s) P[s + 1] += off;
  if (lane == 0) P[0] = 0;
}

// Wave w's share (of weff) of the N decode steps, given the step prefix sums
// P and lengths Ls; NSETS fragment sets in the bf16 ring.
//
// PREFIX: the shared-prefix work list (prefix items after the sequences'
// own items); an instantiation without it holds no prefix path, so the
// plain decode keeps its register budget.
// APPEND: the appending decode.  Only an item's last step reads the slot of
// the sequence's new token; the wave whose piece holds that step takes the
// token's K/V from the call's rows (NewToken / NewToken8 patches of the
// step's fragments) and writes the slot after its whole share, so no load
// waits for a store.  A separate instantiation, so that the plain decode's
// K/V stay read-only to the compiler.
template <int D, bool FP8, int NSETS, bool PREFIX = false, bool APPEND = false>
__device__ __forceinline__ void decode_share(const AttnArgs& a, const int* P, const int* Ls,
                                             int64_t N, int64_t weff, int w,
                                             uint8_t* tok_lds = nullptr) {
  constexpr int STEP = FP8 ? 64 : 32;
  const int S = a.num_seqs + prefix_items(a.num_seqs, a.prefix_group);  // work-list entries
  const int Hkv = a.num_kv_heads;
  int64_t g = (int64_t)w * N / weff;
  const int64_t g_end = (int64_t)(w + 1) * N / weff;
  // Sequence holding step g: the largest s with Hkv * P[s] <= g.
  int s;
  {
    int lo = 0, hi = S - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if ((int64_t)Hkv * P[mid] <= g) lo = mid;
      else hi = mid - 1;
    }
    s = lo;
  }
  const int s_first = s;
  while (g < g_end) {
    while ((int64_t)Hkv * P[s + 1] <= g) ++s;
    const int cost = P[s + 1] - P[s];  // steps + kPieceCostSteps
    const int nch = cost - kPieceCostSteps;
    const int64_t base = (int64_t)Hkv * P[s];
    const int kvh = (int)((g - base) / cost);
    const int64_t g_item = base + (int64_t)kvh * cost + kPieceCostSteps;  // the item's step 0
    const int c0 = (int)max((int64_t)0, g - g_item);
    const int c1 = (int)min((int64_t)nch, g_end - g_item);
    g = g_item + nch;  // next item (or past g_end)
    if (c1 <= c0) continue;  // the share holds only the start-up cost of this item
    const int64_t wf = wave_of_step(g_item, weff, N);
    const int64_t wl = wave_of_step(g_item + nch - 1, weff, N);
    const int piece = (int)(w - wf);
    if (PREFIX && s >= a.num_seqs) {
      // A prefix item: the prefix blocks through table row 0, for the query
      // rows of a group of sequences (PT 16-row tiles that share every K/V
      // load).  Chunk token j of this view is sequence r0 + j,
      // every row sees all prefix keys, and the loads go through the caches.
      const int k = s - a.num_seqs;
      const int qg = min(a.prefix_group, a.num_seqs - a.prefix_group * k);
      SeqView v;
      v.s = 0;
      v.kvh = kvh;
      v.L = a.prefix_keys + qg;
      v.r0 = a.prefix_group * k;
      v.qn = qg;
      v.nblk = a.prefix_keys >> a.log2_block;
      v.kcap = a.prefix_keys;
      const int kl = a.prefix_keys;
      constexpr int PT = prefix_tiles(FP8);
      RowState<D, PT> st;
      load_rows<D, PT, FP8>(a, v, 0, st);
      const int k_begin = c0 * STEP;
      const int k_end = min(c1 * STEP, kl);
      if constexpr (FP8) attend_fp8<D, false, PT>(a, v, kl, kl, k_begin, k_end, st);
      else attend<D, PT, false, NSETS>(a, v, kl, kl, k_begin, k_end, st);
      // prefix pieces sit in the last prefix_slots slots of each row
      write_rows<D, PT>(a, v, 0, st, false, a.sk_slots - a.prefix_slots + piece,
                        PartialDst{a.sk_part_o, a.sk_part_ml, a.sk_slots, -1});
      continue;
    }
    int r0, qn;
    seq_rows(a.query_start_loc, s, a.num_tokens, r0, qn);
    const SeqView v = seq_view(a, s, kvh, Ls[s], r0, 1);
    const int kl = min(v.L, v.kcap);
    // Appending: the step that holds the new token takes its K/V from the
    // call's rows (bf16: in registers, or in LDS in the shared-prefix
    // kernel; e4m3: its codes in LDS); the cache write comes after the share
    // (below).
    NewToken<D> nt;
    NewToken8 nt8;
    nt.c = -1;
    nt8.c = -1;
    const int new_pos = Ls[s] - 1;
    const int new_id = APPEND && c1 == nch && new_pos >= 0 && new_pos < kl
                           ? a.block_tables[(int64_t)s * a.max_blocks + (new_pos >> a.log2_block)]
                           : -1;
    if constexpr (APPEND && FP8) {
      if (new_id >= 0 && new_id < a.num_blocks) {  // exactly when the write happens
        const int lane = threadIdx.x & 63;
        const int u = new_pos & 63;                 // the token within its 64-key step
        nt8.c = new_pos - u;
        nt8.kx = (u >> 2) & 3;
        nt8.k_sel = (lane & 15) == 4 * (u >> 4) + (u & 3);
        nt8.v_sel = (lane >> 4) == (u >> 4);
        nt8.vd = (u & 15) >> 2;
        nt8.sh = 8 * (u & 3);
        nt8.codes = tok_lds;
        // codes as the cache write makes them (x / scale rounded once,
        // clamped to +-448, e4m3 with round to nearest even); lane l makes
        // those of dims D/64 * l .. of the K row and the V column
        constexpr int PER = D / 64;
        const int64_t hb = (int64_t)new_id * Hkv + kvh;
        const float ks = a.k_scales[hb], vs = a.v_scales[hb];
        const int64_t src = ((int64_t)r0 * Hkv + kvh) * D + PER * lane;
        const uint16_t* nk = static_cast<const uint16_t*>(a.new_k) + src;
        const uint16_t* nv = static_cast<const uint16_t*>(a.new_v) + src;
        float xk[2] = {0.f, 0.f}, xv[2] = {0.f, 0.f};
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          xk[e] = sat_e4m3(__fdiv_rn(__uint_as_float((uint32_t)nk[e] << 16), ks));
          xv[e] = sat_e4m3(__fdiv_rn(__uint_as_float((uint32_t)nv[e] << 16), vs));
        }
        const uint32_t ck = __builtin_amdgcn_cvt_pk_fp8_f32(xk[0], xk[1], 0, false);
        const uint32_t cv = __builtin_amdgcn_cvt_pk_fp8_f32(xv[0], xv[1], 0, false);
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          tok_lds[PER * lane + e] = (uint8_t)(ck >> (8 * e));
          tok_lds[D + PER * lane + e] = (uint8_t)(cv >> (8 * e));
        }
      }
    }
    NewTokenL ntl;
    ntl.c = -1;
    if constexpr (APPEND && !FP8 && PREFIX) {
      if (new_id >= 0 && new_id < a.num_blocks) {  // exactly when the write happens
        const int lane = threadIdx.x & 63;
        const int u = new_pos & 31;
        const bool b = (u & 4) != 0;
        const int ua = b ? u - 4 : u;
        const bool krow = (lane & 15) == 4 * (ua >> 3) + (ua & 3);
        ntl.c = new_pos - u;
        ntl.ka = krow && !b;
        ntl.kb = krow && b;
        ntl.v_sel = (lane >> 4) == (u >> 3);
        ntl.vd = (u & 7) >> 1;
        ntl.sh = 16 * (u & 1);
        uint16_t* row = reinterpret_cast<uint16_t*>(tok_lds);
        ntl.row = row;
        constexpr int PER = D / 64;
        const int64_t src = ((int64_t)r0 * Hkv + kvh) * D + PER * lane;
        const uint16_t* nk = static_cast<const uint16_t*>(a.new_k) + src;
        const uint16_t* nv = static_cast<const uint16_t*>(a.new_v) + src;
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          row[PER * lane + e] = nk[e];
          row[D + PER * lane + e] = nv[e];
        }
      }
    }
    if constexpr (APPEND && !FP8 && !PREFIX) {
      const int pos = new_pos;
      const int id = new_id;
      if (id >= 0 && id < a.num_blocks) {  // exactly when the write happens
        const int lane = threadIdx.x & 63;
        const int u = pos & 31;                  // the token within its step
        const bool b = (u & 4) != 0;             // "b" rows are the "a" tokens + 4
        const int ua = b ? u - 4 : u;
        const bool krow = (lane & 15) == 4 * (ua >> 3) + (ua & 3);
        const bool vcol = (lane >> 4) == (u >> 3);
        nt.c = pos - u;
        nt.ka = krow && !b;
        nt.kb = krow && b;
        nt.vd = (u & 7) >> 1;
        const int sh = 16 * (u & 1);
        nt.vmask = vcol ? 0xFFFFu << sh : 0u;
        const int64_t row = ((int64_t)r0 * Hkv + kvh) * D;
        const uint16_t* nk = static_cast<const uint16_t*>(a.new_k) + row;
        const uint16_t* nv = static_cast<const uint16_t*>(a.new_v) + row;
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk)
          nt.k[kk] = krow ? __builtin_bit_cast(u32x4, load_bf16x8(nk + 8 * (lane >> 4) + 32 * kk))
                          : u32x4{0, 0, 0, 0};
#pragma unroll
        for (int n = 0; n < D / 16; ++n)
          nt.v[n] = vcol ? (uint32_t)nv[(lane & 15) + 16 * n] << sh : 0u;
      }
    }
    constexpr int PATCH = APPEND && !FP8 ? (PREFIX ? 2 : 1) : 0;
    RowState<D, 1> st;
    load_rows<D, 1, FP8>(a, v, 0, st);
    const int kb0 = a.prefix_keys;  // step 0 of an own item starts after the shared prefix
    const int k_begin = kb0 + c0 * STEP;
    const int k_end = min(kb0 + c1 * STEP, kl);
    // Keys read through the caches: with a shared prefix none (what the
    // table shares past the prefix is less than a step), else the leading
    // shared blocks.
    const int k_sh = a.prefix_keys > 0 ? 0
                     : k_begin < (64 << a.log2_block) ? leading_shared_keys(a, v) & ~(STEP - 1)
                                                      : 0;
    if constexpr (FP8) {
      constexpr bool PATCH8 = APPEND;
      if (k_sh > k_begin)
        attend_fp8<D, false, 1, NSETS, PATCH8>(a, v, kl, kl, k_begin, min(k_sh, k_end), st, &nt8);
      if (k_end > max(k_begin, k_sh))
        attend_fp8<D, true, 1, NSETS, PATCH8>(a, v, kl, kl, max(k_begin, k_sh), k_end, st, &nt8);
    } else {
      if (k_sh > k_begin)
        attend<D, 1, false, NSETS, PATCH>(a, v, kl, kl, k_begin, min(k_sh, k_end), st, &nt, &ntl);
      if (k_end > max(k_begin, k_sh))
        attend<D, 1, true, NSETS, PATCH>(a, v, kl, kl, max(k_begin, k_sh), k_end, st, &nt, &ntl);
    }
    if (a.prefix_keys > 0) {
      // every row is merged with its prefix part: own pieces in slots
      // [0, own); a piece past that range (out-of-contract lengths) is dropped
      const int own = a.sk_slots - a.prefix_slots;
      write_rows<D, 1>(a, v, 0, st, false, piece < own ? piece : a.sk_slots,
                       PartialDst{a.sk_part_o, a.sk_part_ml, a.sk_slots, -1});
    } else {
      write_rows<D, 1>(a, v, 0, st, wf == wl, piece,
                       PartialDst{a.sk_part_o, a.sk_part_ml, a.sk_slots, (int64_t)s * a.num_q_heads});
    }
  }
  if constexpr (APPEND) {
    // The cache writes of the new tokens whose last step this share held,
    // once its attention is done: stores issued while every wave streams
    // K/V would hold up the wave's next loads until they complete.  The
    // same walk over the share's items as above.
    int64_t g2 = (int64_t)w * N / weff;
    int s2 = s_first;
    while (g2 < g_end) {
      while ((int64_t)Hkv * P[s2 + 1] <= g2) ++s2;
      const int cost = P[s2 + 1] - P[s2];
      const int nch = cost - kPieceCostSteps;
      const int64_t base = (int64_t)Hkv * P[s2];
      const int kvh = (int)((g2 - base) / cost);
      const int64_t g_item = base + (int64_t)kvh * cost + kPieceCostSteps;
      const int c0 = (int)max((int64_t)0, g2 - g_item);
      const int c1 = (int)min((int64_t)nch, g_end - g_item);
      g2 = g_item + nch;
      if (c1 <= c0 || c1 != nch || (PREFIX && s2 >= a.num_seqs)) continue;  // prefix items hold none
      int r0, qn;
      seq_rows(a.query_start_loc, s2, a.num_tokens, r0, qn);
      append_token<2, D, FP8>(a, s2, kvh, Ls[s2], r0);
    }
  }
}


template <int D, bool FP8, bool PREFIX = false, bool APPEND = false>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(
    (FP8 ? kFp8Sets : kDecodeSets) > 2 ? 1 : 2, (FP8 ? kFp8Sets : kDecodeSets) > 2 ? 1 : 2)))
void decode_streamk_kernel(AttnArgs a, int waves, StreamKHeader* hdr) {
  extern __shared__ int smem[];
  const int S = a.num_seqs + prefix_items(a.num_seqs, a.prefix_group);  // work-list entries
  int* P = smem;           // [S + 1] steps before entry s (per KV head)
  int* Ls = smem + S + 1;  // [S]     sequence lengths
  const int lane = threadIdx.x;
  decode_prefix_fill<FP8>(a, P, Ls, lane, 64);
  __syncthreads();
  decode_prefix_scan(P, S, lane);
  __syncthreads();
  const int64_t N = (int64_t)a.num_kv_heads * P[S];
  const int64_t weff = N == 0 ? 0 : min((int64_t)waves, max((int64_t)1, N / kMinStepsPerWave));
  if (blockIdx.x == 0) {
    if (lane == 0) {
      hdr->total_steps = N;
      hdr->waves = weff;
    }
    int* hp = reinterpret_cast<int*>(hdr + 1);
    for (int s = lane; s <= S; s += 64) hp[s] = P[s];
  }
  if ((int64_t)blockIdx.x >= weff) return;
  // Workgroups are dealt to the 8 XCDs round-robin; each XCD takes a
  // contiguous run of the weff shares, so the KV heads of one sequence
  // (neighbours in the work list) run under one L2 and share its lines of
  // the block table and of the fp8 scales.  A bijection of [0, weff).
  const int nb = (int)weff, xq = nb >> 3, xr = nb & 7, xk = blockIdx.x & 7;
  const int w = xk * xq + min(xk, xr) + (blockIdx.x >> 3);
  // appending e4m3 decode: the new token's codes (K row, V column) after Ls
  uint8_t* tok_lds = reinterpret_cast<uint8_t*>(smem + ((2 * S + 1 + 3) & ~3));
  decode_share<D, FP8, FP8 ? kFp8Sets : kDecodeSets, PREFIX, APPEND>(a, P, Ls, N, weff, w,
                                                                      tok_lds);
}

// Up to kMergeBatch pieces of one row held in registers, so that all of
// their loads are in flight together (lane b also holds piece b's (m, l)).
constexpr int kMergeBatch = 8;
template <int D>
struct RowPieces {
  float o[kMergeBatch][D / 64];
  float m, l;
};

// Loads pieces 0 .. ns-1 (ns <= kMergeBatch) of a row; slot(b) is piece b's
// partial slot.
template <int D, typename SlotFn>
__device__ __forceinline__ void load_pieces(const float* ml, const float* po, int ns, SlotFn slot,
                                            int lane, RowPieces<D>& rp) {
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) {
    if (k < ns) {
      const float* p = po + (int64_t)slot(k) * D + lane;
#pragma unroll
      for (int dd = 0; dd < D / 64; ++dd) rp.o[k][dd] = p[64 * dd];
    }
  }
  rp.m = lane < ns ? ml[2 * slot(lane)] : neg_inf();
  rp.l = lane < ns ? ml[2 * slot(lane) + 1] : 0.f;
}

// out = sum_b 2^(m_b - M) o_b / sum_b 2^(m_b - M) l_b over the loaded pieces
// (the same operations, in the same order, as the general loops below).
template <int ES, int D>
__device__ __forceinline__ void combine_pieces(const RowPieces<D>& rp, int ns, void* out,
                                               int64_t orow, int lane) {
  constexpr int DD = D / 64;
  // lanes past ns may hold slots loaded ahead of time that this row does
  // not use: they take no part in the max
  float M = lane < ns ? rp.m : neg_inf();
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) M = fmaxf(M, __shfl_xor(M, w));
  const float wt = lane < ns ? fast_exp2(rp.m - M) : 0.f;
  float den = lane < ns ? wt * rp.l : 0.f;
  float acc[DD];
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) acc[dd] = 0.f;
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) {
    if (k < ns) {
      const float wk = __shfl(wt, k);
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) acc[dd] += wk * rp.o[k][dd];
    }
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) den += __shfl_xor(den, w);
  const float inv = 1.f / den;
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) store_elem<ES>(out, orow * D + lane + 64 * dd, acc[dd] * inv);
}

// Pieces of work-list entry e for KV head kvh: the waves whose shares
// intersect the entry's step range (0 when the entry has no steps).
__device__ __forceinline__ int entry_pieces(const int* P, int e, int Hkv, int kvh, int64_t weff,
                                            int64_t N) {
  const int cost = P[e + 1] - P[e];
  if (cost <= 0) return 0;
  const int64_t g_item = (int64_t)Hkv * P[e] + (int64_t)kvh * cost + kPieceCostSteps;
  const int64_t wf = wave_of_step(g_item, weff, N);
  const int64_t wl = wave_of_step(g_item + (cost - kPieceCostSteps) - 1, weff, N);
  return (int)(wl - wf + 1);
}

// Merge for the balanced decode: the pieces of row (s, h) are the waves whose
// shares intersect the row's step range.  With a shared prefix the row also
// has the pieces of its group's prefix entry, in the last prefix_slots slots,
// and is always merged (its decode wrote no final row).
template <int ES, int D>
__global__ __launch_bounds__(256) void merge_streamk_kernel(AttnArgs a, const StreamKHeader* hdr) {
  constexpr int DD = D / 64;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + wave;
  const int s = blockIdx.y;
  if (h >= a.num_q_heads) return;
  const bool pfx = a.prefix_keys > 0;
  const int64_t N = hdr->total_steps;
  const int64_t weff = hdr->waves;
  if (N <= 0 || weff <= 0) return;
  const int* P = reinterpret_cast<const int*>(hdr + 1);
  const int G = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / G;
  const int own_slots = a.sk_slots - (pfx ? a.prefix_slots : 0);
  const int n_own = min(entry_pieces(P, s, a.num_kv_heads, kvh, weff, N), own_slots);
  const int n_pfx =
      pfx ? min(entry_pieces(P, a.num_seqs + s / a.prefix_group, a.num_kv_heads, kvh, weff, N),
                a.prefix_slots)
          : 0;
  const int ns = n_own + n_pfx;
  if (pfx ? ns == 0 : ns <= 1) return;
  int r0, qn;
  seq_rows(a.query_start_loc, s, a.num_tokens, r0, qn);
  const int64_t orow = (int64_t)r0 * a.num_q_heads + h;
  const int64_t prow = pfx ? orow : (int64_t)s * a.num_q_heads + h;
  const float* ml = a.sk_part_ml + prow * a.sk_slots * 2;
  const float* po = a.sk_part_o + prow * a.sk_slots * D;
  // piece b -> its slot: the row's own pieces first, then the prefix's
  auto slot = [&](int b) { return b < n_own ? b : own_slots + (b - n_own); };
  if (ns <= kMergeBatch) {  // all loads in flight together
    RowPieces<D> rp;
    load_pieces<D>(ml, po, ns, slot, lane, rp);
    combine_pieces<ES, D>(rp, ns, a.out, orow, lane);
    return;
  }
  float M = neg_inf();
  for (int b = lane; b < ns; b += 64) M = fmaxf(M, ml[2 * slot(b)]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) M = fmaxf(M, __shfl_xor(M, w));
  float acc[DD];
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) acc[dd] = 0.f;
  float den = 0.f;
  for (int b0 = 0; b0 < ns; b0 += 64) {
    const int b = b0 + lane;
    const float w = b < ns ? fast_exp2(ml[2 * slot(b)] - M) : 0.f;
    den += b < ns ? w * ml[2 * slot(b) + 1] : 0.f;
    const int nb = min(64, ns - b0);
    for (int k = 0; k < nb; ++k) {
      const float wk = __shfl(w, k);
      const float* p = po + (int64_t)slot(b0 + k) * D + lane;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) acc[dd] += wk * p[64 * dd];
    }
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) den += __shfl_xor(den, w);
  const float inv = 1.f / den;
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) store_elem<ES>(a.out, orow * D + lane + 64 * dd, acc[dd] * inv);
}

// ---------------------------------------------------------------------------
// Query-chunk attention (chunked prefill) on v_mfma_f32_32x32x16_bf16 with
// K/V staged in LDS.
//
// Work.  A unit is (sequence with q_len > 1, KV head, tile of 256 query rows,
// row = j * G + g for chunk token j and group head g).  It needs
// ceil(klim / 32) steps of 32 keys, klim being the causal key limit of its
// last row.  The steps of all units, laid end to end (sequence, KV head,
// tile; tile fastest, so that the tiles sharing one stretch of K/V are
// neighbours), are cut into ranges of equal length, one range per resident
// workgroup ("stream-K").  A unit that a range boundary cuts leaves one
// partial (o, m, l) per piece; merge_kernel combines them.  Ranges go to
// workgroups so that each XCD (workgroups are dealt to the 8 XCDs
// round-robin) takes a contiguous run, which keeps a unit's K/V in one L2.
//
// One workgroup per CU: 8 waves (two per SIMD, up to 256 registers each)
// for head_dim 128, 4 for head_dim 64; a wave owns 32 query rows
// (PrefillShape).  Per 32-key step a wave issues D/16 MFMAs for
// S^T = K Q^T and D/16 for O^T = V^T P^T.
//
// S^T = K Q^T (A = K rows of the step, B = Q^T): the accumulator gives lane
// l the 16 scores of query row l%32 at MFMA rows (r/4)*8 + 4*(l/32) + r%4.
// Mapping MFMA row m to step token sigma32(m) (quads 1 and 2 of every 16
// swapped) makes registers 8k..8k+7 of that accumulator hold tokens
// 16k + 8*(l/32) .. +7 -- exactly the B operand P^T of O^T = V^T P^T for the
// k-th 16-key MFMA step.  In O^T every register of lane l belongs to query
// row l%32, so the online-softmax rescale is lane-local.
//
// LDS holds a ring of kPrefillStages steps of [K tile 32 x D | V^T tile],
// filled by direct global->LDS loads (16 bytes per lane, no registers)
// kPrefillStages-1 steps ahead of the step being computed.  Every load
// instruction reads from one physical block, so its address is a scalar
// block base plus a per-lane offset fixed for the whole kernel.  K rows keep
// the pool's token-row order; the V^T tile is block-major ([block of the
// step][head_dim row][8-key chunk]) so that it, too, copies whole runs of one
// block.  The 16-byte chunks are XOR-swizzled so that the MFMA operand reads
// (ds_read_b128, 16 lanes per LDS cycle) touch 16 distinct bank groups.
// Each wave waits for its own loads with vmcnt; one workgroup barrier per
// step publishes the stage and frees the oldest one.
// ---------------------------------------------------------------------------
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Shape of the chunk kernel per head_dim: query rows per wave (32 * halves)
// and waves per workgroup; a unit is the workgroup's rows.
template <int D>
struct PrefillShape {
  static constexpr int kHalves = 1;
  static constexpr int kWaves = D == 128 ? 8 : 4;
  static constexpr int kRows = 32 * kHalves * kWaves;
};
constexpr int kPrefillGroup = 4;                        // steps between barriers
constexpr int kPrefillStages = 2 * kPrefillGroup + 1;   // LDS ring of K/V steps


// global_load_lds of 16 bytes: lane l's bytes land at lds_base + 16 * l.
__device__ __forceinline__ void load_to_lds(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void*)src,
                                   (__attribute__((address_space(3))) void*)lds_base, 16, 0, 0);
}

__device__ __forceinline__ int sigma32(int m) {
  const int q = (m >> 2) & 3;
  const int qq = q == 1 ? 2 : (q == 2 ? 1 : q);
  return (m & 16) | (qq << 2) | (m & 3);
}

// Swizzle of the 16-byte chunks of K row t (D/8 chunks per row; rows of
// 2*D bytes, 128/D rows per 256-byte bank sweep).
template <int D>
__device__ __forceinline__ int ksw(int t) {
  return (t / (128 / D)) % (D / 8);
}

// Steps of 32 keys that tile `tile` of a sequence needs: up to the causal
// limit of its last row, capped by what the table addresses.
__device__ __forceinline__ int tile_steps(int rows, int tile, int nrows, int G, int L, int qn,
                                          int kcap) {
  const int row_last = min((tile + 1) * rows, nrows) - 1;
  const int klim = min(L - qn + row_last / G + 1, kcap);
  return klim > 0 ? (klim + 31) >> 5 : 0;
}

// Steps of all units of sequence s for one KV head (0 for decode rows).
__device__ __forceinline__ int seq_unit_steps(const AttnArgs& a, int s, int G, int rows) {
  int r0, qn;
  seq_rows(a.query_start_loc, s, a.num_tokens, r0, qn);
  if (qn <= 1) return 0;
  const int L = a.seq_lens[s];
  const int kcap = table_blocks(L, a.log2_block, a.max_blocks) << a.log2_block;
  const int nrows = qn * G;
  const int tiles = (nrows + rows - 1) / rows;
  int n = 0;
  for (int t = 0; t < tiles; ++t) n += tile_steps(rows, t, nrows, G, L, qn, kcap);
  return n;
}

// Steps per sequence (all KV heads) of the chunk units, then their prefix
// sums: seq_prefix[s] = steps before sequence s.  All threads of the
// workgroup take part; ends synchronised.
template <int D>
__device__ __forceinline__ void prefill_prefix(const AttnArgs& a, int* seq_prefix) {
  constexpr int NW = PrefillShape<D>::kWaves;
  const int tid = threadIdx.x;
  const int S = a.num_seqs;
  const int G = a.num_q_heads / a.num_kv_heads;
  for (int s = tid; s < S; s += 64 * NW)
    seq_prefix[s + 1] = a.num_kv_heads * seq_unit_steps(a, s, G, PrefillShape<D>::kRows);
  __syncthreads();
  if (tid == 0) {
    seq_prefix[0] = 0;
    for (int s = 0; s < S; ++s) seq_prefix[s + 1] += seq_prefix[s];
  }
  __syncthreads();
}

// The chunk units' work of workgroup wg of num_wgs (a multiple of 8), given
// the step prefix sums.  Every wave of the workgroup takes part (barriers).
// CPB is the number of 8-key chunks one block holds inside a 32-key step
// (min(B, 32) / 8): fixed at compile time, so the V^T tile's head_dim tiles
// sit at constant offsets from a lane's read address.
template <int D, int LGB>
__device__ __forceinline__ void prefill_ranges(const AttnArgs& a, const int* seq_prefix, int wg,
                                               int num_wgs, uint16_t (*smem)[2][32 * D]) {
  constexpr int H = PrefillShape<D>::kHalves;    // 32-row halves per wave
  constexpr int NW = PrefillShape<D>::kWaves;
  constexpr int ROWS = PrefillShape<D>::kRows;
  constexpr int KS = D / 16;                     // S^T MFMA steps over head_dim
  constexpr int DT = D / 32;                     // O^T head_dim tiles
  constexpr int CPR = D / 8;                     // 16-byte chunks per K row
  constexpr int RPI = 1024 / (2 * D);            // K rows per 1 KiB load
  constexpr int IPW = (D / 16) / NW;            // 1 KiB loads per wave per tile
  static_assert(IPW >= 1, "every wave loads part of each tile");
  constexpr int NS = kPrefillStages;
  constexpr int GS = kPrefillGroup;
  constexpr int TILE = 32 * D;                   // elements of one K or V^T tile
  static_assert(TILE == 32 * D, "stage layout");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // known wave-uniform
  const int h = lane >> 5;
  const int c32 = lane & 31;
  const int S = a.num_seqs;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int Hkv = a.num_kv_heads;
  constexpr int lg = LGB;        // block size B = 2^LGB, 8 to 64 on this path
  constexpr int B = 1 << lg;
  constexpr int cpb = (B < 32 ? B : 32) / 8;  // 8-key chunks of one block inside a step (1, 2, 4)
  constexpr int Bs = 8 * cpb;    // keys of one block inside a step
  constexpr int lcpb = cpb == 4 ? 2 : cpb - 1;

  const int N = seq_prefix[S];
  if (N == 0) return;
  const int chunk = a.chunk_auto ? max((N + num_wgs - 1) / num_wgs, a.chunk_steps) : a.chunk_steps;
  const int nranges = (N + chunk - 1) / chunk;

  // Per-lane pieces of the load and read addresses, fixed for the kernel.
  int k_voff[IPW], v_voff[IPW], v_bi[IPW];
#pragma unroll
  for (int x2 = 0; x2 < IPW; ++x2) {
    const int x = w * IPW + x2;
    const int t = x * RPI + lane / CPR;  // token row of the step
    const int chunk16 = (lane % CPR) ^ ksw<D>(t);
    k_voff[x2] = ((lane / CPR) * D + chunk16 * 8) * 2;
    const int p = 64 * x + lane;              // 16-byte position in the V^T tile
    v_bi[x2] = __builtin_amdgcn_readfirstlane(p / (D * cpb));  // block of the step (wave-uniform)
    const int d = (p % (D * cpb)) >> lcpb;    // head_dim row
    const int vs = (d >> (4 - lcpb)) & (cpb - 1);
    const int u = (p & (cpb - 1)) ^ vs;       // 8-key chunk inside the block
    v_voff[x2] = (d * B + 8 * u) * 2;
  }
  const int tk = sigma32(c32);
  int k_roff[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) k_roff[ks] = tk * D + (((2 * ks + h) ^ ksw<D>(tk)) * 8);
  int v_roff[2];
#pragma unroll
  for (int k2 = 0; k2 < 2; ++k2) {
    const int c = 2 * k2 + h;  // 8-key chunk of the step
    const int bi = c >> lcpb, u = c & (cpb - 1);
    const int vs = (c32 >> (4 - lcpb)) & (cpb - 1);
    v_roff[k2] = (bi * D * cpb + c32 * cpb + (u ^ vs)) * 8;
  }
  const float sl2 = a.scale_log2;  // > 0 (checked by the host)
  const int64_t blk_stride = (int64_t)Hkv * B * D;

  for (int r = (wg & 7) * (num_wgs >> 3) + (wg >> 3); r < nranges; r += num_wgs) {
    int g = r * chunk;
    const int gend = min(g + chunk, N);
    // -- unit holding step g ---------------------------------------------
    int s;
    {
      int lo = 0, hi = S - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (seq_prefix[mid] <= g) lo = mid;
        else hi = mid - 1;
      }
      s = lo;
    }
    int rem = g - seq_prefix[s];
    int kvh = 0, tile = 0;
    {
      const int per_head = (seq_prefix[s + 1] - seq_prefix[s]) / Hkv;
      kvh = rem / per_head;
      rem -= kvh * per_head;
    }
    bool located = false;
    // Next unit in (sequence, KV head, tile) order; false past the last one.
    auto advance = [&](int tiles) {
      if (++tile < tiles) return true;
      tile = 0;
      if (++kvh < Hkv) return true;
      kvh = 0;
      do {
        ++s;
      } while (s < S && seq_prefix[s + 1] == seq_prefix[s]);
      return s < S;
    };
    while (g < gend) {
      int r0, qn;
      seq_rows(a.query_start_loc, s, a.num_tokens, r0, qn);
      const int L = a.seq_lens[s];
      const SeqView v = seq_view(a, s, kvh, L, r0, qn);
      const int nrows = qn * G;
      const int tiles = (nrows + ROWS - 1) / ROWS;
      if (!located) {  // tile holding step rem of this (sequence, KV head)
        for (;;) {
          const int n = tile_steps(ROWS, tile, nrows, G, L, qn, v.kcap);
          if (rem < n) break;
          rem -= n;
          ++tile;
        }
        located = true;
      }
      const int nst = tile_steps(ROWS, tile, nrows, G, L, qn, v.kcap);
      if (nst == 0) {  // rows that see no keys (q_len > seq_len): nothing to do
        if (!advance(tiles)) break;
        continue;
      }
      const int a_step = rem;
      const int b_step = min(nst, rem + (gend - g));
      const int u_first = (g - a_step) / chunk;            // range of the unit's first step
      const int u_last = (g - a_step + nst - 1) / chunk;   // range of its last step
      const int npieces = u_last - u_first + 1;
      const int slot = r - u_first;

      // -- one piece: steps [a_step, b_step) of unit (s, kvh, tile) --------
      const int row0 = tile * ROWS;
      const int row_last = min(row0 + ROWS, nrows) - 1;
      const int kv_t = min(L - qn + row_last / G + 1, v.kcap);  // keys the unit sees
      const int k_begin = 32 * a_step;
      const int nsteps = b_step - a_step;
      const int wrow0 = row0 + 32 * H * w;
      const bool wave_active = wrow0 < nrows;
      const int kv_wmin = wave_active ? min(L - qn + wrow0 / G + 1, v.kcap) : 0;

      int jr[H], gr[H], klim[H];
      bool ok[H];
      bf16x8 qf[H][KS];
#pragma unroll
      for (int hf = 0; hf < H; ++hf) {
        const int row = wrow0 + 32 * hf + c32;
        ok[hf] = row < nrows;
        jr[hf] = ok[hf] ? row / G : 0;
        gr[hf] = ok[hf] ? row - jr[hf] * G : 0;
        klim[hf] = ok[hf] ? min(L - qn + jr[hf] + 1, v.kcap) : 0;
        const uint16_t* qp = static_cast<const uint16_t*>(a.q) +
                             ((int64_t)(r0 + jr[hf]) * a.num_q_heads + kvh * G + gr[hf]) * D + 8 * h;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[hf][ks] = ok[hf] ? load_bf16x8(qp + 16 * ks) : bf16x8{};
      }

      const int64_t trow = (int64_t)s * a.max_blocks;
      // Block ids: a window of 64 logical blocks, one per lane, read with
      // readlane.  Ids are clamped when a window becomes current, not when it
      // is loaded: the prefetched next window is not waited for early.  The
      // current window is kept as each block's offset in the pool in 256-byte
      // units (a block is a multiple of 256 bytes, and the host keeps the
      // pool under 2^40 bytes), so a load's block base is one readlane, a
      // shift and an add.
      auto window = [&](int b0) { return a.block_tables[trow + min(b0 + lane, a.max_blocks - 1)]; };
      const uint32_t blk_units = (uint32_t)(blk_stride * 2 / 256);
      uint32_t woff;
      auto set_window = [&](int id) { woff = (uint32_t)clampi(id, 0, a.num_blocks - 1) * blk_units; };
      auto block_off = [&](int idx) {
        return (uint64_t)(uint32_t)__builtin_amdgcn_readlane(woff, idx) << 8;
      };
      int blk0 = k_begin >> lg;
      set_window(window(blk0));
      int wid_next = window(blk0 + 64);
      const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * B * D;
      const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + (int64_t)kvh * D * B;

      // This wave's share of one step (key c) into stage st: IPW 1 KiB pieces
      // of the K tile and of the V^T tile, each from one block.
      auto dma = [&](int c, int st) {
        if ((c >> lg) - blk0 >= 64) {  // wave-uniform: next window of block ids
          blk0 += 64;
          set_window(wid_next);
          wid_next = window(blk0 + 64);
        }
        const int cb = (c >> lg) - blk0;
        const int cmax = v.nblk - 1 - blk0;          // keys past the table reuse its last block
        const int cin = B > 32 ? (c & (B - 1)) : 0;  // token offset of the step in its block
#pragma unroll
        for (int x2 = 0; x2 < IPW; ++x2) {
          const int x = w * IPW + x2;
          const int kb = (x * RPI) >> lg;  // block of these K rows inside the step
          const char* ksrc = reinterpret_cast<const char*>(
                                 kbase + (cin + ((x * RPI) & (Bs - 1))) * D) +
                             block_off(min(cb + kb, cmax));
          load_to_lds(ksrc + k_voff[x2], &smem[st][0][x * 512]);
          const char* vsrc =
              reinterpret_cast<const char*>(vbase + cin) + block_off(min(cb + v_bi[x2], cmax));
          load_to_lds(vsrc + v_voff[x2], &smem[st][1][x * 512]);
        }
      };

      float m[H], l[H];
      f32x16 o[H][DT];
#pragma unroll
      for (int hf = 0; hf < H; ++hf) {
        m[hf] = neg_inf();
        l[hf] = 0.f;
      }
#pragma unroll
      for (int hf = 0; hf < H; ++hf)
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[hf][dt] = f32x16{};

      // S^T of one step for every half (unscaled scores).
      auto scores = [&](int st, f32x16* sc) {
        const uint16_t* kt = smem[st][0];
        bf16x8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = *reinterpret_cast<const bf16x8*>(kt + k_roff[ks]);
#pragma unroll
        for (int hf = 0; hf < H; ++hf) sc[hf] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int hf = 0; hf < H; ++hf)
            sc[hf] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[hf][ks], sc[hf], 0, 0, 0);
      };

      // Keys past a row's limit get score -inf (scores sc of the step at key c).
      auto mask_scores = [&](f32x16* sc, int c) {
#pragma unroll
        for (int hf = 0; hf < H; ++hf)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int tok = 16 * (r >> 3) + 8 * h + (r & 7);
            sc[hf][r] = c + tok < klim[hf] ? sc[hf][r] : neg_inf();
          }
      };
      // Row maxima of (masked) scores, in log2 units.
      auto row_max = [&](const f32x16* sc, float* mx) {
#pragma unroll
        for (int hf = 0; hf < H; ++hf) {
          float t = sc[hf][0];
#pragma unroll
          for (int r = 1; r < 16; ++r) t = fmaxf(t, sc[hf][r]);
          auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
          mx[hf] = fmaxf(__uint_as_float(q[0]), __uint_as_float(q[1])) * sl2;
        }
      };

      // Ring of NS = 2 * GS + 1 stages, filled GS steps at a time.  Before
      // group g (steps g*GS .. g*GS + GS - 1) every wave waits for its own
      // loads of steps up to g*GS + GS (the group and the step after it,
      // whose K the group's last step reads), and one barrier publishes
      // everyone's loads and guarantees that all waves left group g-1; the
      // loads of steps g*GS + GS + 1 .. g*GS + 2*GS then go to the stages
      // group g-1 used.  Between barriers the waves of a workgroup run
      // freely, so the two waves sharing a SIMD drift apart and overlap
      // their matrix and vector work.  Loads past the end re-read the last
      // step.
      //
      // Within a step, the S^T of step i+1 is computed between the (masked)
      // scores of step i and its softmax and PV.  The running maximum m is
      // the true maximum of the piece's first step, then raised only when a
      // step's probabilities grow too large: p = exp2(s * scale_log2 - m)
      // is computed with the current m, and when a lane's sum of its 16 p
      // exceeds 2^8 (or is not finite) the wave takes the rare path, which
      // raises m of those rows to their true maximum, rescales o and l and
      // recomputes the step's p.  Every kept p is then at most 2^8, m is at
      // most the rows' running maximum (so each row with a visible key has a
      // p >= 1), and no per-step maximum is needed.
      int st_load = 0;  // stage of the next load
      auto load_step = [&](int p) {
        dma(k_begin + 32 * min(p, nsteps - 1), st_load);
        st_load = st_load + 1 == NS ? 0 : st_load + 1;
      };
#pragma unroll
      for (int p = 0; p <= GS; ++p) load_step(p);
      f32x16 cur[H];
      float nm[H];        // -m, or 0 while the row has seen no key
      int st_cur = 0;     // stage of step i
      for (int g0 = 0; g0 < nsteps; g0 += GS) {
        __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int p = GS + 1; p <= 2 * GS; ++p) load_step(g0 + p);
        if (!wave_active) continue;
        if (g0 == 0) {
          scores(0, cur);
          if (k_begin + 32 > kv_wmin) mask_scores(cur, k_begin);
          float mx[H];
          row_max(cur, mx);
#pragma unroll
          for (int hf = 0; hf < H; ++hf) {
            m[hf] = mx[hf];
            nm[hf] = (m[hf] == neg_inf()) ? 0.f : -m[hf];
          }
        }
#pragma unroll
        for (int ii = 0; ii < GS; ++ii) {
          const int i = g0 + ii;
          if (i >= nsteps) break;
          const int st_next = st_cur + 1 == NS ? 0 : st_cur + 1;
          const int c = k_begin + 32 * i;
          f32x16 nxt[H];
          scores(st_next, nxt);
          // probabilities of step i (bf16 for the PV MFMA) and their lane sums
          float ps[H];
          bf16x8 pf[H][2];
          auto softmax = [&](int hf) {
            float t = 0.f;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const float p = fast_exp2(fmaf(cur[hf][r], sl2, nm[hf]));
              t = r == 0 ? p : t + p;  // p >= +0: the same sum as from 0, one add fewer
              pf[hf][r >> 3][r & 7] = static_cast<__bf16>(p);
            }
            ps[hf] = t;
          };
          bool over = false;
#pragma unroll
          for (int hf = 0; hf < H; ++hf) {
            softmax(hf);
            over = over || !(ps[hf] <= kLazyRescaleSum);
          }
          if (__builtin_amdgcn_ballot_w64(over) != 0) {
            // some row's probabilities grew past 2^8: raise its m to its
            // true maximum so far, rescale, recompute this step's p
            rare_branch();
            float mx[H];
            row_max(cur, mx);
#pragma unroll
            for (int hf = 0; hf < H; ++hf) {
              const float mnew = fmaxf(m[hf], mx[hf]);
              if (mnew > m[hf]) {
                const float alpha = fast_exp2(m[hf] - mnew);   // 0 when m was -inf
                l[hf] *= alpha;
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                  for (int r = 0; r < 16; ++r) o[hf][dt][r] *= alpha;
                m[hf] = mnew;
                nm[hf] = -mnew;
              }
              softmax(hf);
            }
          }
#pragma unroll
          for (int hf = 0; hf < H; ++hf) {
            auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(ps[hf]), __float_as_uint(ps[hf]), false, false);
            l[hf] += __uint_as_float(q[0]) + __uint_as_float(q[1]);
          }
          const uint16_t* vt = smem[st_cur][1];
          bf16x8 vf[DT][2];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
              vf[dt][k2] = *reinterpret_cast<const bf16x8*>(vt + v_roff[k2] + dt * 32 * cpb * 8);
          if (c + 32 > kv_t) {
            // keys past the unit's last visible one may be unwritten slots:
            // their V must not reach the accumulators even with p = 0
            rare_branch();
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2) {
              const int lim = kv_t - (c + 16 * k2 + 8 * h);  // valid keys of this lane's 8
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) {
                u32x4 bits = __builtin_bit_cast(u32x4, vf[dt][k2]);
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                  const uint32_t keep = (2 * e2 < lim ? 0xFFFFu : 0u) | (2 * e2 + 1 < lim ? 0xFFFF0000u : 0u);
                  bits[e2] &= keep;
                }
                vf[dt][k2] = __builtin_bit_cast(bf16x8, bits);
              }
            }
          }
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int k2 = 0; k2 < 2; ++k2)
#pragma unroll
              for (int hf = 0; hf < H; ++hf)
                o[hf][dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[dt][k2], pf[hf][k2], o[hf][dt], 0, 0, 0);
          // next step's scores: keys past a row's limit get -inf
          if (c + 64 > kv_wmin) mask_scores(nxt, c + 32);
#pragma unroll
          for (int hf = 0; hf < H; ++hf) cur[hf] = nxt[hf];
          st_cur = st_next;
        }
      }
      __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // the ring is quiet
      __builtin_amdgcn_s_waitcnt(0xC07F);        // lgkmcnt(0)
      __builtin_amdgcn_s_barrier();              // before the next piece refills it
      // -- results ----------------------------------------------------------
#pragma unroll
      for (int hf = 0; hf < H; ++hf) {
        if (!ok[hf]) continue;
        const int64_t orow = (int64_t)(r0 + jr[hf]) * a.num_q_heads + kvh * G + gr[hf];
        if (npieces == 1) {
          if (klim[hf] <= 0) continue;
          const float inv = 1.f / l[hf];
          uint16_t* out = static_cast<uint16_t*>(a.out) + orow * D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
              const uint32_t lo = f32_to_bf16_bits(o[hf][dt][4 * r4] * inv) |
                                  ((uint32_t)f32_to_bf16_bits(o[hf][dt][4 * r4 + 1] * inv) << 16);
              const uint32_t hi = f32_to_bf16_bits(o[hf][dt][4 * r4 + 2] * inv) |
                                  ((uint32_t)f32_to_bf16_bits(o[hf][dt][4 * r4 + 3] * inv) << 16);
              *reinterpret_cast<uint2*>(out + 32 * dt + 8 * r4 + 4 * h) = make_uint2(lo, hi);
            }
        } else if (slot < a.max_splits) {
          const int64_t pidx = orow * a.max_splits + slot;
          float* po = a.part_o + pidx * D;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4)
              *reinterpret_cast<f32x4*>(po + 32 * dt + 8 * r4 + 4 * h) =
                  f32x4{o[hf][dt][4 * r4], o[hf][dt][4 * r4 + 1], o[hf][dt][4 * r4 + 2],
                        o[hf][dt][4 * r4 + 3]};
          if (h == 0) {
            a.part_ml[2 * pidx] = m[hf];
            a.part_ml[2 * pidx + 1] = l[hf];
          }
        }
        if (a_step == 0 && h == 0) a.row_pieces[orow] = npieces;
      }

      // -- next unit ----------------------------------------------------------
      g += nsteps;
      rem = 0;
      if (!advance(tiles)) break;
    }
  }
}


// prefill_ranges for the block size of the call (B >= 8 on this path).
template <int D>
__device__ __forceinline__ void prefill_ranges_any(const AttnArgs& a, const int* seq_prefix,
                                                   int wg, int num_wgs) {
  // The ring of K / V^T stages (one per workgroup, whatever the block size).
  __shared__ __attribute__((aligned(16))) uint16_t smem[kPrefillStages][2][32 * D];
  switch (a.log2_block) {
    case 3: prefill_ranges<D, 3>(a, seq_prefix, wg, num_wgs, smem); break;
    case 4: prefill_ranges<D, 4>(a, seq_prefix, wg, num_wgs, smem); break;
    case 5: prefill_ranges<D, 5>(a, seq_prefix, wg, num_wgs, smem); break;
    default: prefill_ranges<D, 6>(a, seq_prefix, wg, num_wgs, smem); break;
  }
}

template <int D>
__global__ __launch_bounds__(64 * PrefillShape<D>::kWaves) __attribute__((
    amdgpu_waves_per_eu(PrefillShape<D>::kHalves == 1 ? 2 : 1, PrefillShape<D>::kHalves == 1 ? 2 : 1)))
void prefill_kernel(AttnArgs a, int num_wgs) {
  extern __shared__ int seq_prefix[];  // [num_seqs + 1] steps
  prefill_prefix<D>(a, seq_prefix);
  prefill_ranges_any<D>(a, seq_prefix, blockIdx.x, num_wgs);
}

// Chunk units and single-token rows of one call in one persistent launch:
// the resident workgroups are split between the two kinds of work, so that
// the matrix-bound chunk units and the memory-bound decode rows run at the
// same time on different CUs instead of one after the other.  Every
// workgroup builds both step prefix sums and derives the same split from
// them: the CUs are shared in proportion to the estimated CU-time of each
// kind (kChunkStepNs per 256-row chunk step, kDecodeStepNs per 32-key decode
// step), in multiples of 8 so that every XCD gets the same mix.  Chunk
// workgroups run prefill_ranges; each wave of a decode workgroup is one wave
// of the balanced decode (two fragment sets, so that both kinds fit the same
// 256-register budget).
// Relative CU-time per step (D = 128; half at D = 64), in ns of one CU,
// each measured on a batch of one kind only, with every CU on it: 4 query
// chunks of 512 tokens over 1-8K context (45,056 chunk steps in 291 us on
// 256 CUs -> 1,650 ns) and 60 decode rows of 256-4,096 keys through the
// same launch (35,744 decode steps in 107 us -> 770 ns).  The decode step
// costs a CU more than its bytes at the HBM rate: one CU streams far below
// its share of HBM bandwidth.  On four mixes (4 x 512 chunks + 60 decode
// rows, 1 x 2,048 + 200, 8 x 512 + 8, 2 x 256 + 120) the split these give
// is within 1.5-3% of the best split found by sweeping it.
constexpr int64_t kChunkStepNs = 1650;
constexpr int64_t kDecodeStepNs = 770;
// An e4m3 decode step (64 keys, the same 16 KiB) in the fused launch runs
// with two fragment sets in a 256-register budget: on workload 5 over e4m3
// pools, 1,000 ns gave the fastest call of 600-1,700 ns, with the Infinity
// Cache flushed between calls and without.
constexpr int64_t kDecodeStepNsFp8 = 1000;

// dec holds the single-token rows' view (the e4m3 pools when FP8), chunk the
// chunk units' view (the same arguments for a bf16 cache; for e4m3 the
// staged bf16 pools and their table).
template <int D, bool FP8>
__device__ __forceinline__ void chunk_mix_body(const AttnArgs& dec, const AttnArgs& chunk,
                                               int num_wgs, StreamKHeader* hdr) {
  constexpr int NW = PrefillShape<D>::kWaves;
  static_assert(PrefillShape<D>::kHalves == 1, "decode waves need the two-wave register budget");
  extern __shared__ int lds_i[];
  const int S = dec.num_seqs;
  int* seq_prefix = lds_i;        // [S + 1] chunk steps before sequence s
  int* P = lds_i + S + 1;         // [S + 1] decode steps before sequence s (per KV head)
  int* Ls = P + S + 1;            // [S]     sequence lengths
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  decode_prefix_fill<FP8>(dec, P, Ls, tid, 64 * NW);
  prefill_prefix<D>(chunk, seq_prefix);  // synchronises: P and Ls are filled too
  if (w == 0) decode_prefix_scan(P, S, lane);
  __syncthreads();
  const int64_t n_pf = seq_prefix[S];
  const int64_t n_dec = (int64_t)dec.num_kv_heads * P[S];
  int w_dec = 0;
  if (n_dec > 0) {
    const int64_t pf = n_pf * (kChunkStepNs * D / 128);
    const int64_t dc = n_dec * ((FP8 ? kDecodeStepNsFp8 : kDecodeStepNs) * D / 128);
    w_dec = (int)(((int64_t)num_wgs * dc / (pf + dc) + 4) / 8 * 8);
    w_dec = max(w_dec, 8);
    if (n_pf > 0) w_dec = min(w_dec, num_wgs - 8);
  }
  const int w_pf = num_wgs - w_dec;
  if ((int)blockIdx.x < w_pf) {
    if (w_dec == 0 && blockIdx.x == 0 && tid == 0) {  // no decode rows: an empty header
      hdr->total_steps = 0;
      hdr->waves = 0;
    }
    prefill_ranges_any<D>(chunk, seq_prefix, blockIdx.x, w_pf);
    return;
  }
  const int64_t waves = (int64_t)w_dec * NW;
  const int64_t weff = n_dec == 0 ? 0 : min(waves, max((int64_t)1, n_dec / kMinStepsPerWave));
  const int dw = (blockIdx.x - w_pf) * NW + w;
  if (dw == 0) {
    if (lane == 0) {
      hdr->total_steps = n_dec;
      hdr->waves = weff;
    }
    int* hp = reinterpret_cast<int*>(hdr + 1);
    for (int s = lane; s <= S; s += 64) hp[s] = P[s];
  }
  if (dw >= weff) return;
  decode_share<D, FP8, 2>(dec, P, Ls, n_dec, weff, dw);
}

template <int D>
__global__ __launch_bounds__(64 * PrefillShape<D>::kWaves) __attribute__((
    amdgpu_waves_per_eu(PrefillShape<D>::kHalves == 1 ? 2 : 1, PrefillShape<D>::kHalves == 1 ? 2 : 1)))
void chunk_mix_kernel(AttnArgs a, int num_wgs, StreamKHeader* hdr) {
  chunk_mix_body<D, false>(a, a, num_wgs, hdr);
}

// The same over an e4m3 cache: chunk units on the staged bf16 pools, the
// single-token rows on the e4m3 pools (two fragment sets per decode wave).
template <int D>
__global__ __launch_bounds__(64 * PrefillShape<D>::kWaves) __attribute__((
    amdgpu_waves_per_eu(PrefillShape<D>::kHalves == 1 ? 2 : 1, PrefillShape<D>::kHalves == 1 ? 2 : 1)))
void chunk_mix_fp8_kernel(AttnArgs dec, AttnArgs chunk, int num_wgs, StreamKHeader* hdr) {
  chunk_mix_body<D, true>(dec, chunk, num_wgs, hdr);
}

// ---------------------------------------------------------------------------
// Vector-ALU attention: one wave per (query token, KV head, split) serving
// the G heads of the group.  Lanes own keys for QK^T and head_dim columns for
// PV.  Used for fp32 caches and for bf16 caches with blocks under 8 tokens.
// ---------------------------------------------------------------------------
template <int ES, int D>
__global__ __launch_bounds__(64) void attn_valu_kernel(AttnArgs a) {
  constexpr int GM = 16;     // largest group size
  constexpr int DD = D / 64; // head_dim columns per lane
  __shared__ float sq[GM][D];
  __shared__ float sp[GM][64];
  __shared__ int sid[64];
  const int lane = threadIdx.x;
  const int s = blockIdx.x / a.num_kv_heads;   // (sequence, KV head) fastest: XCD balance
  const int kvh = blockIdx.x - s * a.num_kv_heads;
  const int j = blockIdx.y;
  const int split = blockIdx.z;
  const int T = a.num_tokens;
  int r0, qn;
  seq_rows(a.query_start_loc, s, T, r0, qn);
  if (j >= qn) return;
  const int L = a.seq_lens[s];
  const int lg = a.log2_block;
  const int B = 1 << lg;
  const int nblk = table_blocks(L, lg, a.max_blocks);
  const int kl = min(L - qn + j + 1, nblk << lg);
  const int k_begin = split * a.split_tokens;
  if (k_begin >= kl) return;
  const int k_end = min(k_begin + a.split_tokens, kl);
  const int G = a.num_q_heads / a.num_kv_heads;
  const int Hq = a.num_q_heads;
  const int64_t qrow0 = (int64_t)(r0 + j) * Hq + kvh * G;

  for (int idx = lane; idx < G * D; idx += 64) {
    const int g = idx / D;
    sq[g][idx - g * D] = load_elem<ES>(a.q, qrow0 * D + idx);
  }
  __syncthreads();

  float m[GM], l[GM], acc[GM][DD];
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    m[g] = neg_inf();
    l[g] = 0.f;
#pragma unroll
    for (int dd = 0; dd < DD; ++dd) acc[g][dd] = 0.f;
  }
  const int64_t blk_stride = (int64_t)a.num_kv_heads * B * D;
  const float sl2 = a.scale_log2;

  for (int t0 = k_begin; t0 < k_end; t0 += 64) {
    const int t = t0 + lane;
    const bool valid = t < k_end;
    const int lb = min(t >> lg, nblk - 1);
    const int id = clampi(a.block_tables[(int64_t)s * a.max_blocks + lb], 0, a.num_blocks - 1);
    sid[lane] = id;
    const int64_t krow = id * blk_stride + (int64_t)kvh * B * D + (int64_t)(t & (B - 1)) * D;
    float sc[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) sc[g] = 0.f;
    for (int d = 0; d < D; ++d) {
      const float kv = load_elem<ES>(a.k_cache, krow + d);
#pragma unroll
      for (int g = 0; g < GM; ++g)
        if (g < G) sc[g] += sq[g][d] * kv;
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) {
      if (g >= G) break;
      const float x = valid ? sc[g] * sl2 : neg_inf();
      float mx = x;
#pragma unroll
      for (int w = 32; w >= 1; w >>= 1) mx = fmaxf(mx, __shfl_xor(mx, w));
      const float mnew = fmaxf(m[g], mx);
      const float muse = (mnew == neg_inf()) ? 0.f : mnew;
      const float alpha = fast_exp2(m[g] - muse);
      const float p = fast_exp2(x - muse);
      float ps = p;
#pragma unroll
      for (int w = 32; w >= 1; w >>= 1) ps += __shfl_xor(ps, w);
      l[g] = l[g] * alpha + ps;
      m[g] = mnew;
      sp[g][lane] = p;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) acc[g][dd] *= alpha;
    }
    __syncthreads();
    const int nt = min(64, k_end - t0);
    for (int tt = 0; tt < nt; ++tt) {
      const int tok = t0 + tt;
      const int64_t vcol = sid[tt] * blk_stride + (int64_t)kvh * D * B + (tok & (B - 1));
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) {
        const float v = load_elem<ES>(a.v_cache, vcol + (int64_t)(lane + 64 * dd) * B);
#pragma unroll
        for (int g = 0; g < GM; ++g)
          if (g < G) acc[g][dd] += sp[g][tt] * v;
      }
    }
    __syncthreads();
  }

  const int ns = min((kl + a.split_tokens - 1) / a.split_tokens, a.max_splits);
#pragma unroll
  for (int g = 0; g < GM; ++g) {
    if (g >= G) break;
    const int64_t orow = qrow0 + g;
    if (ns == 1) {
      const float inv = 1.f / l[g];
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) store_elem<ES>(a.out, orow * D + lane + 64 * dd, acc[g][dd] * inv);
    } else {
      const int64_t pidx = orow * a.max_splits + split;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) a.part_o[pidx * D + lane + 64 * dd] = acc[g][dd];
      if (lane == 0) {
        a.part_ml[2 * pidx] = m[g];
        a.part_ml[2 * pidx + 1] = l[g];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Merge of split partials: out = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i.
// One wave per (query token, head); lanes first read the splits' (m, l)
// pairs in parallel, then own head_dim columns while summing the weighted
// partial outputs.
// ---------------------------------------------------------------------------
// The sequence holding query row t (the largest s with qsl[s] <= t; qsl is
// non-decreasing) by a 64-way search: every lane tests one candidate and a
// ballot picks the answer, two rounds of loads for up to 4,096 sequences
// (more rounds beyond).  All 64 lanes of the wave call it.
__device__ __forceinline__ int seq_of_row(const int32_t* qsl, int S, int t, int lane) {
  int lo = 0, n = S;  // the answer lies in [lo, lo + n)
  while (n > 1) {
    const int k = (n + 63) >> 6;  // candidates lo, lo + k, lo + 2k, ...
    const int c = lo + lane * k;
    const bool ok = lane * k < n && qsl[c] <= t;
    const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
    const int last = m ? 63 - __builtin_clzll(m) : 0;  // qsl[0] = 0 <= t always holds
    lo += last * k;
    n = min(k, n - last * k);
  }
  return lo;
}

template <int ES, int D>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a, int skip_single) {
  constexpr int DD = D / 64;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int h = blockIdx.x * 4 + wave;
  const int t = blockIdx.y;  // query token row
  if (h >= a.num_q_heads) return;
  const int64_t orow = (int64_t)t * a.num_q_heads + h;
  const float* ml = a.part_ml + orow * a.max_splits * 2;
  const float* po = a.part_o + orow * a.max_splits * D;
  // With recorded piece counts the row's partials are loaded before the
  // sequence lookup, which they do not depend on (a row that turns out not
  // to be merged here only wasted the in-bounds loads).
  const int pieces = a.row_pieces ? a.row_pieces[orow] : 0;
  RowPieces<D> rp;
  if (a.row_pieces) {
    if (pieces <= 1) return;  // whole (written by the chunk kernel) or merged elsewhere
    if (pieces <= kMergeBatch)
      load_pieces<D>(ml, po, min(pieces, a.max_splits), [](int b) { return b; }, lane, rp);
  }
  int s = t;
  if (a.query_start_loc) s = seq_of_row(a.query_start_loc, a.num_seqs, t, lane);
  int r0, qn;
  seq_rows(a.query_start_loc, s, a.num_tokens, r0, qn);
  const int j = t - r0;
  if (j < 0 || j >= qn) return;
  if (skip_single && qn == 1) return;  // merged by the balanced decode's pass
  const int L = a.seq_lens[s];
  const int nblk = table_blocks(L, a.log2_block, a.max_blocks);
  const int kl = min(L - qn + j + 1, nblk << a.log2_block);
  if (kl <= 0) return;
  const int ns = min(a.row_pieces ? pieces : (kl + a.split_tokens - 1) / a.split_tokens,
                     a.max_splits);
  if (ns <= 1) return;
  if (ns <= kMergeBatch) {
    if (!a.row_pieces || pieces > kMergeBatch)
      load_pieces<D>(ml, po, ns, [](int b) { return b; }, lane, rp);
    combine_pieces<ES, D>(rp, ns, a.out, orow, lane);
    return;
  }
  float acc[DD];
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) acc[dd] = 0.f;
  float M = neg_inf();
  for (int b = lane; b < ns; b += 64) M = fmaxf(M, ml[2 * b]);
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) M = fmaxf(M, __shfl_xor(M, w));
  float den = 0.f;
  for (int b0 = 0; b0 < ns; b0 += 64) {
    const int b = b0 + lane;
    const float w = b < ns ? fast_exp2(ml[2 * b] - M) : 0.f;
    den += b < ns ? w * ml[2 * b + 1] : 0.f;
    const int nb = min(64, ns - b0);
#pragma unroll 4
    for (int k = 0; k < nb; ++k) {
      const float wk = __shfl(w, k);
      const float* p = po + (int64_t)(b0 + k) * D + lane;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) acc[dd] += wk * p[64 * dd];
    }
  }
#pragma unroll
  for (int w = 32; w >= 1; w >>= 1) den += __shfl_xor(den, w);
  const float inv = 1.f / den;
#pragma unroll
  for (int dd = 0; dd < DD; ++dd) store_elem<ES>(a.out, orow * D + lane + 64 * dd, acc[dd] * inv);
}

// Resident workgroups of a persistent kernel on the current device: CUs
// times its occupancy at this LDS size (cached for the last call site,
// device and sequence count).
struct Residency {
  int dev = -1, seqs = -1, n = 0;
};

template <typename K>
hipError_t resident(Residency& c, K kernel, int threads, size_t lds, int seqs, int& n) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev != c.dev || seqs != c.seqs) {
    int cus = 0, per_cu = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds);
    if (err != hipSuccess) return err;
    c.dev = dev;
    c.seqs = seqs;
    c.n = cus * (per_cu > 0 ? per_cu : 1);
  }
  n = c.n;
  return hipSuccess;
}

template <int D, bool FP8 = false>
hipError_t launch_streamk(const AttnArgs& a, void* header, hipStream_t st) {
  static thread_local Residency cache, cache_p, cache_a, cache_pa;
  const int entries = a.num_seqs + prefix_items(a.num_seqs, a.prefix_group);
  const bool prefix = a.prefix_keys > 0;
  const bool append = a.new_k != nullptr;
  // P and Ls, then (appending decode) the new token's K row and V column at a
  // 16-byte boundary: 2 * D e4m3 codes, or 2 * D bf16 values
  const size_t lds = append ? (size_t)((2 * entries + 1 + 3) & ~3) * sizeof(int) + (FP8 ? 2 : 4) * D
                            : (size_t)(2 * entries + 1) * sizeof(int);
  int waves = 0;
  hipError_t err =
      prefix && append
          ? resident(cache_pa, decode_streamk_kernel<D, FP8, true, true>, 64, lds, entries, waves)
      : prefix ? resident(cache_p, decode_streamk_kernel<D, FP8, true>, 64, lds, entries, waves)
      : append ? resident(cache_a, decode_streamk_kernel<D, FP8, false, true>, 64, lds, entries, waves)
               : resident(cache, decode_streamk_kernel<D, FP8>, 64, lds, entries, waves);
  if (err != hipSuccess) return err;
  StreamKHeader* hdr = static_cast<StreamKHeader*>(header);
  if (prefix && append) decode_streamk_kernel<D, FP8, true, true><<<waves, 64, lds, st>>>(a, waves, hdr);
  else if (prefix) decode_streamk_kernel<D, FP8, true><<<waves, 64, lds, st>>>(a, waves, hdr);
  else if (append) decode_streamk_kernel<D, FP8, false, true><<<waves, 64, lds, st>>>(a, waves, hdr);
  else decode_streamk_kernel<D, FP8><<<waves, 64, lds, st>>>(a, waves, hdr);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  merge_streamk_kernel<2, D><<<dim3((a.num_q_heads + 3) / 4, a.num_seqs), 256, 0, st>>>(a, hdr);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill(const AttnArgs& a, hipStream_t st) {
  static thread_local Residency cache;
  const size_t lds = (size_t)(a.num_seqs + 1) * sizeof(int);
  int n = 0;
  hipError_t err =
      resident(cache, prefill_kernel<D>, 64 * PrefillShape<D>::kWaves, lds, a.num_seqs, n);
  if (err != hipSuccess) return err;
  n = n >= 8 ? n / 8 * 8 : 8;  // the item walk deals runs of items to the 8 XCDs
  prefill_kernel<D><<<n, 64 * PrefillShape<D>::kWaves, lds, st>>>(a, n);
  return hipGetLastError();
}

// Chunk units and decode rows together (chunk_mix_kernel), then the merges.
template <int D>
hipError_t launch_mix(const AttnArgs& a, void* header, hipStream_t st) {
  static thread_local Residency cache;
  const size_t lds = (size_t)(3 * a.num_seqs + 2) * sizeof(int);
  int n = 0;
  hipError_t err =
      resident(cache, chunk_mix_kernel<D>, 64 * PrefillShape<D>::kWaves, lds, a.num_seqs, n);
  if (err != hipSuccess) return err;
  n = n >= 16 ? n / 8 * 8 : 16;  // both kinds of work get whole multiples of 8
  StreamKHeader* hdr = static_cast<StreamKHeader*>(header);
  chunk_mix_kernel<D><<<n, 64 * PrefillShape<D>::kWaves, lds, st>>>(a, n, hdr);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  merge_streamk_kernel<2, D><<<dim3((a.num_q_heads + 3) / 4, a.num_seqs), 256, 0, st>>>(a, hdr);
  return hipGetLastError();
}

// The e4m3 call's chunk units (staged pools) and decode rows in one launch.
template <int D>
hipError_t launch_mix_fp8(const AttnArgs& dec, const AttnArgs& chunk, void* header,
                          hipStream_t st) {
  static thread_local Residency cache;
  const size_t lds = (size_t)(3 * dec.num_seqs + 2) * sizeof(int);
  int n = 0;
  hipError_t err = resident(cache, chunk_mix_fp8_kernel<D>, 64 * PrefillShape<D>::kWaves, lds,
                            dec.num_seqs, n);
  if (err != hipSuccess) return err;
  n = n >= 16 ? n / 8 * 8 : 16;  // both kinds of work get whole multiples of 8
  StreamKHeader* hdr = static_cast<StreamKHeader*>(header);
  chunk_mix_fp8_kernel<D><<<n, 64 * PrefillShape<D>::kWaves, lds, st>>>(dec, chunk, n, hdr);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  merge_streamk_kernel<2, D><<<dim3((dec.num_q_heads + 3) / 4, dec.num_seqs), 256, 0, st>>>(dec, hdr);
  return hipGetLastError();
}

template <int ES, int D>
hipError_t launch_merge(const AttnArgs& a, int skip_single, hipStream_t st) {
  merge_kernel<ES, D><<<dim3((a.num_q_heads + 3) / 4, a.num_tokens), 256, 0, st>>>(a, skip_single);
  return hipGetLastError();
}

template <int D>
hipError_t launch_mfma(const AttnArgs& a, bool has_chunks, void* header, hipStream_t st) {
  hipError_t err;
  if (has_chunks) {
    // Query chunks on the persistent chunk kernel, single-token rows on the
    // balanced decode -- both in one launch when the prefix sums fit next to
    // the LDS ring -- then the merge of split chunk rows.
    if (a.max_query_len > 1 && a.num_seqs <= kMaxMixSeqs) {
      err = launch_mix<D>(a, header, st);
    } else {
      if (a.max_query_len > 1) {
        err = launch_prefill<D>(a, st);
        if (err != hipSuccess) return err;
      }
      err = launch_streamk<D>(a, header, st);
    }
    if (err != hipSuccess) return err;
    return a.max_splits > 1 ? launch_merge<2, D>(a, 1, st) : hipSuccess;
  }
  const int G = a.num_q_heads / a.num_kv_heads;
  const unsigned z = (unsigned)a.num_seqs * a.num_kv_heads;
  const unsigned narrow_tiles = (unsigned)((G + 15) / 16);
  attn_mfma_kernel<D><<<dim3(z, narrow_tiles, a.max_splits), 64, 0, st>>>(a);
  err = hipGetLastError();
  if (err != hipSuccess) return err;
  return a.max_splits > 1 ? launch_merge<2, D>(a, 0, st) : hipSuccess;
}

template <int ES, int D>
hipError_t launch_valu(const AttnArgs& a, hipStream_t st) {
  const unsigned z = (unsigned)a.num_seqs * a.num_kv_heads;
  attn_valu_kernel<ES, D><<<dim3(z, a.max_query_len, a.max_splits), 64, 0, st>>>(a);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return a.max_splits > 1 ? launch_merge<ES, D>(a, 0, st) : hipSuccess;
}

// ---------------------------------------------------------------------------
// Query chunks over an e4m3 cache.  Chunked prefill is bound by the matrix
// cores and the chunk kernel by its vector work per score, so widening codes
// inside it would cost more than one pass over the context: the blocks of
// every multi-token sequence are first staged as bf16 (value(code) * scale,
// rounded to nearest even) into a staging pool, and the bf16 chunk kernel
// runs on that pool.  Single-token rows read the e4m3 pools directly through
// the e4m3 balanced decode, in the same launch as the chunk units
// (chunk_mix_fp8_kernel) up to kMaxMixSeqs sequences, else after them.
// ---------------------------------------------------------------------------

// Staged blocks of sequence s: nblk(s) = its table blocks when it has more
// than one query row, else 0.  off[s] = sum of nblk over sequences before s,
// off[S] = the total.  One workgroup of 256 threads.
__global__ __launch_bounds__(256) void stage_offsets_kernel(AttnArgs a, int32_t* __restrict__ off) {
  __shared__ int part[256];
  const int S = a.num_seqs;
  const int tid = threadIdx.x;
  const int per = (S + 255) / 256;
  const int lo = min(tid * per, S), hi = min(lo + per, S);
  auto nblk = [&](int s) {
    int r0, qn;
    seq_rows(a.query_start_loc, s, a.num_tokens, r0, qn);
    return qn > 1 ? table_blocks(a.seq_lens[s], a.log2_block, a.max_blocks) : 0;
  };
  int run = 0;
  for (int s = lo; s < hi; ++s) run += nblk(s);
  part[tid] = run;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int t = 0; t < 256; ++t) {
      const int x = part[t];
      part[t] = acc;
      acc += x;
    }
    off[S] = acc;
  }
  __syncthreads();
  int acc = part[tid];
  for (int s = lo; s < hi; ++s) {
    off[s] = acc;
    acc += nblk(s);
  }
}

// Workgroup b: staging block b, i.e. logical block j = b - off[s] of the
// multi-token sequence s with off[s] <= b < off[s + 1] (workgroups past
// off[S] or past the pool's capacity exit): K and V of every KV head widened
// to bf16 with their scales, and the staging table entry of (s, j).  The
// workgroup of a sequence's last block also fills its table entries past its
// blocks with that block.  The sequence is found by a 256-way search (every
// thread probes one offset per level: one level up to 256 sequences, two up
// to 65,536), and each thread issues its K, V and scale loads together
// before it converts any.
template <int D, int NKV>
__global__ __launch_bounds__(256) void stage_fp8_kernel(AttnArgs a, const int32_t* __restrict__ off,
                                                        int64_t cap, uint16_t* __restrict__ sk,
                                                        uint16_t* __restrict__ sv,
                                                        int32_t* __restrict__ stab) {
  const int64_t bidx = blockIdx.x;
  const int S = a.num_seqs;
  if (bidx >= off[S] || bidx >= cap) return;
  // the last sequence s with off[s] <= b: off is non-decreasing, so the
  // probes at or below b form a prefix; [lo, hi) always holds the answer
  int lo = 0, hi = S;
  while (hi - lo > 1) {
    const int step = (hi - lo + 255) >> 8;
    const int idx = lo + (int)threadIdx.x * step;
    const int cnt = __syncthreads_count(idx < hi && off[idx] <= bidx);  // >= 1: off[lo] <= b
    const int nlo = lo + (cnt - 1) * step;
    hi = min(lo + cnt * step, hi);
    lo = nlo;
  }
  const int s = lo;
  const int j = (int)(bidx - off[s]);
  const int nblk = off[s + 1] - off[s];   // > j: sequence s owns staging block b
  int32_t* trow = stab + (int64_t)s * a.max_blocks;
  if (threadIdx.x == 0) trow[j] = (int32_t)bidx;
  if (j == nblk - 1)
    for (int x = nblk + threadIdx.x; x < a.max_blocks; x += 256) trow[x] = (int32_t)bidx;
  const int phys = clampi(a.block_tables[(int64_t)s * a.max_blocks + j], 0, a.num_blocks - 1);
  const int Hkv = a.num_kv_heads;
  const int64_t tile = (int64_t)D << a.log2_block;  // elements of one (block, KV head) tile
  const int64_t n = Hkv * tile;
  const uint8_t* k8 = static_cast<const uint8_t*>(a.k_cache) + phys * n;
  const uint8_t* v8 = static_cast<const uint8_t*>(a.v_cache) + phys * n;
  const float* ksc = a.k_scales + (int64_t)phys * Hkv;
  const float* vsc = a.v_scales + (int64_t)phys * Hkv;
  uint16_t* k16 = sk + bidx * n;
  uint16_t* v16 = sv + bidx * n;
  // NKV 8-byte pieces per thread and pool cover the block when n == NKV * 256 * 8
  // (8 KV heads of D x B bytes, B * D = 2048); other sizes loop.  Each
  // load and each 16-byte store instruction covers one contiguous run.
  for (int64_t e0 = (int64_t)threadIdx.x * 8; e0 < n; e0 += (int64_t)NKV * 256 * 8) {
    uint2 ck[NKV], cv[NKV];
    float ks[NKV], vs[NKV];
#pragma unroll
    for (int u = 0; u < NKV; ++u) {
      const int64_t e = e0 + (int64_t)u * 256 * 8;
      if (e < n) {
        const int h = (int)(e / tile);  // 8 elements never straddle a tile (tile % 8 == 0)
        // the codes are read once: streamed past the caches (the staged
        // copies are written through them, for the chunk kernel to re-read)
        const uint64_t k64 = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(k8 + e));
        const uint64_t v64 = __builtin_nontemporal_load(reinterpret_cast<const uint64_t*>(v8 + e));
        ck[u] = make_uint2((uint32_t)k64, (uint32_t)(k64 >> 32));
        cv[u] = make_uint2((uint32_t)v64, (uint32_t)(v64 >> 32));
        ks[u] = ksc[h];
        vs[u] = vsc[h];
      }
    }
#pragma unroll
    for (int u = 0; u < NKV; ++u) {
      const int64_t e = e0 + (int64_t)u * 256 * 8;
      if (e >= n) continue;
#pragma unroll
      for (int pool = 0; pool < 2; ++pool) {
        const uint2 c = pool ? cv[u] : ck[u];
        const float sc = pool ? vs[u] : ks[u];
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 2; ++q) {
          const uint32_t cq = q ? c.y : c.x;
          const auto lo2 = __builtin_amdgcn_cvt_pk_f32_fp8(cq, false);
          const auto hi2 = __builtin_amdgcn_cvt_pk_f32_fp8(cq, true);
          w[2 * q] = f32_to_bf16_bits(lo2[0] * sc) | ((uint32_t)f32_to_bf16_bits(lo2[1] * sc) << 16);
          w[2 * q + 1] =
              f32_to_bf16_bits(hi2[0] * sc) | ((uint32_t)f32_to_bf16_bits(hi2[1] * sc) << 16);
        }
        *reinterpret_cast<u32x4*>((pool ? v16 : k16) + e) = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  }
}

template <int D>
hipError_t launch_chunked_fp8_d(const AttnArgs& dec, const AttnArgs& chunk, void* header,
                                int64_t cap, int32_t* off, hipStream_t st) {
  stage_offsets_kernel<<<1, 256, 0, st>>>(dec, off);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  if (dec.max_query_len > 1 && cap > 0) {
    stage_fp8_kernel<D, 8><<<(unsigned)cap, 256, 0, st>>>(
        dec, off, cap, static_cast<uint16_t*>(const_cast<void*>(chunk.k_cache)),
        static_cast<uint16_t*>(const_cast<void*>(chunk.v_cache)),
        const_cast<int32_t*>(chunk.block_tables));
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    // as for a bf16 cache: one launch for both kinds of rows when the
    // prefix sums fit next to the LDS ring
    err = dec.num_seqs <= kMaxMixSeqs ? launch_mix_fp8<D>(dec, chunk, header, st)
                                      : launch_prefill<D>(chunk, st);
    if (err != hipSuccess) return err;
    if (dec.num_seqs > kMaxMixSeqs) err = launch_streamk<D, true>(dec, header, st);
  } else {
    err = launch_streamk<D, true>(dec, header, st);
  }
  if (err != hipSuccess) return err;
  return chunk.max_splits > 1 ? launch_merge<2, D>(chunk, 1, st) : hipSuccess;
}

}  // namespace

hipError_t launch_chunked_fp8(const AttnArgs& dec, const AttnArgs& chunk, void* header,
                              int64_t cap_blocks, int32_t* offsets, hipStream_t stream) {
  return dec.head_dim == 128
             ? launch_chunked_fp8_d<128>(dec, chunk, header, cap_blocks, offsets, stream)
             : launch_chunked_fp8_d<64>(dec, chunk, header, cap_blocks, offsets, stream);
}

hipError_t launch_decode_streamk(const AttnArgs& a, void* header, hipStream_t stream) {
  if (a.kv_fp8)
    return a.head_dim == 128 ? launch_streamk<128, true>(a, header, stream)
                             : launch_streamk<64, true>(a, header, stream);
  return a.head_dim == 128 ? launch_streamk<128>(a, header, stream)
                           : launch_streamk<64>(a, header, stream);
}

bool mfma_path(const AttnArgs& a) {
  return a.bf16 && a.block_size >= 8 && (a.head_dim == 64 || a.head_dim == 128);
}

hipError_t launch_slot_mapping(int64_t* slots, const int32_t* bt, int32_t max_blocks,
                               const int32_t* seq_lens, const int32_t* qsl, int32_t num_seqs,
                               int32_t num_tokens, int32_t block_size, hipStream_t stream) {
  const int lg = __builtin_ctz((unsigned)block_size);
  slot_mapping_kernel<<<num_seqs, 256, 0, stream>>>(slots, bt, max_blocks, seq_lens, qsl,
                                                    num_tokens, lg);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slots, int32_t num_tokens,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                    int32_t num_blocks, int32_t elem_bytes, hipStream_t stream) {
  const int lg = __builtin_ctz((unsigned)block_size);
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const dim3 grid((num_tokens + 15) / 16, num_kv_heads);
#define PA_RC(ES, D)                                                                      \
  reshape_and_cache_kernel<ES, D><<<grid, 16 * D * ES / 16, 0, stream>>>(                 \
      key, value, k_cache, v_cache, slots, num_tokens, num_kv_heads, lg, num_slots)
  if (elem_bytes == 2 && head_dim == 128) PA_RC(2, 128);
  else if (elem_bytes == 2 && head_dim == 64) PA_RC(2, 64);
  else if (elem_bytes == 4 && head_dim == 128) PA_RC(4, 128);
  else PA_RC(4, 64);
#undef PA_RC
  return hipGetLastError();
}

hipError_t launch_append_tokens(const AttnArgs& a, hipStream_t stream) {
  const dim3 grid(a.num_seqs, a.num_kv_heads);
#define PA_AT(ES, D, F8) append_tokens_kernel<ES, D, F8><<<grid, 64, 0, stream>>>(a)
  if (a.kv_fp8) {
    if (a.head_dim == 128) PA_AT(2, 128, true);
    else PA_AT(2, 64, true);
  } else if (a.bf16) {
    if (a.head_dim == 128) PA_AT(2, 128, false);
    else PA_AT(2, 64, false);
  } else {
    if (a.head_dim == 128) PA_AT(4, 128, false);
    else PA_AT(4, 64, false);
  }
#undef PA_AT
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* dst, const void* src, const int64_t* mapping,
                              int32_t num_pairs, int64_t block_bytes, int64_t src_num_blocks,
                              int64_t dst_num_blocks, hipStream_t stream) {
  const bool v16 = block_bytes % 16 == 0 && reinterpret_cast<uintptr_t>(dst) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(src) % 16 == 0;
  const int64_t elems = block_bytes / (v16 ? 16 : 4);
  const unsigned gx = (unsigned)std::min<int64_t>((elems + 255) / 256, 64);
  const unsigned gy = (unsigned)std::min<int32_t>(num_pairs, 65535);
  uint8_t* d = static_cast<uint8_t*>(dst);
  const uint8_t* s = static_cast<const uint8_t*>(src);
  if (v16)
    copy_blocks_kernel<u32x4><<<dim3(gx, gy), 256, 0, stream>>>(d, s, mapping, num_pairs,
                                                               block_bytes, src_num_blocks,
                                                               dst_num_blocks);
  else
    copy_blocks_kernel<uint32_t><<<dim3(gx, gy), 256, 0, stream>>>(d, s, mapping, num_pairs,
                                                                  block_bytes, src_num_blocks,
                                                                  dst_num_blocks);
  return hipGetLastError();
}

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                        void* v_cache, const float* k_scales,
                                        const float* v_scales, const int64_t* slots,
                                        int32_t num_tokens, int32_t num_kv_heads,
                                        int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        hipStream_t stream) {
  const int lg = __builtin_ctz((unsigned)block_size);
  const int64_t num_slots = (int64_t)num_blocks * block_size;
  const dim3 grid((num_tokens + 15) / 16, num_kv_heads);
  const uint16_t* k = static_cast<const uint16_t*>(key);
  const uint16_t* v = static_cast<const uint16_t*>(value);
  uint8_t* kc = static_cast<uint8_t*>(k_cache);
  uint8_t* vc = static_cast<uint8_t*>(v_cache);
  if (head_dim == 128)
    reshape_and_cache_fp8_kernel<128><<<grid, 256, 0, stream>>>(
        k, v, kc, vc, k_scales, v_scales, slots, num_tokens, num_kv_heads, lg, num_slots);
  else
    reshape_and_cache_fp8_kernel<64><<<grid, 128, 0, stream>>>(
        k, v, kc, vc, k_scales, v_scales, slots, num_tokens, num_kv_heads, lg, num_slots);
  return hipGetLastError();
}

hipError_t launch_attention(const AttnArgs& a, bool has_chunks, void* header,
                            hipStream_t stream) {
  if (mfma_path(a)) {
    return a.head_dim == 128 ? launch_mfma<128>(a, has_chunks, header, stream)
                             : launch_mfma<64>(a, has_chunks, header, stream);
  }
  if (a.bf16)
    return a.head_dim == 128 ? launch_valu<2, 128>(a, stream) : launch_valu<2, 64>(a, stream);
  return a.head_dim == 128 ? launch_valu<4, 128>(a, stream) : launch_valu<4, 64>(a, stream);
}

}  // namespace pa
