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
//   slot_mapping_kernel       slot of every query token (index equations)
//   reshape_and_cache_kernel  bit copy of new K/V into their slots
//   attn_mfma_kernel<D, R>    bf16 split-K attention; QK^T and PV on
//                             v_mfma_f32_16x16x32_bf16, online softmax in
//                             fp32 with cross-lane max/sum
//   attn_valu_kernel<ES, D>   fp32 (and small-block bf16) split-K attention
//                             on the vector ALUs
//   merge_kernel<ES, D>       exact log-sum-exp merge of split partials
//
// Cache layout: K [NB, Hkv, B, D] (token rows), V [NB, Hkv, D, B] (each
// head_dim row holds the block's tokens).  The V layout lets one 16-byte
// load fetch 8 consecutive tokens of one head_dim column, which is exactly
// what the PV MFMA's B operand holds per lane.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
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
template <int D, int R>
__global__ __launch_bounds__(64) void attn_mfma_kernel(AttnArgs a, int filter) {
  constexpr int KK = D / 32;  // QK k-steps
  constexpr int NT = D / 16;  // PV head_dim tiles
  const int lane = threadIdx.x;
  const int i = lane & 15;
  const int j4 = lane >> 4;
  const int split = blockIdx.x;
  const int tg = blockIdx.y;
  const int s = blockIdx.z / a.num_kv_heads;
  const int kvh = blockIdx.z - s * a.num_kv_heads;
  const int T = a.num_tokens;

  int r0, qn;
  seq_rows(a.query_start_loc, s, T, r0, qn);
  if (filter == kMultiRowSeqs && qn <= 1) return;
  if (filter == kSingleRowSeqs && qn != 1) return;
  const int G = a.num_q_heads / a.num_kv_heads;
  const int nrows = qn * G;
  const int row0 = tg * 16 * R;
  if (row0 >= nrows) return;
  const int L = a.seq_lens[s];
  const int lg = a.log2_block;
  const int B = 1 << lg;
  const int nblk = table_blocks(L, lg, a.max_blocks);
  const int kcap = nblk << lg;
  const int row_last = min(row0 + 16 * R, nrows) - 1;
  const int kv_wave = min(L - qn + row_last / G + 1, kcap);
  const int k_begin = split * a.split_tokens;
  if (k_begin >= kv_wave) return;
  const int k_end = min(k_begin + a.split_tokens, kv_wave);

  // Block ids of this split, one logical block per lane (the split spans at
  // most 64 blocks); clamped so that any table value stays inside the pool.
  const int blk0 = k_begin >> lg;
  int wid = a.block_tables[(int64_t)s * a.max_blocks + min(blk0 + lane, nblk - 1)];
  wid = clampi(wid, 0, a.num_blocks - 1);

  const int Hq = a.num_q_heads;
  const uint16_t* q = static_cast<const uint16_t*>(a.q);
  int klim[R];
  bf16x8 qf[R][KK];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    const int row = row0 + 16 * t + i;
    klim[t] = 0;
    if (row < nrows) {
      const int j = row / G;
      const int g = row - j * G;
      klim[t] = min(L - qn + j + 1, kcap);
      const uint16_t* qp = q + ((int64_t)(r0 + j) * Hq + kvh * G + g) * D + 8 * j4;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[t][kk] = load_bf16x8(qp + 32 * kk);
    } else {
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) qf[t][kk] = bf16x8{};
    }
  }

  float m[R], l[R];
  f32x4 o[R][NT];
#pragma unroll
  for (int t = 0; t < R; ++t) {
    m[t] = neg_inf();
    l[t] = 0.f;
#pragma unroll
    for (int n = 0; n < NT; ++n) o[t][n] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int64_t blk_stride = (int64_t)a.num_kv_heads * B * D;
  const uint16_t* kbase = static_cast<const uint16_t*>(a.k_cache) + (int64_t)kvh * B * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(a.v_cache) + (int64_t)kvh * D * B;
  const int tok_a = 8 * (i >> 2) + (i & 3);
  const float sl2 = a.scale_log2;

  for (int c = k_begin; c < k_end; c += 32) {
    const int pa_ = c + tok_a;
    const int pb_ = pa_ + 4;
    const int pv_ = c + 8 * j4;
    const int ia = __shfl(wid, min(pa_ >> lg, nblk - 1) - blk0);
    const int ib = __shfl(wid, min(pb_ >> lg, nblk - 1) - blk0);
    const int iv = __shfl(wid, min(pv_ >> lg, nblk - 1) - blk0);
    const uint16_t* ka = kbase + ia * blk_stride + (pa_ & (B - 1)) * D + 8 * j4;
    const uint16_t* kb = kbase + ib * blk_stride + (pb_ & (B - 1)) * D + 8 * j4;
    const uint16_t* vp = vbase + iv * blk_stride + (int64_t)i * B + (pv_ & (B - 1));
    bf16x8 kfa[KK], kfb[KK], vf[NT];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      kfa[kk] = load_bf16x8(ka + 32 * kk);
      kfb[kk] = load_bf16x8(kb + 32 * kk);
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) vf[n] = load_bf16x8(vp + (int64_t)16 * n * B);
    if (c + 32 > kv_wave) {
      // Keys past the last visible one may be unwritten slots: zero their V
      // so that 0-weight * garbage cannot produce NaN.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (pv_ + e >= kv_wave) {
#pragma unroll
          for (int n = 0; n < NT; ++n) vf[n][e] = static_cast<__bf16>(0.f);
        }
      }
    }

#pragma unroll
    for (int t = 0; t < R; ++t) {
      f32x4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfa[kk], qf[t][kk], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfb[kk], qf[t][kk], sb, 0, 0, 0);
      }
      float sv[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        sv[r] = sa[r];
        sv[4 + r] = sb[r];
      }
      float mx = neg_inf();
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sv[e] = (pv_ + e < klim[t]) ? sv[e] * sl2 : neg_inf();
        mx = fmaxf(mx, sv[e]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[t], mx);
      const float muse = (mnew == neg_inf()) ? 0.f : mnew;
      const float alpha = fast_exp2(m[t] - muse);
      float ps = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        sv[e] = fast_exp2(sv[e] - muse);
        ps += sv[e];
      }
      ps += __shfl_xor(ps, 16);
      ps += __shfl_xor(ps, 32);
      l[t] = l[t] * alpha + ps;
      m[t] = mnew;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * j4 + r);
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 8; ++e) pf[e] = static_cast<__bf16>(sv[e]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
#pragma unroll
        for (int r = 0; r < 4; ++r) o[t][n][r] *= ar[r];
        o[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf, vf[n], o[t][n], 0, 0, 0);
      }
    }
  }

  // Lane l holds output rows 4*(l/16)+r, head_dim columns 16*n + l%16.
  const int ST = a.split_tokens;
  uint16_t* out = static_cast<uint16_t*>(a.out);
#pragma unroll
  for (int t = 0; t < R; ++t) {
    float lr[4], mr[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      lr[r] = __shfl(l[t], 4 * j4 + r);
      mr[r] = __shfl(m[t], 4 * j4 + r);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = row0 + 16 * t + 4 * j4 + r;
      if (row >= nrows) continue;
      const int j = row / G;
      const int g = row - j * G;
      const int kl = min(L - qn + j + 1, kcap);
      if (kl <= k_begin) continue;
      const int ns = min((kl + ST - 1) / ST, a.max_splits);
      const int64_t orow = (int64_t)(r0 + j) * Hq + kvh * G + g;
      if (ns == 1) {
        const float inv = 1.f / lr[r];
#pragma unroll
        for (int n = 0; n < NT; ++n) out[orow * D + 16 * n + i] = f32_to_bf16_bits(o[t][n][r] * inv);
      } else {
        const int64_t pidx = orow * a.max_splits + split;
        float* po = a.part_o + pidx * D;
#pragma unroll
        for (int n = 0; n < NT; ++n) po[16 * n + i] = o[t][n][r];
        if (i == 0) {
          a.part_ml[2 * pidx] = mr[r];
          a.part_ml[2 * pidx + 1] = lr[r];
        }
      }
    }
  }
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
  const int split = blockIdx.x;
  const int j = blockIdx.y;
  const int s = blockIdx.z / a.num_kv_heads;
  const int kvh = blockIdx.z - s * a.num_kv_heads;
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
// One workgroup per query token; each wave takes every fourth head.
// ---------------------------------------------------------------------------
template <int ES, int D>
__global__ __launch_bounds__(256) void merge_kernel(AttnArgs a) {
  constexpr int DD = D / 64;
  const int j = blockIdx.x;
  const int s = blockIdx.y;
  int r0, qn;
  seq_rows(a.query_start_loc, s, a.num_tokens, r0, qn);
  if (j >= qn) return;
  const int L = a.seq_lens[s];
  const int nblk = table_blocks(L, a.log2_block, a.max_blocks);
  const int kl = min(L - qn + j + 1, nblk << a.log2_block);
  if (kl <= 0) return;
  const int ns = min((kl + a.split_tokens - 1) / a.split_tokens, a.max_splits);
  if (ns <= 1) return;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  for (int h = wave; h < a.num_q_heads; h += 4) {
    const int64_t orow = (int64_t)(r0 + j) * a.num_q_heads + h;
    const float* ml = a.part_ml + orow * a.max_splits * 2;
    float M = neg_inf();
    for (int sp = 0; sp < ns; ++sp) M = fmaxf(M, ml[2 * sp]);
    float acc[DD];
#pragma unroll
    for (int dd = 0; dd < DD; ++dd) acc[dd] = 0.f;
    float den = 0.f;
    for (int sp = 0; sp < ns; ++sp) {
      const float w = fast_exp2(ml[2 * sp] - M);
      den += w * ml[2 * sp + 1];
      const float* po = a.part_o + (orow * a.max_splits + sp) * D;
#pragma unroll
      for (int dd = 0; dd < DD; ++dd) acc[dd] += w * po[lane + 64 * dd];
    }
    const float inv = 1.f / den;
#pragma unroll
    for (int dd = 0; dd < DD; ++dd) store_elem<ES>(a.out, orow * D + lane + 64 * dd, acc[dd] * inv);
  }
}

template <int D>
hipError_t launch_mfma(const AttnArgs& a, bool has_chunks, hipStream_t st) {
  const int G = a.num_q_heads / a.num_kv_heads;
  const unsigned z = (unsigned)a.num_seqs * a.num_kv_heads;
  const unsigned narrow_tiles = (unsigned)((G + 15) / 16);
  if (has_chunks) {
    constexpr int R = 4;
    const unsigned tiles = (unsigned)(((int64_t)a.max_query_len * G + 16 * R - 1) / (16 * R));
    attn_mfma_kernel<D, R><<<dim3(a.max_splits, tiles, z), 64, 0, st>>>(a, kMultiRowSeqs);
    attn_mfma_kernel<D, 1><<<dim3(a.max_splits, narrow_tiles, z), 64, 0, st>>>(a, kSingleRowSeqs);
  } else {
    attn_mfma_kernel<D, 1><<<dim3(a.max_splits, narrow_tiles, z), 64, 0, st>>>(a, kAllSeqs);
  }
  return hipGetLastError();
}

template <int ES, int D>
hipError_t launch_valu(const AttnArgs& a, hipStream_t st) {
  const unsigned z = (unsigned)a.num_seqs * a.num_kv_heads;
  attn_valu_kernel<ES, D><<<dim3(a.max_splits, a.max_query_len, z), 64, 0, st>>>(a);
  return hipGetLastError();
}

template <int ES, int D>
hipError_t launch_merge(const AttnArgs& a, hipStream_t st) {
  merge_kernel<ES, D><<<dim3(a.max_query_len, a.num_seqs), 256, 0, st>>>(a);
  return hipGetLastError();
}

}  // namespace

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

hipError_t launch_attention(const AttnArgs& a, bool has_chunks, hipStream_t stream) {
  hipError_t err;
  const bool mfma = mfma_path(a);
  if (mfma) {
    err = a.head_dim == 128 ? launch_mfma<128>(a, has_chunks, stream)
                            : launch_mfma<64>(a, has_chunks, stream);
  } else if (a.bf16) {
    err = a.head_dim == 128 ? launch_valu<2, 128>(a, stream) : launch_valu<2, 64>(a, stream);
  } else {
    err = a.head_dim == 128 ? launch_valu<4, 128>(a, stream) : launch_valu<4, 64>(a, stream);
  }
  if (err != hipSuccess) return err;
  if (a.max_splits > 1) {
    if (a.bf16)
      err = a.head_dim == 128 ? launch_merge<2, 128>(a, stream) : launch_merge<2, 64>(a, stream);
    else
      err = a.head_dim == 128 ? launch_merge<4, 128>(a, stream) : launch_merge<4, 64>(a, stream);
  }
  return err;
}

}  // namespace pa
