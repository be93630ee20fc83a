// libpa_probe: measurement probes for bench.py, not part of libpa's ABI.
//
// pa_probe_read_tiles reads whole tiles of a device pool in a random order
// (the tile ids are a permutation the caller draws) with the same access
// the paged decode makes: 16-byte non-temporal loads, each tile read by one
// wave, several tiles in flight per wave, one wave per SIMD or more.  Its
// bytes / time is the read ceiling that pool gathers of that tile size can
// reach on the device -- the second denominator bench.py reports beside the
// nominal HBM peak.  Every load stays inside the pool: tile ids are taken
// modulo the number of tiles, and each lane reads offsets below tile_bytes.
//
// pa_probe_read_rows reads the same kind of tiles (4 KiB) in the layout of an
// MFMA A operand, 64 bytes of each of 16 rows per load, as the decode reads
// K: the L1 then sends 64-byte requests instead of whole 128-byte lines.
//
// pa_probe_mfma issues v_mfma_f32_32x32x16_bf16 back to back (four
// independent accumulators per wave, two waves per SIMD), the instruction
// the chunked-prefill kernel runs on.  Its flops / time is the matrix-core
// rate the device sustains, the second denominator beside the 2.5 PFLOP/s
// dense bf16 peak.  It touches no memory but one sink word per thread.
//
// pa_probe_overlap times bursts of matrix work (8 MFMAs) and of vector work
// (16 exponentials and 32 fmas per lane, the mix of a softmax step) on every
// SIMD, one workgroup per CU: in separate launches, one after the other in
// each wave, interleaved one MFMA to ten vector instructions in each wave,
// or split between waves (half the waves of a workgroup do only one kind).
// How much the two kinds overlap bounds any kernel that issues both from
// the same waves, as the chunked-prefill kernel does.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWaveLanes = 64;
constexpr int kTilesInFlight = 4;

template <int TILE_BYTES>
__global__ __launch_bounds__(256) void read_tiles_kernel(const u32x4* __restrict__ pool,
                                                         const int32_t* __restrict__ tile_ids,
                                                         int32_t num_ids, int32_t num_tiles,
                                                         uint32_t* __restrict__ sink) {
  constexpr int kVecPerTile = TILE_BYTES / 16;
  constexpr int kPerLane = kVecPerTile / kWaveLanes;
  const int lane = threadIdx.x & (kWaveLanes - 1);
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWaveLanes;
  const int num_waves = gridDim.x * blockDim.x / kWaveLanes;
  uint32_t acc = 0;
  for (int t0 = wave * kTilesInFlight; t0 < num_ids; t0 += num_waves * kTilesInFlight) {
    u32x4 v[kTilesInFlight][kPerLane];
#pragma unroll
    for (int u = 0; u < kTilesInFlight; ++u) {
      const int t = t0 + u;
      const int id = t < num_ids ? (int)((uint32_t)tile_ids[t] % (uint32_t)num_tiles) : -1;
      const u32x4* base = pool + (int64_t)(id < 0 ? 0 : id) * kVecPerTile + lane;
#pragma unroll
      for (int k = 0; k < kPerLane; ++k)
        v[u][k] = id >= 0 ? __builtin_nontemporal_load(base + k * kWaveLanes)
                          : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kTilesInFlight; ++u)
#pragma unroll
      for (int k = 0; k < kPerLane; ++k) acc ^= v[u][k].x ^ v[u][k].y ^ v[u][k].z ^ v[u][k].w;
  }
  sink[wave * kWaveLanes + lane] = acc;
}

// The same random 4 KiB tiles (16 rows of 256 bytes, a bf16 K tile of one
// block and KV head) read in the layout of an MFMA A operand: load k gives
// lane (i, j) = (l % 16, l / 16) bytes 64k + 16j .. +15 of row i, so every
// load reads 64 bytes of each of 16 rows (the decode's K loads).
__global__ __launch_bounds__(256) void read_rows_kernel(const char* __restrict__ pool,
                                                        const int32_t* __restrict__ tile_ids,
                                                        int32_t num_ids, int32_t num_tiles,
                                                        uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & (kWaveLanes - 1);
  const int wave = (blockIdx.x * blockDim.x + threadIdx.x) / kWaveLanes;
  const int num_waves = gridDim.x * blockDim.x / kWaveLanes;
  const int off = (lane & 15) * 256 + (lane >> 4) * 16;
  uint32_t acc = 0;
  for (int t0 = wave * kTilesInFlight; t0 < num_ids; t0 += num_waves * kTilesInFlight) {
    u32x4 v[kTilesInFlight][4];
#pragma unroll
    for (int u = 0; u < kTilesInFlight; ++u) {
      const int t = t0 + u;
      const int id = t < num_ids ? (int)((uint32_t)tile_ids[t] % (uint32_t)num_tiles) : -1;
      const char* base = pool + (int64_t)(id < 0 ? 0 : id) * 4096 + off;
#pragma unroll
      for (int k = 0; k < 4; ++k)
        v[u][k] = id >= 0 ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + 64 * k))
                          : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kTilesInFlight; ++u)
#pragma unroll
      for (int k = 0; k < 4; ++k) acc ^= v[u][k].x ^ v[u][k].y ^ v[u][k].z ^ v[u][k].w;
  }
  sink[wave * kWaveLanes + lane] = acc;
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
constexpr int kMfmaChains = 4;

__global__ __launch_bounds__(256) void mfma_kernel(int32_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & (kWaveLanes - 1);
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<__bf16>(0.001f * (float)(lane + e));
    b[e] = static_cast<__bf16>(0.002f * (float)(lane - e));
  }
  f32x16 acc[kMfmaChains];
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k) acc[k] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < kMfmaChains; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < kMfmaChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) t += acc[k][r];
  sink[(int64_t)blockIdx.x * blockDim.x + threadIdx.x] = t;
}

struct OverlapState {
  f32x16 c[4];
  float x[16];
  bf16x8 a, b;
};

__device__ __forceinline__ void matrix_burst(OverlapState& s) {
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) s.c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(s.a, s.b, s.c[j], 0, 0, 0);
}

// EXP: the softmax-like mix (16 exponentials and 32 fmas per lane); without
// it, 48 fmas.
template <bool EXP>
__device__ __forceinline__ void vector_burst(OverlapState& s) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float y = EXP ? __builtin_amdgcn_exp2f(__builtin_fmaf(s.x[i], 0.5f, -0.25f))
                        : __builtin_fmaf(s.x[i], 0.5f, -0.25f);
    s.x[i] = __builtin_fmaf(y, 0.999f, -s.x[i] * 1e-3f);
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) s.x[i] = __builtin_fmaf(s.x[i], 1.0001f, 1e-7f);
}

// MODE 0: matrix bursts only; 1: vector bursts only; 2: both in every wave,
// one after the other; 3: both in every wave, interleaved one MFMA to ten
// vector instructions; 4: waves 0-3 matrix only, waves 4-7 vector only;
// 5: even waves matrix only, odd waves vector only.  (Which waves share a
// SIMD is the hardware's choice; modes 4 and 5 pair them two ways.)
template <int MODE, bool EXP>
__global__ void overlap_kernel(int32_t iters, float* __restrict__ sink) {
  extern __shared__ float pad[];  // sized by the host: one workgroup per CU
  const int tid = blockIdx.x * blockDim.x + threadIdx.x;
  const int wave = threadIdx.x >> 6;
  OverlapState s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    s.a[e] = static_cast<__bf16>(0.001f * (float)(tid & 255) + (float)e);
    s.b[e] = static_cast<__bf16>(0.5f * (float)e);
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) s.c[j] = f32x16{};
#pragma unroll
  for (int i = 0; i < 16; ++i) s.x[i] = 1e-6f * (float)(tid & 1023) + 1e-3f * (float)i;
  for (int it = 0; it < iters; ++it) {
    if constexpr (MODE == 0) matrix_burst(s);
    if constexpr (MODE == 1) vector_burst<EXP>(s);
    if constexpr (MODE == 2) {
      matrix_burst(s);
      __builtin_amdgcn_sched_barrier(0);
      vector_burst<EXP>(s);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE == 3) {
      matrix_burst(s);
      vector_burst<EXP>(s);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // ten vector instructions
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (MODE == 4) {
      if (wave < 4) matrix_burst(s);
      else vector_burst<EXP>(s);
    }
    if constexpr (MODE == 5) {
      if ((wave & 1) == 0) matrix_burst(s);
      else vector_burst<EXP>(s);
    }
  }
  if (threadIdx.x > 1u << 20) pad[0] = 0.f;  // never: keeps the LDS request
  float t = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) t += s.c[0][r] + s.c[1][r] + s.c[2][r] + s.c[3][r] + s.x[r];
  sink[tid] = t;
}

template <int MODE, bool EXP>
hipError_t launch_overlap(int32_t num_wgs, int32_t threads, int32_t iters, float* sink,
                          hipStream_t st) {
  const size_t lds = 96 * 1024;  // more than half a CU's LDS: one workgroup per CU
  (void)hipFuncSetAttribute(reinterpret_cast<const void*>(&overlap_kernel<MODE, EXP>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  hipLaunchKernelGGL((overlap_kernel<MODE, EXP>), dim3(num_wgs), dim3(threads), lds, st, iters,
                     sink);
  return hipGetLastError();
}

template <bool EXP>
hipError_t launch_overlap_mode(int32_t mode, int32_t num_wgs, int32_t threads, int32_t iters,
                               float* sink, hipStream_t st) {
  switch (mode) {
    case 0: return launch_overlap<0, EXP>(num_wgs, threads, iters, sink, st);
    case 1: return launch_overlap<1, EXP>(num_wgs, threads, iters, sink, st);
    case 2: return launch_overlap<2, EXP>(num_wgs, threads, iters, sink, st);
    case 3: return launch_overlap<3, EXP>(num_wgs, threads, iters, sink, st);
    case 4: return launch_overlap<4, EXP>(num_wgs, threads, iters, sink, st);
    default: return launch_overlap<5, EXP>(num_wgs, threads, iters, sink, st);
  }
}

template <int TILE_BYTES>
hipError_t launch(const void* pool, const int32_t* ids, int32_t num_ids, int32_t num_tiles,
                  uint32_t* sink, int32_t num_waves, hipStream_t st) {
  hipLaunchKernelGGL(read_tiles_kernel<TILE_BYTES>, dim3(num_waves / 4), dim3(256), 0, st,
                     static_cast<const u32x4*>(pool), ids, num_ids, num_tiles, sink);
  return hipGetLastError();
}

}  // namespace

// Reads num_ids tiles of tile_bytes (1, 2, 4, 8 or 16 KiB) from `pool`
// (pool_bytes long, 16-byte aligned), tile tile_ids[i] % (pool_bytes /
// tile_bytes) for each i, with num_waves waves (a positive multiple of 4);
// `sink` receives one word per lane (uint32 [num_waves * 64]).  Returns 0,
// -2 for bad sizes, -7 when the launch fails.
extern "C" int pa_probe_read_tiles(const void* pool, int64_t pool_bytes, const int32_t* tile_ids,
                                   int32_t num_ids, int32_t tile_bytes, uint32_t* sink,
                                   int32_t num_waves, void* stream) {
  if (!pool || !tile_ids || !sink || num_ids <= 0 || num_waves <= 0 || num_waves % 4 != 0)
    return -2;
  if (tile_bytes <= 0 || pool_bytes < tile_bytes || pool_bytes / tile_bytes > INT32_MAX) return -2;
  const int32_t num_tiles = (int32_t)(pool_bytes / tile_bytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (tile_bytes) {
    case 1024: e = launch<1024>(pool, tile_ids, num_ids, num_tiles, sink, num_waves, st); break;
    case 2048: e = launch<2048>(pool, tile_ids, num_ids, num_tiles, sink, num_waves, st); break;
    case 4096: e = launch<4096>(pool, tile_ids, num_ids, num_tiles, sink, num_waves, st); break;
    case 8192: e = launch<8192>(pool, tile_ids, num_ids, num_tiles, sink, num_waves, st); break;
    case 16384: e = launch<16384>(pool, tile_ids, num_ids, num_tiles, sink, num_waves, st); break;
    default: return -2;
  }
  return e == hipSuccess ? 0 : -7;
}

// pa_probe_read_tiles with 4 KiB tiles, read in the MFMA A-operand layout
// (read_rows_kernel: 64 bytes of each of 16 rows per load instead of 1 KiB
// contiguous).  Same arguments and returns, without tile_bytes.
extern "C" int pa_probe_read_rows(const void* pool, int64_t pool_bytes, const int32_t* tile_ids,
                                  int32_t num_ids, uint32_t* sink, int32_t num_waves,
                                  void* stream) {
  if (!pool || !tile_ids || !sink || num_ids <= 0 || num_waves <= 0 || num_waves % 4 != 0)
    return -2;
  if (pool_bytes < 4096 || pool_bytes / 4096 > INT32_MAX) return -2;
  hipLaunchKernelGGL(read_rows_kernel, dim3(num_waves / 4), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const char*>(pool), tile_ids,
                     num_ids, (int32_t)(pool_bytes / 4096), sink);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// Runs num_wgs workgroups of 256 threads, each wave issuing iters x 4
// v_mfma_f32_32x32x16_bf16 (32 x 32 x 16 multiply-adds each); `sink`
// receives one float per thread (float [num_wgs * 256]).  Returns 0, -2 for
// bad sizes, -7 when the launch fails.
extern "C" int pa_probe_mfma(float* sink, int32_t num_wgs, int32_t iters, void* stream) {
  if (!sink || num_wgs <= 0 || iters <= 0) return -2;
  hipLaunchKernelGGL(mfma_kernel, dim3(num_wgs), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -7;
}

// One overlap run: num_wgs workgroups (one per CU) of waves_per_simd * 4
// waves, each wave running `iters` bursts of the kind `mode` selects (0-5,
// see overlap_kernel; modes 4 and 5 need two waves per SIMD), with the
// softmax-like vector mix when `exp_mix` is non-zero, else fmas only.
// `sink` receives one float per thread (float [num_wgs * waves_per_simd *
// 256]).  Returns 0, -2 for bad arguments, -7 when the launch fails.
extern "C" int pa_probe_overlap(float* sink, int32_t mode, int32_t exp_mix, int32_t num_wgs,
                                int32_t waves_per_simd, int32_t iters, void* stream) {
  if (!sink || num_wgs <= 0 || iters <= 0 || (waves_per_simd != 1 && waves_per_simd != 2) ||
      mode < 0 || mode > 5 || (mode >= 4 && waves_per_simd != 2))
    return -2;
  const int threads = 256 * waves_per_simd;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const hipError_t e = exp_mix ? launch_overlap_mode<true>(mode, num_wgs, threads, iters, sink, st)
                               : launch_overlap_mode<false>(mode, num_wgs, threads, iters, sink, st);
  return e == hipSuccess ? 0 : -7;
}
