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
// pa_probe_mfma issues v_mfma_f32_32x32x16_bf16 back to back (four
// independent accumulators per wave, two waves per SIMD), the instruction
// the chunked-prefill kernel runs on.  Its flops / time is the matrix-core
// rate the device sustains, the second denominator beside the 2.5 PFLOP/s
// dense bf16 peak.  It touches no memory but one sink word per thread.
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
