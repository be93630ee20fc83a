// pa_decode_noalloc: pa_decode with its workspace in a static device array
// instead of a caller buffer, for callers that cannot allocate device memory
// (code under stream capture, tight serving loops, hosts that forbid
// hipMalloc).  The entry point allocates nothing and calls pa_decode's own
// validation, planning and kernels.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <mutex>

#include "pa.h"

// One copy per GPU, resident from module load until the process ends.  Host
// code never names this array directly (its host-side symbol is a stand-in,
// not a device address): it uses the address hipGetSymbolAddress returns on
// each device.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr size_t kScratchBytes = (size_t)PA_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up once per
// device with that device current.
int scratch_address(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return PA_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return PA_OK;
}

}  // namespace

extern "C" int pa_decode_noalloc(void* out, const void* query, const void* k_cache,
                                 const void* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* block_refcounts,
                                 const int32_t* seq_lens, int32_t num_seqs, int32_t max_seq_len,
                                 int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, float scale,
                                 int32_t dtype, int32_t kv_split_tokens, void* stream) {
  // pa_decode checks every argument before it looks at the workspace: with
  // none it returns PA_ERR_WORKSPACE exactly when the arguments are valid
  // (PA_OK for an empty batch), touching neither the GPU nor the stream.
  const int arg_rc = pa_decode(out, query, k_cache, v_cache, block_tables, max_blocks_per_seq,
                               block_refcounts, seq_lens, num_seqs, max_seq_len, num_q_heads,
                               num_kv_heads, head_dim, block_size, num_blocks, scale, dtype,
                               kv_split_tokens, nullptr, 0, stream);
  if (arg_rc != PA_ERR_WORKSPACE) return arg_rc;
  const size_t need = pa_decode_workspace_bytes(num_seqs, num_q_heads, head_dim, max_seq_len,
                                                block_size, kv_split_tokens);
  if (need == 0) return PA_ERR_SHAPE;
  if (need > kScratchBytes) return PA_ERR_SCRATCH;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc != PA_OK) return rc;
  // pa_decode's workspace needs no initialisation: nothing is cleared.
  return pa_decode(out, query, k_cache, v_cache, block_tables, max_blocks_per_seq,
                   block_refcounts, seq_lens, num_seqs, max_seq_len, num_q_heads, num_kv_heads,
                   head_dim, block_size, num_blocks, scale, dtype, kv_split_tokens, ws,
                   kScratchBytes, stream);
}
