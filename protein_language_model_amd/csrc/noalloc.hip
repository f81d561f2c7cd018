// esm_attn_fwd_noalloc: the forward for callers that cannot allocate device
// memory. Its workspace is a fixed buffer in device global memory owned by
// the library (one copy per GPU, alive while the library is loaded), so the
// call itself allocates nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "esm_attn.h"

namespace {

// The buffer. In host code this name is only a stand-in for the device
// symbol: it is never passed to a kernel, a copy or a fill. The device
// address of the current GPU's copy comes from hipGetSymbolAddress, looked
// up once per device with that device current.
__device__ __align__(256) unsigned char scratch[ESM_ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The current GPU's copy of `scratch`; nullptr if the device query or the
// symbol lookup fails.
void* current_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return nullptr;
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" esm_attn_status_t esm_attn_fwd_noalloc(
    const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* cu_seqlens,
    int32_t batch, int32_t total_tokens, int32_t max_seqlen, int32_t num_heads,
    int32_t head_dim, float softmax_scale, float rope_base, uint16_t* o, float* lse,
    void* stream) {
  // Argument checks first, exactly those of esm_attn_fwd: given a zero-byte
  // workspace it validates every argument and, if all are fine, returns
  // ESM_ATTN_ERR_WORKSPACE_TOO_SMALL without enqueuing anything (the dummy
  // workspace pointer is never dereferenced). OK means there is nothing to do.
  alignas(16) static unsigned char no_workspace[16];
  esm_attn_status_t s = esm_attn_fwd(q, k, v, cu_seqlens, batch, total_tokens, max_seqlen,
                                     num_heads, head_dim, softmax_scale, rope_base, o, lse,
                                     no_workspace, 0, stream);
  if (s != ESM_ATTN_ERR_WORKSPACE_TOO_SMALL) return s;
  const size_t need = esm_attn_fwd_workspace_bytes(batch, total_tokens, max_seqlen, num_heads,
                                                   head_dim);
  if (need > ESM_ATTN_NOALLOC_SCRATCH_BYTES) return ESM_ATTN_ERR_SCRATCH_TOO_SMALL;
  void* ws = current_scratch();
  if (ws == nullptr) return ESM_ATTN_ERR_HIP;
  return esm_attn_fwd(q, k, v, cu_seqlens, batch, total_tokens, max_seqlen, num_heads,
                      head_dim, softmax_scale, rope_base, o, lse, ws,
                      ESM_ATTN_NOALLOC_SCRATCH_BYTES, stream);
}
