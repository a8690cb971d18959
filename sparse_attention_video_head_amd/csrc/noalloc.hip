// svg2_varblock_attn_noalloc: the variable-block attention with its scratch
// memory in a fixed device array of this library instead of a caller
// workspace, for callers that cannot allocate (code under HIP graph capture,
// serving loops that must not call hipMalloc, harnesses that forbid it).
//
// `scratch` is a file-scope device array: each GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code its
// name is only a host-side stand-in, so the device address is resolved once
// per device with hipGetSymbolAddress (with that device current) and that
// pointer is what the kernels receive.  Every call on one GPU shares that
// GPU's array: calls that overlap on one GPU (two streams, two threads) race.
// The attention's kernels rewrite every scratch word they read on each call
// (its work-queue counters included, which the plan kernel resets), so no
// clearing is needed between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "svg2.h"
#include "internal.hpp"

using svg2::record_hip_error;

namespace {

constexpr size_t kScratchBytes = size_t(16) << 20;      // 16 MiB
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];                            // per device, resolved on first use

// The device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    record_hip_error((int)e);
    return SVG2_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return SVG2_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      record_hip_error((int)(e != hipSuccess ? e : hipErrorInvalidSymbol));
      return SVG2_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SVG2_OK;
}

}  // namespace

extern "C" {

size_t svg2_varblock_attn_noalloc_max_scratch(void) { return kScratchBytes; }

int svg2_varblock_attn_noalloc(const void* q, const void* k, const void* v, int32_t dtype, int32_t bh,
                               int32_t n_tokens, int32_t head_dim, const int32_t* q_offsets, int32_t n_q,
                               const int32_t* k_offsets, int32_t n_k, const int32_t* sel_count,
                               const int32_t* sel_idx, float scale, void* out, float* lse, hipStream_t stream) {
  // every argument check of svg2_varblock_attn, on the host: with no
  // workspace it returns the argument error, or SVG2_ERR_WORKSPACE when the
  // arguments are valid (it checks the workspace last)
  const int chk = svg2_varblock_attn(q, k, v, dtype, bh, n_tokens, head_dim, q_offsets, n_q, k_offsets, n_k,
                                     sel_count, sel_idx, scale, out, lse, nullptr, 0, stream);
  if (chk != SVG2_ERR_WORKSPACE) return chk;
  const size_t need = svg2_varblock_attn_workspace_size(bh, n_tokens, n_q, n_k, head_dim);
  if (need > kScratchBytes) return SVG2_ERR_WORKSPACE;   // larger than the fixed scratch array
  void* ws = nullptr;
  const int st = scratch_address(&ws);
  if (st != SVG2_OK) return st;
  return svg2_varblock_attn(q, k, v, dtype, bh, n_tokens, head_dim, q_offsets, n_q, k_offsets, n_k, sel_count,
                            sel_idx, scale, out, lse, ws, kScratchBytes, stream);
}

}  // extern "C"
