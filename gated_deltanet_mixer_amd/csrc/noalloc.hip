// gdn_prefill_noalloc: gdn_prefill with the chunked algorithm's scratch in a
// fixed device array of the library instead of a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ object: every GPU the library runs on
// holds its own copy (GDN_NOALLOC_SCRATCH_BYTES) until the process ends.  In
// host code its name is only a host-side stand-in, so its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and that address is what the kernels receive.  Every call on a GPU
// shares the array: calls that overlap on one GPU (other streams, other
// threads) race on it.  The chunked kernels write every scratch element they
// read, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/gdn.h"

namespace {

__device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device).  No allocation, no synchronisation.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return GDN_ERR_LAUNCH;
  if (dev < 0 || dev >= kMaxDevices) return GDN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return GDN_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GDN_OK;
}

}  // namespace

extern "C" int gdn_prefill_noalloc(const void* q, int64_t q_tok_stride, const void* k,
                                   int64_t k_tok_stride, const void* v, int64_t v_tok_stride,
                                   int32_t qkv_dt, const void* a, const void* b, int32_t gate_dt,
                                   const float* A_log, const float* dt_bias,
                                   const float* state_in, float* state_out, void* o,
                                   int32_t o_dt, int32_t B, int32_t T, gdn_dims dims,
                                   float q_scale, int32_t algo, void* stream) {
  const size_t need = gdn_prefill_workspace_bytes(B, T, dims, qkv_dt, algo);
  if (need > (size_t)GDN_NOALLOC_SCRATCH_BYTES) return GDN_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(&ws);
    if (st != GDN_OK) return st;
  }
  // Same validation and kernels as gdn_prefill, with the fixed scratch as
  // the workspace.
  return gdn_prefill(q, q_tok_stride, k, k_tok_stride, v, v_tok_stride, qkv_dt, a, b, gate_dt,
                     A_log, dt_bias, state_in, state_out, o, o_dt, B, T, dims, q_scale, algo, ws,
                     need, stream);
}
