// The decode step without a caller-provided workspace: its workspace is a
// static device array of the library (one per GPU), for callers that cannot
// allocate device memory (HIP graph capture, serving loops).
#include <mutex>

#include "host_plan.h"
#include "kernels.h"
#include "sparse_attn.h"

// The step's workspace.  In host code this name stands for the array but is
// not its device address: the address comes from hipGetSymbolAddress, per
// device, and only that address is ever passed to a kernel.
static __device__ __align__(256) unsigned char scratch[SA_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace sa;

constexpr size_t kScratchBytes = SA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % kAlign == 0, "scratch size");

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device (null: not yet)

// The current device's address of `scratch`, looked up on the first call on
// that device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SA_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return SA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return SA_OK;
}

}  // namespace

extern "C" int sparse_attn_decode_step_noalloc(const sa_shape* shape, const int32_t* pos,
                                               int32_t T, const void* k_new, const void* v_new,
                                               const void* q, const float* P, void* k_cache,
                                               void* v_cache, uint8_t* kp_cache,
                                               const int32_t* seq_lens, int32_t n_max, int32_t M,
                                               float softmax_scale, int32_t* idx, void* out,
                                               float* lse, void* stream) {
  const int st = check_shape(shape);
  if (st != SA_OK) return st;
  const size_t need = workspace_bytes(*shape, n_max, M);
  if (need == 0) return SA_ERR_INVALID;              // n_max or M out of range
  if (need > kScratchBytes) return SA_ERR_TOO_LARGE;
  void* ws = nullptr;
  const int sst = scratch_address(&ws);
  if (sst != SA_OK) return sst;
  return sparse_attn_decode_step(shape, pos, T, k_new, v_new, q, P, k_cache, v_cache, kp_cache,
                                 seq_lens, n_max, M, softmax_scale, idx, out, lse, ws,
                                 kScratchBytes, stream);
}
