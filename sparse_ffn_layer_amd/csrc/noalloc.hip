// moe_layer_forward_noalloc: the layer on a workspace the library owns, for
// callers that cannot allocate device memory (graph capture, serving loops,
// harnesses that forbid allocation).
//
// The workspace is `scratch`, a file-scope device array of
// MOE_NOALLOC_SCRATCH_BYTES.  Every GPU the library runs on holds its own
// copy at its own address.  In host code the array's name is only a
// host-side stand-in, so the device address of each GPU's copy is looked up
// once (hipGetSymbolAddress with that GPU current) and only that address is
// ever handed to kernels.  No kernel of the layer needs the workspace zeroed:
// each one writes the state it later reads.
#include <hip/hip_runtime.h>

#include <mutex>

#include "layer.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices] = {};
std::mutex g_scratch_mu;

// Device address of `scratch` on the stream's GPU, looked up on the first
// call for that GPU and kept; null with *status set on failure.
void* scratch_on(hipStream_t st, int32_t* status) {
  int dev = -1;
  hipError_t e = st != nullptr ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) {
    *status = MOE_ERR_HIP;
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *status = MOE_ERR_UNSUPPORTED;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) {
      *status = MOE_ERR_HIP;
      return nullptr;
    }
    // the lookup gives the copy of the current device
    if (cur != dev && hipSetDevice(dev) != hipSuccess) {
      *status = MOE_ERR_HIP;
      return nullptr;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || ptr == nullptr) {
      *status = MOE_ERR_HIP;
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" int32_t moe_layer_forward_noalloc(const moe_problem* mp, const void* x, const void* W_r,
                                             const float* router_bias, const float* select_bias,
                                             const void* W1, const void* b1, const void* W2,
                                             const void* b2, const float* w1_scale, const float* w2_scale,
                                             void* y, int32_t* topk_idx_out, float* topk_gate_out,
                                             float* logits_out, int32_t* expert_counts_out, void* stream) {
  const sfl::LayerArgs a{x, W_r, router_bias, select_bias, W1, b1, W2, b2, w1_scale, w2_scale, y,
                         topk_idx_out, topk_gate_out, logits_out, expert_counts_out};
  size_t need = 0;
  int32_t s = sfl::layer_validate(mp, a, &need);
  if (s != MOE_OK || need == 0) return s;
  if (need > MOE_NOALLOC_SCRATCH_BYTES) return MOE_ERR_TOO_LARGE;
  hipStream_t st = (hipStream_t)stream;
  void* ws = scratch_on(st, &s);
  if (ws == nullptr) return s;
  return sfl::layer_run(mp, a, ws, st);
}
