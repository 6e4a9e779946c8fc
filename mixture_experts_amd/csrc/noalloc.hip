// moe_forward for callers that cannot allocate device memory (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
// launch sequence as moe_forward, with its scratch in a static device array of
// fixed size instead of a caller workspace.
#include <mutex>
#include <vector>

#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(128) << 20;   // 128 MiB per GPU, held until the process ends

// Scratch of moe_forward_noalloc.  In host code this name is only a stand-in
// for the symbol; the device address of each GPU's copy comes from
// hipGetSymbolAddress (scratch_on_current_device).
__device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
std::vector<void*> g_ptr;                              // per device, filled on first use

// Device address of `scratch` on the current device, looked up once per device
// with that device current; nullptr if the lookup fails.
void* scratch_on_current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return nullptr;
  std::lock_guard<std::mutex> lock(g_mu);
  if (size_t(dev) >= g_ptr.size()) g_ptr.resize(size_t(dev) + 1, nullptr);
  if (!g_ptr[size_t(dev)]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_ptr[size_t(dev)] = p;
  }
  return g_ptr[size_t(dev)];
}

}  // namespace

extern "C" {

size_t moe_forward_noalloc_scratch_bytes(void) { return kScratchBytes; }

moe_status_t moe_forward_noalloc(const moe_config_t* cfg, const void* x, const float* gate_w, const float* bias,
                                 const moe_weights_t* experts, const moe_weights_t* shared, void* out,
                                 int32_t* topk_idx_out, float* topk_w_out, void* stream) {
  const size_t need = moe_workspace_bytes(cfg);
  if (need == 0)   // an invalid or unsupported configuration: moe_forward's own status, nothing enqueued
    return moe_forward(cfg, x, gate_w, bias, experts, shared, out, topk_idx_out, topk_w_out, nullptr, 0, stream);
  if (need > kScratchBytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
  if (cfg->num_tokens == 0) return MOE_OK;
  void* ws = scratch_on_current_device();
  if (!ws) return MOE_ERR_LAUNCH;
  return moe_forward(cfg, x, gate_w, bias, experts, shared, out, topk_idx_out, topk_w_out, ws, kScratchBytes, stream);
}

}  // extern "C"
