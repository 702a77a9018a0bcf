// mmdit_step_noalloc: the denoising step on a workspace the library holds in
// a file-scope device array, for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops).
//
// `scratch` below is a device symbol. In host code its name stands for a
// host-side shadow, not for device memory, so host code never passes it to a
// kernel or a copy: the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device (with that device current) and
// kept in g_scratch.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/mmdit.h"
#include "api_internal.h"

namespace {

// 256 MiB per GPU: the step at 512x512 (1280 tokens) and h 3072 needs about
// 150 MB; the 1024x1024 step (4608 tokens) needs more and is refused.
constexpr size_t kScratchBytes = size_t(256) << 20;
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's scratch, resolved on the first call
// on that device.
int scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return mmdit::fail(MMDIT_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return mmdit::fail(MMDIT_ERR_UNSUPPORTED, "device %d: mmdit_step_noalloc supports devices 0..%d", dev,
                       kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return mmdit::fail(MMDIT_ERR_HIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MMDIT_OK;
}

}  // namespace

extern "C" int mmdit_step_noalloc(const mmdit_config* cfg, const mmdit_model_w* w, void* x_packed, void* v_out,
                                  const void* txt_emb, const void* y, const int32_t* ids, double sigma,
                                  double sigma_next, const mmdit_step_opts* opts, void* hip_stream) {
  size_t need = 0;
  int r = mmdit_step_workspace_ex(cfg, w, opts, &need);
  if (r != MMDIT_OK) return r;
  if (need > kScratchBytes)
    return mmdit::fail(MMDIT_ERR_WORKSPACE,
                       "mmdit_step_noalloc: this configuration needs %zu bytes of workspace; the library's "
                       "scratch holds %zu (use mmdit_step_ex with a caller workspace)",
                       need, kScratchBytes);
  void* ws = nullptr;
  if ((r = scratch_of_current_device(&ws)) != MMDIT_OK) return r;
  return mmdit::step_impl(cfg, w, x_packed, v_out, txt_emb, y, ids, sigma, sigma_next, opts, ws, kScratchBytes,
                          hip_stream);
}
