// decode_layer_step_noalloc: one layer-step with no handle and no device
// allocation, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// Its scratch is the static device array `scratch` below: one area per
// device, which each device that runs the library holds until the process
// ends, shared by every call on that device.  The launch sequence, the
// kernels and the scratch layout are those of decode_layer_step; only where
// the scratch lives differs, and the multi-launch path runs its shared-expert
// projection on the caller's stream instead of a second stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "../../include/decode_layer.h"
#include "kernels.h"
#include "layer_host.h"

using namespace dl;
using namespace dl::host;

namespace {

constexpr size_t kStaticScratchBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;

}  // namespace

// In host code this name is only a handle for hipGetSymbolAddress, never a
// device address; kernels get the per-device address that call returns.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

struct StaticDevice {
  std::atomic<char *> ptr{nullptr};  // device address of `scratch` on this device
  std::atomic<int> cleared{0};       // the hand-off region was cleared by zero_words
  int n_cu = 0;
  int fused_ok = 0;                  // the single-launch kernel fits on a CU
};
StaticDevice g_static[kMaxDevices];
std::mutex g_static_mu;

__global__ void zero_words(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = 0u;
}

// Looks up this device's address of `scratch` (with the device current) once
// per device, with the device's CU count and whether the single-launch kernel
// fits.
int static_setup(int dev, StaticDevice **out) {
  if (dev < 0 || dev >= kMaxDevices)
    return fail(nullptr, DL_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  StaticDevice &d = g_static[dev];
  if (!d.ptr.load(std::memory_order_acquire)) {
    std::lock_guard<std::mutex> lk(g_static_mu);
    if (!d.ptr.load(std::memory_order_relaxed)) {
      void *p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return fail(nullptr, DL_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d failed: %s", dev,
                    hipGetErrorString(e));
      d.n_cu = cu_count(dev);
      d.fused_ok = fused_blocks_per_cu() >= 1;
      d.ptr.store((char *)p, std::memory_order_release);
    }
  }
  *out = &d;
  return DL_OK;
}

}  // namespace

extern "C" {

size_t decode_layer_noalloc_max_scratch(void) { return kStaticScratchBytes; }

int decode_layer_step_noalloc(const decode_layer_config *cfg, const decode_layer_weights *w,
                              const decode_layer_io *io, void *hip_stream) {
  int rc = check_config(cfg, nullptr);
  if (rc != DL_OK) return rc;
  rc = check_weights(cfg, w, nullptr);
  if (rc != DL_OK) return rc;
  rc = check_io(cfg, io, nullptr);
  if (rc != DL_OK) return rc;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(nullptr, DL_ERR_HIP, "hipGetDevice failed");
  StaticDevice *d = nullptr;
  rc = static_setup(dev, &d);
  if (rc != DL_OK) return rc;
  SinglePlan sp = plan_single(*cfg, d->n_cu);
  if (sp.max_batch > 0 && !d->fused_ok) sp = SinglePlan{};
  if (cfg->path == DL_PATH_SINGLE && sp.max_batch == 0)
    return fail(nullptr, DL_ERR_UNSUPPORTED, "the single-launch path cannot run this configuration on this device");
  if (cfg->path == DL_PATH_BATCHED && !batched_ok(*cfg))
    return fail(nullptr, DL_ERR_UNSUPPORTED, "the batched path needs hidden %% 512 == 0 and attn_dim %% 128 == 0");
  const Layout L = layout_of(*cfg, sp);
  if (L.total > kStaticScratchBytes)
    return fail(nullptr, DL_ERR_UNSUPPORTED,
                "this configuration needs %zu bytes of scratch; the static area holds %zu (use a handle, a "
                "smaller max_batch or another path)",
                L.total, kStaticScratchBytes);
  if (io->batch == 0) return DL_OK;
  const hipStream_t st = (hipStream_t)hip_stream;
  char *base = d->ptr.load(std::memory_order_acquire);
  if (!d->cleared.load(std::memory_order_acquire)) {
    // Set-up on this device: the hand-off state (tagged slots, the step
    // counter, arrival counters) must start at zero.  Static device memory
    // starts zeroed; it is cleared here as well, once, by a kernel on the
    // caller's stream (not while the stream is being captured: a captured
    // clear would run again at every replay).
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess)
      return fail(nullptr, DL_ERR_HIP, "hipStreamIsCapturing failed");
    if (cs == hipStreamCaptureStatusNone) {
      std::lock_guard<std::mutex> lk(g_static_mu);
      if (!d->cleared.load(std::memory_order_relaxed)) {
        const size_t words = L.off[kBHg] / 4;  // the configuration-independent hand-off region
        hipLaunchKernelGGL(zero_words, dim3(64), dim3(256), 0, st, (uint32_t *)base, words);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return fail(nullptr, DL_ERR_HIP, "clearing the static scratch failed: %s", hipGetErrorString(e));
        d->cleared.store(1, std::memory_order_release);
      }
    }
  }
  const Scratch S = bind_scratch(base, L);
  const StepCtx x{cfg, w, &S, &sp, 2 * std::max(1, d->n_cu), nullptr, nullptr, nullptr,
                  kDefaultSpinLimit, nullptr, nullptr, nullptr};
  return enqueue_step(x, io, st);
}

}  // extern "C"
