// The static scratch of chunk_attn_fwd_noalloc: the attention's split-row
// workspace (arrival words, partial tags, partial results) held in a device
// array of this library instead of memory the caller allocates, for callers
// that cannot allocate (graph capture, serving loops, harnesses that forbid
// hipMalloc).  Nothing here allocates or frees device memory.
//
// The array's name is a host-side stand-in in host code: its device address
// on each GPU is taken once, with that GPU current, through
// hipGetSymbolAddress, and only that address is handed to kernels.  Every
// call on a GPU shares that GPU's array; calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvc_internal.hpp"

namespace kvc {
namespace {

constexpr size_t kScratchBytes = KVC_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

struct PerDevice {
  void* ptr = nullptr;     // device address of `scratch` on this device
  uint32_t epoch = 0;      // epoch of the last call handed out
  bool ready = false;      // a call that zeroes the arrival words and tags was enqueued
};
constexpr int kMaxDevices = 64;
PerDevice g_dev[kMaxDevices];
std::mutex g_mu;

}  // namespace

kvc_status static_workspace(size_t need, StaticWork& w) {
  // the layout bound the array is sized for
  static_assert(KVC_NOALLOC_SCRATCH_BYTES ==
                    sizeof(unsigned long long) * KVC_NOALLOC_MAX_ROWS + 4u * 2 * kAttnMaxWg +
                        4u * 2 * kAttnMaxWg * 2 * kAttnRowQueries +
                        4u * 2 * kAttnMaxWg * kAttnRowQueries * 128,
                "KVC_NOALLOC_SCRATCH_BYTES holds KVC_NOALLOC_MAX_ROWS rows at head_dim 128");
  if (need > kScratchBytes) return KVC_E_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVC_E_DEVICE;
  std::lock_guard<std::mutex> lock(g_mu);
  PerDevice& p = g_dev[dev];
  if (!p.ptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return KVC_E_DEVICE;
    p.ptr = ptr;
  }
  w.ptr = p.ptr;
  w.bytes = kScratchBytes;
  w.ready = p.ready;
  p.epoch = p.epoch + 1 == 0 ? 1 : p.epoch + 1;
  w.epoch = p.epoch;
  w.device = dev;
  return KVC_OK;
}

void static_workspace_launched(const StaticWork& w) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (w.device >= 0 && w.device < kMaxDevices) g_dev[w.device].ready = true;
}

}  // namespace kvc
