// sdpa_bwd_run_noalloc: the backward for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  Its workspace is a file-scope device
// array of the library, `scratch`, of kScratchBytes: every GPU the library
// runs on holds one copy until the process ends.  Host code never passes the
// array's name to a kernel or a copy (in host code it names a host-side
// stand-in, not device memory): on its first call on a device the entry
// point looks up that device's address of the array with
// hipGetSymbolAddress, with the device current, and from then on uses only
// that per-device pointer.  The kernels are those of sdpa_bwd_run; they
// clear what must start at zero (relay counters, tickets, accumulator
// slots) themselves, so the array's contents from an earlier call are
// harmless.  Calls that overlap on one GPU share the array and race.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "api_internal.h"
#include "swa_sdpa.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per GPU
constexpr int kMaxDevices = 64;

}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // per-device address of `scratch`, once looked up

// Device address of `scratch` on the current device (looked up once per
// device, with that device current), or NULL with the error text in *err.
void* scratch_ptr(char* err, size_t n) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    std::snprintf(err, n, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    std::snprintf(err, n, "device %d is beyond the %d devices the scratch table holds", dev, kMaxDevices);
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      std::snprintf(err, n, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch[dev] = ptr;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

sdpa_status sdpa_bwd_run_noalloc(const sdpa_bwd_plan_t* plan, const sdpa_bwd_tensors* tensors,
                                 hipStream_t stream) {
  char err[256];
  if (!plan) return swa::set_error(SDPA_ERR_INVALID_ARG, "plan is NULL");
  const size_t need = swa::bwd_plan_workspace_bytes(plan);
  if (need > kScratchBytes) {
    std::snprintf(err, sizeof err,
                  "the plan needs %zu bytes of workspace, more than the %zu-byte scratch of "
                  "sdpa_bwd_run_noalloc: use sdpa_bwd_run with a caller workspace",
                  need, kScratchBytes);
    return swa::set_error(SDPA_ERR_WORKSPACE, err);
  }
  void* ws = scratch_ptr(err, sizeof err);
  if (!ws) return swa::set_error(SDPA_ERR_HIP, err);
  return swa::bwd_run(plan, tensors, ws, kScratchBytes, stream, nullptr, nullptr, false);
}

}  // extern "C"
