// muon_ns_batched without any device allocation by library or caller: the
// workspace is a fixed array in the library's own device memory.
//
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).  The array is a
// file-scope __device__ object: every device the library runs on holds its
// own copy, at its own address, from module load until the process ends.
// In host code the array's name is only a stand-in for the symbol, so the
// device address of this device's copy is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is
// ever handed to kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <string>

#include "../../include/muon_ns.h"
#include "launch.hpp"

namespace muon {
namespace {

constexpr size_t kScratchBytes = MUON_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size must keep 256-byte alignment");

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`.
muon_status_t scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    set_last_error("no current HIP device");
    return MUON_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) {
    set_last_error("device index " + std::to_string(dev) + " above the supported 63");
    return MUON_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      set_last_error(std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
      return MUON_ERR_HIP;
    }
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MUON_OK;
}

}  // namespace
}  // namespace muon

extern "C" muon_status_t muon_ns_batched_noalloc(const muon_ns_desc_t* desc, int32_t count,
                                                 int32_t steps, const float coeffs[3],
                                                 muon_dtype_t dtype, float eps, void* stream) {
  using namespace muon;
  // the scalar checks of muon_ns_batched, made here too so that no HIP call
  // (the device lookup below) precedes a rejected request
  if (count > 0) {
    if (steps < 0 || steps > 64) {
      set_last_error("steps out of range [0, 64]");
      return MUON_ERR_INVALID_ARG;
    }
    if (!coeffs || !std::isfinite(coeffs[0]) || !std::isfinite(coeffs[1]) || !std::isfinite(coeffs[2])) {
      set_last_error("coeffs NULL or not finite");
      return MUON_ERR_INVALID_ARG;
    }
    if (!std::isfinite(eps) || eps < 0) {
      set_last_error("eps must be finite and >= 0");
      return MUON_ERR_INVALID_ARG;
    }
  }
  size_t need = 0;
  muon_status_t s = muon_ns_workspace_size(desc, count, dtype, &need);
  if (s != MUON_OK) return s;
  if (need > kScratchBytes) {
    set_last_error("these matrices need " + std::to_string(need) +
                   " bytes of workspace; the static scratch of muon_ns_batched_noalloc holds " +
                   std::to_string(kScratchBytes) + " (use muon_ns_batched with a workspace)");
    return MUON_ERR_WORKSPACE;
  }
  if (count == 0) return muon_ns_batched(desc, count, steps, coeffs, dtype, eps, nullptr, 0, stream);
  void* ws = nullptr;
  s = scratch_for_current_device(&ws);
  if (s != MUON_OK) return s;
  set_no_events(true);
  s = muon_ns_batched(desc, count, steps, coeffs, dtype, eps, ws, kScratchBytes, stream);
  set_no_events(false);
  return s;
}
