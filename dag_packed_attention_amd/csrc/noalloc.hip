// dag_attn_fwd_noalloc: the forward with its workspace in a static device array, for
// callers that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid hipMalloc).
//
// The array `scratch` below is a device-side object: in host code its name is only a
// host stand-in.  Its device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept in scratch_ptr[]; only that
// address is ever handed to kernels.  Every device that runs this library holds its own
// copy until the process ends.  All calls on one device share it, so calls that overlap
// on one device (concurrent streams or threads) race; calls in order on one stream do not.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "abi_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

void* scratch_ptr[kMaxDevices] = {};
std::mutex scratch_mu;

// The device address of this device's copy of `scratch`, looked up on first use.
dag_status current_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return dagattn::set_error(DAG_E_DEVICE, "hipGetDevice failed");
  }
  if (dev < 0 || dev >= kMaxDevices)
    return dagattn::set_error(DAG_E_UNSUPPORTED, "device index " + std::to_string(dev) + " beyond the static table");
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      (void)hipGetLastError();
      return dagattn::set_error(DAG_E_DEVICE, std::string("hipGetSymbolAddress(scratch) failed: ") +
                                                  hipGetErrorString(e));
    }
    scratch_ptr[dev] = p;
  }
  *out = scratch_ptr[dev];
  return DAG_OK;
}

}  // namespace

extern "C" dag_status dag_attn_fwd_noalloc(dag_plan* plan, const dag_attn_params* p, const void* q, const void* k,
                                           const void* v, void* o, float* lse, void* o_lo, void* hip_stream) {
  size_t need = 0;
  const dag_status st = dag_attn_workspace(plan, p, &need, nullptr);
  if (st != DAG_OK) return st;
  if (need > kScratchBytes)
    return dagattn::set_error(DAG_E_WORKSPACE, "the forward needs " + std::to_string(need) +
                                                   " workspace bytes; the static scratch holds " +
                                                   std::to_string(kScratchBytes) + " (use dag_attn_fwd)");
  void* ws = nullptr;
  const dag_status sst = current_scratch(&ws);
  if (sst != DAG_OK) return sst;
  // the forward overwrites every workspace byte it reads (the q/k/v maxima are cleared by
  // a kernel first), so the previous call's contents never leak into this one
  return dagattn::attn_fwd_impl(plan, p, q, k, v, o, lse, o_lo, ws, kScratchBytes, hip_stream,
                                /*allow_upload=*/false);
}
