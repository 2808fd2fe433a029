// flare_encode_static: the encoder of flare_encode with its split partials in
// a static device array instead of a caller workspace, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops,
// harnesses that forbid allocation).
//
// The array lives in the library's code object: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  In host
// code the array's name is only a host-side stand-in, so its device address
// is looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address reaches a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/flare.h"
#include "api_internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;  // per device
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of the current device's scratch array (nullptr on error).
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_once[dev], [dev] {
    void* ptr = nullptr;
    g_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? ptr : nullptr;
  });
  return g_ptr[dev];
}

}  // namespace

extern "C" {

size_t flare_encode_static_scratch_bytes(void) { return kScratchBytes; }

flare_status flare_encode_static(const flare_tensor* Q, const flare_tensor* K, const flare_tensor* V,
                                 const flare_tensor* Z, float* lse, int B, int H, int M, int64_t N,
                                 int D, float scale, unsigned flags, void* stream) {
  const flare_status v = flare::encode_validate(Q, K, V, Z, lse, B, H, M, N, D, scale, flags);
  if (v != FLARE_OK) return v;
  const int S = flare::encode_splits_within(B, H, M, N, D, K->dtype == FLARE_F32, kScratchBytes);
  if (S < 1) return FLARE_E_SCRATCH;
  void* ws = scratch_address();
  if (!ws) return FLARE_E_HIP;
  return flare::encode_run(Q, K, V, Z, lse, B, H, M, N, D, scale, flags, ws, S, stream);
}

}  // extern "C"
