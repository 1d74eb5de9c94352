// monarch_bwd_noalloc: the backward pass of monarch_bwd with its workspace
// taken from a static device array instead of a caller buffer, for callers
// that cannot allocate device memory (code under HIP graph capture, serving
// loops, harnesses that forbid hipMalloc). It runs exactly monarch_bwd's
// kernels; only where the intermediates and partial sums live changes.
//
// `scratch` below is a host-side stand-in for a per-device array: each GPU
// the library runs on holds its own copy, at its own address, until the
// process ends. The address is fetched once per device (hipGetSymbolAddress
// with that device current) and only that address is handed to kernels.
// Nothing in the backward reads scratch before writing it, so no clearing is
// needed between calls; calls that overlap on one GPU share the array and
// race.
#include <mutex>

#include "api_internal.h"
#include "monarch.h"

namespace monarch {

static __device__ __align__(256) unsigned char scratch[MONARCH_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// Device address of `scratch` on the current device (fetched once per device).
int scratch_address(void** out) {
  int dev = -1;
  int st = record_hip(hipGetDevice(&dev));
  if (st) return st;
  if (dev < 0 || dev >= kMaxDevices) return record_hip(hipErrorInvalidDevice);
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
  });
  st = record_hip(g_scratch_err[dev]);
  if (st) return st;
  if (!g_scratch[dev]) return record_hip(hipErrorInvalidSymbol);
  *out = g_scratch[dev];
  return MONARCH_OK;
}

}  // namespace
}  // namespace monarch

using namespace monarch;

extern "C" int monarch_bwd_noalloc(const void* dy, const void* x, const void* w1, const void* w2,
                                   const void* z, const void* y, void* dx, void* dw1, void* dw2,
                                   int64_t in_features, int64_t out_features, int64_t nblocks1,
                                   int64_t nblocks2, int64_t batch, int dtype, int act,
                                   void* stream) {
  Problem pr;
  int st = make_problem(in_features, out_features, nblocks1, nblocks2, batch, dtype, act, &pr);
  if (st) return st;
  st = bwd_check(pr, dy, x, w1, w2, z, y, dx, dw1, dw2, nullptr);
  if (st) return st;
  const size_t need = workspace_bytes(pr);
  if (need > static_cast<size_t>(MONARCH_NOALLOC_SCRATCH_BYTES)) return MONARCH_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0) {
    st = scratch_address(&ws);
    if (st) return st;
  }
  return bwd_impl(pr, dy, x, w1, w2, z, y, dx, dw1, dw2, nullptr, ws, need, stream, nullptr, 0);
}
