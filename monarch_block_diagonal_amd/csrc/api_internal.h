// Shared by the C-ABI translation units (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "plan.h"

namespace monarch {

// Records a HIP error for monarch_status_string(MONARCH_ERR_HIP) on the
// calling thread; returns MONARCH_OK or MONARCH_ERR_HIP.
int record_hip(hipError_t e);

// Null and alignment checks of the backward's pointers (not the workspace);
// no HIP call. Returns a monarch_status.
int bwd_check(const Problem& pr, const void* dy, const void* x, const void* w1, const void* w2,
              const void* z, const void* y, const void* dx, const void* dw1, const void* dw2,
              const void* dbias);

// bwd_check, the workspace checks, then the backward plan's launches on `stream`
// (ws: ws_bytes of device memory, at least workspace_bytes(pr)).
int bwd_impl(const Problem& pr, const void* dy, const void* x, const void* w1, const void* w2,
             const void* z, const void* y, void* dx, void* dw1, void* dw2, void* dbias, void* ws,
             size_t ws_bytes, void* stream, void* const* events, int n_events);

}  // namespace monarch
