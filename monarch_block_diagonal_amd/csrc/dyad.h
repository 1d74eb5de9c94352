// Planning of the DYAD-style layer (internal).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "steps.h"

namespace monarch {

struct DyadProblem {
  int64_t in = 0, out = 0, nb = 0, qi = 0, qo = 0, batch = 0;
  int dtype = 0;
  int64_t esize = 4;
  int64_t splits = 1, chunk = 0;   // batch split of both weight gradients
  // backward workspace: partial sums of dA and dB, block-major X and dY;
  // forward workspace: block-major X and term B's block-major rows (ws_fwd
  // bytes)
  size_t ws_pa = 0, ws_pb = 0, ws_xp = 0, ws_dyp = 0, ws_total = 0, ws_fwd = 0;
  size_t ws_fwd_yp = 0;   // forward: term B's block-major rows after Xp
};

struct DyadBuffers {
  const void* x = nullptr;
  const void* wa = nullptr;
  const void* wb = nullptr;
  void* y = nullptr;
  const void* dy = nullptr;
  void* dx = nullptr;
  void* dwa = nullptr;
  void* dwb = nullptr;
  void* ws = nullptr;
};

constexpr int kDyadMaxSteps = 8;

// Checks the shape (in and out divisible by nb), batch and dtype; returns a
// monarch_status.
int make_dyad(int64_t in, int64_t out, int64_t nb, int64_t batch, int dtype, DyadProblem* dp);
int dyad_plan_fwd(const DyadProblem& dp, const DyadBuffers& b, SeqStep* steps);
int dyad_plan_bwd(const DyadProblem& dp, const DyadBuffers& b, SeqStep* steps);

}  // namespace monarch
