// Planning of the k-factor ("hypercube") Monarch layer (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"
#include "steps.h"

namespace monarch {

constexpr int kHyperMaxDims = 4;

struct HyperProblem {
  int k = 0;                        // lattice dimensions
  int64_t dims[kHyperMaxDims] = {};
  int64_t N = 0, batch = 0;
  int dtype = 0;
  int64_t esize = 4;
  int64_t splits[kHyperMaxDims] = {}, chunk[kHyperMaxDims] = {};   // batch split of dw_j
  // backward workspace: two gradient buffers, the weight-gradient partials
  // and per-fiber transposed weights for the fiber kernel's data products
  size_t ws_g[2] = {}, ws_part[kHyperMaxDims] = {}, ws_wt = 0, ws_total = 0;
};

struct HyperBuffers {
  const void* x = nullptr;
  const void* w[kHyperMaxDims] = {};
  void* y = nullptr;
  void* saved = nullptr;            // k * batch * N elements (k >= 2)
  const void* saved_in = nullptr;
  const void* dy = nullptr;
  void* dx = nullptr;
  void* dw[kHyperMaxDims] = {};
  void* ws = nullptr;
};

constexpr int kHyperMaxSteps = 4 * kHyperMaxDims + 4;

// Checks the lattice (1..4 dimensions, positive, N < 2^31), batch and dtype;
// returns a monarch_status. hyper_saved_elems: elements the forward keeps.
int make_hyper(int ndims, const int64_t* dims, int64_t batch, int dtype, HyperProblem* hp);
int64_t hyper_saved_elems(const HyperProblem& hp);
// Steps of the forward / backward pass; returns their count.
int hyper_plan_fwd(const HyperProblem& hp, const HyperBuffers& b, SeqStep* steps);
int hyper_plan_bwd(const HyperProblem& hp, const HyperBuffers& b, SeqStep* steps);

}  // namespace monarch
