// Planning of the k-factor ("hypercube") Monarch layer (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"

namespace monarch {

constexpr int kHyperMaxDims = 4;

struct HyperProblem {
  int k = 0;                        // lattice dimensions
  int64_t dims[kHyperMaxDims] = {};
  int64_t N = 0, batch = 0;
  int dtype = 0;
  int64_t esize = 4;
  int64_t splits[kHyperMaxDims] = {}, chunk[kHyperMaxDims] = {};   // batch split of dw_j
  size_t ws_g[2] = {}, ws_part[kHyperMaxDims] = {}, ws_total = 0;
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

enum HyperKind { HYPER_GEMM, HYPER_REDUCE, HYPER_ZERO, HYPER_TRANSPOSE };

struct HyperStep {
  HyperKind kind = HYPER_GEMM;
  const char* name = "";
  GemmArgs g;
  ReduceArgs r[3];
  void* zero_ptr = nullptr;
  size_t zero_bytes = 0;
  // HYPER_TRANSPOSE: every row of `rows` is an R x C matrix, written as C x R
  const void* t_in = nullptr;
  void* t_out = nullptr;
  int64_t t_rows = 0, t_R = 0, t_C = 0;
};

constexpr int kHyperMaxSteps = 3 * kHyperMaxDims + 4;

// Checks the lattice (1..4 dimensions, positive, N < 2^31), batch and dtype;
// returns a monarch_status. hyper_saved_elems: elements the forward keeps.
int make_hyper(int ndims, const int64_t* dims, int64_t batch, int dtype, HyperProblem* hp);
int64_t hyper_saved_elems(const HyperProblem& hp);
// Steps of the forward / backward pass; returns their count.
int hyper_plan_fwd(const HyperProblem& hp, const HyperBuffers& b, HyperStep* steps);
int hyper_plan_bwd(const HyperProblem& hp, const HyperBuffers& b, HyperStep* steps);
hipError_t hyper_launch(const HyperStep& st, bool bf16, hipStream_t s);

}  // namespace monarch
