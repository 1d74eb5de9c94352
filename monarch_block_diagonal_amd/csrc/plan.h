// Problem description, kernel plans and step launches (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "small.h"
#include "square.h"

namespace monarch {

enum Path { PATH_GENERIC = 0, PATH_SQ128 = 1, PATH_SM32 = 2 };

struct Problem {
  int64_t in = 0, out = 0, mid = 0, b1 = 0, b2 = 0;
  int64_t q1i = 0, q1o = 0, q2i = 0, q2o = 0;
  // whole-block extents: the input is zero-padded to in_ext = b1*q1i and the
  // output keeps the first `out` of out_ext = b2*q2o features
  int64_t in_ext = 0, out_ext = 0;
  bool bias = false;
  // bias-gradient batch chunks (rows per chunk, chunk count)
  int64_t bias_chunk = 0, bias_chunks = 0;
  int64_t batch = 0;
  int dtype = 0, act = 0;
  int64_t esize = 4;
  int path = PATH_GENERIC;
  // generic path: z holds stage 2's input in stage 2's order,
  // W[b, g*q2i + t] = Z[b, t*b2 + g] (needs q1o % b2 == 0; else Z's own order)
  bool z_stage2_order = false;
  // batch split of the weight-gradient reductions (stage 2 and stage 1)
  int64_t s2 = 1, kc2 = 0, s1 = 1, kc1 = 0;
  SqPlan sq;  // launch geometry of PATH_SQ128
  // workspace layout (byte offsets)
  size_t ws_dz = 0, ws_p2 = 0, ws_p1 = 0, ws_dv = 0, ws_pb = 0, ws_total = 0;
};

struct Buffers {
  const void* x = nullptr;
  const void* w1 = nullptr;
  const void* w2 = nullptr;
  const void* dy = nullptr;
  const void* y = nullptr;  // forward output (read by the ReLU backward)
  const void* z = nullptr;  // saved stage-2 input (read by the backward)
  const void* bias = nullptr;
  void* dbias = nullptr;
  void* y_out = nullptr;
  void* z_out = nullptr;
  void* dx = nullptr;
  void* dw1 = nullptr;
  void* dw2 = nullptr;
  void* ws = nullptr;
};

enum StepKind {
  GEN_DV_GATHER,
  GEN_BIAS_PARTIALS,
  GEN_STAGE1_FWD,
  GEN_STAGE2_FWD,
  GEN_STAGE2_BWD_DATA,
  GEN_STAGE2_BWD_WEIGHT,
  GEN_STAGE1_BWD_DATA,
  GEN_STAGE1_BWD_WEIGHT,
  REDUCE_DW,
  ZERO_DW,
  SQ_DV_PANELS,
  SQ_STAGE1_FWD,
  SQ_STAGE2_FWD,
  SQ_STAGE2_BWD_DATA,
  SQ_STAGE2_BWD_WEIGHT,
  SQ_STAGE1_BWD,
  SM_FWD,
  SM_BWD_DATA,
  SM_WGRAD,
};

struct Plan {
  int n = 0;
  StepKind kind[16];
  void add(StepKind k) { kind[n++] = k; }
};

// Checks dtype/act/shape and fills the derived sizes, path and workspace
// layout. Returns a monarch_status. make_problem takes mid = out and needs
// whole blocks (in % nb1 == 0, out % nb2 == 0); make_problem_ex takes any
// mid divisible by both block counts and pads in and out to whole blocks.
int make_problem(int64_t in, int64_t out, int64_t nb1, int64_t nb2, int64_t batch, int dtype,
                 int act, Problem* pr);
int make_problem_ex(int64_t in, int64_t out, int64_t mid, int64_t nb1, int64_t nb2, int64_t batch,
                    int dtype, int act, bool bias, Problem* pr);
size_t workspace_bytes(const Problem& pr);
Plan plan_fwd(const Problem& pr);
Plan plan_bwd(const Problem& pr);
const char* step_name(StepKind k);
hipError_t launch_step(StepKind k, const Problem& pr, const Buffers& b, hipStream_t s);

}  // namespace monarch
