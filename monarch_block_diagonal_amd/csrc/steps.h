// A launch sequence of the library: the layers that are not the two-stage
// Monarch product (the k-factor lattice, the DYAD sum) run as lists of these
// steps (internal).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "kernels.h"

namespace monarch {

// base + off bytes, or null when base is null: the planners also run with
// null buffers (to name a call's kernels), and arithmetic on a null pointer is
// undefined.
inline char* byte_at(void* base, size_t off) {
  return base ? static_cast<char*>(base) + off : nullptr;
}
inline const char* byte_at(const void* base, size_t off) {
  return base ? static_cast<const char*>(base) + off : nullptr;
}

enum SeqKind {
  SEQ_GEMM, SEQ_REDUCE, SEQ_ZERO, SEQ_SWAP, SEQ_FIBER, SEQ_FIBER_WGRAD, SEQ_FIBER_SWAP,
  SEQ_FIBER_STRIDED
};

struct SeqStep {
  SeqKind kind = SEQ_GEMM;
  const char* name = "";
  GemmArgs g;
  ReduceArgs r[3];
  void* zero_ptr = nullptr;
  size_t zero_bytes = 0;
  // SEQ_SWAP: `rows` A x M x C arrays, written as C x M x A
  const void* t_in = nullptr;
  void* t_out = nullptr;
  int64_t t_rows = 0, t_A = 0, t_M = 1, t_C = 0;
  int t_accum = 0;   // SEQ_SWAP: add into t_out
  // SEQ_FIBER: t_out[b, f*f_n + p] = sum_t f_w[f][p][t] t_in[b, f*f_n + t]
  // for t_rows rows of f_N elements
  const void* f_w = nullptr;
  int64_t f_N = 0, f_n = 0;
  // SEQ_FIBER_SWAP: SEQ_FIBER on rows of [t_A][t_M][f_n] arrays, each written
  // as [f_n][t_M][t_A] in the same place (t_out may equal t_in)
  // SEQ_FIBER_STRIDED: round 0 with the change between the natural layout and
  // L_0 (f_dir 0: natural -> L_0, the L_0 input copy to f_save; 1: L_0 ->
  // natural)
  void* f_save = nullptr;
  int f_dir = 0;
  // SEQ_FIBER_WGRAD: f_part[c][f][p][t] = sum over chunk c (f_chunk rows) of
  // t_in[b, f*f_n + p] f_in2[b, f*f_n + t], for t_rows rows
  const void* f_in2 = nullptr;
  float* f_part = nullptr;
  int64_t f_chunk = 0;
};

hipError_t seq_launch(const SeqStep& st, bool bf16, hipStream_t s);

}  // namespace monarch
