// Kernel planning for one Monarch problem and the launch of each step.
//
// Generic path (any shape): every step is one strided batched GEMM
// (tiled.hip when its operands are contiguous along a tile dimension,
// generic.hip otherwise). With Z[b, r*q1o + k] the stage-1 output:
//   stage 1 fwd   Z(r; b, k)  = sum_s X[b, r*q1i+s] w1[r,k,s]
//   stage 2 fwd   Y(g; b, p)  = act(sum_t Z[b, t*b2+g] w2[g,p,t])   -> Y[b, p*b2+g]
//   dV gather     dV[b, g*q2o+p] = dYe[b, p*b2+g]
//   stage 2 bwd   dZ(g; b, t) = sum_p dV[b, g*q2o+p] w2[g,p,t]      -> dZ[b, t*b2+g]
//                 dw2(g; p, t) = sum_b dV[b, g*q2o+p] Z[b, t*b2+g]   (batch split)
//   stage 1 bwd   dX(r; b, s) = sum_k dZ[b, r*q1o+k] w1[r,k,s]
//                 dw1(r; k, s) = sum_b dZ[b, r*q1o+k] X[b, r*q1i+s]  (batch split)
// where dYe = dY masked by Y > 0 after a fused ReLU. The index maps are the
// stride permutation and its inverse (scatterbrain issues page, "hypercube"
// thread) folded into the operand strides. When q1o % b2 == 0 the saved z
// holds Z in stage 2's order, W[b, g*q2i + t] = Z[b, t*b2 + g]: stage 1
// enumerates its output columns of block r as j = g*n1 + tt (k = tt*b2 + g,
// n1 = q1o/b2), so it writes runs of n1 consecutive elements and stage 2 and
// the dw2 product read z contiguously.
//
// Fused path (bf16, 32 x 32 blocks, at most 1024 features, small.hip): the
// forward, the data part of the backward and both weight gradients are one
// launch each (the weight gradients as batch-chunk partials from the dV and
// dZ the data kernel stores), then the shared reduction.
#include "kernels.h"
#include "monarch.h"
#include "plan.h"

namespace monarch {

namespace {

constexpr int64_t kDimLimit = int64_t(1) << 31;

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Batch split for a weight-gradient GEMM with nblk blocks of M x N and
// reduction length K: enough workgroups to fill the chip, chunks >= 128 rows.
void choose_splits(int64_t nblk, int64_t M, int64_t N, int64_t K, bool bf16, int64_t* splits,
                   int64_t* chunk) {
  if (K <= 0) {
    *splits = 1;
    *chunk = 0;
    return;
  }
  int64_t s;
  if (bf16 && M >= 256 && (N >= 256 || (N > 128 && N <= 192))) {
    // 256 x 256 (or 256 x 192) tiles, one workgroup per CU: about one wave
    // of 256 of them
    const int64_t base = nblk * ((M + 255) / 256) * ((N + 255) / 256);
    s = 256 / base;
  } else {
    const int64_t base = nblk * ((M + 63) / 64) * ((N + 63) / 64);
    s = (2048 + base - 1) / base;
  }
  const int64_t smax_k = (K + 127) / 128;
  if (s > smax_k) s = smax_k;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  int64_t c = (K + s - 1) / s;
  c = (c + kSplitK - 1) / kSplitK * kSplitK;
  *chunk = c;
  *splits = (K + c - 1) / c;
}

}  // namespace

int make_problem_ex(int64_t in, int64_t out, int64_t mid, int64_t nb1, int64_t nb2, int64_t batch,
                    int dtype, int act, bool bias, Problem* pr) {
  if (dtype != MONARCH_F32 && dtype != MONARCH_BF16) return MONARCH_ERR_DTYPE;
  if (act != MONARCH_ACT_NONE && act != MONARCH_ACT_RELU) return MONARCH_ERR_DTYPE;
  if (in <= 0 || out <= 0 || mid <= 0 || nb1 <= 0 || nb2 <= 0 || batch < 0)
    return MONARCH_ERR_SHAPE;
  if (in >= kDimLimit || out >= kDimLimit || mid >= kDimLimit || batch >= kDimLimit ||
      nb1 >= kDimLimit || nb2 >= kDimLimit)
    return MONARCH_ERR_SHAPE;
  if (mid % nb1 || mid % nb2) return MONARCH_ERR_SHAPE;
  Problem p;
  p.in = in;
  p.out = out;
  p.mid = mid;
  p.b1 = nb1;
  p.b2 = nb2;
  p.q1i = (in + nb1 - 1) / nb1;
  p.q1o = mid / nb1;
  p.q2i = mid / nb2;
  p.q2o = (out + nb2 - 1) / nb2;
  p.in_ext = p.q1i * nb1;
  p.out_ext = p.q2o * nb2;
  if (p.in_ext >= kDimLimit || p.out_ext >= kDimLimit) return MONARCH_ERR_SHAPE;
  p.bias = bias;
  p.batch = batch;
  p.dtype = dtype;
  p.act = act;
  p.esize = dtype == MONARCH_BF16 ? 2 : 4;
  p.path = PATH_GENERIC;
  p.z_stage2_order = p.q1o % nb2 == 0;
  const bool whole = p.in_ext == in && p.out_ext == out && mid == out && !bias;
  if (batch > 0 && whole && sq_applicable(in, out, nb1, nb2, batch, dtype == MONARCH_BF16)) {
    p.path = PATH_SQ128;
    p.sq = sq_plan(batch, nb1);
    p.s2 = p.sq.w2_chunks;
    p.s1 = p.sq.b1_chunks;
  } else {
    if (batch > 0 && whole && sm_applicable(in, out, nb1, nb2, batch, dtype == MONARCH_BF16)) {
      p.path = PATH_SM32;
      sm_wgrad_split(batch, &p.s2, &p.kc2);
      p.s1 = p.s2, p.kc1 = p.kc2;
    } else {
      choose_splits(p.b2, p.q2o, p.q2i, batch, dtype == MONARCH_BF16, &p.s2, &p.kc2);
      choose_splits(p.b1, p.q1o, p.q1i, batch, dtype == MONARCH_BF16, &p.s1, &p.kc1);
    }
  }
  if (batch > 0) {
    size_t off = 0;
    p.ws_dz = off;
    off = align_up(off + static_cast<size_t>(batch) * mid * p.esize, 256);
    p.ws_p2 = off;
    off = align_up(off + static_cast<size_t>(p.s2) * nb2 * p.q2o * p.q2i * 4, 256);
    p.ws_p1 = off;
    off = align_up(off + static_cast<size_t>(p.s1) * nb1 * p.q1o * p.q1i * 4, 256);
    // dY in block-major order (sq path: panels, generic path: rows)
    p.ws_dv = off;
    off = align_up(off + static_cast<size_t>(batch) * p.out_ext * p.esize, 256);
    if (bias) {
      // bias-gradient partials: about 256 rows per chunk, at most 256 chunks
      int64_t chunks = (batch + 255) / 256;
      if (chunks > 256) chunks = 256;
      p.bias_chunk = (batch + chunks - 1) / chunks;
      p.bias_chunks = (batch + p.bias_chunk - 1) / p.bias_chunk;
      p.ws_pb = off;
      off = align_up(off + static_cast<size_t>(p.bias_chunks) * out * 4, 256);
    }
    p.ws_total = off;
  }
  *pr = p;
  return MONARCH_OK;
}

int make_problem(int64_t in, int64_t out, int64_t nb1, int64_t nb2, int64_t batch, int dtype,
                 int act, Problem* pr) {
  if (dtype != MONARCH_F32 && dtype != MONARCH_BF16) return MONARCH_ERR_DTYPE;
  if (act != MONARCH_ACT_NONE && act != MONARCH_ACT_RELU) return MONARCH_ERR_DTYPE;
  if (in <= 0 || out <= 0 || nb1 <= 0 || nb2 <= 0 || batch < 0) return MONARCH_ERR_SHAPE;
  if (in % nb1 || out % nb1 || out % nb2) return MONARCH_ERR_SHAPE;
  return make_problem_ex(in, out, out, nb1, nb2, batch, dtype, act, false, pr);
}

size_t workspace_bytes(const Problem& pr) { return pr.ws_total; }

Plan plan_fwd(const Problem& pr) {
  Plan p;
  if (pr.batch == 0) return p;
  if (pr.path == PATH_SQ128) {
    p.add(SQ_STAGE1_FWD);
    p.add(SQ_STAGE2_FWD);
    return p;
  }
  if (pr.path == PATH_SM32) {
    p.add(SM_FWD);
    return p;
  }
  p.add(GEN_STAGE1_FWD);
  p.add(GEN_STAGE2_FWD);
  return p;
}

Plan plan_bwd(const Problem& pr) {
  Plan p;
  if (pr.batch == 0) {
    p.add(ZERO_DW);
    return p;
  }
  if (pr.path == PATH_SQ128) {
    p.add(SQ_DV_PANELS);
    p.add(SQ_STAGE2_BWD_DATA);
    p.add(SQ_STAGE2_BWD_WEIGHT);
    p.add(SQ_STAGE1_BWD);
    p.add(REDUCE_DW);
    return p;
  }
  if (pr.path == PATH_SM32) {
    p.add(SM_BWD_DATA);
    p.add(SM_WGRAD);
    p.add(REDUCE_DW);
    return p;
  }
  p.add(GEN_DV_GATHER);
  if (pr.bias) p.add(GEN_BIAS_PARTIALS);
  p.add(GEN_STAGE2_BWD_DATA);
  p.add(GEN_STAGE2_BWD_WEIGHT);
  p.add(GEN_STAGE1_BWD_DATA);
  p.add(GEN_STAGE1_BWD_WEIGHT);
  p.add(REDUCE_DW);
  return p;
}

const char* step_name(StepKind k) {
  switch (k) {
    case GEN_DV_GATHER: return "generic_dv_gather";
    case GEN_BIAS_PARTIALS: return "generic_bias_partials";
    case GEN_STAGE1_FWD: return "generic_stage1_fwd";
    case GEN_STAGE2_FWD: return "generic_stage2_fwd";
    case GEN_STAGE2_BWD_DATA: return "generic_stage2_bwd_data";
    case GEN_STAGE2_BWD_WEIGHT: return "generic_stage2_bwd_weight";
    case GEN_STAGE1_BWD_DATA: return "generic_stage1_bwd_data";
    case GEN_STAGE1_BWD_WEIGHT: return "generic_stage1_bwd_weight";
    case REDUCE_DW: return "reduce_dw";
    case ZERO_DW: return "zero_dw";
    case SQ_DV_PANELS: return "sq128_dv_panels";
    case SQ_STAGE1_FWD: return "sq128_stage1_fwd";
    case SQ_STAGE2_FWD: return "sq128_stage2_fwd";
    case SQ_STAGE2_BWD_DATA: return "sq128_stage2_bwd_data";
    case SQ_STAGE2_BWD_WEIGHT: return "sq128_stage2_bwd_weight";
    case SQ_STAGE1_BWD: return "sq128_stage1_bwd";
    case SM_FWD: return "sm32_fwd";
    case SM_BWD_DATA: return "sm32_bwd_data";
    case SM_WGRAD: return "sm32_bwd_weight";
  }
  return "?";
}

hipError_t launch_step(StepKind k, const Problem& pr, const Buffers& b, hipStream_t s) {
  const bool bf16 = pr.dtype == MONARCH_BF16;
  char* ws = static_cast<char*>(b.ws);
  void* dz = ws ? ws + pr.ws_dz : nullptr;
  float* p2 = ws ? reinterpret_cast<float*>(ws + pr.ws_p2) : nullptr;
  float* p1 = ws ? reinterpret_cast<float*>(ws + pr.ws_p1) : nullptr;
  const void* mask = pr.act == MONARCH_ACT_RELU ? b.y : nullptr;
  void* dv = ws ? ws + pr.ws_dv : nullptr;
  float* pb = ws && pr.bias ? reinterpret_cast<float*>(ws + pr.ws_pb) : nullptr;
  GemmArgs a;
  switch (k) {
    case GEN_DV_GATHER:
      return launch_dv_gather(b.dy, mask, dv, pr.batch, pr.out, pr.b2, pr.q2o, bf16, s);
    case GEN_BIAS_PARTIALS:
      return launch_bias_partials(dv, pb, pr.batch, pr.bias_chunk, pr.bias_chunks, pr.out, pr.b2,
                                  pr.q2o, bf16, s);
    case GEN_STAGE1_FWD:
      // X is zero-padded to whole blocks: block r sums over k < in - r*q1i
      a.A = b.x;
      a.a_sb = pr.q1i, a.a_si = pr.in, a.a_sk = 1;
      a.k_lim = pr.in, a.k_lim_bs = pr.q1i;
      a.B = b.w1;
      a.b_sb = pr.q1o * pr.q1i, a.b_sk = 1;
      a.C = b.z_out;
      a.c_si = pr.mid;
      if (pr.z_stage2_order) {
        // column j = g*n1 + tt of block r is k = tt*b2 + g, stored at W
        // position g*q2i + r*n1 + tt
        const int64_t n1 = pr.q1o / pr.b2;
        a.nsplit = n1;
        a.b_sj_hi = pr.q1i, a.b_sj = pr.b2 * pr.q1i;
        a.c_sb = n1, a.c_sj_hi = pr.q2i, a.c_sj = 1;
      } else {
        a.b_sj = pr.q1i;
        a.c_sb = pr.q1o, a.c_sj = 1;
      }
      a.M = pr.batch, a.N = pr.q1o, a.K = pr.q1i, a.nblk = pr.b1;
      return launch_gemm(a, bf16, s);
    case GEN_STAGE2_FWD:
      // outputs past `out` are dropped; bias and ReLU in the epilogue
      a.A = b.z_out;
      if (pr.z_stage2_order)
        a.a_sb = pr.q2i, a.a_si = pr.mid, a.a_sk = 1;
      else
        a.a_sb = 1, a.a_si = pr.mid, a.a_sk = pr.b2;
      a.B = b.w2;
      a.b_sb = pr.q2o * pr.q2i, a.b_sk = 1, a.b_sj = pr.q2i;
      a.C = b.y_out;
      a.c_sb = 1, a.c_si = pr.out, a.c_sj = pr.b2, a.c_cols = pr.out < pr.out_ext ? pr.out : -1;
      a.bias = b.bias;
      a.M = pr.batch, a.N = pr.q2o, a.K = pr.q2i, a.nblk = pr.b2;
      a.relu = pr.act == MONARCH_ACT_RELU;
      return launch_gemm(a, bf16, s);
    case GEN_STAGE2_BWD_DATA:
      a.A = dv;
      a.a_sb = pr.q2o, a.a_si = pr.out_ext, a.a_sk = 1;
      a.B = b.w2;
      a.b_sb = pr.q2o * pr.q2i, a.b_sk = pr.q2i, a.b_sj = 1;
      a.C = dz;
      a.c_sb = 1, a.c_si = pr.mid, a.c_sj = pr.b2;
      a.M = pr.batch, a.N = pr.q2i, a.K = pr.q2o, a.nblk = pr.b2;
      return launch_gemm(a, bf16, s);
    case GEN_STAGE2_BWD_WEIGHT:
      a.A = dv;
      a.a_sb = pr.q2o, a.a_si = 1, a.a_sk = pr.out_ext;
      a.B = b.z;
      if (pr.z_stage2_order)
        a.b_sb = pr.q2i, a.b_sk = pr.mid, a.b_sj = 1;
      else
        a.b_sb = 1, a.b_sk = pr.mid, a.b_sj = pr.b2;
      a.partial = p2, a.splits = pr.s2, a.k_chunk = pr.kc2;
      a.M = pr.q2o, a.N = pr.q2i, a.K = pr.batch, a.nblk = pr.b2;
      return launch_gemm(a, bf16, s);
    case GEN_STAGE1_BWD_DATA:
      // dX of the padded input positions is dropped
      a.A = dz;
      a.a_sb = pr.q1o, a.a_si = pr.mid, a.a_sk = 1;
      a.B = b.w1;
      a.b_sb = pr.q1o * pr.q1i, a.b_sk = pr.q1i, a.b_sj = 1;
      a.C = b.dx;
      a.c_sb = pr.q1i, a.c_si = pr.in, a.c_sj = 1, a.c_cols = pr.in < pr.in_ext ? pr.in : -1;
      a.M = pr.batch, a.N = pr.q1i, a.K = pr.q1o, a.nblk = pr.b1;
      return launch_gemm(a, bf16, s);
    case GEN_STAGE1_BWD_WEIGHT:
      // padded input positions read as zero: their weight gradient is 0
      a.A = dz;
      a.a_sb = pr.q1o, a.a_si = 1, a.a_sk = pr.mid;
      a.B = b.x;
      a.b_sb = pr.q1i, a.b_sk = pr.in, a.b_sj = 1;
      a.n_lim = pr.in, a.n_lim_bs = pr.q1i;
      a.partial = p1, a.splits = pr.s1, a.k_chunk = pr.kc1;
      a.M = pr.q1o, a.N = pr.q1i, a.K = pr.batch, a.nblk = pr.b1;
      return launch_gemm(a, bf16, s);
    case REDUCE_DW: {
      ReduceArgs r2, r1, rb;
      r2.partial = p2, r2.out = b.dw2, r2.n = pr.b2 * pr.q2o * pr.q2i, r2.splits = pr.s2;
      r1.partial = p1, r1.out = b.dw1, r1.n = pr.b1 * pr.q1o * pr.q1i, r1.splits = pr.s1;
      if (pr.bias) rb.partial = pb, rb.out = b.dbias, rb.n = pr.out, rb.splits = pr.bias_chunks;
      return launch_reduce_partials(r2, r1, rb, bf16, s);
    }
    case SQ_DV_PANELS:
      return sq_launch_dv_panels(b.dy, mask, dv, pr.batch, pr.b2, s);
    case SQ_STAGE1_FWD:
      return sq_launch_stage1_fwd(b.x, b.w1, b.z_out, pr.batch, pr.b1, pr.sq, s);
    case SQ_STAGE2_FWD:
      return sq_launch_stage2_fwd(b.z_out, b.w2, b.y_out, pr.batch, pr.b2,
                                  pr.act == MONARCH_ACT_RELU, pr.sq, s);
    case SQ_STAGE2_BWD_DATA:
      return sq_launch_stage2_bwd_data(dv, b.w2, dz, pr.batch, pr.b2, pr.sq, s);
    case SQ_STAGE2_BWD_WEIGHT:
      return sq_launch_stage2_bwd_weight(dv, b.z, p2, pr.batch, pr.b2, pr.sq, s);
    case SQ_STAGE1_BWD:
      return sq_launch_stage1_bwd(dz, b.x, b.w1, b.dx, p1, pr.batch, pr.b1, pr.sq, s);
    case SM_FWD:
      return sm_launch_fwd(b.x, b.w1, b.w2, b.y_out, b.z_out, pr.batch, pr.b1,
                           pr.act == MONARCH_ACT_RELU, s);
    case SM_BWD_DATA:
      return sm_launch_bwd_data(b.dy, mask, b.w1, b.w2, b.dx, dv, dz, pr.batch, pr.b1, s);
    case SM_WGRAD:
      return sm_launch_wgrad(dv, b.z, dz, b.x, p2, p1, pr.batch, pr.b1, s);
    case ZERO_DW: {
      hipError_t e = launch_zero(b.dw2, static_cast<size_t>(pr.b2 * pr.q2o * pr.q2i) * pr.esize, s);
      if (e != hipSuccess) return e;
      e = launch_zero(b.dw1, static_cast<size_t>(pr.b1 * pr.q1o * pr.q1i) * pr.esize, s);
      if (e != hipSuccess || !pr.bias) return e;
      return launch_zero(b.dbias, static_cast<size_t>(pr.out) * pr.esize, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace monarch
