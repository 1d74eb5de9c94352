// DYAD-style layer (DYAD page, abstract: a weight matrix that is the sum of
// two matrices, each a permutation of a block-sparse one, stored as 3D
// tensors): with nb blocks, qi = in/nb, qo = out/nb,
//   Y = X · (BD(A) + Q_out · BD(B) · P_in)ᵀ,
//   term A: Y[b, r*qo + k] += sum_s A[r,k,s] X[b, r*qi + s]   (contiguous blocks)
//   term B: Y[b, p*nb + g] += sum_t B[g,p,t] X[b, t*nb + g]   (residue-g features)
// Term B's operands are strided by nb. An axis swap (generic.hip) first
// gathers X into block-major order, Xp[b, g*qi + t] = X[b, t*nb + g] (and the
// backward also dY, dYp[b, g*qo + p] = dY[b, p*nb + g]), so that every GEMM
// reads 16-byte pieces. Term B's results are written block-major too (the
// stride-nb positions would take element-by-element stores) and added into
// the output by an accumulating axis swap. The forward runs term B into its
// block-major rows, term A into Y, and adds term B; the backward takes both
// weight gradients as batch-split sums (reduced in a fixed order), term B's
// data product into block-major rows (in Xp's place), term A's into dX, and
// adds term B's.
#include "dyad.h"
#include "monarch.h"

namespace monarch {
namespace {

constexpr int64_t kLimit = int64_t(1) << 31;

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

void splits_for(int64_t nblk, int64_t M, int64_t N, int64_t K, bool bf16, int64_t* splits,
                int64_t* chunk) {
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
  const int64_t smax = (K + 127) / 128;
  if (s > smax) s = smax;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  int64_t c = (K + s - 1) / s;
  c = (c + kSplitK - 1) / kSplitK * kSplitK;
  *chunk = c;
  *splits = (K + c - 1) / c;
}

// term A and term B GEMMs of the forward
void term_a_fwd(GemmArgs& a, const DyadProblem& dp, const void* x, const void* wa, void* y) {
  a.A = x, a.a_sb = dp.qi, a.a_si = dp.in, a.a_sk = 1;
  a.B = wa, a.b_sb = dp.qo * dp.qi, a.b_sk = 1, a.b_sj = dp.qi;
  a.C = y, a.c_sb = dp.qo, a.c_si = dp.out, a.c_sj = 1;
  a.M = dp.batch, a.N = dp.qo, a.K = dp.qi, a.nblk = dp.nb;
}
// term B into block-major rows, yp[b, g*qo + p] (added into Y by an axis
// swap: its stride-nb positions would be written element by element)
void term_b_fwd(GemmArgs& a, const DyadProblem& dp, const void* xp, const void* wb, void* yp) {
  a.A = xp, a.a_sb = dp.qi, a.a_si = dp.in, a.a_sk = 1;
  a.B = wb, a.b_sb = dp.qo * dp.qi, a.b_sk = 1, a.b_sj = dp.qi;
  a.C = yp, a.c_sb = dp.qo, a.c_si = dp.out, a.c_sj = 1;
  a.M = dp.batch, a.N = dp.qo, a.K = dp.qi, a.nblk = dp.nb;
}
// [rows][a][c] -> [rows][c][a], one row of `cols` = a*c elements per batch row
void gather(SeqStep& st, const char* name, const void* in, void* out, int64_t rows, int64_t a,
            int64_t c) {
  st.kind = SEQ_SWAP;
  st.name = name;
  st.t_in = in, st.t_out = out;
  st.t_rows = rows, st.t_A = a, st.t_M = 1, st.t_C = c;
}

}  // namespace

int make_dyad(int64_t in, int64_t out, int64_t nb, int64_t batch, int dtype, DyadProblem* dp) {
  if (dtype != MONARCH_F32 && dtype != MONARCH_BF16) return MONARCH_ERR_DTYPE;
  if (in <= 0 || out <= 0 || nb <= 0 || batch < 0) return MONARCH_ERR_SHAPE;
  if (in >= kLimit || out >= kLimit || batch >= kLimit || in % nb || out % nb)
    return MONARCH_ERR_SHAPE;
  DyadProblem p;
  p.in = in, p.out = out, p.nb = nb, p.qi = in / nb, p.qo = out / nb, p.batch = batch;
  p.dtype = dtype;
  p.esize = dtype == MONARCH_BF16 ? 2 : 4;
  if (batch > 0) {
    splits_for(nb, p.qo, p.qi, batch, dtype == MONARCH_BF16, &p.splits, &p.chunk);
    const size_t part = static_cast<size_t>(p.splits) * nb * p.qo * p.qi * 4;
    p.ws_pa = 0;
    p.ws_pb = align256(part);
    p.ws_xp = align256(p.ws_pb + part);
    p.ws_dyp = align256(p.ws_xp + static_cast<size_t>(batch) * in * p.esize);
    p.ws_total = align256(p.ws_dyp + static_cast<size_t>(batch) * out * p.esize);
    p.ws_fwd_yp = align256(static_cast<size_t>(batch) * in * p.esize);
    p.ws_fwd = align256(p.ws_fwd_yp + static_cast<size_t>(batch) * out * p.esize);
  }
  *dp = p;
  return MONARCH_OK;
}

int dyad_plan_fwd(const DyadProblem& dp, const DyadBuffers& b, SeqStep* steps) {
  if (dp.batch == 0) return 0;
  void* xp = b.ws;   // the forward's workspace: Xp, then term B's block-major rows
  void* yp = byte_at(b.ws, dp.ws_fwd_yp);
  gather(steps[0], "dyad_gather_x", b.x, xp, dp.batch, dp.qi, dp.nb);
  steps[1].kind = SEQ_GEMM;
  steps[1].name = "dyad_term_b_fwd";
  term_b_fwd(steps[1].g, dp, xp, b.wb, yp);
  steps[2].kind = SEQ_GEMM;
  steps[2].name = "dyad_term_a_fwd";
  term_a_fwd(steps[2].g, dp, b.x, b.wa, b.y);
  // Y[b, p*nb + g] += yp[b, g*qo + p]
  gather(steps[3], "dyad_add_term_b", yp, b.y, dp.batch, dp.nb, dp.qo);
  steps[3].t_accum = 1;
  return 4;
}

int dyad_plan_bwd(const DyadProblem& dp, const DyadBuffers& b, SeqStep* steps) {
  const size_t wbytes = static_cast<size_t>(dp.nb * dp.qo * dp.qi) * dp.esize;
  if (dp.batch == 0) {
    steps[0].kind = SEQ_ZERO, steps[0].name = "zero_dw";
    steps[0].zero_ptr = b.dwa, steps[0].zero_bytes = wbytes;
    steps[1].kind = SEQ_ZERO, steps[1].name = "zero_dw";
    steps[1].zero_ptr = b.dwb, steps[1].zero_bytes = wbytes;
    return 2;
  }
  float* pa = reinterpret_cast<float*>(byte_at(b.ws, dp.ws_pa));
  float* pb = reinterpret_cast<float*>(byte_at(b.ws, dp.ws_pb));
  void* xp = byte_at(b.ws, dp.ws_xp);
  void* dyp = byte_at(b.ws, dp.ws_dyp);
  int n = 0;
  gather(steps[n++], "dyad_gather_x", b.x, xp, dp.batch, dp.qi, dp.nb);
  gather(steps[n++], "dyad_gather_dy", b.dy, dyp, dp.batch, dp.qo, dp.nb);
  {
    // dA[r] = sum_b dY[b, r-block]ᵀ X[b, r-block]
    SeqStep& st = steps[n++];
    st.name = "dyad_term_a_bwd_weight";
    GemmArgs& a = st.g;
    a.A = b.dy, a.a_sb = dp.qo, a.a_si = 1, a.a_sk = dp.out;
    a.B = b.x, a.b_sb = dp.qi, a.b_sk = dp.in, a.b_sj = 1;
    a.partial = pa, a.splits = dp.splits, a.k_chunk = dp.chunk;
    a.M = dp.qo, a.N = dp.qi, a.K = dp.batch, a.nblk = dp.nb;
  }
  {
    // dB[g] = sum_b dYp[b, g*qo + p] Xp[b, g*qi + t]
    SeqStep& st = steps[n++];
    st.name = "dyad_term_b_bwd_weight";
    GemmArgs& a = st.g;
    a.A = dyp, a.a_sb = dp.qo, a.a_si = 1, a.a_sk = dp.out;
    a.B = xp, a.b_sb = dp.qi, a.b_sk = dp.in, a.b_sj = 1;
    a.partial = pb, a.splits = dp.splits, a.k_chunk = dp.chunk;
    a.M = dp.qo, a.N = dp.qi, a.K = dp.batch, a.nblk = dp.nb;
  }
  // term B's data product goes to block-major rows in Xp's place (both
  // weight products, which read Xp, come first)
  void* dxp = xp;
  {
    // dXp[b, g*qi + t] = sum_p dYp[b, g*qo + p] B[g,p,t]
    SeqStep& st = steps[n++];
    st.name = "dyad_term_b_bwd_data";
    GemmArgs& a = st.g;
    a.A = dyp, a.a_sb = dp.qo, a.a_si = dp.out, a.a_sk = 1;
    a.B = b.wb, a.b_sb = dp.qo * dp.qi, a.b_sk = dp.qi, a.b_sj = 1;
    a.C = dxp, a.c_sb = dp.qi, a.c_si = dp.in, a.c_sj = 1;
    a.M = dp.batch, a.N = dp.qi, a.K = dp.qo, a.nblk = dp.nb;
  }
  {
    // dX[b, r*qi + s] = sum_k dY[b, r*qo + k] A[r,k,s]
    SeqStep& st = steps[n++];
    st.name = "dyad_term_a_bwd_data";
    GemmArgs& a = st.g;
    a.A = b.dy, a.a_sb = dp.qo, a.a_si = dp.out, a.a_sk = 1;
    a.B = b.wa, a.b_sb = dp.qo * dp.qi, a.b_sk = dp.qi, a.b_sj = 1;
    a.C = b.dx, a.c_sb = dp.qi, a.c_si = dp.in, a.c_sj = 1;
    a.M = dp.batch, a.N = dp.qi, a.K = dp.qo, a.nblk = dp.nb;
  }
  // dX[b, t*nb + g] += dXp[b, g*qi + t]
  gather(steps[n], "dyad_add_term_b", dxp, b.dx, dp.batch, dp.nb, dp.qi);
  steps[n++].t_accum = 1;
  {
    SeqStep& st = steps[n++];
    st.kind = SEQ_REDUCE;
    st.name = "reduce_dw";
    const int64_t nw = dp.nb * dp.qo * dp.qi;
    st.r[0].partial = pa, st.r[0].out = b.dwa, st.r[0].n = nw, st.r[0].splits = dp.splits;
    st.r[1].partial = pb, st.r[1].out = b.dwb, st.r[1].n = nw, st.r[1].splits = dp.splits;
  }
  return n;
}

}  // namespace monarch
