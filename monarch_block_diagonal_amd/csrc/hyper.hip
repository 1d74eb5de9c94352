// k-factor ("hypercube") Monarch layer: planning of its rounds (scatterbrain
// issues page, "hypercube" thread: the N units form a lattice [n_1, ..., n_k];
// round j multiplies along axis j with one matrix per index of the other
// axes, rounds in axis order).
//
// A round is one launch: the fiber kernel (fiber.hip) for bf16 fibers of 16,
// 24 or 32 units, else the tiled GEMM (tiled.hip) with one block per fiber of
// its axis; the weight gradients likewise. Layouts: L_j denotes the lattice with axis j moved to
// the end (the other axes in order), so a fiber of round j is a contiguous
// run of n_j elements and the fiber index equals the weight index; L_{k-1} is
// the natural row-major layout. A round reads and writes L_j, and an axis
// swap moves the result on: L_j = [pre][n_{j+1}][mid][n_j] and L_{j+1} =
// [pre][n_j][mid][n_{j+1}] (pre = axes before j, mid = axes after j+1), so
// the change is the swap of the outer and inner axis of [n_{j+1}][mid][n_j],
// a pass at copy speed where writing L_{j+1} from the GEMM would scatter
// every element. The forward transposes x into L_0, runs round j into y
// (scratch until the last round) and swaps it into the saved slot j + 1; it
// keeps x in L_0 and the inputs of rounds 1..k-1 (k saved tensors). The
// backward walks the rounds in reverse: the weight gradient of round j sums
// g_{j+1}[fiber]ᵀ · input_j[fiber] over the batch (split in chunks, summed in
// a fixed order), and the data gradient g_j = F_jᵀ g_{j+1}, written in L_j,
// is swapped into L_{j-1}; g_0 is transposed back into dx. A one-dimensional
// lattice needs no layout change. Where a swap's arrays are small, a bf16
// fiber round and the swap after it are one kernel (fiber_swap_kernel), in
// place in the backward.
#include "hyper.h"
#include "monarch.h"

namespace monarch {
namespace {

constexpr int64_t kLimit = int64_t(1) << 31;

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// batch split of a weight-gradient GEMM with nblk blocks of n x n: about
// 2048 tiles of 64 x 64 in flight, chunks of at least 128 rows, multiples of
// kSplitK
void splits_for(int64_t nblk, int64_t n, int64_t K, int64_t* splits, int64_t* chunk) {
  if (K <= 0) {
    *splits = 1;
    *chunk = kSplitK;
    return;
  }
  const int64_t t = (n + 63) / 64;
  const int64_t base = nblk * t * t;
  int64_t s = (2048 + base - 1) / base;
  const int64_t smax = (K + 127) / 128;
  if (s > smax) s = smax;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  int64_t c = (K + s - 1) / s;
  c = (c + kSplitK - 1) / kSplitK * kSplitK;
  *chunk = c;
  *splits = (K + c - 1) / c;
}

int64_t prod(const int64_t* d, int lo, int hi) {
  int64_t p = 1;
  for (int i = lo; i < hi; ++i) p *= d[i];
  return p;
}

// round j on fibers of n_j by the fiber kernel (inputs and outputs in L_j)
void set_fiber(SeqStep& st, const HyperProblem& hp, int j, const void* in, const void* w,
               void* out) {
  st.kind = SEQ_FIBER;
  st.t_in = in, st.t_out = out, st.f_w = w;
  st.t_rows = hp.batch, st.f_N = hp.N, st.f_n = hp.dims[j];
}

// arrays of the swap after round j: L_j = [pre][A][M][n_j] with A = n_{j+1}
// (up) or n_{j-1} (down) and M the product of the axes after the pair
void swap_array(const HyperProblem& hp, int j, bool up, int64_t* A, int64_t* M) {
  const int lo = up ? j : j - 1;
  *A = up ? hp.dims[lo + 1] : hp.dims[lo];
  *M = prod(hp.dims, lo + 2, hp.k);
}

// round j on fibers together with the swap that follows it, when the
// swap's arrays fit the fused kernel
bool set_fiber_swap(SeqStep& st, const HyperProblem& hp, int j, bool up, const void* in,
                    const void* w, void* out) {
  int64_t A, M;
  swap_array(hp, j, up, &A, &M);
  if (!fiber_swap_applicable(hp.dims[j], A, M, hp.dtype == MONARCH_BF16)) return false;
  st.kind = SEQ_FIBER_SWAP;
  st.t_in = in, st.t_out = out, st.f_w = w;
  st.t_rows = hp.batch, st.f_N = hp.N, st.f_n = hp.dims[j], st.t_A = A, st.t_M = M;
  return true;
}

// round 0 joined with the layout change natural <-> L_0 (bf16 fibers of 16,
// 24 or 32 units, a multiple of 8 of them)
bool strided_round0(const HyperProblem& hp) {
  return hp.k > 1 && fiber_strided_applicable(hp.dims[0], hp.N, hp.dtype == MONARCH_BF16);
}
void set_strided(SeqStep& st, const HyperProblem& hp, int dir, const void* in, const void* w,
                 void* out, void* save) {
  st.kind = SEQ_FIBER_STRIDED;
  st.t_in = in, st.t_out = out, st.f_w = w, st.f_save = save, st.f_dir = dir;
  st.t_rows = hp.batch, st.f_N = hp.N, st.f_n = hp.dims[0];
}

// the axis swap L_j -> L_{j+1} (up = true) or L_j -> L_{j-1} (up = false)
void set_swap(SeqStep& st, const HyperProblem& hp, int j, bool up, const void* in, void* out) {
  const int lo = up ? j : j - 1;   // the swap exchanges axes lo and lo + 1
  st.kind = SEQ_SWAP;
  st.name = "hyper_permute";
  st.t_in = in, st.t_out = out;
  st.t_rows = hp.batch * prod(hp.dims, 0, lo);
  st.t_M = prod(hp.dims, lo + 2, hp.k);
  // L_lo = [pre][n_{lo+1}][mid][n_lo], L_{lo+1} = [pre][n_lo][mid][n_{lo+1}]
  st.t_A = up ? hp.dims[lo + 1] : hp.dims[lo];
  st.t_C = up ? hp.dims[lo] : hp.dims[lo + 1];
}

}  // namespace

int make_hyper(int ndims, const int64_t* dims, int64_t batch, int dtype, HyperProblem* hp) {
  if (dtype != MONARCH_F32 && dtype != MONARCH_BF16) return MONARCH_ERR_DTYPE;
  if (ndims < 1 || ndims > kHyperMaxDims || !dims || batch < 0 || batch >= kLimit)
    return MONARCH_ERR_SHAPE;
  HyperProblem p;
  p.k = ndims;
  int64_t n = 1;
  for (int i = 0; i < ndims; ++i) {
    if (dims[i] <= 0 || dims[i] >= kLimit) return MONARCH_ERR_SHAPE;
    p.dims[i] = dims[i];
    n *= dims[i];
    if (n >= kLimit) return MONARCH_ERR_SHAPE;
  }
  p.N = n;
  p.batch = batch;
  p.dtype = dtype;
  p.esize = dtype == MONARCH_BF16 ? 2 : 4;
  size_t off = 0;
  if (batch > 0) {
    for (int g = 0; g < 2; ++g) {
      p.ws_g[g] = off;
      off = align256(off + static_cast<size_t>(batch) * n * p.esize);
    }
    for (int j = 0; j < ndims; ++j) {
      const int64_t nj = p.dims[j];
      if (fiber_applicable(nj, dtype == MONARCH_BF16))
        fiber_wgrad_split(batch, n, nj, &p.splits[j], &p.chunk[j]);
      else
        splits_for(n / nj, nj, batch, &p.splits[j], &p.chunk[j]);
      p.ws_part[j] = off;
      off = align256(off + static_cast<size_t>(p.splits[j]) * (n / nj) * nj * nj * 4);
    }
    size_t wt = 0;
    for (int j = 0; j < ndims; ++j)
      if (fiber_applicable(p.dims[j], dtype == MONARCH_BF16))
        wt = static_cast<size_t>(n) * p.dims[j] * p.esize > wt ? static_cast<size_t>(n) * p.dims[j] * p.esize : wt;
    p.ws_wt = off;
    off = align256(off + wt);
  }
  p.ws_total = off;
  *hp = p;
  return MONARCH_OK;
}

int64_t hyper_saved_elems(const HyperProblem& hp) { return hp.k > 1 ? hp.k * hp.batch * hp.N : 0; }

int hyper_plan_fwd(const HyperProblem& hp, const HyperBuffers& b, SeqStep* steps) {
  if (hp.batch == 0) return 0;
  const int k = hp.k;
  const int64_t BN = hp.batch * hp.N;
  // saved slot j: the input of round j in L_j (slot 0 = x)
  auto slot = [&](int sidx) { return byte_at(b.saved, sidx * BN * hp.esize); };
  int ns = 0;
  const bool strided = strided_round0(hp);
  if (k > 1 && !strided) {
    SeqStep& st = steps[ns++];
    st.kind = SEQ_SWAP;
    st.name = "hyper_transpose";
    st.t_in = b.x, st.t_out = slot(0);
    st.t_rows = hp.batch, st.t_A = hp.dims[0], st.t_M = 1, st.t_C = hp.N / hp.dims[0];
  }
  for (int j = 0; j < k; ++j) {
    const int64_t n = hp.dims[j];
    const void* in = k > 1 ? static_cast<const void*>(slot(j)) : b.x;   // L_j
    if (j == 0 && strided) {
      // x (natural) -> its L_0 copy in slot 0 and round 0's output in L_0
      set_strided(steps[ns], hp, 0, b.x, b.w[0], b.y, slot(0));
      steps[ns++].name = "hyper_transpose_round_fwd";
      set_swap(steps[ns++], hp, j, true, b.y, slot(j + 1));
      continue;
    }
    if (j < k - 1 && set_fiber_swap(steps[ns], hp, j, true, in, b.w[j], slot(j + 1))) {
      steps[ns++].name = "hyper_round_fwd_swap";
      continue;
    }
    SeqStep& st = steps[ns++];
    st.name = "hyper_round_fwd";
    if (fiber_applicable(n, hp.dtype == MONARCH_BF16)) {
      set_fiber(st, hp, j, in, b.w[j], b.y);
    } else {
      st.kind = SEQ_GEMM;
      GemmArgs& a = st.g;
      a.A = in;
      a.a_sb = n, a.a_sk = 1, a.a_si = hp.N;
      a.B = b.w[j];
      a.b_sb = n * n, a.b_sk = 1, a.b_sj = n;
      a.C = b.y;                                                // L_j
      a.c_sb = n, a.c_sj = 1, a.c_si = hp.N;
      a.M = hp.batch, a.N = n, a.K = n, a.nblk = hp.N / n;
    }
    if (j < k - 1) set_swap(steps[ns++], hp, j, true, b.y, slot(j + 1));
  }
  return ns;
}

int hyper_plan_bwd(const HyperProblem& hp, const HyperBuffers& b, SeqStep* steps) {
  const int k = hp.k;
  int ns = 0;
  if (hp.batch == 0) {
    for (int j = 0; j < k; ++j) {
      SeqStep& st = steps[ns++];
      st.kind = SEQ_ZERO;
      st.name = "zero_dw";
      st.zero_ptr = b.dw[j];
      st.zero_bytes = static_cast<size_t>(hp.N) * hp.dims[j] * hp.esize;
    }
    return ns;
  }
  const int64_t BN = hp.batch * hp.N;
  void* ws = b.ws;
  // input of round j in L_j: the saved copies (slot j), or x itself when the
  // lattice has one dimension
  auto input = [&](int j) -> const void* {
    return k > 1 ? byte_at(b.saved_in, j * BN * hp.esize) : b.x;
  };
  // g_{j+1} (gradient w.r.t. round j's output, in L_j) is dy for the last
  // round, else buffer 1; round j's data gradient goes to buffer 0 (in L_j)
  // and is swapped into buffer 1 (in L_{j-1})
  void* g0 = byte_at(ws, hp.ws_g[0]);
  void* g1 = byte_at(ws, hp.ws_g[1]);
  for (int j = k - 1; j >= 0; --j) {
    const int64_t n = hp.dims[j], nf = hp.N / n;
    const void* g = j == k - 1 ? b.dy : g1;
    const bool fib = fiber_applicable(n, hp.dtype == MONARCH_BF16);
    if (fib) {
      SeqStep& st = steps[ns++];
      st.kind = SEQ_FIBER_WGRAD;
      st.name = "hyper_round_bwd_weight";
      st.t_in = g, st.f_in2 = input(j);
      st.f_part = reinterpret_cast<float*>(byte_at(ws, hp.ws_part[j]));
      st.t_rows = hp.batch, st.f_N = hp.N, st.f_n = n, st.f_chunk = hp.chunk[j];
    } else {
      SeqStep& st = steps[ns++];
      st.kind = SEQ_GEMM;
      st.name = "hyper_round_bwd_weight";
      GemmArgs& a = st.g;
      a.A = g;
      a.a_sb = n, a.a_si = 1, a.a_sk = hp.N;
      a.B = input(j);
      a.b_sb = n, a.b_sk = hp.N, a.b_sj = 1;
      a.partial = reinterpret_cast<float*>(byte_at(ws, hp.ws_part[j]));
      a.splits = hp.splits[j], a.k_chunk = hp.chunk[j];
      a.M = n, a.N = n, a.K = hp.batch, a.nblk = nf;
    }
    void* gout = k > 1 ? g0 : b.dx;                // L_j
    if (fib) {
      // per-fiber transposed weights, then the fiber products with them
      void* wt = byte_at(ws, hp.ws_wt);
      SeqStep& sw = steps[ns++];
      sw.kind = SEQ_SWAP;
      sw.name = "hyper_weight_transpose";
      sw.t_in = b.w[j], sw.t_out = wt;
      sw.t_rows = nf, sw.t_A = n, sw.t_M = 1, sw.t_C = n;
      if (j == 0 && strided_round0(hp)) {
        // round 0's data product straight into dx (natural layout)
        set_strided(steps[ns], hp, 1, g, wt, b.dx, nullptr);
        steps[ns++].name = "hyper_round_bwd_data_transpose";
        continue;
      }
      // g1 may be both the input and the output: the fused kernel reads
      // each region before writing it
      if (j > 0 && set_fiber_swap(steps[ns], hp, j, false, g, wt, g1)) {
        steps[ns++].name = "hyper_round_bwd_data_swap";
        continue;
      }
      SeqStep& st = steps[ns++];
      st.name = "hyper_round_bwd_data";
      set_fiber(st, hp, j, g, wt, gout);
    } else {
      SeqStep& st = steps[ns++];
      st.kind = SEQ_GEMM;
      st.name = "hyper_round_bwd_data";
      GemmArgs& a = st.g;
      a.A = g;
      a.a_sb = n, a.a_si = hp.N, a.a_sk = 1;
      a.B = b.w[j];
      a.b_sb = n * n, a.b_sk = n, a.b_sj = 1;
      a.C = gout;
      a.c_sb = n, a.c_sj = 1, a.c_si = hp.N;
      a.M = hp.batch, a.N = n, a.K = n, a.nblk = nf;
    }
    if (j > 0) set_swap(steps[ns++], hp, j, false, g0, g1);
  }
  if (k > 1 && !strided_round0(hp)) {
    SeqStep& st = steps[ns++];
    st.kind = SEQ_SWAP;
    st.name = "hyper_transpose";
    st.t_in = g0, st.t_out = b.dx;
    st.t_rows = hp.batch, st.t_A = hp.N / hp.dims[0], st.t_M = 1, st.t_C = hp.dims[0];
  }
  // fixed-order sums of the weight-gradient chunks, three rounds per launch
  for (int j0 = 0; j0 < k; j0 += 3) {
    SeqStep& st = steps[ns++];
    st.kind = SEQ_REDUCE;
    st.name = "reduce_dw";
    for (int i = 0; i < 3 && j0 + i < k; ++i) {
      const int j = j0 + i;
      st.r[i].partial = reinterpret_cast<const float*>(byte_at(ws, hp.ws_part[j]));
      st.r[i].out = b.dw[j];
      st.r[i].n = hp.N * hp.dims[j];
      st.r[i].splits = hp.splits[j];
    }
  }
  return ns;
}

hipError_t seq_launch(const SeqStep& st, bool bf16, hipStream_t s) {
  switch (st.kind) {
    case SEQ_GEMM: return launch_gemm(st.g, bf16, s);
    case SEQ_REDUCE: return launch_reduce_partials(st.r[0], st.r[1], st.r[2], bf16, s);
    case SEQ_ZERO: return launch_zero(st.zero_ptr, st.zero_bytes, s);
    case SEQ_SWAP:
      return launch_swap(st.t_in, st.t_out, st.t_rows, st.t_A, st.t_M, st.t_C, bf16, s,
                         st.t_accum != 0);
    case SEQ_FIBER:
      return launch_fiber(st.t_in, st.f_w, st.t_out, st.t_rows, st.f_N, st.f_n, bf16, s);
    case SEQ_FIBER_SWAP:
      return launch_fiber_swap(st.t_in, st.f_w, st.t_out, st.t_rows, st.f_N, st.f_n, st.t_A,
                               st.t_M, bf16, s);
    case SEQ_FIBER_STRIDED:
      return launch_fiber_strided(st.t_in, st.f_w, st.t_out, st.f_save, st.t_rows, st.f_N, st.f_n,
                                  st.f_dir, bf16, s);
    case SEQ_FIBER_WGRAD:
      return launch_fiber_wgrad(st.t_in, st.f_in2, st.f_part, st.t_rows, st.f_N, st.f_n,
                                st.f_chunk, bf16, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace monarch
