// Host-side launchers of the Monarch kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace monarch {

// A batched GEMM over independent blocks with arbitrary element strides:
//   C[blk](i, j) = act( sum_k A[blk](i, k) * B[blk](k, j) ),  i < M, j < N, k < K
// with A element (blk, i, k) at A + blk*a_sb + i*a_si + k*a_sk (elements of the
// I/O type), likewise B and C. Every step of the two-stage Monarch product and
// of its backward pass is one such GEMM whose strides encode the block layout
// and the stride permutation. When `mask` is set, A(blk, i, k) is replaced by
// 0 wherever mask at the same offset is <= 0 (ReLU derivative). When
// `partial` is set, K is cut into `splits` chunks of k_chunk and chunk s writes
// its fp32 sum to partial[((s*nblk + blk)*M + i)*N + j] instead of C.
// When nsplit > 0 (not with `partial`), column j is split as
// (j / nsplit, j % nsplit) and sits at (j / nsplit)*b_sj_hi + (j % nsplit)*b_sj
// in B and (j / nsplit)*c_sj_hi + (j % nsplit)*c_sj in C: a reordering of the
// output columns that lets stage 1 write its result in stage 2's order.
struct GemmArgs {
  const void* A = nullptr;
  const void* B = nullptr;
  void* C = nullptr;
  const void* mask = nullptr;
  float* partial = nullptr;
  int64_t a_sb = 0, a_si = 0, a_sk = 0;
  int64_t b_sb = 0, b_sk = 0, b_sj = 0;
  int64_t c_sb = 0, c_si = 0, c_sj = 0;
  int64_t nsplit = 0, b_sj_hi = 0, c_sj_hi = 0;
  // Zero padding and truncation (all optional, -1 = none): in block blk only
  // k < k_lim - blk*k_lim_bs takes part in the sum (A and B), only B columns
  // j < n_lim - blk*n_lim_bs are read (others count as zero), and only C
  // entries whose row-relative offset blk*c_sb + (column offset) is below
  // c_cols are written.
  int64_t k_lim = -1, k_lim_bs = 0, n_lim = -1, n_lim_bs = 0, c_cols = -1;
  // Optional bias (I/O type) added before `relu`, indexed by the row-relative
  // C offset.
  const void* bias = nullptr;
  // accum: C += the product (C read back before the store; not with `partial`)
  int accum = 0;
  int64_t M = 0, N = 0, K = 0;
  int64_t nblk = 1;
  int64_t splits = 1;
  int64_t k_chunk = 0;
  int relu = 0;
  // set by launch_gemm: C columns are contiguous and every 4-column group is
  // aligned and inside or outside the limits as a whole (4-wide epilogue)
  int cvec = 0;
};

// Reduction-chunk granularity of batch-split GEMMs (a multiple of both
// kernels' K steps).
constexpr int kSplitK = 64;

// Runs any GemmArgs: the block-diagonal kernel (bd_mode) or the K-split
// kernel (skinny_mode) where those take the product, otherwise the tiled
// GEMM (tiled.hip), whose operands move as 16-byte pieces when they are
// contiguous along a tile dimension with 16-byte aligned rows, element by
// element otherwise.
hipError_t launch_gemm(const GemmArgs& a, bool bf16, hipStream_t s);

// dV[b, g*q2o + p] = dY[b, p*b2 + g] for p*b2 + g < out, else 0, times
// 1[Y > 0] when ymask is set: dY (and the ReLU derivative) gathered into the
// block-major order of stage 2's backward products. dY and Y are rows x out,
// dV is rows x (b2*q2o).
hipError_t launch_dv_gather(const void* dy, const void* ymask, void* dv, int64_t rows, int64_t out,
                            int64_t b2, int64_t q2o, bool bf16, hipStream_t s);

// Per-fiber products of a lattice round on fibers of n (bf16, n in
// {16, 24, 32}): out[b, f*n + p] = sum_t w[f][p][t] in[b, f*n + t] for
// `batch` rows of N elements (fiber.hip).
bool fiber_applicable(int64_t n, bool bf16);
hipError_t launch_fiber(const void* in, const void* w, void* out, int64_t batch, int64_t N,
                        int64_t n, bool bf16, hipStream_t s);
// Weight gradient of such a round as fp32 partials [splits][N/n][n][n]:
// partial[c][f][p][t] = sum over the rows of chunk c of g[b, f*n + p]
// in[b, f*n + t]; fiber_wgrad_split picks the chunks (multiples of 32 rows).
void fiber_wgrad_split(int64_t batch, int64_t N, int64_t n, int64_t* splits, int64_t* chunk);
// A round followed by its layout swap, fused: rows of N/S arrays of
// S = A*M*n elements, [A][M][n] in (fibers of n), each written in place as
// [n][M][A]; w as for launch_fiber. Needs A % 8 == 0 and S <= 1024; in may
// equal out.
bool fiber_swap_applicable(int64_t n, int64_t A, int64_t M, bool bf16);
// Round 0 (fibers of n at stride N/n in the natural layout) joined with the
// layout change: dir 0 reads natural rows, writes the L_0 copy of the input
// to `save` and the results in L_0 to `out`; dir 1 reads L_0 rows and writes
// the results in the natural layout. w as for launch_fiber. Needs N/n a
// multiple of 8.
bool fiber_strided_applicable(int64_t n, int64_t N, bool bf16);
hipError_t launch_fiber_strided(const void* in, const void* w, void* out, void* save,
                                int64_t batch, int64_t N, int64_t n, int dir, bool bf16,
                                hipStream_t s);
hipError_t launch_fiber_swap(const void* in, const void* w, void* out, int64_t batch, int64_t N,
                             int64_t n, int64_t A, int64_t M, bool bf16, hipStream_t s);
hipError_t launch_fiber_wgrad(const void* g, const void* in, float* partial, int64_t batch,
                              int64_t N, int64_t n, int64_t chunk, bool bf16, hipStream_t s);

// Axis swap of `rows` row-major A x M x C arrays: out[b][c][m][a] =
// in[b][a][m][c] (M = 1: a per-row transpose; lattice layout changes); with
// accum, out[b][c][m][a] += in[b][a][m][c] (fp32 sum, one rounding).
hipError_t launch_swap(const void* in, void* out, int64_t rows, int64_t A, int64_t M, int64_t C,
                       bool bf16, hipStream_t s, bool accum = false);

// Bias gradient partial sums: partial[c][p*b2 + g] = sum over rows
// [c*chunk, (c+1)*chunk) of dV[b, g*q2o + p], for p*b2 + g < out (fp32,
// rows in increasing order).
hipError_t launch_bias_partials(const void* dv, float* partial, int64_t rows, int64_t chunk,
                                int64_t chunks, int64_t out, int64_t b2, int64_t q2o, bool bf16,
                                hipStream_t s);

// bf16 block-diagonal products with K = 192 or 256 per block and N a
// multiple of 256, weights held in registers (blockdiag.hip): both DYAD
// terms and the stage-1 forward at those block shapes. bd_mode returns 1
// (K = 256) or 3 (K = 192) when W_blk(k, j) is B[blk][row(j)][k] (b_sk = 1,
// rows under the optional column split), 2 when it is B[blk][k][j] with
// K = N = 256, and 0 when the GemmArgs are not such a product (then
// launch_gemm's tiled kernels run).
int bd_mode(const GemmArgs& a, bool bf16);
hipError_t launch_bd(const GemmArgs& a, int mode, hipStream_t s);

// Products whose K is split over the eight waves of a workgroup, both
// operands contiguous along k (skinny.hip), the waves' tiles summed in a
// fixed order: skinny_mode returns 1 for at most 16 rows and K >= 128 (one
// block and 16 output columns per workgroup), 2 for fp32 products with
// K >= 512 and at most 512 tiles of 64 x 64 (one such tile per workgroup),
// and 0 otherwise (also with batch-split partials, accumulation or a column
// limit). Bias, ReLU, the column split and the output column guard are
// applied in the epilogue.
int skinny_mode(const GemmArgs& a, bool bf16);
hipError_t launch_skinny(const GemmArgs& a, int mode, bool bf16, hipStream_t s);

// Writes `bytes` zero bytes (a plain kernel, not hipMemsetAsync, so callers may
// capture it in a graph). p must be 2-byte aligned and bytes a multiple of 2.
hipError_t launch_zero(void* p, size_t bytes, hipStream_t s);

// Up to three gradients in one launch: out[e] = sum_{s < splits} partial[s*n + e]
// in increasing s, stored in the I/O type (fixed order: bit-reproducible).
// An entry with n == 0 is skipped.
struct ReduceArgs {
  const float* partial = nullptr;
  void* out = nullptr;
  int64_t n = 0, splits = 1;
};
hipError_t launch_reduce_partials(const ReduceArgs& a, const ReduceArgs& b, const ReduceArgs& c,
                                  bool bf16, hipStream_t s);

// Plain device copy of `bytes` bytes (16-byte aligned src and dst): the
// measured-bandwidth reference of the HBM rooflines.
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t s);

// Dense -> Monarch projection: one workgroup per (g, r) slice of M
// [out = nb1*nb2, in]; writes w1 [nb1, nb2, q1i], w2 [nb2, q2o, nb1] and, when
// status is set, status[r*nb2 + g] = the products with AᵀA a converged slice
// used (> 0), or 0 when it did not converge.
// project_pad is the padded slice size (16, 32, 64 or 128), 0 when a slice
// side exceeds 128.
int project_pad(int64_t q1i, int64_t q2o);
hipError_t launch_project(const void* m, void* w1, void* w2, int* status, int64_t in,
                          int64_t nb1, int64_t nb2, int64_t q1i, int64_t q2o, int max_steps,
                          bool bf16, hipStream_t s);

}  // namespace monarch
