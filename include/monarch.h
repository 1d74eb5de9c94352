/*
 * monarch.h -- C ABI of the MI355X (gfx950) Monarch multiply library.
 *
 * Operation (Monarch paper, abstract: a product of two block-diagonal
 * matrices; scatterbrain issues page, "Definition C.3" thread: the block
 * counts and the MonarchLinear parameter layout; "hypercube" thread: the
 * stride permutation between the two products):
 *
 *   y = Qout · L · P · R · x        for every row x of X, i.e. Y = X · Mᵀ
 *
 *   in  = in_features, out = out_features, mid = out (intermediate width),
 *   b1  = nblocks1, b2 = nblocks2,
 *   q1i = in/b1, q1o = mid/b1, q2i = mid/b2, q2o = out/b2.
 *
 *   stage 1   Z[b, r*q1o + k] = sum_s w1[r, k, s] * X[b, r*q1i + s]
 *   P         W[b, g*q2i + t] = Z[b, t*b2 + g]          (stride-b2 gather)
 *   stage 2   V[b, g*q2o + p] = sum_t w2[g, p, t] * W[b, g*q2i + t]
 *   Qout      Y[b, p*b2 + g]  = act(V[b, g*q2o + p])    (inverse stride scatter)
 *
 * Layouts (all row-major, contiguous):
 *   x  [batch, in]            y  [batch, out]
 *   w1 [b1, q1o, q1i]  (R)    w2 [b2, q2o, q2i]  (L)
 *   z  batch*mid elements of the I/O dtype: stage 2's input W, in a layout
 *      private to the library. It is written by monarch_fwd and must be
 *      passed unchanged to monarch_bwd with the same shape arguments.
 *   dtype MONARCH_F32: every buffer is fp32.  MONARCH_BF16: every buffer is
 *   bfloat16; all sums accumulate in fp32 and results are rounded to
 *   nearest-even bf16 when stored.
 *
 * Common rules for every entry point:
 *   - Calls are asynchronous and ordered on `stream` (a hipStream_t; NULL is
 *     the default stream). The library never allocates, frees or
 *     synchronises, and keeps no state between calls (reentrant); the one
 *     exception is monarch_bwd_noalloc's static scratch, described there.
 *   - The caller owns every buffer. Outputs must not alias inputs.
 *   - Every argument is checked before any HIP call; a rejected call has no
 *     side effects. Checks, in order:
 *       dtype or act out of range                      -> MONARCH_ERR_DTYPE
 *       a size <= 0 (batch < 0), a block count that
 *       does not divide in, mid or out, or a size
 *       beyond 2^31 elements per dimension              -> MONARCH_ERR_SHAPE
 *       a required pointer is NULL                      -> MONARCH_ERR_NULL
 *       a pointer not 16-byte aligned                   -> MONARCH_ERR_ALIGN
 *       workspace smaller than required                 -> MONARCH_ERR_WORKSPACE
 *     A failed kernel launch returns MONARCH_ERR_HIP; the HIP error text is
 *     then available from monarch_status_string(MONARCH_ERR_HIP) on the same
 *     thread.
 */
#ifndef MONARCH_H_
#define MONARCH_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MONARCH_ABI_VERSION 4

typedef enum {
  MONARCH_OK = 0,
  MONARCH_ERR_NULL = -1,
  MONARCH_ERR_SHAPE = -2,
  MONARCH_ERR_DTYPE = -3,
  MONARCH_ERR_ALIGN = -4,
  MONARCH_ERR_WORKSPACE = -5,
  MONARCH_ERR_HIP = -6,
  MONARCH_ERR_SCRATCH = -7   /* monarch_bwd_noalloc: problem too large for its scratch */
} monarch_status;

typedef enum { MONARCH_F32 = 0, MONARCH_BF16 = 1 } monarch_dtype;

/* Activation fused after the inverse permutation (the ReLU between the two
 * layers of the recommender MLP, scatterbrain issues page, "efficiency
 * testing numbers" thread). Its derivative at 0 is taken as 0. */
typedef enum { MONARCH_ACT_NONE = 0, MONARCH_ACT_RELU = 1 } monarch_act;

/* Forward pass: y = act(X · Mᵀ); also writes z (stage 2's input, kept for
 * the backward pass). x, w1, w2 are read; y and z are overwritten.
 * batch == 0 returns MONARCH_OK without launching anything (x, y, z may then
 * be NULL). */
int monarch_fwd(const void* x, const void* w1, const void* w2, void* y, void* z,
                int64_t in_features, int64_t out_features, int64_t nblocks1,
                int64_t nblocks2, int64_t batch, int dtype, int act, void* stream);

/* Bytes of device workspace monarch_bwd needs for this problem (0 when
 * batch == 0). Returns 0 and sets nothing for invalid shapes. */
size_t monarch_bwd_workspace_bytes(int64_t in_features, int64_t out_features,
                                   int64_t nblocks1, int64_t nblocks2, int64_t batch,
                                   int dtype);

/* Backward pass. Given dy = dL/dy [batch, out], computes
 *   dx  [batch, in]        = dY_eff · M,
 *   dw1 [b1, q1o, q1i]     = block r of (dY_eff·Qout·L·P)ᵀ · X   (sum over batch),
 *   dw2 [b2, q2o, q2i]     = block g of (dY_eff·Qout)ᵀ · W      (sum over batch),
 * with dY_eff = dy ⊙ 1[y > 0] when act == MONARCH_ACT_RELU (y is then the
 * forward output and must be non-NULL) and dY_eff = dy otherwise (y unused,
 * may be NULL). z must be the buffer monarch_fwd wrote for the same x, w1
 * and shapes. dx, dw1 and dw2 are overwritten, never accumulated into. The
 * batch reduction of dw1/dw2 runs in a fixed order, so results are
 * bit-reproducible from run to run. workspace must hold
 * monarch_bwd_workspace_bytes(...) bytes; its contents are scratch.
 * batch == 0 writes zeros to dw1 and dw2 and touches nothing else. */
int monarch_bwd(const void* dy, const void* x, const void* w1, const void* w2,
                const void* z, const void* y, void* dx, void* dw1, void* dw2,
                void* workspace, size_t workspace_bytes, int64_t in_features,
                int64_t out_features, int64_t nblocks1, int64_t nblocks2,
                int64_t batch, int dtype, int act, void* stream);

/* Same as monarch_fwd / monarch_bwd, and in addition records events[i]
 * (hipEvent_t) on the stream just before kernel i of the call and
 * events[n] after the last kernel, where n is the kernel count that
 * monarch_describe reports for the same problem. events may be NULL. Used to
 * time single kernels inside a timed region. */
int monarch_fwd_traced(const void* x, const void* w1, const void* w2, void* y, void* z,
                       int64_t in_features, int64_t out_features, int64_t nblocks1,
                       int64_t nblocks2, int64_t batch, int dtype, int act, void* stream,
                       void* const* events, int n_events);
int monarch_bwd_traced(const void* dy, const void* x, const void* w1, const void* w2,
                       const void* z, const void* y, void* dx, void* dw1, void* dw2,
                       void* workspace, size_t workspace_bytes, int64_t in_features,
                       int64_t out_features, int64_t nblocks1, int64_t nblocks2,
                       int64_t batch, int dtype, int act, void* stream,
                       void* const* events, int n_events);

/* Describes the kernels monarch_fwd (direction 0) or monarch_bwd (direction
 * 1) launches for a problem: returns their count (negative status for an
 * invalid problem) and writes their names, separated by ';', into buf
 * (truncated to buf_len including the terminating NUL; buf may be NULL). */
int monarch_describe(int direction, int64_t in_features, int64_t out_features,
                     int64_t nblocks1, int64_t nblocks2, int64_t batch, int dtype,
                     int act, char* buf, size_t buf_len);

/* Dense -> Monarch projection (scatterbrain issues page, "projection"
 * thread: M rearranged as '(p k) (r s) -> k r p s', every (k, r) slice fitted
 * on its own; Monarch paper, abstract: an analytical optimal solution).
 *
 * Defined for the Definition C.3 case out_features = nblocks1 * nblocks2 with
 * in_features % nblocks1 == 0 (then q1o = nblocks2 and q2i = nblocks1). The
 * Monarch matrix has M[p*b2 + g, r*q1i + s] = w2[g, p, r] * w1[r, g, s], so
 * slice (g, r) over (p, s) is an outer product and the nearest Monarch matrix
 * (Frobenius) takes each slice's nearest rank-one matrix.
 *
 *   m  [out, in] row-major, read;  w1 [b1, b2, q1i] and w2 [b2, q2o, b1],
 *   overwritten, in the layouts monarch_fwd takes.
 *
 * A slice A (q2o x q1i) is fitted by x, the unit vector maximising xᵀAᵀAx
 * (the fit (A x) xᵀ leaves ||A||² - xᵀAᵀAx): Lanczos on AᵀA in fp32 with
 * full reorthogonalisation, in cycles of up to 32 products restarted from the
 * Ritz vector, until ||AᵀA x - theta x|| <= 1e-4 * theta (theta = xᵀAᵀAx) or
 * max_steps (1..4096) products with AᵀA have been spent. The factors split
 * sqrt(sigma) evenly (sigma = ||A x||), with the sign making the
 * largest-magnitude entry of w1[r, g, :] (the first on ties) positive.
 * converged (may be NULL): int32 [nb1 * nb2] device array; element
 * r*nb2 + g is set to the number of products with AᵀA slice (g, r) used
 * (> 0) when it met the tolerance, 0 when the budget ran out first (its
 * factors are then the last Ritz vector's fit).
 * Slices up to 128 x 128 (q1i, q2o <= 128). Errors as for monarch_fwd;
 * shapes outside the case, max_steps out of range or a slice too large give
 * MONARCH_ERR_SHAPE. */
int monarch_project(const void* m, void* w1, void* w2, int64_t in_features,
                    int64_t out_features, int64_t nblocks1, int64_t nblocks2, int dtype,
                    int max_steps, int* converged, void* stream);

/* ---------------------------------------------------------------------------
 * monarch_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Arguments, layouts, results and errors as for
 * monarch_bwd; the same kernels run. The intermediates and partial sums live
 * in a static array of MONARCH_NOALLOC_SCRATCH_BYTES bytes per GPU, which
 * the library holds on each GPU it runs on until the process ends (its
 * address is looked up on the first call on a device, with the calling
 * thread's current device, which must be the stream's). A problem whose
 * monarch_bwd_workspace_bytes() exceeds that size returns
 * MONARCH_ERR_SCRATCH before any HIP call. No allocating call is made. The
 * array is shared by every call on one GPU: calls that overlap in time on
 * one GPU (other streams, other threads) race and must be serialised by the
 * caller. */
#define MONARCH_NOALLOC_SCRATCH_BYTES (256ull << 20)

int monarch_bwd_noalloc(const void* dy, const void* x, const void* w1, const void* w2,
                        const void* z, const void* y, void* dx, void* dw1, void* dw2,
                        int64_t in_features, int64_t out_features, int64_t nblocks1,
                        int64_t nblocks2, int64_t batch, int dtype, int act, void* stream);

/* ---------------------------------------------------------------------------
 * General layer shapes (the MonarchLinear constructor in the "Definition C.3"
 * thread of the scatterbrain issues page: block sizes ceil(in/nb) and
 * ceil(out/nb), and mid = in_ext for an expanding layer, out_ext otherwise).
 *
 * The *_ex entry points take the intermediate width mid explicitly (divisible
 * by both block counts) and any in and out:
 *   q1i = ceil(in/b1), q1o = mid/b1, q2i = mid/b2, q2o = ceil(out/b2),
 *   in_ext = b1*q1i >= in, out_ext = b2*q2o >= out.
 * The input is zero-padded to in_ext features (the padded positions of w1
 * take no part in the product and receive zero gradient), the two stages
 * run at the extended sizes as above, and y keeps the first `out` of the
 * out_ext features. An optional bias [out] is added before the activation:
 *   y = act(Qout·L·P·R·pad(x) truncated to out + bias).
 *   w1 [b1, q1o, q1i], w2 [b2, q2o, q2i], bias and dbias [out] in the I/O
 *   dtype; z holds batch*mid elements. With mid = out, in % b1 == 0,
 *   out % b2 == 0 and no bias they compute exactly what monarch_fwd and
 *   monarch_bwd compute. Errors as for monarch_fwd/monarch_bwd, except that
 *   in and out need not be divisible (mid must be: MONARCH_ERR_SHAPE). */

/* The MonarchLinear intermediate width for one block count nb:
 * min-of-branches rule above (in_ext if in_ext < out_ext, else out_ext).
 * Returns MONARCH_ERR_SHAPE for non-positive or too large sizes. */
int64_t monarch_linear_mid(int64_t in_features, int64_t out_features, int64_t nblocks);

/* Forward of the general layer. bias may be NULL (no bias). events: as for
 * monarch_fwd_traced (may be NULL, with n_events 0). */
int monarch_fwd_ex(const void* x, const void* w1, const void* w2, const void* bias, void* y,
                   void* z, int64_t in_features, int64_t out_features, int64_t mid_features,
                   int64_t nblocks1, int64_t nblocks2, int64_t batch, int dtype, int act,
                   void* stream, void* const* events, int n_events);

/* Workspace bytes of monarch_bwd_ex (with_bias: whether dbias is requested). */
size_t monarch_bwd_ex_workspace_bytes(int64_t in_features, int64_t out_features,
                                      int64_t mid_features, int64_t nblocks1, int64_t nblocks2,
                                      int64_t batch, int dtype, int with_bias);

/* Backward of the general layer: dx [batch, in], dw1, dw2 as for
 * monarch_bwd, and dbias[o] = sum over rows of dY_eff[b, o] when dbias is
 * non-NULL (fixed-order sums, bit-reproducible). dx, dw1, dw2 and dbias are
 * overwritten. batch == 0 writes zeros to dw1, dw2 and dbias. */
int monarch_bwd_ex(const void* dy, const void* x, const void* w1, const void* w2, const void* z,
                   const void* y, void* dx, void* dw1, void* dw2, void* dbias, void* workspace,
                   size_t workspace_bytes, int64_t in_features, int64_t out_features,
                   int64_t mid_features, int64_t nblocks1, int64_t nblocks2, int64_t batch,
                   int dtype, int act, void* stream, void* const* events, int n_events);

/* monarch_describe for the general layer (with_bias as above). */
int monarch_describe_ex(int direction, int64_t in_features, int64_t out_features,
                        int64_t mid_features, int64_t nblocks1, int64_t nblocks2, int64_t batch,
                        int dtype, int act, int with_bias, char* buf, size_t buf_len);

/* ---------------------------------------------------------------------------
 * k-factor ("hypercube") Monarch layer (scatterbrain issues page, "hypercube"
 * thread: the N units of a layer as a lattice, one round of block products
 * per lattice dimension).
 *
 * dims[0..ndims-1] (1 <= ndims <= 4, N = prod dims < 2^31) is a row-major
 * lattice: unit u has multi-index (a_1..a_k), u = ((a_1*n_2 + a_2)*n_3 + ...).
 * Round j (in axis order j = 1..k) multiplies along axis j with one
 * n_j x n_j matrix per combination of the other axes' indices:
 *   w[j] [N/n_j, n_j, n_j], w[j][f][o, i] the weight from position i to o,
 *   f = the other axes' indices flattened row-major in axis order.
 * y = F_k ... F_1 x for every row (x, y [batch, N]). The forward also writes
 * what the backward reads to `saved` (monarch_hyper_saved_elems elements of
 * the I/O dtype, k * batch * N for k >= 2: x and the outputs of rounds
 * 1..k-1, in layouts private to the library). w and dw are host arrays of ndims device pointers.
 * dtype, streams, ownership, alignment and errors as for monarch_fwd
 * (a bad lattice gives MONARCH_ERR_SHAPE). */
size_t monarch_hyper_saved_elems(int ndims, const int64_t* dims, int64_t batch);

int monarch_hyper_fwd(const void* x, const void* const* w, void* y, void* saved, int ndims,
                      const int64_t* dims, int64_t batch, int dtype, void* stream,
                      void* const* events, int n_events);

size_t monarch_hyper_bwd_workspace_bytes(int ndims, const int64_t* dims, int64_t batch,
                                         int dtype);

/* dx [batch, N] and dw[j] [N/n_j, n_j, n_j] (overwritten; fixed-order batch
 * sums) from dy, x, w and the forward's `saved`. batch == 0 zeroes dw. */
int monarch_hyper_bwd(const void* dy, const void* x, const void* const* w, const void* saved,
                      void* dx, void* const* dw, void* workspace, size_t workspace_bytes,
                      int ndims, const int64_t* dims, int64_t batch, int dtype, void* stream,
                      void* const* events, int n_events);

/* Kernel names of monarch_hyper_fwd (direction 0) / monarch_hyper_bwd (1). */
int monarch_hyper_describe(int direction, int ndims, const int64_t* dims, int64_t batch,
                           int dtype, char* buf, size_t buf_len);

/* ---------------------------------------------------------------------------
 * DYAD-style layer (DYAD page, abstract: the weight matrix is the sum of two
 * matrices, each a permutation of a block-sparse one, stored as 3D tensors).
 * With nb = nblocks, qi = in/nb, qo = out/nb (both divisible):
 *   y = (BD(A) + Qout · BD(B) · P) x            for every row,
 *   Y[b, r*qo + k] += sum_s A[r, k, s] X[b, r*qi + s]     (contiguous blocks)
 *   Y[b, p*nb + g] += sum_t B[g, p, t] X[b, t*nb + g]     (stride-nb features)
 * w_a = A and w_b = B are [nb, qo, qi]; x [batch, in], y [batch, out]. No
 * saved intermediate. Each term is rounded to the I/O type and their sum is
 * rounded again (three roundings of y in bf16). The caller's workspace
 * (monarch_dyad_fwd_workspace_bytes, 16-byte aligned, contents unspecified
 * on return) holds x and the second term in block-major order. Errors and
 * conventions as for monarch_bwd. */
size_t monarch_dyad_fwd_workspace_bytes(int64_t in_features, int64_t out_features,
                                        int64_t nblocks, int64_t batch, int dtype);
int monarch_dyad_fwd(const void* x, const void* w_a, const void* w_b, void* y, void* workspace,
                     size_t workspace_bytes, int64_t in_features, int64_t out_features,
                     int64_t nblocks, int64_t batch, int dtype, void* stream,
                     void* const* events, int n_events);

size_t monarch_dyad_bwd_workspace_bytes(int64_t in_features, int64_t out_features,
                                        int64_t nblocks, int64_t batch, int dtype);

/* dx = dy · M, dw_a / dw_b = the block gradients (fixed-order batch sums),
 * all overwritten. batch == 0 zeroes dw_a and dw_b. */
int monarch_dyad_bwd(const void* dy, const void* x, const void* w_a, const void* w_b, void* dx,
                     void* dw_a, void* dw_b, void* workspace, size_t workspace_bytes,
                     int64_t in_features, int64_t out_features, int64_t nblocks, int64_t batch,
                     int dtype, void* stream, void* const* events, int n_events);

int monarch_dyad_describe(int direction, int64_t in_features, int64_t out_features,
                          int64_t nblocks, int64_t batch, int dtype, char* buf, size_t buf_len);

/* ---------------------------------------------------------------------------
 * Stream copy: copies `bytes` bytes from src to dst (device buffers, 16-byte
 * aligned, not overlapping), reading and writing each byte once with 16-byte
 * non-temporal accesses. Not part of the Monarch operator: it is the
 * reference for the HBM rooflines, the rate a kernel that streams its data
 * through HBM can reach on this memory system (2 * bytes moved per call).
 * bytes == 0 launches nothing. Errors: NULL -> MONARCH_ERR_NULL,
 * misaligned -> MONARCH_ERR_ALIGN. */
int monarch_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/* Static text for a status code; for MONARCH_ERR_HIP the last HIP error
 * message recorded on the calling thread. Never NULL. */
const char* monarch_status_string(int status);

/* MONARCH_ABI_VERSION of the built library. */
int monarch_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MONARCH_H_ */
