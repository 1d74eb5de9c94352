// C ABI of the Monarch library: argument checks, kernel planning, launches.
//
// The operator and its backward pass are stated in include/monarch.h. Every
// check runs before the first HIP call, so a rejected call has no side
// effects and the checks work on machines without a GPU.
#include <stdio.h>
#include <string.h>

#include "dyad.h"
#include "hyper.h"
#include "kernels.h"
#include "monarch.h"
#include "plan.h"
#include "api_internal.h"

namespace monarch {

namespace {
thread_local char g_hip_error[256] = "no HIP error recorded";
}  // namespace

int record_hip(hipError_t e) {
  if (e == hipSuccess) return MONARCH_OK;
  snprintf(g_hip_error, sizeof(g_hip_error), "HIP error %d: %s", static_cast<int>(e),
           hipGetErrorString(e));
  return MONARCH_ERR_HIP;
}

namespace {

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

struct Tracer {
  void* const* ev;
  int n;
  int idx = 0;
  hipStream_t s;
  hipError_t mark() {
    hipError_t e = hipSuccess;
    if (ev && idx < n && ev[idx]) e = hipEventRecord(static_cast<hipEvent_t>(ev[idx]), s);
    ++idx;
    return e;
  }
};

int run_plan(const Plan& plan, const Problem& pr, const Buffers& b, hipStream_t s,
             void* const* events, int n_events) {
  Tracer tr{events, n_events, 0, s};
  for (int i = 0; i < plan.n; ++i) {
    int st = record_hip(tr.mark());
    if (st) return st;
    st = record_hip(launch_step(plan.kind[i], pr, b, s));
    if (st) return st;
  }
  return record_hip(tr.mark());
}

int fwd_impl(const Problem& pr, const void* x, const void* w1, const void* w2, const void* bias,
             void* y, void* z, void* stream, void* const* events, int n_events) {
  if (!w1 || !w2) return MONARCH_ERR_NULL;
  if (pr.bias && !bias) return MONARCH_ERR_NULL;
  if (pr.batch > 0 && (!x || !y || !z)) return MONARCH_ERR_NULL;
  if (misaligned(x) || misaligned(w1) || misaligned(w2) || misaligned(y) || misaligned(z) ||
      misaligned(bias))
    return MONARCH_ERR_ALIGN;
  if (pr.batch == 0) return MONARCH_OK;
  Buffers b;
  b.x = x;
  b.w1 = w1;
  b.w2 = w2;
  b.bias = bias;
  b.y_out = y;
  b.z_out = z;
  Plan plan = plan_fwd(pr);
  return run_plan(plan, pr, b, static_cast<hipStream_t>(stream), events, n_events);
}

int run_seq(const SeqStep* steps, int n, bool bf16, hipStream_t s, void* const* events,
              int n_events) {
  Tracer tr{events, n_events, 0, s};
  for (int i = 0; i < n; ++i) {
    int st = record_hip(tr.mark());
    if (st) return st;
    st = record_hip(seq_launch(steps[i], bf16, s));
    if (st) return st;
  }
  return record_hip(tr.mark());
}

int write_names(const char* const* names, int n, char* buf, size_t buf_len) {
  if (buf && buf_len) {
    buf[0] = '\0';
    size_t used = 0;
    for (int i = 0; i < n; ++i) {
      int w = snprintf(buf + used, buf_len - used, "%s%s", i ? ";" : "", names[i]);
      if (w < 0) break;
      used += static_cast<size_t>(w);
      if (used >= buf_len) {
        buf[buf_len - 1] = '\0';
        break;
      }
    }
  }
  return n;
}

int describe_plan(const Problem& pr, int direction, char* buf, size_t buf_len) {
  if (direction != 0 && direction != 1) return MONARCH_ERR_DTYPE;
  Plan plan;
  if (direction == 0)
    plan = pr.batch == 0 ? Plan{} : plan_fwd(pr);
  else
    plan = plan_bwd(pr);
  if (buf && buf_len) {
    buf[0] = '\0';
    size_t used = 0;
    for (int i = 0; i < plan.n; ++i) {
      const char* nm = step_name(plan.kind[i]);
      int w = snprintf(buf + used, buf_len - used, "%s%s", i ? ";" : "", nm);
      if (w < 0) break;
      used += static_cast<size_t>(w);
      if (used >= buf_len) {
        buf[buf_len - 1] = '\0';
        break;
      }
    }
  }
  return plan.n;
}

}  // namespace

int bwd_check(const Problem& pr, const void* dy, const void* x, const void* w1, const void* w2,
              const void* z, const void* y, const void* dx, const void* dw1, const void* dw2,
              const void* dbias) {
  if (!w1 || !w2 || !dw1 || !dw2) return MONARCH_ERR_NULL;
  if (pr.bias && !dbias) return MONARCH_ERR_NULL;
  if (pr.batch > 0) {
    if (!dy || !x || !z || !dx) return MONARCH_ERR_NULL;
    if (pr.act == MONARCH_ACT_RELU && !y) return MONARCH_ERR_NULL;
  }
  if (misaligned(dy) || misaligned(x) || misaligned(w1) || misaligned(w2) || misaligned(z) ||
      misaligned(y) || misaligned(dx) || misaligned(dw1) || misaligned(dw2) || misaligned(dbias))
    return MONARCH_ERR_ALIGN;
  return MONARCH_OK;
}

int bwd_impl(const Problem& pr, const void* dy, const void* x, const void* w1, const void* w2,
             const void* z, const void* y, void* dx, void* dw1, void* dw2, void* dbias, void* ws,
             size_t ws_bytes, void* stream, void* const* events, int n_events) {
  int st = bwd_check(pr, dy, x, w1, w2, z, y, dx, dw1, dw2, dbias);
  if (st) return st;
  const size_t need = workspace_bytes(pr);
  if (need > 0 && !ws) return MONARCH_ERR_NULL;
  if (misaligned(ws)) return MONARCH_ERR_ALIGN;
  if (ws_bytes < need) return MONARCH_ERR_WORKSPACE;
  Buffers b;
  b.dy = dy;
  b.x = x;
  b.w1 = w1;
  b.w2 = w2;
  b.z = z;
  b.y = y;
  b.dx = dx;
  b.dw1 = dw1;
  b.dw2 = dw2;
  b.dbias = dbias;
  b.ws = ws;
  Plan plan = plan_bwd(pr);
  return run_plan(plan, pr, b, static_cast<hipStream_t>(stream), events, n_events);
}

}  // namespace monarch

using namespace monarch;

extern "C" {

int monarch_fwd(const void* x, const void* w1, const void* w2, void* y, void* z,
                int64_t in_features, int64_t out_features, int64_t nblocks1, int64_t nblocks2,
                int64_t batch, int dtype, int act, void* stream) {
  return monarch_fwd_traced(x, w1, w2, y, z, in_features, out_features, nblocks1, nblocks2, batch,
                            dtype, act, stream, nullptr, 0);
}

int monarch_fwd_traced(const void* x, const void* w1, const void* w2, void* y, void* z,
                       int64_t in_features, int64_t out_features, int64_t nblocks1,
                       int64_t nblocks2, int64_t batch, int dtype, int act, void* stream,
                       void* const* events, int n_events) {
  Problem pr;
  int st = make_problem(in_features, out_features, nblocks1, nblocks2, batch, dtype, act, &pr);
  if (st) return st;
  return fwd_impl(pr, x, w1, w2, nullptr, y, z, stream, events, n_events);
}

size_t monarch_bwd_workspace_bytes(int64_t in_features, int64_t out_features, int64_t nblocks1,
                                   int64_t nblocks2, int64_t batch, int dtype) {
  Problem pr;
  if (make_problem(in_features, out_features, nblocks1, nblocks2, batch, dtype, 0, &pr))
    return 0;
  return workspace_bytes(pr);
}

int monarch_bwd(const void* dy, const void* x, const void* w1, const void* w2, const void* z,
                const void* y, void* dx, void* dw1, void* dw2, void* workspace,
                size_t workspace_bytes, int64_t in_features, int64_t out_features,
                int64_t nblocks1, int64_t nblocks2, int64_t batch, int dtype, int act,
                void* stream) {
  return monarch_bwd_traced(dy, x, w1, w2, z, y, dx, dw1, dw2, workspace, workspace_bytes,
                            in_features, out_features, nblocks1, nblocks2, batch, dtype, act,
                            stream, nullptr, 0);
}

int monarch_bwd_traced(const void* dy, const void* x, const void* w1, const void* w2,
                       const void* z, const void* y, void* dx, void* dw1, void* dw2,
                       void* workspace, size_t workspace_bytes, int64_t in_features,
                       int64_t out_features, int64_t nblocks1, int64_t nblocks2, int64_t batch,
                       int dtype, int act, void* stream, void* const* events, int n_events) {
  Problem pr;
  int st = make_problem(in_features, out_features, nblocks1, nblocks2, batch, dtype, act, &pr);
  if (st) return st;
  return bwd_impl(pr, dy, x, w1, w2, z, y, dx, dw1, dw2, nullptr, workspace, workspace_bytes,
                  stream, events, n_events);
}

int64_t monarch_linear_mid(int64_t in_features, int64_t out_features, int64_t nblocks) {
  const int64_t lim = int64_t(1) << 31;
  if (in_features <= 0 || out_features <= 0 || nblocks <= 0 || in_features >= lim ||
      out_features >= lim || nblocks >= lim)
    return MONARCH_ERR_SHAPE;
  const int64_t in_ext = (in_features + nblocks - 1) / nblocks * nblocks;
  const int64_t out_ext = (out_features + nblocks - 1) / nblocks * nblocks;
  return in_ext < out_ext ? in_ext : out_ext;
}

int monarch_fwd_ex(const void* x, const void* w1, const void* w2, const void* bias, void* y,
                   void* z, int64_t in_features, int64_t out_features, int64_t mid_features,
                   int64_t nblocks1, int64_t nblocks2, int64_t batch, int dtype, int act,
                   void* stream, void* const* events, int n_events) {
  Problem pr;
  int st = make_problem_ex(in_features, out_features, mid_features, nblocks1, nblocks2, batch,
                           dtype, act, bias != nullptr, &pr);
  if (st) return st;
  return fwd_impl(pr, x, w1, w2, bias, y, z, stream, events, n_events);
}

size_t monarch_bwd_ex_workspace_bytes(int64_t in_features, int64_t out_features,
                                      int64_t mid_features, int64_t nblocks1, int64_t nblocks2,
                                      int64_t batch, int dtype, int with_bias) {
  Problem pr;
  if (make_problem_ex(in_features, out_features, mid_features, nblocks1, nblocks2, batch, dtype, 0,
                      with_bias != 0, &pr))
    return 0;
  return workspace_bytes(pr);
}

int monarch_bwd_ex(const void* dy, const void* x, const void* w1, const void* w2, const void* z,
                   const void* y, void* dx, void* dw1, void* dw2, void* dbias, void* workspace,
                   size_t workspace_bytes, int64_t in_features, int64_t out_features,
                   int64_t mid_features, int64_t nblocks1, int64_t nblocks2, int64_t batch,
                   int dtype, int act, void* stream, void* const* events, int n_events) {
  Problem pr;
  int st = make_problem_ex(in_features, out_features, mid_features, nblocks1, nblocks2, batch,
                           dtype, act, dbias != nullptr, &pr);
  if (st) return st;
  return bwd_impl(pr, dy, x, w1, w2, z, y, dx, dw1, dw2, dbias, workspace, workspace_bytes, stream,
                  events, n_events);
}

int monarch_describe_ex(int direction, int64_t in_features, int64_t out_features,
                        int64_t mid_features, int64_t nblocks1, int64_t nblocks2, int64_t batch,
                        int dtype, int act, int with_bias, char* buf, size_t buf_len) {
  Problem pr;
  int st = make_problem_ex(in_features, out_features, mid_features, nblocks1, nblocks2, batch,
                           dtype, act, with_bias != 0, &pr);
  if (st) return st;
  return describe_plan(pr, direction, buf, buf_len);
}

int monarch_project(const void* m, void* w1, void* w2, int64_t in_features,
                    int64_t out_features, int64_t nblocks1, int64_t nblocks2, int dtype,
                    int max_steps, int* converged, void* stream) {
  if (dtype != MONARCH_F32 && dtype != MONARCH_BF16) return MONARCH_ERR_DTYPE;
  const int64_t lim = int64_t(1) << 31;
  if (in_features <= 0 || out_features <= 0 || nblocks1 <= 0 || nblocks2 <= 0 ||
      in_features >= lim || out_features >= lim || in_features % nblocks1 != 0 ||
      out_features != nblocks1 * nblocks2 || max_steps < 1 || max_steps > 4096)
    return MONARCH_ERR_SHAPE;
  const int64_t q1i = in_features / nblocks1, q2o = out_features / nblocks2;
  if (!project_pad(q1i, q2o)) return MONARCH_ERR_SHAPE;
  if (!m || !w1 || !w2) return MONARCH_ERR_NULL;
  if (misaligned(m) || misaligned(w1) || misaligned(w2)) return MONARCH_ERR_ALIGN;
  if (reinterpret_cast<uintptr_t>(converged) & 3u) return MONARCH_ERR_ALIGN;
  return record_hip(launch_project(m, w1, w2, converged, in_features, nblocks1, nblocks2, q1i,
                                   q2o, max_steps, dtype == MONARCH_BF16,
                                   static_cast<hipStream_t>(stream)));
}

int monarch_describe(int direction, int64_t in_features, int64_t out_features, int64_t nblocks1,
                     int64_t nblocks2, int64_t batch, int dtype, int act, char* buf,
                     size_t buf_len) {
  Problem pr;
  int st = make_problem(in_features, out_features, nblocks1, nblocks2, batch, dtype, act, &pr);
  if (st) return st;
  return describe_plan(pr, direction, buf, buf_len);
}

size_t monarch_hyper_saved_elems(int ndims, const int64_t* dims, int64_t batch) {
  HyperProblem hp;
  if (make_hyper(ndims, dims, batch, MONARCH_F32, &hp)) return 0;
  return static_cast<size_t>(hyper_saved_elems(hp));
}

int monarch_hyper_fwd(const void* x, const void* const* w, void* y, void* saved, int ndims,
                      const int64_t* dims, int64_t batch, int dtype, void* stream,
                      void* const* events, int n_events) {
  HyperProblem hp;
  int st = make_hyper(ndims, dims, batch, dtype, &hp);
  if (st) return st;
  if (!w) return MONARCH_ERR_NULL;
  HyperBuffers b;
  for (int j = 0; j < hp.k; ++j) {
    if (!w[j]) return MONARCH_ERR_NULL;
    if (misaligned(w[j])) return MONARCH_ERR_ALIGN;
    b.w[j] = w[j];
  }
  if (batch > 0 && (!x || !y || (hp.k > 1 && !saved))) return MONARCH_ERR_NULL;
  if (misaligned(x) || misaligned(y) || misaligned(saved)) return MONARCH_ERR_ALIGN;
  if (batch == 0) return MONARCH_OK;
  b.x = x;
  b.y = y;
  b.saved = saved;
  SeqStep steps[kHyperMaxSteps];
  const int n = hyper_plan_fwd(hp, b, steps);
  return run_seq(steps, n, dtype == MONARCH_BF16, static_cast<hipStream_t>(stream), events,
                   n_events);
}

size_t monarch_hyper_bwd_workspace_bytes(int ndims, const int64_t* dims, int64_t batch,
                                         int dtype) {
  HyperProblem hp;
  if (make_hyper(ndims, dims, batch, dtype, &hp)) return 0;
  return hp.ws_total;
}

int monarch_hyper_bwd(const void* dy, const void* x, const void* const* w, const void* saved,
                      void* dx, void* const* dw, void* workspace, size_t workspace_bytes,
                      int ndims, const int64_t* dims, int64_t batch, int dtype, void* stream,
                      void* const* events, int n_events) {
  HyperProblem hp;
  int st = make_hyper(ndims, dims, batch, dtype, &hp);
  if (st) return st;
  if (!w || !dw) return MONARCH_ERR_NULL;
  HyperBuffers b;
  for (int j = 0; j < hp.k; ++j) {
    if (!w[j] || !dw[j]) return MONARCH_ERR_NULL;
    if (misaligned(w[j]) || misaligned(dw[j])) return MONARCH_ERR_ALIGN;
    b.w[j] = w[j];
    b.dw[j] = dw[j];
  }
  if (batch > 0 && (!dy || !x || !dx || (hp.k > 1 && !saved))) return MONARCH_ERR_NULL;
  if (hp.ws_total > 0 && !workspace) return MONARCH_ERR_NULL;
  if (misaligned(dy) || misaligned(x) || misaligned(saved) || misaligned(dx) ||
      misaligned(workspace))
    return MONARCH_ERR_ALIGN;
  if (workspace_bytes < hp.ws_total) return MONARCH_ERR_WORKSPACE;
  b.dy = dy;
  b.x = x;
  b.saved_in = saved;
  b.dx = dx;
  b.ws = workspace;
  SeqStep steps[kHyperMaxSteps];
  const int n = hyper_plan_bwd(hp, b, steps);
  return run_seq(steps, n, dtype == MONARCH_BF16, static_cast<hipStream_t>(stream), events,
                   n_events);
}

int monarch_hyper_describe(int direction, int ndims, const int64_t* dims, int64_t batch,
                           int dtype, char* buf, size_t buf_len) {
  HyperProblem hp;
  int st = make_hyper(ndims, dims, batch, dtype, &hp);
  if (st) return st;
  if (direction != 0 && direction != 1) return MONARCH_ERR_DTYPE;
  HyperBuffers b;
  SeqStep steps[kHyperMaxSteps];
  const int n = direction == 0 ? hyper_plan_fwd(hp, b, steps) : hyper_plan_bwd(hp, b, steps);
  const char* names[kHyperMaxSteps];
  for (int i = 0; i < n; ++i) names[i] = steps[i].name;
  return write_names(names, n, buf, buf_len);
}

size_t monarch_dyad_fwd_workspace_bytes(int64_t in_features, int64_t out_features,
                                        int64_t nblocks, int64_t batch, int dtype) {
  DyadProblem dp;
  if (make_dyad(in_features, out_features, nblocks, batch, dtype, &dp)) return 0;
  return dp.ws_fwd;
}

int monarch_dyad_fwd(const void* x, const void* w_a, const void* w_b, void* y, void* workspace,
                     size_t workspace_bytes, int64_t in_features, int64_t out_features,
                     int64_t nblocks, int64_t batch, int dtype, void* stream,
                     void* const* events, int n_events) {
  DyadProblem dp;
  int st = make_dyad(in_features, out_features, nblocks, batch, dtype, &dp);
  if (st) return st;
  if (!w_a || !w_b) return MONARCH_ERR_NULL;
  if (batch > 0 && (!x || !y)) return MONARCH_ERR_NULL;
  if (dp.ws_fwd > 0 && !workspace) return MONARCH_ERR_NULL;
  if (misaligned(x) || misaligned(w_a) || misaligned(w_b) || misaligned(y) ||
      misaligned(workspace))
    return MONARCH_ERR_ALIGN;
  if (workspace_bytes < dp.ws_fwd) return MONARCH_ERR_WORKSPACE;
  if (batch == 0) return MONARCH_OK;
  DyadBuffers b;
  b.x = x, b.wa = w_a, b.wb = w_b, b.y = y, b.ws = workspace;
  SeqStep steps[kDyadMaxSteps];
  const int n = dyad_plan_fwd(dp, b, steps);
  return run_seq(steps, n, dtype == MONARCH_BF16, static_cast<hipStream_t>(stream), events,
                 n_events);
}

size_t monarch_dyad_bwd_workspace_bytes(int64_t in_features, int64_t out_features,
                                        int64_t nblocks, int64_t batch, int dtype) {
  DyadProblem dp;
  if (make_dyad(in_features, out_features, nblocks, batch, dtype, &dp)) return 0;
  return dp.ws_total;
}

int monarch_dyad_bwd(const void* dy, const void* x, const void* w_a, const void* w_b, void* dx,
                     void* dw_a, void* dw_b, void* workspace, size_t workspace_bytes,
                     int64_t in_features, int64_t out_features, int64_t nblocks, int64_t batch,
                     int dtype, void* stream, void* const* events, int n_events) {
  DyadProblem dp;
  int st = make_dyad(in_features, out_features, nblocks, batch, dtype, &dp);
  if (st) return st;
  if (!w_a || !w_b || !dw_a || !dw_b) return MONARCH_ERR_NULL;
  if (batch > 0 && (!dy || !x || !dx)) return MONARCH_ERR_NULL;
  if (dp.ws_total > 0 && !workspace) return MONARCH_ERR_NULL;
  if (misaligned(dy) || misaligned(x) || misaligned(w_a) || misaligned(w_b) || misaligned(dx) ||
      misaligned(dw_a) || misaligned(dw_b) || misaligned(workspace))
    return MONARCH_ERR_ALIGN;
  if (workspace_bytes < dp.ws_total) return MONARCH_ERR_WORKSPACE;
  DyadBuffers b;
  b.dy = dy, b.x = x, b.wa = w_a, b.wb = w_b, b.dx = dx, b.dwa = dw_a, b.dwb = dw_b;
  b.ws = workspace;
  SeqStep steps[kDyadMaxSteps];
  const int n = dyad_plan_bwd(dp, b, steps);
  return run_seq(steps, n, dtype == MONARCH_BF16, static_cast<hipStream_t>(stream), events,
                 n_events);
}

int monarch_dyad_describe(int direction, int64_t in_features, int64_t out_features,
                          int64_t nblocks, int64_t batch, int dtype, char* buf, size_t buf_len) {
  DyadProblem dp;
  int st = make_dyad(in_features, out_features, nblocks, batch, dtype, &dp);
  if (st) return st;
  if (direction != 0 && direction != 1) return MONARCH_ERR_DTYPE;
  DyadBuffers b;
  SeqStep steps[kDyadMaxSteps];
  const int n = direction == 0 ? dyad_plan_fwd(dp, b, steps) : dyad_plan_bwd(dp, b, steps);
  const char* names[kDyadMaxSteps];
  for (int i = 0; i < n; ++i) names[i] = steps[i].name;
  return write_names(names, n, buf, buf_len);
}

int monarch_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return MONARCH_OK;
  if (!src || !dst) return MONARCH_ERR_NULL;
  if (misaligned(src) || misaligned(dst)) return MONARCH_ERR_ALIGN;
  return record_hip(launch_stream_copy(src, dst, bytes, static_cast<hipStream_t>(stream)));
}

const char* monarch_status_string(int status) {
  switch (status) {
    case MONARCH_OK: return "ok";
    case MONARCH_ERR_NULL: return "a required pointer is NULL";
    case MONARCH_ERR_SHAPE: return "invalid shape: sizes must be positive and divisible by the block counts";
    case MONARCH_ERR_DTYPE: return "dtype or activation out of range";
    case MONARCH_ERR_ALIGN: return "a pointer is not 16-byte aligned";
    case MONARCH_ERR_WORKSPACE: return "workspace smaller than monarch_bwd_workspace_bytes()";
    case MONARCH_ERR_HIP: return g_hip_error;
    case MONARCH_ERR_SCRATCH:
      return "problem needs more than MONARCH_NOALLOC_SCRATCH_BYTES of scratch (use monarch_bwd)";
    default: return "unknown status";
  }
}

int monarch_abi_version(void) { return MONARCH_ABI_VERSION; }

}  // extern "C"
