// C ABI of libpgo (include/pgo.h): handle, arena, LM loop, inspection and
// timing.  Every step of the iteration runs in pgo_kernels.hip; this file
// plans the structure once and enqueues work on the handle's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "pgo.h"
#include "pgo_kernels.h"

using namespace pgo;

namespace {

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPC(expr)                                                  \
  do {                                                              \
    hipError_t e_ = (expr);                                         \
    if (e_ != hipSuccess) {                                         \
      g_err = std::string(#expr) + ": " + hipGetErrorString(e_);    \
      return PGO_ERR_DEVICE;                                        \
    }                                                               \
  } while (0)

#define CHECK_RC(expr)              \
  do {                              \
    int rc_ = (expr);               \
    if (rc_ != PGO_OK) return rc_;  \
  } while (0)

constexpr int kBatch = 4;   // PCG iterations per batch; the host waits one batch behind

struct Arena {
  char* base = nullptr;
  std::vector<std::pair<void**, size_t>> plan;
  template <class T>
  void add(T*& p, int64_t count) {
    plan.emplace_back(reinterpret_cast<void**>(&p), sizeof(T) * (size_t)std::max<int64_t>(count, 1));
  }
  int commit() {
    size_t total = 0;
    for (auto& e : plan) total += (e.second + 255) & ~size_t(255);
    if (hipMalloc(&base, total) != hipSuccess) {
      base = nullptr;
      return fail(PGO_ERR_ALLOC, "hipMalloc arena");
    }
    size_t off = 0;
    for (auto& e : plan) {
      *e.first = base + off;
      off += (e.second + 255) & ~size_t(255);
    }
    plan.clear();
    return PGO_OK;
  }
};

struct ProfRec {
  int kernel;
  int pcg_iter;
  hipEvent_t a, b;
};

}  // namespace

struct pgo_problem {
  int64_t n = 0, m = 0;
  int n_fixed = 0;
  pgo_options opt{};
  hipStream_t stream = nullptr;
  Arena arena;
  double* poses[2] = {nullptr, nullptr};
  double* tab[2] = {nullptr, nullptr};
  int cur = 0;
  int2* edges = nullptr;
  double *meas = nullptr, *meas_tab = nullptr, *info = nullptr;
  int32_t* half_ptr = nullptr;
  int2* nbr = nullptr;
  double *r = nullptr, *Ji = nullptr, *Jj = nullptr, *Hc = nullptr, *half = nullptr,
         *cost_part = nullptr;
  double *Hd = nullptr, *Hdd = nullptr, *Minv = nullptr, *g = nullptr;
  double *x = nullptr, *rv = nullptr, *z = nullptr, *p = nullptr, *q = nullptr, *red = nullptr;
  PcgState* pcg = nullptr;
  StepOut* out = nullptr;
  int* flags = nullptr;
  StepOut* h_out = nullptr;
  int* h_done = nullptr;
  int* h_done_dev = nullptr;
  hipEvent_t batch_ev[2] = {nullptr, nullptr};
  int last_iters = 0;
  double lambda = 0.0, cost = 0.0;
  int linearized = 0;
  int prof_on = 0, prof_every = 1;
  int64_t prof_seen[PGO_K_NUM] = {0};
  std::vector<ProfRec> prof_recs;
  std::vector<hipEvent_t> prof_pool;
  size_t prof_used = 0;
  int64_t prof_count[PGO_K_NUM] = {0};
  double prof_ms[PGO_K_NUM] = {0};
};

namespace {

Dev make_dev(const pgo_problem* h) {
  Dev d{};
  d.n = h->n;
  d.m = h->m;
  d.n_fixed = h->n_fixed;
  d.lambda = h->lambda;
  d.diag_floor = h->opt.diag_floor;
  d.tol = h->opt.pcg_rel_tol;
  d.poses = h->poses[h->cur];
  d.trial = h->poses[1 - h->cur];
  d.tab = h->tab[h->cur];
  d.tab_trial = h->tab[1 - h->cur];
  d.edges = h->edges;
  d.meas_tab = h->meas_tab;
  d.info = h->info;
  d.half_ptr = h->half_ptr;
  d.nbr = h->nbr;
  d.r = h->r;
  d.Ji = h->Ji;
  d.Jj = h->Jj;
  d.Hc = h->Hc;
  d.half = h->half;
  d.cost_part = h->cost_part;
  d.n_cost_parts = edge_blocks(h->m);
  d.Hd = h->Hd;
  d.Hdd = h->Hdd;
  d.Minv = h->Minv;
  d.g = h->g;
  d.x = h->x;
  d.rv = h->rv;
  d.z = h->z;
  d.p = h->p;
  d.q = h->q;
  d.red = h->red;
  d.red_nb = red_blocks(h->n);
  d.n_chunks = pcg_chunks(h->n);
  d.pcg = h->pcg;
  d.host_done = h->h_done_dev;
  d.out = h->out;
  d.flags = h->flags;
  return d;
}

int prof_begin(pgo_problem* h, int kernel, int it, hipEvent_t* stop) {
  *stop = nullptr;
  if (!((h->prof_on >> kernel) & 1)) return PGO_OK;
  if (h->prof_seen[kernel]++ % h->prof_every != 0) return PGO_OK;
  if (h->prof_used + 2 > h->prof_pool.size())
    for (int i = 0; i < 64; ++i) {
      hipEvent_t e;
      HIPC(hipEventCreate(&e));
      h->prof_pool.push_back(e);
    }
  hipEvent_t a = h->prof_pool[h->prof_used++], b = h->prof_pool[h->prof_used++];
  DispatchEvents& ev = dispatch_events();
  ev.start = a;
  ev.stop = b;
  ev.used = false;
  h->prof_recs.push_back({kernel, it, a, b});
  *stop = b;
  return PGO_OK;
}

int prof_end(pgo_problem* h, hipEvent_t stop) {
  if (!stop) return PGO_OK;
  DispatchEvents& ev = dispatch_events();
  if (!ev.used) {
    h->prof_recs.pop_back();
    h->prof_used -= 2;
  }
  ev = DispatchEvents{};
  return PGO_OK;
}

// PCG launches from the stopping iteration on exit at once; not counted.
int prof_collect(pgo_problem* h, int pcg_iters) {
  for (auto& r : h->prof_recs) {
    if (r.pcg_iter >= 0 && r.pcg_iter >= pcg_iters) continue;
    float ms = 0.f;
    HIPC(hipEventElapsedTime(&ms, r.a, r.b));
    h->prof_ms[r.kernel] += ms;
    h->prof_count[r.kernel] += 1;
  }
  h->prof_recs.clear();
  h->prof_used = 0;
  return PGO_OK;
}

#define TIMED(kid, it, call)                          \
  do {                                                \
    hipEvent_t stop_;                                 \
    CHECK_RC(prof_begin(h, (kid), (it), &stop_));     \
    call;                                             \
    CHECK_RC(prof_end(h, stop_));                     \
  } while (0)

int stage_linearize(pgo_problem* h, bool jac) {
  Dev d = make_dev(h);
  TIMED(PGO_K_EDGE, -1, launch_edge(d, jac, h->stream));
  HIPC(hipGetLastError());
  return PGO_OK;
}

// Damping, block-Jacobi inverses, and PCG queued in batches: the host waits
// for batch b only once batch b + 1 is queued, then reads the host-mapped
// stop flag; launches past the stopping iteration exit at once.
int stage_step(pgo_problem* h) {
  Dev d = make_dev(h);
  HIPC(hipMemsetAsync(h->flags, 0, 2 * sizeof(int), h->stream));
  TIMED(PGO_K_POSE, -1, launch_pose(d, h->stream));
  launch_pcg_init(d, h->stream);
  *h->h_done = 0;
  const int maxit = h->opt.pcg_max_iters;
  int next = 0;
  auto enqueue = [&](int k) -> int {
    for (int u = 0; u < k && next < maxit; ++u, ++next) {
      TIMED(PGO_K_PCG_A, next, launch_pcg_a(d, next, h->stream));
      TIMED(PGO_K_PCG_B, next, launch_pcg_b(d, next, h->stream));
    }
    return PGO_OK;
  };
  int queued = 0, waited = 0;
  if (maxit > 0) {
    CHECK_RC(enqueue(std::max(kBatch, h->last_iters - kBatch)));
    HIPC(hipEventRecord(h->batch_ev[0], h->stream));
    queued = 1;
    while (next < maxit) {
      CHECK_RC(enqueue(kBatch));
      HIPC(hipEventRecord(h->batch_ev[queued & 1], h->stream));
      ++queued;
      HIPC(hipEventSynchronize(h->batch_ev[waited & 1]));
      ++waited;
      if (__atomic_load_n(h->h_done, __ATOMIC_ACQUIRE)) break;
    }
  }
  launch_pcg_final(d, next, h->stream);
  HIPC(hipGetLastError());
  return PGO_OK;
}

int read_out(pgo_problem* h) {
  HIPC(hipMemcpyAsync(h->h_out, h->out, sizeof(StepOut), hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  return PGO_OK;
}

int current_cost(pgo_problem* h, double* c) {
  Dev d = make_dev(h);
  launch_cost(d, d.tab, h->stream);
  launch_cost_final(d, h->stream);
  HIPC(hipGetLastError());
  CHECK_RC(read_out(h));
  *c = h->h_out->trial_cost;
  return PGO_OK;
}

int lm_step(pgo_problem* h, pgo_step_info* info) {
  if (!h->linearized) CHECK_RC(stage_linearize(h, false));
  h->linearized = 1;
  CHECK_RC(stage_step(h));
  Dev d = make_dev(h);
  TIMED(PGO_K_RETRACT, -1, launch_retract(d, h->stream));
  TIMED(PGO_K_PREP, -1, launch_prep(d.trial, d.tab_trial, h->n, h->stream));
  TIMED(PGO_K_COST, -1, launch_cost(d, d.tab_trial, h->stream));
  launch_cost_final(d, h->stream);
  HIPC(hipGetLastError());
  CHECK_RC(read_out(h));
  const StepOut o = *h->h_out;
  h->last_iters = o.pcg_iters;
  if (h->prof_on) CHECK_RC(prof_collect(h, o.pcg_iters));
  if (o.not_spd) return fail(PGO_ERR_NOT_SPD, "a damped 6x6 block is not positive definite");
  pgo_step_info inf{};
  inf.cost_before = h->cost;
  inf.cost_after = o.trial_cost;
  inf.lambda = h->lambda;
  inf.pcg_iters = o.pcg_iters;
  inf.pcg_rel_res = o.pcg_rel_res;
  if (std::isfinite(o.trial_cost) && o.trial_cost < h->cost) {
    inf.accepted = 1;
    h->cur = 1 - h->cur;
    h->cost = o.trial_cost;
    h->linearized = 0;
    h->lambda = std::max(h->lambda / h->opt.lambda_down, h->opt.lambda_min);
  } else {
    inf.accepted = 0;
    h->lambda = std::min(h->lambda * h->opt.lambda_up, h->opt.lambda_max);
  }
  if (info) *info = inf;
  return PGO_OK;
}

int check_options(const pgo_options& o) {
  if (!(o.lambda0 >= 0.0) || !(o.lambda_up >= 1.0) || !(o.lambda_down >= 1.0) ||
      !(o.lambda_min >= 0.0) || !(o.lambda_max >= o.lambda_min))
    return fail(PGO_ERR_ARG, "bad damping schedule");
  if (!(o.diag_floor >= 0.0)) return fail(PGO_ERR_ARG, "diag_floor must be >= 0");
  if (o.pcg_max_iters < 0 || !(o.pcg_rel_tol >= 0.0)) return fail(PGO_ERR_ARG, "bad PCG options");
  if (o.mem != PGO_MEM_HOST && o.mem != PGO_MEM_DEVICE) return fail(PGO_ERR_ARG, "bad mem");
  return PGO_OK;
}

}  // namespace

extern "C" {

int pgo_options_default(pgo_options* o) {
  if (!o) return PGO_ERR_ARG;
  o->lambda0 = 1e-3;
  o->lambda_up = 10.0;
  o->lambda_down = 10.0;
  o->lambda_min = 1e-16;
  o->lambda_max = 1e16;
  o->diag_floor = 1e-6;
  o->pcg_max_iters = 200;
  o->pcg_rel_tol = 1e-8;
  o->mem = PGO_MEM_HOST;
  o->stream = nullptr;
  return PGO_OK;
}

void pgo_destroy(pgo_problem* h) {
  if (!h) return;
  if (h->stream) (void)hipStreamSynchronize(h->stream);
  else (void)hipDeviceSynchronize();
  (void)hipFree(h->arena.base);
  if (h->h_out) (void)hipHostFree(h->h_out);
  if (h->h_done) (void)hipHostFree(h->h_done);
  for (hipEvent_t e : h->batch_ev)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : h->prof_pool) (void)hipEventDestroy(e);
  delete h;
}

int pgo_create(const double* poses, int64_t n, const int32_t* edges, const double* meas,
               const double* info, int64_t m, int n_fixed, const pgo_options* opts,
               pgo_problem** out) {
  if (!out) return fail(PGO_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!poses || n <= 0 || m < 0 || (m > 0 && (!edges || !meas || !info)) || n_fixed < 0 ||
      n_fixed > n || n >= (int64_t)INT32_MAX || m >= (int64_t)INT32_MAX / 2)
    return fail(PGO_ERR_ARG, "bad arguments");
  pgo_problem* h = new pgo_problem();
  if (opts) h->opt = *opts;
  else pgo_options_default(&h->opt);
  int rc = check_options(h->opt);
  if (rc != PGO_OK) {
    delete h;
    return rc;
  }
  h->stream = reinterpret_cast<hipStream_t>(h->opt.stream);
  h->n = n;
  h->m = m;
  h->n_fixed = n_fixed;
  hipStream_t s = h->stream;
  auto bail = [&](int code) {
    pgo_destroy(h);
    return code;
  };
  if (hipHostMalloc(reinterpret_cast<void**>(&h->h_out), sizeof(StepOut), hipHostMallocDefault) !=
          hipSuccess ||
      hipHostMalloc(reinterpret_cast<void**>(&h->h_done), sizeof(int), hipHostMallocMapped) !=
          hipSuccess ||
      hipHostGetDevicePointer(reinterpret_cast<void**>(&h->h_done_dev), h->h_done, 0) != hipSuccess ||
      hipEventCreateWithFlags(&h->batch_ev[0], hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&h->batch_ev[1], hipEventDisableTiming) != hipSuccess)
    return bail(fail(PGO_ERR_ALLOC, "pinned buffers or events"));
  *h->h_done = 0;
  // edges on the host for the per-pose lists
  std::vector<int32_t> eh(2 * (size_t)m);
  const hipMemcpyKind kin = h->opt.mem == PGO_MEM_DEVICE ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
  if (m) {
    if (h->opt.mem == PGO_MEM_DEVICE) {
      if (hipMemcpy(eh.data(), edges, sizeof(int32_t) * 2 * m, hipMemcpyDeviceToHost) != hipSuccess)
        return bail(fail(PGO_ERR_DEVICE, "copy of the edges"));
    } else {
      std::memcpy(eh.data(), edges, sizeof(int32_t) * 2 * m);
    }
  }
  for (int64_t e = 0; e < m; ++e) {
    const int32_t a = eh[2 * e], b = eh[2 * e + 1];
    if (a < 0 || a >= n || b < 0 || b >= n || a == b) return bail(fail(PGO_ERR_ARG, "bad edge"));
  }
  std::vector<int32_t> half_ptr(n + 1, 0);
  std::vector<int2> nbr(2 * (size_t)m);
  for (int64_t k = 0; k < 2 * m; ++k) ++half_ptr[eh[k] + 1];
  for (int64_t i = 0; i < n; ++i) half_ptr[i + 1] += half_ptr[i];
  {
    std::vector<int32_t> fill(half_ptr.begin(), half_ptr.end() - 1);
    for (int64_t k = 0; k < 2 * m; ++k)   // k = 2 e + side; the other end is eh[k ^ 1]
      nbr[fill[eh[k]]++] = make_int2((int)k, eh[k ^ 1]);
  }
  Arena& A = h->arena;
  for (int c = 0; c < 2; ++c) {
    A.add(h->poses[c], 6 * n);
    A.add(h->tab[c], 12 * n);
  }
  A.add(h->edges, m);
  A.add(h->meas, 6 * m);
  A.add(h->meas_tab, 12 * m);
  A.add(h->info, 2 * m);
  A.add(h->half_ptr, n + 1);
  A.add(h->nbr, 2 * m);
  A.add(h->r, 6 * m);
  A.add(h->Ji, 36 * m);
  A.add(h->Jj, 36 * m);
  A.add(h->Hc, (int64_t)kCoupVals * m);
  A.add(h->half, (int64_t)kHalfVals * 2 * m);
  A.add(h->cost_part, edge_blocks(m));
  A.add(h->Hd, 36 * n);
  A.add(h->Hdd, (int64_t)kSymVals * n);
  A.add(h->Minv, (int64_t)kSymVals * n);
  A.add(h->g, 6 * n);
  A.add(h->x, 6 * n);
  A.add(h->rv, 6 * n);
  A.add(h->z, 6 * n);
  A.add(h->p, 6 * n);
  A.add(h->q, 6 * n);
  A.add(h->red, kNumSums * (int64_t)red_blocks(n));
  A.add(h->pcg, 1);
  A.add(h->out, 1);
  A.add(h->flags, 2);
  if ((rc = A.commit()) != PGO_OK) return bail(rc);
  auto cp = [&](void* dst, const void* src, size_t bytes, hipMemcpyKind k) -> bool {
    return bytes == 0 || hipMemcpyAsync(dst, src, bytes, k, s) == hipSuccess;
  };
  bool ok = cp(h->poses[0], poses, sizeof(double) * 6 * n, kin) &&
            cp(h->edges, eh.data(), sizeof(int32_t) * 2 * m, hipMemcpyHostToDevice) &&
            cp(h->meas, meas, sizeof(double) * 6 * m, kin) &&
            cp(h->info, info, sizeof(double) * 2 * m, kin) &&
            cp(h->half_ptr, half_ptr.data(), sizeof(int32_t) * (n + 1), hipMemcpyHostToDevice) &&
            cp(h->nbr, nbr.data(), sizeof(int2) * 2 * m, hipMemcpyHostToDevice) &&
            hipMemsetAsync(h->flags, 0, 2 * sizeof(int), s) == hipSuccess &&
            hipMemsetAsync(h->x, 0, sizeof(double) * 6 * n, s) == hipSuccess &&
            hipMemsetAsync(h->pcg, 0, sizeof(PcgState), s) == hipSuccess;
  if (!ok) return bail(fail(PGO_ERR_DEVICE, "copy of the inputs"));
  h->cur = 0;
  h->lambda = h->opt.lambda0;
  Dev d = make_dev(h);
  launch_validate(d, h->meas, h->flags, s);
  int flags[2] = {0, 0};
  if (hipMemcpyAsync(flags, h->flags, sizeof(flags), hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return bail(fail(PGO_ERR_DEVICE, "validation"));
  if (flags[1]) return bail(fail(PGO_ERR_ARG, "non-positive information weight"));
  if (flags[0]) return bail(fail(PGO_ERR_NONFINITE, "non-finite input"));
  if (hipMemsetAsync(h->flags, 0, 2 * sizeof(int), s) != hipSuccess)
    return bail(fail(PGO_ERR_DEVICE, "flags"));
  launch_meas_prep(h->meas, h->meas_tab, m, s);
  launch_prep(h->poses[0], h->tab[0], n, s);
  double c = 0.0;
  rc = current_cost(h, &c);
  if (rc == PGO_OK && !std::isfinite(c)) rc = fail(PGO_ERR_NONFINITE, "initial cost is not finite");
  if (rc != PGO_OK) return bail(rc);
  h->cost = c;
  *out = h;
  return PGO_OK;
}

int pgo_lm_step(pgo_problem* h, pgo_step_info* info) {
  if (!h) return fail(PGO_ERR_ARG, "null handle");
  return lm_step(h, info);
}

int pgo_solve(pgo_problem* h, int n_iters, pgo_step_info* infos) {
  if (!h || n_iters < 0) return fail(PGO_ERR_ARG, "bad arguments");
  for (int k = 0; k < n_iters; ++k) CHECK_RC(lm_step(h, infos ? infos + k : nullptr));
  return PGO_OK;
}

int pgo_cost(pgo_problem* h, double* cost_out) {
  if (!h || !cost_out) return fail(PGO_ERR_ARG, "bad arguments");
  return current_cost(h, cost_out);
}

int pgo_get_poses(pgo_problem* h, double* out) {
  if (!h || !out) return fail(PGO_ERR_ARG, "bad arguments");
  HIPC(hipMemcpyAsync(out, h->poses[h->cur], sizeof(double) * 6 * h->n, hipMemcpyDeviceToHost,
                      h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  return PGO_OK;
}

int pgo_set_lambda(pgo_problem* h, double lambda) {
  if (!h || !(lambda >= 0.0)) return fail(PGO_ERR_ARG, "bad arguments");
  h->lambda = lambda;
  return PGO_OK;
}

int pgo_get_lambda(const pgo_problem* h, double* lambda_out) {
  if (!h || !lambda_out) return fail(PGO_ERR_ARG, "bad arguments");
  *lambda_out = h->lambda;
  return PGO_OK;
}

int pgo_debug_run(pgo_problem* h, int upto) {
  if (!h || upto < PGO_STAGE_LINEARIZE || upto > PGO_STAGE_STEP) return fail(PGO_ERR_ARG, "bad arguments");
  CHECK_RC(stage_linearize(h, true));
  h->linearized = 1;
  if (upto >= PGO_STAGE_STEP) {
    CHECK_RC(stage_step(h));
  } else {
    // per-pose sums of H and g (and the damped blocks at the current lambda)
    Dev d = make_dev(h);
    launch_pose(d, h->stream);
    HIPC(hipGetLastError());
  }
  HIPC(hipStreamSynchronize(h->stream));
  return PGO_OK;
}

int64_t pgo_debug_size(const pgo_problem* h, int which) {
  if (!h) return PGO_ERR_ARG;
  switch (which) {
    case PGO_DBG_R: return 6 * h->m;
    case PGO_DBG_JI: case PGO_DBG_JJ: case PGO_DBG_HO: return 36 * h->m;
    case PGO_DBG_HD: return 36 * h->n;
    case PGO_DBG_G: case PGO_DBG_DX: return 6 * h->n;
    case PGO_DBG_PCG: return 2;
    default: return PGO_ERR_ARG;
  }
}

int pgo_debug_get(pgo_problem* h, int which, double* out, int64_t count) {
  if (!h || !out) return fail(PGO_ERR_ARG, "bad arguments");
  const int64_t need = pgo_debug_size(h, which);
  if (need < 0 || count != need) return fail(PGO_ERR_ARG, "bad array id or count");
  const double* src = nullptr;
  switch (which) {
    case PGO_DBG_R: src = h->r; break;
    case PGO_DBG_JI: src = h->Ji; break;
    case PGO_DBG_JJ: src = h->Jj; break;
    case PGO_DBG_HD: src = h->Hd; break;
    case PGO_DBG_HO: {
      if (count == 0) return PGO_OK;
      double* tmp = nullptr;
      HIPC(hipMallocAsync(reinterpret_cast<void**>(&tmp), sizeof(double) * count, h->stream));
      launch_expand_coupling(make_dev(h), tmp, h->stream);
      hipError_t e1 = hipGetLastError();
      hipError_t e2 = hipMemcpyAsync(out, tmp, sizeof(double) * count, hipMemcpyDeviceToHost, h->stream);
      hipError_t e3 = hipFreeAsync(tmp, h->stream);
      hipError_t e4 = hipStreamSynchronize(h->stream);
      for (hipError_t e : {e1, e2, e3, e4})
        if (e != hipSuccess) return fail(PGO_ERR_DEVICE, std::string("coupling blocks: ") + hipGetErrorString(e));
      return PGO_OK;
    }
    case PGO_DBG_G: src = h->g; break;
    case PGO_DBG_DX: src = h->x; break;
    case PGO_DBG_PCG: {
      PcgState st;
      HIPC(hipMemcpyAsync(&st, h->pcg, sizeof(st), hipMemcpyDeviceToHost, h->stream));
      HIPC(hipStreamSynchronize(h->stream));
      out[0] = st.iters;
      out[1] = st.rhs_norm > 0.0 ? st.res_norm / st.rhs_norm : 0.0;
      return PGO_OK;
    }
    default: return fail(PGO_ERR_ARG, "bad array id");
  }
  if (count) HIPC(hipMemcpyAsync(out, src, sizeof(double) * count, hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  return PGO_OK;
}

int pgo_profile_enable(pgo_problem* h, int kernel_mask, int every) {
  if (!h || every < 1) return fail(PGO_ERR_ARG, "bad arguments");
  h->prof_on = kernel_mask;
  h->prof_every = every;
  for (int k = 0; k < PGO_K_NUM; ++k) {
    h->prof_seen[k] = 0;
    h->prof_count[k] = 0;
    h->prof_ms[k] = 0.0;
  }
  return PGO_OK;
}

int pgo_profile_get(pgo_problem* h, int kernel, int64_t* launches, double* total_ms) {
  if (!h || kernel < 0 || kernel >= PGO_K_NUM) return fail(PGO_ERR_ARG, "bad arguments");
  if (launches) *launches = h->prof_count[kernel];
  if (total_ms) *total_ms = h->prof_ms[kernel];
  return PGO_OK;
}

const char* pgo_status_string(int code) {
  static thread_local std::string msg;
  const char* base = "unknown status";
  switch (code) {
    case PGO_OK: base = "ok"; break;
    case PGO_ERR_ARG: base = "invalid argument"; break;
    case PGO_ERR_NONFINITE: base = "non-finite value"; break;
    case PGO_ERR_NOT_SPD: base = "matrix not positive definite"; break;
    case PGO_ERR_DEVICE: base = "device error"; break;
    case PGO_ERR_ALLOC: base = "allocation failed"; break;
  }
  msg = base;
  if (code != PGO_OK && !g_err.empty()) msg += ": " + g_err;
  return msg.c_str();
}

}  // extern "C"
