// C ABI of libba: handle, device arena, structure build and the LM loop.
// Declarations and argument documentation live in include/ba.h.
#include <hip/hip_runtime.h>
#include <hipcub/hipcub.hpp>

#include <algorithm>
#include <chrono>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "../../include/ba.h"

#include "ba_kernels.h"

using namespace ba;

namespace {

thread_local std::string g_err;

#define HIPC(expr)                                                                   \
  do {                                                                               \
    hipError_t e_ = (expr);                                                          \
    if (e_ != hipSuccess) {                                                          \
      g_err = std::string(#expr) + ": " + hipGetErrorString(e_);                     \
      return BA_ERR_DEVICE;                                                          \
    }                                                                                \
  } while (0)

#define CHECK_RC(expr)      \
  do {                      \
    int rc_ = (expr);       \
    if (rc_ != BA_OK) return rc_; \
  } while (0)

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

struct Arena {
  char* base = nullptr;
  size_t size = 0, used = 0;
  std::vector<std::pair<void**, size_t>> plan;
  template <class T>
  void add(T*& p, int64_t count) {
    plan.emplace_back(reinterpret_cast<void**>(&p), sizeof(T) * (size_t)std::max<int64_t>(count, 1));
  }
  int commit() {
    size_t total = 0;
    for (auto& e : plan) total += (e.second + 255) & ~size_t(255);
    hipError_t err = hipMalloc(&base, total);
    if (err != hipSuccess) {
      base = nullptr;
      return fail(BA_ERR_ALLOC, std::string("hipMalloc arena: ") + hipGetErrorString(err));
    }
    size = total;
    size_t off = 0;
    for (auto& e : plan) {
      *e.first = base + off;
      off += (e.second + 255) & ~size_t(255);
    }
    used = off;
    plan.clear();
    return BA_OK;
  }
};

struct ProfRec {
  int kernel;
  int pcg_iter;
  int step;          // queued LM step (0 otherwise)
  hipEvent_t a, b;
};

}  // namespace

int ba::set_error(int code, const std::string& msg) { return fail(code, msg); }

struct ba_problem {
  int64_t nc = 0, np = 0, nobs = 0;
  ba_options opt{};
  hipStream_t stream = nullptr;
  int n_chunks = 0, lds_blocks = 0,
      cam_lds_bytes = 0, cam_layout = 0, n_chunk_blocks = 0;
  Arena arena;   // everything sized by n_cams, n_pts, n_obs
  Arena arena2;  // partitions and partial sums, sized after the CSR offsets
  Arena arena3;  // dense solver: runs, block pair lists, S
  // parameters: [cur] current, [1 - cur] trial
  double* cams[2] = {nullptr, nullptr};
  double* pts[2] = {nullptr, nullptr};
  CamT* tab[2] = {nullptr, nullptr};
  double* camq[2] = {nullptr, nullptr};
  int cur = 0;
  // structure
  int32_t *perm_pt = nullptr, *perm_cam = nullptr, *pt_ptr = nullptr, *cam_ptr = nullptr;
  int32_t *o_cam = nullptr, *o_pt = nullptr, *c_pt = nullptr, *run_len = nullptr;
  double *o_uv = nullptr, *c_uv = nullptr;
  int32_t *cam_chunk_ptr = nullptr, *wave_begin = nullptr;
  int4* blk_chunk = nullptr;
  // dense solver
  int ds_ld = 0, ds_T = 0, ds_nruns = 0, ds_nblk = 0;
  int32_t *ds_run = nullptr, *ds_blk_ptr = nullptr;
  int2 *ds_blk = nullptr, *ds_pair = nullptr;
  double *ds_F = nullptr, *ds_S = nullptr, *ds_diag = nullptr, *ds_diagT = nullptr, *ds_dinv = nullptr, *ds_v = nullptr,
         *ds_cov = nullptr;
  // work arrays
  double *w_pt = nullptr, *w_cam = nullptr, *C = nullptr, *gp = nullptr, *B = nullptr,
         *gc = nullptr, *lin_part = nullptr;
  double *Cinv = nullptr, *Bd = nullptr, *rhs = nullptr, *Minv = nullptr,
         *Mfull = nullptr, *schur_part = nullptr;
  double *x = nullptr, *r = nullptr, *zc = nullptr, *pbuf = nullptr, *q = nullptr, *prec = nullptr,
         *pcg_part = nullptr, *red_part = nullptr, *pt_dot = nullptr, *cam_rows = nullptr;
  PcgState* pcg = nullptr;
  double *dp = nullptr, *cost_part = nullptr;
  double* vjp = nullptr;     // backward: df/du in the original observation order
  // dogleg: partials and sums of the step's model, the step's camera part
  double *dl_vpart = nullptr, *dl_opart = nullptr, *dl_out = nullptr, *dl_hc = nullptr;
  double radius = 0.0;
  int dl_valid = 0, dl_iters = 0;
  double dl_rel = 0.0;
  double dl_sums[6] = {0, 0, 0, 0, 0, 0};   // g.g, h.h, g.h, |Jg|^2, Jg.Jh, |Jh|^2
  StepOut* out = nullptr;
  int* flags = nullptr;
  StepOut* h_out = nullptr;  // pinned
  long long* h_done = nullptr;  // pinned, device-mapped, tagged with the solve's number in
                                // the upper 32 bits: [0] the solve stopped (low bits: its
                                // iteration count), [1] the last iteration whose stop test
                                // found the solve still running
  long long* h_done_dev = nullptr;
  long long pcg_seq = 0;        // PCG solves started on this handle
  int last_pcg_iters = 0;       // -1: the last solve's count was not yet seen
  // queued LM steps (ba_solve): the device state, its staging copy, the records
  LmDev* lm = nullptr;
  LmDev* h_lm = nullptr;        // pinned
  LmLog* lm_log = nullptr;
  int64_t lm_log_cap = 0;
  int queued = 0, q_step = 0;   // stages are building queued step q_step
  // work a stage left to the next one's launch: k_lin_final's (to the damping
  // launch) and k_pcg_final's, for a solve capped at this many iterations (to
  // the back-substitution; -1: none)
  int lin_final_pending = 0;
  int pcg_final_iters = -1;
  // LM state
  double lambda = 0.0, cost = 0.0;
  int linearized = 0;
  int64_t iteration = 0;
  // timing
  int prof_on = 0;
  int prof_every = 1;
  int64_t prof_seen[BA_K_NUM] = {0};
  std::vector<ProfRec> prof_recs;
  std::vector<hipEvent_t> prof_pool;
  size_t prof_used = 0;
  int64_t prof_count[BA_K_NUM] = {0};
  double prof_ms[BA_K_NUM] = {0};
};

namespace {

Dev make_dev(const ba_problem* h) {
  Dev d{};
  d.nc = h->nc;
  d.np = h->np;
  d.nobs = h->nobs;
  d.n_chunks = h->n_chunks;
  d.n_chunk_blocks = h->n_chunk_blocks;
  d.blk_chunk = h->blk_chunk;
  d.lds_blocks = h->lds_blocks;
  d.cam_lds_bytes = h->cam_lds_bytes;
  d.cam_layout = h->cam_layout;
  d.wave_begin = h->wave_begin;
  d.loss = h->opt.loss;
  d.delta = h->opt.huber_delta;
  d.diag_floor = h->opt.diag_floor;
  d.lambda = h->opt.strategy == BA_STRATEGY_DOGLEG ? h->opt.dl_gn_damping : h->lambda;
  d.tol = h->opt.pcg_rel_tol;
  const int c = h->cur, t = 1 - h->cur;
  d.cams = h->cams[c];
  d.pts = h->pts[c];
  d.tab = h->tab[c];
  d.camq = h->camq[c];
  d.cams_trial = h->cams[t];
  d.pts_trial = h->pts[t];
  d.tab_trial = h->tab[t];
  d.camq_trial = h->camq[t];
  d.o_cam = h->o_cam;
  d.o_pt = h->o_pt;
  d.o_uv = h->o_uv;
  d.c_pt = h->c_pt;
  d.c_uv = h->c_uv;
  d.run_len = h->run_len;
  d.pt_ptr = h->pt_ptr;
  d.cam_chunk_ptr = h->cam_chunk_ptr;
  d.w_pt = h->w_pt;
  d.w_cam = h->w_cam;
  d.C = h->C;
  d.gp = h->gp;
  d.B = h->B;
  d.gc = h->gc;
  d.lin_part = h->lin_part;
  d.Cinv = h->Cinv;
  d.Bd = h->Bd;
  d.rhs = h->rhs;
  d.Minv = h->Minv;
  d.Mfull = h->Mfull;
  d.schur_part = h->schur_part;
  d.x = h->x;
  d.r = h->r;
  d.zc = h->zc;
  d.pbuf = h->pbuf;
  d.q = h->q;
  d.prec = h->prec;
  d.pcg_part = h->pcg_part;
  d.red_part = h->red_part;
  d.pt_dot = h->pt_dot;
  d.cam_rows = h->cam_rows;
  d.red_nb = pcg_red_blocks(h->nc);
  d.host_done = h->h_done_dev;
  d.pcg_seq = h->pcg_seq;
  d.lm = h->queued ? h->lm : nullptr;
  d.lm_log = h->queued ? h->lm_log : nullptr;
  d.lm_up = h->opt.lambda_up;
  d.lm_down = h->opt.lambda_down;
  d.lm_min = h->opt.lambda_min;
  d.lm_max = h->opt.lambda_max;
  d.pcg = h->pcg;
  d.dp = h->dp;
  d.cost_part = h->cost_part;
  d.out = h->out;
  d.flags = h->flags;
  d.ds_n = (int)(9 * h->nc);
  d.ds_ld = h->ds_ld;
  d.ds_T = h->ds_T;
  d.ds_nruns = h->ds_nruns;
  d.ds_nblk = h->ds_nblk;
  d.ds_run = h->ds_run;
  d.ds_blk = h->ds_blk;
  d.ds_blk_ptr = h->ds_blk_ptr;
  d.ds_pair = h->ds_pair;
  d.ds_F = h->ds_F;
  d.ds_S = h->ds_S;
  d.ds_diag = h->ds_diag;
  d.ds_diagT = h->ds_diagT;
  d.ds_dinv = h->ds_dinv;
  d.ds_v = h->ds_v;
  return d;
}

// ---- kernel timing --------------------------------------------------------

// A timed launch hands a pair of pool events to the next kernel dispatch,
// which records them at its own start and end.
int prof_begin(ba_problem* h, int kernel, int pcg_iter, hipEvent_t* stop) {
  *stop = nullptr;
  if (!((h->prof_on >> kernel) & 1)) return BA_OK;
  if (h->prof_seen[kernel]++ % h->prof_every != 0) return BA_OK;
  if (h->prof_used + 2 > h->prof_pool.size()) {
    for (int i = 0; i < 64; ++i) {
      hipEvent_t e;
      HIPC(hipEventCreate(&e));
      h->prof_pool.push_back(e);
    }
  }
  hipEvent_t a = h->prof_pool[h->prof_used++], b = h->prof_pool[h->prof_used++];
  DispatchEvents& ev = dispatch_events();
  ev.start = a;
  ev.stop = b;
  ev.used = false;
  h->prof_recs.push_back({kernel, pcg_iter, h->queued ? h->q_step : 0, a, b});
  *stop = b;
  return BA_OK;
}

// Drops the record when nothing was launched (an empty launch).
int prof_end(ba_problem* h, hipEvent_t stop) {
  if (!stop) return BA_OK;
  DispatchEvents& ev = dispatch_events();
  if (!ev.used) {
    h->prof_recs.pop_back();
    h->prof_used -= 2;
  }
  ev = DispatchEvents{};
  return BA_OK;
}

// After a synchronisation: fold the recorded pairs into the totals.  PCG
// launches after convergence exit at once and are not counted, nor are the
// linearisation launches of queued steps that followed a rejected one
// (lin_ran[step] == 0; null: all ran).
int prof_collect_steps(ba_problem* h, const int* step_iters, const int* lin_ran) {
  for (auto& r : h->prof_recs) {
    if (r.pcg_iter >= 0 && r.pcg_iter >= step_iters[r.step]) continue;
    if (lin_ran && !lin_ran[r.step] && (r.kernel == BA_K_LIN_PT || r.kernel == BA_K_LIN_CAM))
      continue;
    float ms = 0.f;
    HIPC(hipEventElapsedTime(&ms, r.a, r.b));
    h->prof_ms[r.kernel] += ms;
    h->prof_count[r.kernel] += 1;
  }
  h->prof_recs.clear();
  h->prof_used = 0;
  return BA_OK;
}

int prof_collect(ba_problem* h, int pcg_iters) {
  return prof_collect_steps(h, &pcg_iters, nullptr);
}

#define TIMED(kid, it, call)                   \
  do {                                         \
    hipEvent_t stop_;                          \
    CHECK_RC(prof_begin(h, (kid), (it), &stop_)); \
    call;                                      \
    CHECK_RC(prof_end(h, stop_));              \
  } while (0)

// ---- pieces of one LM iteration -------------------------------------------

// defer_final: the per-camera sums are left to stage_schur's first launch,
// which must follow.
int stage_linearize(ba_problem* h, bool defer_final = false) {
  Dev d = make_dev(h);
  TIMED(BA_K_LIN_PT, -1, launch_lin_pt(d, h->stream));
  TIMED(BA_K_LIN_CAM, -1, launch_lin_cam(d, h->stream));
  h->lin_final_pending = defer_final ? 1 : 0;
  if (!defer_final) launch_lin_final(d, h->stream);
  HIPC(hipGetLastError());
  return BA_OK;
}

int stage_schur(ba_problem* h) {
  Dev d = make_dev(h);
  // a queued step after the first finds the flags cleared by the last decision
  if (!(h->queued && h->q_step > 0)) HIPC(hipMemsetAsync(h->flags, 0, 2 * sizeof(int), h->stream));
  TIMED(BA_K_DAMP_PT, -1, launch_damp_pt(d, h->stream, h->lin_final_pending != 0));
  h->lin_final_pending = 0;
  TIMED(BA_K_SCHUR_CAM, -1, launch_schur_cam(d, h->stream));
  // the PCG, which always follows, starts in the same launch
  TIMED(BA_K_PRECOND, -1, launch_precond(d, h->stream, h->opt.solver != BA_SOLVER_DENSE_SCHUR));
  HIPC(hipGetLastError());
  return BA_OK;
}

// PCG iterations: the first batch is three shorter than the previous solve
// (the iteration count changes slowly across LM steps); after it the host
// queues one iteration at a time, as soon as the stop test of the last queued
// one (made at the start of its point pass) has found the solve still running,
// which block 0 reports in host-mapped memory.  The new iteration is then
// queued while the last one's camera pass and update run, so the device does
// not wait for the host and always has the next kernels in its queue, and once
// the test stops the solve no further iteration has been queued.  The kernels
// raise the host-mapped stop flag when the solve stops; every launch after
// that exits at once.  Both host-mapped words carry the solve's number, so a
// late write of an earlier solve (queued LM steps do not wait for one to
// finish) is never taken for this one's.  A wait that takes far longer than
// an iteration falls back to synchronising the stream, which also reports
// device errors.
int stage_pcg(ba_problem* h, bool defer_final) {
  const int maxit = h->opt.pcg_max_iters;
  if (h->last_pcg_iters < 0) {
    // the last solve was queued to its cap before its stop was seen
    const long long v = __atomic_load_n(&h->h_done[0], __ATOMIC_ACQUIRE);
    h->last_pcg_iters = v >= (h->pcg_seq << 32) ? (int)(v & 0xffffffffll) : maxit;
  }
  h->pcg_seq += 1;
  const long long tag = h->pcg_seq << 32;
  Dev d = make_dev(h);   // the start (r, x, z, partials) was made by k_precond
  int next_it = 0;
  auto enqueue = [&](int n) -> int {
    for (int k = 0; k < n; ++k, ++next_it) {
      TIMED(BA_K_PCG_PT, next_it, launch_pcg_pt(d, next_it, h->stream));
      TIMED(BA_K_PCG_CAM, next_it, launch_pcg_cam(d, h->stream));
      TIMED(BA_K_PCG_XR, next_it, launch_pcg_step(d, next_it, h->stream));
    }
    return BA_OK;
  };
  int launched = std::min(maxit, std::max(1, h->last_pcg_iters - 3));
  if (maxit > 0) {
    CHECK_RC(enqueue(launched));
    while (launched < maxit) {
      // wait for the stop test of iteration launched - 1
      const auto t0 = std::chrono::steady_clock::now();
      bool synced = false;
      for (;;) {
        if (__atomic_load_n(&h->h_done[0], __ATOMIC_ACQUIRE) >= tag) break;
        if (__atomic_load_n(&h->h_done[1], __ATOMIC_ACQUIRE) >= tag + launched - 1) break;
        if (synced) break;   // everything queued has run: nothing more will change
        if (std::chrono::steady_clock::now() - t0 > std::chrono::milliseconds(20)) {
          HIPC(hipStreamSynchronize(h->stream));
          synced = true;
        }
      }
      if (__atomic_load_n(&h->h_done[0], __ATOMIC_ACQUIRE) >= tag) break;
      CHECK_RC(enqueue(1));
      launched += 1;
    }
  }
  const long long v = __atomic_load_n(&h->h_done[0], __ATOMIC_ACQUIRE);
  h->last_pcg_iters = v >= tag ? (int)(v & 0xffffffffll) : -1;
  // a capped solve's record: here, or with defer_final in the back-substitution
  // launch of stage_update, which must follow
  h->pcg_final_iters = defer_final ? next_it : -1;
  if (!defer_final) launch_pcg_final(d, next_it, h->stream);
  HIPC(hipGetLastError());
  return BA_OK;
}

// Explicit S and its Cholesky factorisation by tile columns, the rhs as an
// extra row (it ends as L^-1 rhs); with `cov` the same launches also form
// Z = L^-T in the upper tiles.
int stage_dense_factor(ba_problem* h, int cov) {
  Dev d = make_dev(h);
  hipStream_t s = h->stream;
  TIMED(BA_K_DS_RUNS, -1, launch_ds_runs(d, s));
  TIMED(BA_K_DS_FILL, -1, launch_ds_fill(d, s));
  TIMED(BA_K_DS_ASSEMBLE, -1, launch_ds_assemble(d, s));
  // with `cov` the upper tiles, which take Z's off-diagonal tiles, start at zero
  if (cov) TIMED(BA_K_COV_ZERO, -1, launch_cov_zero(d, s));
  for (int k = -1; k < h->ds_T - 1; ++k)
    TIMED(k < 0 ? BA_K_DS_PANEL : BA_K_DS_UPDATE, -1, launch_ds_step(d, k, cov, s));
  HIPC(hipGetLastError());
  return BA_OK;
}

// Dense solve of S dc = rhs: factorisation, then back-substitution.
int stage_dense(ba_problem* h) {
  CHECK_RC(stage_dense_factor(h, 0));
  Dev d = make_dev(h);
  TIMED(BA_K_DS_BACKSOLVE, -1, launch_ds_backsolve(d, h->stream));
  HIPC(hipGetLastError());
  return BA_OK;
}

int stage_solve(ba_problem* h, bool defer_final = false) {
  h->pcg_final_iters = -1;
  return h->opt.solver == BA_SOLVER_DENSE_SCHUR ? stage_dense(h) : stage_pcg(h, defer_final);
}

int stage_update(ba_problem* h) {
  Dev d = make_dev(h);
  // the trial cameras (and a capped PCG solve's record) ride on the
  // back-substitution launch
  TIMED(BA_K_BACKSUB, -1, launch_backsub(d, h->stream, h->pcg_final_iters, true));
  h->pcg_final_iters = -1;
  TIMED(BA_K_COST, -1, launch_cost(d, d.pts_trial, d.tab_trial, d.camq_trial, h->stream,
                                   h->queued ? h->q_step : -1));
  if (h->queued) launch_lm_commit(d, h->stream);
  HIPC(hipGetLastError());
  return BA_OK;
}

int read_out(ba_problem* h) {
  HIPC(hipMemcpyAsync(h->h_out, h->out, sizeof(StepOut), hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  return BA_OK;
}

int current_cost(ba_problem* h, double* c) {
  Dev d = make_dev(h);
  launch_cost(d, d.pts, d.tab, d.camq, h->stream);
  HIPC(hipGetLastError());
  CHECK_RC(read_out(h));
  *c = h->h_out->trial_cost;
  return BA_OK;
}

int dogleg_step(ba_problem* h, ba_step_info* info);

int lm_step(ba_problem* h, ba_step_info* info) {
  if (h->opt.strategy == BA_STRATEGY_DOGLEG) return dogleg_step(h, info);
  if (!h->linearized) CHECK_RC(stage_linearize(h, true));
  CHECK_RC(stage_schur(h));
  h->linearized = 1;
  CHECK_RC(stage_solve(h, true));
  CHECK_RC(stage_update(h));
  CHECK_RC(read_out(h));
  const StepOut o = *h->h_out;
  h->last_pcg_iters = o.pcg_iters;
  if (h->prof_on) CHECK_RC(prof_collect(h, o.pcg_iters));
  if (o.not_spd) return fail(BA_ERR_NOT_SPD, "a damped block is not positive definite");
  ba_step_info inf{};
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
  h->iteration += 1;
  if (info) *info = inf;
  return BA_OK;
}

// One dogleg iteration (BA_STRATEGY_DOGLEG in include/ba.h): at a new point
// of linearisation the Gauss-Newton step of the system damped by
// dl_gn_damping (Schur elimination, the configured solver,
// back-substitution) and the six sums of the quadratic model; then the step
// h = s_g g + s_n h_gn for the current radius, the trial cost and the gain
// ratio.  The step's coefficients are chosen on the host from the sums.
int dogleg_step(ba_problem* h, ba_step_info* info) {
  hipStream_t s = h->stream;
  int pcg_iters = 0;
  double pcg_rel = 0.0;
  if (!h->dl_valid) {
    if (!h->linearized) CHECK_RC(stage_linearize(h));
    h->linearized = 1;
    CHECK_RC(stage_schur(h));
    CHECK_RC(stage_solve(h));
    Dev d = make_dev(h);
    TIMED(BA_K_BACKSUB, -1, launch_backsub(d, s));
    launch_dl_vec(d, h->dl_vpart, s);
    TIMED(BA_K_DL_OBS, -1, launch_dl_obs(d, h->dl_opart, s));
    launch_dl_final(d, h->dl_vpart, h->dl_opart, h->dl_out, s);
    HIPC(hipGetLastError());
    PcgState st;
    int flags[2] = {0, 0};
    HIPC(hipMemcpyAsync(h->dl_sums, h->dl_out, sizeof(h->dl_sums), hipMemcpyDeviceToHost, s));
    HIPC(hipMemcpyAsync(&st, h->pcg, sizeof(st), hipMemcpyDeviceToHost, s));
    HIPC(hipMemcpyAsync(flags, h->flags, sizeof(flags), hipMemcpyDeviceToHost, s));
    HIPC(hipStreamSynchronize(s));
    if (flags[1]) return fail(BA_ERR_NOT_SPD, "a damped block is not positive definite");
    h->dl_iters = pcg_iters = st.iters;
    h->dl_rel = pcg_rel = st.rhs_norm > 0.0 ? st.res_norm / st.rhs_norm : 0.0;
    h->last_pcg_iters = st.iters;
    h->dl_valid = 1;
  }
  const double gg = h->dl_sums[0], nn = h->dl_sums[1], gn = h->dl_sums[2];
  const double JgJg = h->dl_sums[3], JgJn = h->dl_sums[4], JnJn = h->dl_sums[5];
  const double R = h->radius, gnorm = std::sqrt(gg), nnorm = std::sqrt(nn);
  double s_g = 0.0, s_n = 0.0;
  int kind = 0;
  if (gg == 0.0) {
    kind = 0;   // stationary: no step
  } else if (nnorm <= R) {
    s_n = 1.0;
  } else {
    const double alpha = JgJg > 0.0 ? gg / JgJg : INFINITY;
    if (alpha * gnorm >= R) {
      s_g = -R / gnorm;
      kind = 1;
    } else {
      // a = -alpha g, b = h_gn: |a + beta (b - a)| = R
      const double aa = alpha * alpha * gg;
      const double c = -alpha * gn - aa;
      const double dd = nn + 2.0 * alpha * gn + aa;
      const double disc = std::sqrt(c * c + dd * (R * R - aa));
      const double beta = c <= 0.0 ? (-c + disc) / dd : (R * R - aa) / (c + disc);
      s_g = -alpha * (1.0 - beta);
      s_n = beta;
      kind = 2;
    }
  }
  const double hh = s_g * s_g * gg + 2.0 * s_g * s_n * gn + s_n * s_n * nn;
  const double hnorm = std::sqrt(hh > 0.0 ? hh : 0.0);
  const double model = -(s_g * gg + s_n * gn) - 0.5 * (s_g * s_g * JgJg + 2.0 * s_g * s_n * JgJn +
                                                       s_n * s_n * JnJn);
  Dev d = make_dev(h);
  TIMED(BA_K_DL_STEP, -1, launch_dl_step(d, s_g, s_n, h->dl_hc, s));
  Dev dr = d;
  dr.x = h->dl_hc;
  TIMED(BA_K_RETRACT, -1, launch_retract(dr, s));
  TIMED(BA_K_COST, -1, launch_cost(d, d.pts_trial, d.tab_trial, d.camq_trial, s));
  HIPC(hipGetLastError());
  CHECK_RC(read_out(h));
  const double trial = h->h_out->trial_cost;
  if (h->prof_on) CHECK_RC(prof_collect(h, pcg_iters));
  const double rho = model > 0.0 ? (h->cost - trial) / model : 0.0;
  ba_step_info inf{};
  inf.cost_before = h->cost;
  inf.cost_after = trial;
  inf.lambda = h->opt.dl_gn_damping;
  inf.pcg_iters = pcg_iters;
  inf.pcg_rel_res = pcg_rel;
  inf.radius = R;
  inf.gain_ratio = rho;
  inf.step_norm = hnorm;
  inf.step_kind = kind;
  if (rho > 0.75) h->radius = std::max(h->radius, 3.0 * hnorm);
  else if (rho < 0.25) h->radius = 0.5 * h->radius;
  if (std::isfinite(trial) && trial < h->cost) {
    inf.accepted = 1;
    h->cur = 1 - h->cur;
    h->cost = trial;
    h->linearized = 0;
    h->dl_valid = 0;
  }
  h->iteration += 1;
  if (info) *info = inf;
  return BA_OK;
}

// ---- structure build --------------------------------------------------------

int sort_pairs(const int32_t* major, const int32_t* minor, int64_t n_major, int64_t n_minor,
               int64_t n, int32_t* perm_out, hipStream_t s) {
  uint64_t *k_in = nullptr, *k_out = nullptr;
  int32_t* v_in = nullptr;
  void* tmp = nullptr;
  size_t tmp_bytes = 0;
  int end_bit = 1;
  const unsigned long long maxkey = (unsigned long long)n_major * (unsigned long long)n_minor;
  while (end_bit < 64 && (1ull << end_bit) < maxkey) ++end_bit;
  auto cleanup = [&]() {
    (void)hipFree(k_in);
    (void)hipFree(k_out);
    (void)hipFree(v_in);
    (void)hipFree(tmp);
  };
  if (hipMalloc(&k_in, sizeof(uint64_t) * n) != hipSuccess ||
      hipMalloc(&k_out, sizeof(uint64_t) * n) != hipSuccess ||
      hipMalloc(&v_in, sizeof(int32_t) * n) != hipSuccess) {
    cleanup();
    return fail(BA_ERR_ALLOC, "hipMalloc sort buffers");
  }
  launch_make_keys(major, minor, n_minor, n, k_in, v_in, s);
  hipError_t e = hipcub::DeviceRadixSort::SortPairs(nullptr, tmp_bytes, k_in, k_out, v_in, perm_out,
                                                   (int)n, 0, end_bit, s);
  if (e == hipSuccess) e = hipMalloc(&tmp, std::max<size_t>(tmp_bytes, 1));
  if (e == hipSuccess)
    e = hipcub::DeviceRadixSort::SortPairs(tmp, tmp_bytes, k_in, k_out, v_in, perm_out, (int)n, 0,
                                           end_bit, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  cleanup();
  if (e != hipSuccess) return fail(BA_ERR_DEVICE, std::string("radix sort: ") + hipGetErrorString(e));
  return BA_OK;
}

int build(ba_problem* h, const double* cams_in, const double* pts_in, const int32_t* cam_in,
          const int32_t* pt_in, const double* uv_in) {
  const int64_t nc = h->nc, np = h->np, N = h->nobs;
  const hipStream_t s = h->stream;
  const hipMemcpyKind kind =
      h->opt.mem == BA_MEM_DEVICE ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;

  // Raw inputs on the device (temporary).
  int32_t *d_cam = nullptr, *d_pt = nullptr, *d_ccam = nullptr;
  double* d_uv = nullptr;
  int* d_flags = nullptr;
  auto tmp_free = [&]() {
    (void)hipFree(d_cam);
    (void)hipFree(d_pt);
    (void)hipFree(d_uv);
    (void)hipFree(d_flags);
    (void)hipFree(d_ccam);
  };
  const int64_t Na = std::max<int64_t>(N, 1);
  if (hipMalloc(&d_cam, sizeof(int32_t) * Na) != hipSuccess ||
      hipMalloc(&d_pt, sizeof(int32_t) * Na) != hipSuccess ||
      hipMalloc(&d_uv, sizeof(double) * 2 * Na) != hipSuccess ||
      hipMalloc(&d_ccam, sizeof(int32_t) * Na) != hipSuccess ||
      hipMalloc(&d_flags, sizeof(int) * 2) != hipSuccess) {
    tmp_free();
    return fail(BA_ERR_ALLOC, "hipMalloc input staging");
  }

  // Persistent arena.
  Arena& A = h->arena;
  for (int b = 0; b < 2; ++b) {
    A.add(h->cams[b], 9 * nc);
    A.add(h->pts[b], 3 * np);
    A.add(h->tab[b], nc);
    A.add(h->camq[b], 4 * nc);
  }
  A.add(h->perm_pt, N);
  A.add(h->perm_cam, N);
  A.add(h->pt_ptr, np + 1);
  A.add(h->cam_ptr, nc + 1);
  A.add(h->o_cam, N);
  A.add(h->o_pt, N);
  A.add(h->o_uv, 2 * N);
  A.add(h->c_pt, N);
  A.add(h->c_uv, 2 * N);
  A.add(h->run_len, N);
  A.add(h->w_pt, N);
  A.add(h->w_cam, N);
  A.add(h->C, 6 * np);
  A.add(h->gp, 3 * np);
  A.add(h->Cinv, 6 * np);
  A.add(h->prec, 8 * np);
  A.add(h->dp, 3 * np);
  A.add(h->vjp, 2 * N);
  A.add(h->B, 45 * nc);
  A.add(h->gc, 9 * nc);
  A.add(h->Bd, 45 * nc);
  A.add(h->rhs, 9 * nc);
  A.add(h->Minv, 45 * nc);
  A.add(h->Mfull, 45 * nc);
  A.add(h->x, 9 * nc);
  A.add(h->r, 9 * nc);
  A.add(h->zc, 9 * nc);
  A.add(h->pbuf, 9 * nc);
  A.add(h->q, 9 * nc);
  A.add(h->pcg, 1);
  A.add(h->out, 1);
  A.add(h->flags, 2);
  A.add(h->lm, 1);
  A.add(h->cam_chunk_ptr, nc + 1);

  // Partitions need the CSR offsets first, so they get a second small arena
  // piece below; everything above is committed now.
  int rc = A.commit();
  if (rc != BA_OK) {
    tmp_free();
    return rc;
  }
  if (hipMemsetAsync(A.base, 0, A.size, s) != hipSuccess) {
    tmp_free();
    return fail(BA_ERR_DEVICE, "arena clear");
  }

  hipError_t e = hipSuccess;
#define TRY(x)                                                         \
  do {                                                                 \
    e = (x);                                                           \
    if (e != hipSuccess) {                                             \
      tmp_free();                                                      \
      return fail(BA_ERR_DEVICE, std::string(#x) + ": " + hipGetErrorString(e)); \
    }                                                                  \
  } while (0)
  TRY(hipMemcpyAsync(h->cams[0], cams_in, sizeof(double) * 9 * nc, kind, s));
  TRY(hipMemcpyAsync(h->pts[0], pts_in, sizeof(double) * 3 * np, kind, s));
  if (N > 0) {
    TRY(hipMemcpyAsync(d_cam, cam_in, sizeof(int32_t) * N, kind, s));
    TRY(hipMemcpyAsync(d_pt, pt_in, sizeof(int32_t) * N, kind, s));
    TRY(hipMemcpyAsync(d_uv, uv_in, sizeof(double) * 2 * N, kind, s));
  }
  TRY(hipMemsetAsync(d_flags, 0, sizeof(int) * 2, s));
  launch_validate(d_cam, d_pt, d_uv, N, h->cams[0], nc, h->pts[0], np, d_flags, s);
  int flags[2] = {0, 0};
  TRY(hipMemcpyAsync(flags, d_flags, sizeof(flags), hipMemcpyDeviceToHost, s));
  TRY(hipStreamSynchronize(s));
  if (flags[0]) {
    tmp_free();
    return fail(BA_ERR_ARG, "observation index out of range");
  }
  if (flags[1]) {
    tmp_free();
    return fail(BA_ERR_NONFINITE, "non-finite camera, point or observation");
  }

  if (N > 0) {
    rc = sort_pairs(d_pt, d_cam, np, nc, N, h->perm_pt, s);
    if (rc == BA_OK) rc = sort_pairs(d_cam, d_pt, nc, np, N, h->perm_cam, s);
    if (rc != BA_OK) {
      tmp_free();
      return rc;
    }
    launch_gather_obs(h->perm_pt, d_cam, d_pt, d_uv, N, h->o_cam, h->o_pt, h->o_uv, s);
    launch_gather_obs(h->perm_cam, d_cam, d_pt, d_uv, N, d_ccam, h->c_pt, h->c_uv, s);
    launch_run_len(d_ccam, h->c_pt, N, h->run_len, s);
  }
  launch_seg_ptr(h->o_pt, N, np, h->pt_ptr, s);
  launch_seg_ptr(d_ccam, N, nc, h->cam_ptr, s);
  TRY(hipGetLastError());

  std::vector<int32_t> pt_ptr(np + 1), cam_ptr(nc + 1);
  TRY(hipMemcpyAsync(pt_ptr.data(), h->pt_ptr, sizeof(int32_t) * (np + 1), hipMemcpyDeviceToHost, s));
  TRY(hipMemcpyAsync(cam_ptr.data(), h->cam_ptr, sizeof(int32_t) * (nc + 1), hipMemcpyDeviceToHost, s));
  TRY(hipStreamSynchronize(s));
  tmp_free();
  d_cam = d_pt = d_ccam = nullptr;
  d_uv = nullptr;
  d_flags = nullptr;

  // The kernels that keep the camera table in LDS run one block per compute
  // unit; each wavefront takes an equal share of the observations, moved to
  // the nearest point start at or after the even split.
  // The point passes' camera data: up to kCamLdsMaxCams cameras whole rows
  // in LDS; up to kZLdsMaxCams the PCG's 9-vectors there and the geometry in
  // memory; past that everything in memory.  BA_NO_LDS_CAMERAS=1 at creation
  // selects the memory layout, BA_SPLIT_LDS_CAMERAS=1 the vectors layout
  // where it fits (for the tests of those layouts on small scenes).
  std::vector<int32_t> wave_begin;
  {
    int dev = 0, cus = 0;
    TRY(hipGetDevice(&dev));
    TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    h->cam_lds_bytes = 0;
    h->cam_layout = kCamMemory;
    h->lds_blocks = 0;
    const char* off = std::getenv("BA_NO_LDS_CAMERAS");
    const char* spl = std::getenv("BA_SPLIT_LDS_CAMERAS");
    if (!(off && off[0] == '1')) {
      if (nc <= kCamLdsMaxCams && !(spl && spl[0] == '1')) {
        h->cam_layout = kCamRows;
        h->cam_lds_bytes = (int)(kCamLdsStride * 8 * nc);
      } else if (nc <= kZLdsMaxCams) {
        h->cam_layout = kCamVectors;
        h->cam_lds_bytes = (int)(kZLdsStride * 8 * nc);
      }
    }
    if (h->cam_lds_bytes > 0) TRY(set_lds_camera_limit());
    {
      // with no observations one block of empty ranges still makes the
      // PCG's stop test and per-block partials
      constexpr int wpb = kLdsBlock / kWave;
      const int64_t want = (N + (int64_t)wpb * kWave - 1) / ((int64_t)wpb * kWave);
      h->lds_blocks = (int)std::max<int64_t>(1, std::min<int64_t>(std::max(cus, 1), want));
      const int64_t W = (int64_t)h->lds_blocks * wpb;
      wave_begin.resize(W + 1);
      for (int64_t w = 0; w <= W; ++w) {
        const int64_t target = N * w / W;
        wave_begin[w] = *std::lower_bound(pt_ptr.begin(), pt_ptr.end(), (int32_t)target);
      }
      wave_begin[W] = (int32_t)N;
    }
  }
  // Camera chunks: a camera's observations are sorted by point, so those whose
  // points fall in each of kPointBands equal index bands form a contiguous
  // piece, cut into equal chunks of at most kChunk.  Blocks are laid out so
  // that block b takes a chunk of band b % kPointBands (-1 pads short bands).
  std::vector<int32_t> c_pt_h(N);
  if (N) TRY(hipMemcpyAsync(c_pt_h.data(), h->c_pt, sizeof(int32_t) * N, hipMemcpyDeviceToHost, s));
  TRY(hipStreamSynchronize(s));
  std::vector<int32_t> chunk_begin, chunk_cam, cam_chunk_ptr(nc + 1, 0);
  std::vector<std::vector<int32_t>> band_list(kPointBands);
  const int64_t np1 = std::max<int64_t>(np, 1);
  auto band_of = [&](int64_t k) { return (int)((int64_t)c_pt_h[k] * kPointBands / np1); };
  for (int64_t j = 0; j < nc; ++j) {
    int64_t a = cam_ptr[j];
    const int64_t b1 = cam_ptr[j + 1];
    while (a < b1) {
      const int band = band_of(a);
      int64_t e = a;
      while (e < b1 && band_of(e) == band) ++e;
      const int64_t len = e - a, nch = (len + kChunk - 1) / kChunk;
      for (int64_t c = 0; c < nch; ++c) {
        band_list[band].push_back((int32_t)chunk_cam.size());
        chunk_begin.push_back((int32_t)(a + (len * c) / nch));
        chunk_cam.push_back((int32_t)j);
      }
      a = e;
    }
    cam_chunk_ptr[j + 1] = (int32_t)chunk_cam.size();
  }
  chunk_begin.push_back((int32_t)N);
  size_t per_band = 0;
  for (auto& v : band_list) per_band = std::max(per_band, v.size());
  std::vector<int4> blk_chunk(per_band * kPointBands, make_int4(0, 0, 0, -1));
  for (int bnd = 0; bnd < kPointBands; ++bnd)
    for (size_t i = 0; i < band_list[bnd].size(); ++i) {
      const int32_t ch = band_list[bnd][i];
      blk_chunk[i * kPointBands + bnd] = make_int4(chunk_begin[ch], chunk_begin[ch + 1], chunk_cam[ch], ch);
    }
  h->n_chunk_blocks = (int)blk_chunk.size();
  h->n_chunks = (int)chunk_cam.size();

  Arena& P = h->arena2;
  P.add(h->wave_begin, (int64_t)std::max<size_t>(wave_begin.size(), 1));
  const int64_t n_ch1 = std::max(h->n_chunks, 1);
  P.add(h->blk_chunk, (int64_t)std::max<size_t>(blk_chunk.size(), 1));
  P.add(h->lin_part, n_ch1 * kLinCamVals);
  P.add(h->schur_part, n_ch1 * kSchurVals);
  P.add(h->pcg_part, n_ch1 * 9);
  P.add(h->cost_part, (int64_t)std::max(h->lds_blocks, 1));
  P.add(h->red_part, 8 * (int64_t)pcg_red_blocks(nc) + 2);
  P.add(h->pt_dot, (int64_t)std::max(h->lds_blocks, 1));
  P.add(h->cam_rows, h->cam_layout == kCamRows ? (int64_t)kCamLdsFill * kLdsBlock : 1);
  P.add(h->dl_vpart, 3 * (int64_t)dl_vec_blocks(nc, h->np));
  P.add(h->dl_opart, 3 * (int64_t)std::max(h->n_chunk_blocks, 1));
  P.add(h->dl_out, 6);
  P.add(h->dl_hc, 9 * nc);
  rc = P.commit();
  if (rc != BA_OK) return rc;
  TRY(hipMemsetAsync(P.base, 0, P.size, s));
  if (!wave_begin.empty())
    TRY(hipMemcpyAsync(h->wave_begin, wave_begin.data(), sizeof(int32_t) * wave_begin.size(),
                       hipMemcpyHostToDevice, s));
  if (!blk_chunk.empty())
    TRY(hipMemcpyAsync(h->blk_chunk, blk_chunk.data(), sizeof(int4) * blk_chunk.size(),
                       hipMemcpyHostToDevice, s));
  TRY(hipMemcpyAsync(h->cam_chunk_ptr, cam_chunk_ptr.data(), sizeof(int32_t) * (nc + 1),
                     hipMemcpyHostToDevice, s));
  TRY(hipStreamSynchronize(s));
#undef TRY
  return BA_OK;
}

}  // namespace

// ============================================================== C ABI ====

namespace {

// Structure of the dense solver, once per handle: the (point, camera) runs of
// the point order; for every lower 9x9 block (j2, j1) of S with j2 >= j1 the
// pairs of runs (camera j2, camera j1) that share a point, in point order
// (every diagonal block is listed, with no pairs when the camera sees
// nothing); the arena for the run blocks F, S with its rhs rows and the
// factor's diagonal tiles.
int plan_dense(ba_problem* h) {
  hipStream_t s = h->stream;
  const int64_t N = h->nobs, nc = h->nc;
  std::vector<int32_t> oc(N), op(N);
  if (N) {
    HIPC(hipMemcpyAsync(oc.data(), h->o_cam, sizeof(int32_t) * N, hipMemcpyDeviceToHost, s));
    HIPC(hipMemcpyAsync(op.data(), h->o_pt, sizeof(int32_t) * N, hipMemcpyDeviceToHost, s));
  }
  HIPC(hipStreamSynchronize(s));
  std::vector<int32_t> run;
  for (int64_t k = 0; k < N; ++k)
    if (k == 0 || oc[k] != oc[k - 1] || op[k] != op[k - 1]) run.push_back((int32_t)k);
  const int64_t nruns = (int64_t)run.size();
  run.push_back((int32_t)N);
  // runs of one point are consecutive and in camera order
  std::vector<int64_t> off((size_t)(nc * nc), 0);
  auto for_pairs = [&](auto&& fn) {
    for (int64_t g0 = 0; g0 < nruns;) {
      int64_t g1 = g0 + 1;
      while (g1 < nruns && op[run[g1]] == op[run[g0]]) ++g1;
      for (int64_t a = g0; a < g1; ++a)
        for (int64_t b = g0; b <= a; ++b) fn((int64_t)oc[run[a]] * nc + oc[run[b]], a, b);
      g0 = g1;
    }
  };
  for_pairs([&](int64_t key, int64_t, int64_t) { ++off[key]; });
  std::vector<int2> blk;
  std::vector<int32_t> blk_ptr;
  int64_t npairs = 0;
  for (int64_t j2 = 0; j2 < nc; ++j2)
    for (int64_t j1 = 0; j1 <= j2; ++j1) {
      const int64_t key = j2 * nc + j1, cnt = off[key];
      if (cnt == 0 && j1 != j2) continue;
      blk.push_back(make_int2((int)j2, (int)j1));
      blk_ptr.push_back((int32_t)npairs);
      off[key] = npairs;
      npairs += cnt;
    }
  blk_ptr.push_back((int32_t)npairs);
  if (npairs >= (int64_t)INT32_MAX) return fail(BA_ERR_ARG, "too many co-visible run pairs");
  std::vector<int2> pair((size_t)std::max<int64_t>(npairs, 1));
  for_pairs([&](int64_t key, int64_t a, int64_t b) { pair[off[key]++] = make_int2((int)a, (int)b); });
  const int kt = ds_tile();
  h->ds_ld = (int)((9 * nc + kt - 1) / kt * kt);
  h->ds_T = h->ds_ld / kt;
  h->ds_nruns = (int)nruns;
  h->ds_nblk = (int)blk.size();
  Arena& A = h->arena3;
  A.add(h->ds_run, nruns + 1);
  A.add(h->ds_blk, (int64_t)blk.size());
  A.add(h->ds_blk_ptr, (int64_t)blk_ptr.size());
  A.add(h->ds_pair, npairs);
  A.add(h->ds_F, 27 * nruns);
  A.add(h->ds_S, ((int64_t)h->ds_ld + kt) * h->ds_ld);
  A.add(h->ds_diag, (int64_t)h->ds_T * kt * kt);
  A.add(h->ds_diagT, (int64_t)h->ds_T * kt * kt);
  A.add(h->ds_dinv, (int64_t)h->ds_ld);
  A.add(h->ds_v, 2 * (int64_t)h->ds_ld);
  A.add(h->ds_cov, 81 * nc);
  CHECK_RC(A.commit());
  HIPC(hipMemcpyAsync(h->ds_run, run.data(), sizeof(int32_t) * run.size(), hipMemcpyHostToDevice, s));
  HIPC(hipMemcpyAsync(h->ds_blk, blk.data(), sizeof(int2) * blk.size(), hipMemcpyHostToDevice, s));
  HIPC(hipMemcpyAsync(h->ds_blk_ptr, blk_ptr.data(), sizeof(int32_t) * blk_ptr.size(),
                      hipMemcpyHostToDevice, s));
  if (npairs)
    HIPC(hipMemcpyAsync(h->ds_pair, pair.data(), sizeof(int2) * npairs, hipMemcpyHostToDevice, s));
  HIPC(ds_backsolve_limit(h->ds_ld));
  HIPC(hipStreamSynchronize(s));
  return BA_OK;
}

int check_options(const ba_options& o) {
  if (o.loss != BA_LOSS_SQUARED && o.loss != BA_LOSS_HUBER) return fail(BA_ERR_ARG, "bad loss");
  if (!(o.huber_delta > 0.0)) return fail(BA_ERR_ARG, "huber_delta must be > 0");
  if (!(o.lambda0 >= 0.0) || !(o.lambda_up >= 1.0) || !(o.lambda_down >= 1.0) ||
      !(o.lambda_min >= 0.0) || !(o.lambda_max >= o.lambda_min))
    return fail(BA_ERR_ARG, "bad damping schedule");
  if (!(o.diag_floor >= 0.0)) return fail(BA_ERR_ARG, "diag_floor must be >= 0");
  if (o.pcg_max_iters < 0 || !(o.pcg_rel_tol >= 0.0)) return fail(BA_ERR_ARG, "bad PCG options");
  if (o.mem != BA_MEM_HOST && o.mem != BA_MEM_DEVICE) return fail(BA_ERR_ARG, "bad mem");
  if (o.solver != BA_SOLVER_PCG && o.solver != BA_SOLVER_DENSE_SCHUR) return fail(BA_ERR_ARG, "bad solver");
  if (o.strategy != BA_STRATEGY_LM && o.strategy != BA_STRATEGY_DOGLEG) return fail(BA_ERR_ARG, "bad strategy");
  if (!(o.dl_radius0 > 0.0) || !std::isfinite(o.dl_radius0) || !(o.dl_gn_damping >= 0.0))
    return fail(BA_ERR_ARG, "bad dogleg options");
  return BA_OK;
}

void expand_sym(const double* packed, int n, int64_t count, double* full) {
  for (int64_t b = 0; b < count; ++b) {
    const double* p = packed + b * (n * (n + 1) / 2);
    double* f = full + b * n * n;
    for (int i = 0; i < n; ++i)
      for (int j = i; j < n; ++j) f[i * n + j] = f[j * n + i] = p[sym_idx(n, i, j)];
  }
}

int d2h(ba_problem* h, void* dst, const void* src, size_t bytes) {
  if (bytes) HIPC(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  return BA_OK;
}

const char* kKernelNames[BA_K_NUM] = {"lin_pt",   "lin_cam",  "damp_pt",     "schur_cam",
                                      "precond",  "pcg_init", "pcg_pt",      "pcg_cam",
                                      "pcg_q",    "pcg_xr",   "backsub",     "retract",
                                      "cost",     "ds_runs",  "ds_fill",     "ds_assemble",
                                      "ds_panel", "ds_update", "ds_backsolve", "cov_zero",
                                      "cov_blocks", "dl_obs",      "dl_step"};

// n LM steps queued without reading each one back: the accept/reject
// decision, the damping update and the copy of an accepted trial into the
// current parameters run on the device (k_cost_final, k_lm_commit), the
// linearisation is launched every step and runs only after an accepted one,
// and the host waits only for the PCG pacing.  The per-step records are read
// back after the last step.  Same decisions and arithmetic as lm_step.
int solve_queued(ba_problem* h, int n, ba_summary* s) {
  ba_summary sum{};
  sum.initial_cost = h->cost;
  if (n > h->lm_log_cap) {
    if (h->lm_log) HIPC(hipFree(h->lm_log));
    h->lm_log = nullptr;
    h->lm_log_cap = 0;
    HIPC(hipMalloc(reinterpret_cast<void**>(&h->lm_log), sizeof(LmLog) * (size_t)n));
    h->lm_log_cap = n;
  }
  *h->h_lm = LmDev{h->cost, h->lambda, h->linearized ? 0 : 1, 0, {0, 0}};
  HIPC(hipMemcpyAsync(h->lm, h->h_lm, sizeof(LmDev), hipMemcpyHostToDevice, h->stream));
  h->queued = 1;
  int rc = BA_OK;
  for (int k = 0; k < n && rc == BA_OK; ++k) {
    h->q_step = k;
    if (k > 0 || !h->linearized) rc = stage_linearize(h, true);
    if (rc == BA_OK) rc = stage_schur(h);
    if (rc == BA_OK) rc = stage_solve(h, true);
    if (rc == BA_OK) rc = stage_update(h);
  }
  h->queued = 0;
  if (rc != BA_OK) {
    h->lin_final_pending = 0;
    h->pcg_final_iters = -1;
    (void)hipStreamSynchronize(h->stream);
    return rc;
  }
  std::vector<LmLog> log((size_t)n);
  LmDev L{};
  HIPC(hipMemcpyAsync(log.data(), h->lm_log, sizeof(LmLog) * (size_t)n, hipMemcpyDeviceToHost,
                      h->stream));
  HIPC(hipMemcpyAsync(&L, h->lm, sizeof(LmDev), hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  int done = 0;
  for (; done < n && !log[done].not_spd; ++done) {
    sum.accepted += log[done].accepted;
    sum.pcg_iters_total += log[done].pcg_iters;
  }
  h->cost = L.cost;
  h->lambda = L.lambda;
  h->linearized = L.relin ? 0 : 1;
  h->iteration += done;
  h->last_pcg_iters = log[(size_t)n - 1].pcg_iters;
  if (h->prof_on) {
    std::vector<int> iters((size_t)n), lin((size_t)n);
    for (int k = 0; k < n; ++k) {
      iters[k] = log[k].pcg_iters;
      lin[k] = k == 0 ? 1 : log[k - 1].accepted;
    }
    CHECK_RC(prof_collect_steps(h, iters.data(), lin.data()));
  }
  if (done < n) return fail(BA_ERR_NOT_SPD, "a damped block is not positive definite");
  sum.iterations = n;
  sum.final_cost = h->cost;
  sum.lambda = h->lambda;
  if (s) *s = sum;
  return BA_OK;
}

}  // namespace

extern "C" {

int ba_options_default(ba_options* o) {
  if (!o) return BA_ERR_ARG;
  o->loss = BA_LOSS_SQUARED;
  o->huber_delta = 2.0;
  o->lambda0 = 1e-3;
  o->lambda_up = 10.0;
  o->lambda_down = 10.0;
  o->lambda_min = 1e-16;
  o->lambda_max = 1e16;
  o->diag_floor = 1e-6;
  o->pcg_max_iters = 50;
  o->pcg_rel_tol = 1e-6;
  o->mem = BA_MEM_HOST;
  o->stream = nullptr;
  o->solver = BA_SOLVER_PCG;
  o->strategy = BA_STRATEGY_LM;
  o->dl_radius0 = 1.0;
  o->dl_gn_damping = 1e-6;
  return BA_OK;
}

void ba_destroy(ba_problem* h) {
  if (!h) return;
  if (h->stream) (void)hipStreamSynchronize(h->stream);
  else (void)hipDeviceSynchronize();
  (void)hipFree(h->arena.base);
  (void)hipFree(h->arena2.base);
  (void)hipFree(h->arena3.base);
  if (h->h_out) (void)hipHostFree(h->h_out);
  if (h->h_done) (void)hipHostFree(h->h_done);
  if (h->h_lm) (void)hipHostFree(h->h_lm);
  if (h->lm_log) (void)hipFree(h->lm_log);
  for (hipEvent_t e : h->prof_pool) (void)hipEventDestroy(e);
  delete h;
}

int ba_create(const double* cams, int64_t n_cams, const double* points, int64_t n_pts,
              const int32_t* obs_cam_idx, const int32_t* obs_pt_idx, const double* obs_uv,
              int64_t n_obs, const ba_options* opts, ba_problem** out) {
  if (!out) return fail(BA_ERR_ARG, "out is NULL");
  *out = nullptr;
  if (!cams || !points || n_cams <= 0 || n_pts <= 0 || n_obs < 0)
    return fail(BA_ERR_ARG, "null parameters or non-positive sizes");
  if (n_obs > 0 && (!obs_cam_idx || !obs_pt_idx || !obs_uv))
    return fail(BA_ERR_ARG, "null observation arrays");
  if (n_obs > BA_MAX_OBS || n_cams > BA_MAX_CAMS || n_pts > BA_MAX_PTS)
    return fail(BA_ERR_ARG, "sizes beyond BA_MAX_OBS, BA_MAX_CAMS or BA_MAX_PTS");
  ba_problem* h = new ba_problem();
  if (opts) h->opt = *opts;
  else ba_options_default(&h->opt);
  int rc = check_options(h->opt);
  if (rc != BA_OK) {
    delete h;
    return rc;
  }
  h->stream = reinterpret_cast<hipStream_t>(h->opt.stream);
  h->nc = n_cams;
  h->np = n_pts;
  h->nobs = n_obs;
  if (h->opt.solver == BA_SOLVER_DENSE_SCHUR && n_cams > BA_DENSE_MAX_CAMS) {
    delete h;
    return fail(BA_ERR_ARG, "the dense solver takes at most BA_DENSE_MAX_CAMS cameras");
  }
  if (hipHostMalloc(reinterpret_cast<void**>(&h->h_out), sizeof(StepOut), hipHostMallocDefault) !=
      hipSuccess) {
    h->h_out = nullptr;
    ba_destroy(h);
    return fail(BA_ERR_ALLOC, "hipHostMalloc");
  }
  bool ok = hipHostMalloc(reinterpret_cast<void**>(&h->h_done), 2 * sizeof(long long),
                          hipHostMallocMapped) == hipSuccess &&
            hipHostGetDevicePointer(reinterpret_cast<void**>(&h->h_done_dev), h->h_done, 0) ==
                hipSuccess;
  if (!ok) {
    ba_destroy(h);
    return fail(BA_ERR_ALLOC, "pinned flag");
  }
  h->h_done[0] = 0;
  h->h_done[1] = 0;
  if (hipHostMalloc(reinterpret_cast<void**>(&h->h_lm), sizeof(LmDev), hipHostMallocDefault) !=
      hipSuccess) {
    h->h_lm = nullptr;
    ba_destroy(h);
    return fail(BA_ERR_ALLOC, "hipHostMalloc");
  }
  rc = build(h, cams, points, obs_cam_idx, obs_pt_idx, obs_uv);
  if (rc == BA_OK && h->opt.solver == BA_SOLVER_DENSE_SCHUR) rc = plan_dense(h);
  if (rc != BA_OK) {
    ba_destroy(h);
    return rc;
  }
  h->cur = 0;
  h->lambda = h->opt.lambda0;
  h->radius = h->opt.dl_radius0;
  h->linearized = 0;
  h->iteration = 0;
  launch_cam_prep(h->cams[0], h->tab[0], h->camq[0], h->nc, h->stream);
  double c = 0.0;
  rc = current_cost(h, &c);
  if (rc == BA_OK && !std::isfinite(c)) rc = fail(BA_ERR_NONFINITE, "initial cost is not finite");
  if (rc != BA_OK) {
    ba_destroy(h);
    return rc;
  }
  h->cost = c;
  *out = h;
  return BA_OK;
}

int ba_lm_step(ba_problem* h, ba_step_info* info) {
  if (!h) return fail(BA_ERR_ARG, "null handle");
  return lm_step(h, info);
}

int ba_solve(ba_problem* h, int n_iters, ba_summary* s) {
  if (!h || n_iters < 0) return fail(BA_ERR_ARG, "bad arguments");
  if (n_iters > 0 && h->opt.strategy == BA_STRATEGY_LM)
    return solve_queued(h, n_iters, s);
  ba_summary sum{};
  sum.initial_cost = h->cost;
  for (int it = 0; it < n_iters; ++it) {
    ba_step_info inf;
    int rc = lm_step(h, &inf);
    if (rc != BA_OK) return rc;
    sum.accepted += inf.accepted;
    sum.pcg_iters_total += inf.pcg_iters;
  }
  sum.iterations = n_iters;
  sum.final_cost = h->cost;
  sum.lambda = h->lambda;
  if (s) *s = sum;
  return BA_OK;
}

int ba_backward(ba_problem* h, const double* grad_cams, const double* grad_points, double* grad_uv,
                int* pcg_iters) {
  if (!h || !grad_cams || !grad_points || (h->nobs > 0 && !grad_uv))
    return fail(BA_ERR_ARG, "bad arguments");
  const int64_t nc = h->nc, np = h->np, N = h->nobs;
  const bool dev = h->opt.mem == BA_MEM_DEVICE;
  const hipMemcpyKind kin = dev ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
  CHECK_RC(stage_linearize(h));
  // g = -G: the damped step system then solves H~ x = G
  HIPC(hipMemcpyAsync(h->gc, grad_cams, sizeof(double) * 9 * nc, kin, h->stream));
  HIPC(hipMemcpyAsync(h->gp, grad_points, sizeof(double) * 3 * np, kin, h->stream));
  launch_negate(h->gc, 9 * nc, h->stream);
  launch_negate(h->gp, 3 * np, h->stream);
  h->linearized = 0;   // g no longer holds the gradient of the cost
  h->dl_valid = 0;     // nor x and dp the dogleg's Gauss-Newton step
  CHECK_RC(stage_schur(h));
  CHECK_RC(stage_solve(h));
  Dev d = make_dev(h);
  TIMED(BA_K_BACKSUB, -1, launch_backsub(d, h->stream));
  launch_vjp_obs(d, h->perm_cam, dev ? grad_uv : h->vjp, h->stream);
  HIPC(hipGetLastError());
  if (!dev && N) HIPC(hipMemcpyAsync(grad_uv, h->vjp, sizeof(double) * 2 * N, hipMemcpyDeviceToHost,
                                     h->stream));
  PcgState st;
  HIPC(hipMemcpyAsync(&st, h->pcg, sizeof(st), hipMemcpyDeviceToHost, h->stream));
  int flags[2] = {0, 0};
  HIPC(hipMemcpyAsync(flags, h->flags, sizeof(flags), hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  if (h->prof_on) CHECK_RC(prof_collect(h, st.iters));
  if (flags[1]) return fail(BA_ERR_NOT_SPD, "a damped block is not positive definite");
  if (pcg_iters) *pcg_iters = st.iters;
  return BA_OK;
}

int ba_covariance(ba_problem* h, double* cov_out) {
  if (!h || !cov_out) return fail(BA_ERR_ARG, "bad arguments");
  if (h->opt.solver != BA_SOLVER_DENSE_SCHUR)
    return fail(BA_ERR_ARG, "the covariance needs the dense solver (opts.solver = BA_SOLVER_DENSE_SCHUR)");
  const int64_t nc = h->nc;
  CHECK_RC(stage_linearize(h));
  h->linearized = 1;
  h->dl_valid = 0;
  CHECK_RC(stage_schur(h));
  CHECK_RC(stage_dense_factor(h, 1));
  Dev d = make_dev(h);
  hipStream_t s = h->stream;
  const bool dev = h->opt.mem == BA_MEM_DEVICE;
  TIMED(BA_K_COV_BLOCKS, -1, launch_cov_blocks(d, dev ? cov_out : h->ds_cov, nc, s));
  HIPC(hipGetLastError());
  if (!dev) HIPC(hipMemcpyAsync(cov_out, h->ds_cov, sizeof(double) * 81 * nc, hipMemcpyDeviceToHost, s));
  int flags[2] = {0, 0};
  HIPC(hipMemcpyAsync(flags, h->flags, sizeof(flags), hipMemcpyDeviceToHost, s));
  HIPC(hipStreamSynchronize(s));
  if (h->prof_on) CHECK_RC(prof_collect(h, 0));
  if (flags[1]) return fail(BA_ERR_NOT_SPD, "the damped system is not positive definite");
  return BA_OK;
}

int ba_cost(ba_problem* h, double* cost_out) {
  if (!h || !cost_out) return fail(BA_ERR_ARG, "bad arguments");
  return current_cost(h, cost_out);
}

int ba_get_params(ba_problem* h, double* cams_out, double* points_out) {
  if (!h) return fail(BA_ERR_ARG, "null handle");
  if (cams_out) HIPC(hipMemcpyAsync(cams_out, h->cams[h->cur], sizeof(double) * 9 * h->nc,
                                    hipMemcpyDeviceToHost, h->stream));
  if (points_out) HIPC(hipMemcpyAsync(points_out, h->pts[h->cur], sizeof(double) * 3 * h->np,
                                      hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  return BA_OK;
}

// The new parameters are staged in the trial buffers (free between steps) and
// checked there; only when they are finite and give a finite cost do they
// become the current ones, so a rejected call leaves the handle as it was.
int ba_set_params(ba_problem* h, const double* cams, const double* points) {
  if (!h) return fail(BA_ERR_ARG, "null handle");
  const hipMemcpyKind kind =
      h->opt.mem == BA_MEM_DEVICE ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice;
  const int c = h->cur, t = 1 - h->cur;
  hipStream_t s = h->stream;
  if (cams) HIPC(hipMemcpyAsync(h->cams[t], cams, sizeof(double) * 9 * h->nc, kind, s));
  else HIPC(hipMemcpyAsync(h->cams[t], h->cams[c], sizeof(double) * 9 * h->nc, hipMemcpyDeviceToDevice, s));
  if (points) HIPC(hipMemcpyAsync(h->pts[t], points, sizeof(double) * 3 * h->np, kind, s));
  else HIPC(hipMemcpyAsync(h->pts[t], h->pts[c], sizeof(double) * 3 * h->np, hipMemcpyDeviceToDevice, s));
  HIPC(hipMemsetAsync(h->flags, 0, 2 * sizeof(int), s));
  launch_validate(nullptr, nullptr, nullptr, 0, h->cams[t], h->nc, h->pts[t], h->np, h->flags, s);
  int flags[2] = {0, 0};
  HIPC(hipMemcpyAsync(flags, h->flags, sizeof(flags), hipMemcpyDeviceToHost, s));
  HIPC(hipStreamSynchronize(s));
  if (flags[1]) return fail(BA_ERR_NONFINITE, "non-finite parameters");
  launch_cam_prep(h->cams[t], h->tab[t], h->camq[t], h->nc, s);
  Dev d = make_dev(h);
  launch_cost(d, d.pts_trial, d.tab_trial, d.camq_trial, s);
  HIPC(hipGetLastError());
  CHECK_RC(read_out(h));
  const double cost = h->h_out->trial_cost;
  if (!std::isfinite(cost)) return fail(BA_ERR_NONFINITE, "cost is not finite");
  h->cur = t;
  h->cost = cost;
  h->linearized = 0;
  h->dl_valid = 0;
  return BA_OK;
}

int ba_get_state(const ba_problem* h, ba_state* st) {
  if (!h || !st) return fail(BA_ERR_ARG, "bad arguments");
  st->lambda = h->lambda;
  st->cost = h->cost;
  st->iteration = h->iteration;
  st->radius = h->radius;
  return BA_OK;
}

int ba_set_state(ba_problem* h, const ba_state* st) {
  if (!h || !st || !(st->lambda >= 0.0) || !(st->radius >= 0.0) || !std::isfinite(st->radius))
    return fail(BA_ERR_ARG, "bad arguments");
  h->lambda = st->lambda;    // the cost always follows the parameters; st->cost is ignored
  if (st->radius > 0.0) h->radius = st->radius;
  h->iteration = st->iteration;
  return BA_OK;
}

int ba_get_sizes(const ba_problem* h, int64_t* n_cams, int64_t* n_pts, int64_t* n_obs) {
  if (!h) return fail(BA_ERR_ARG, "null handle");
  if (n_cams) *n_cams = h->nc;
  if (n_pts) *n_pts = h->np;
  if (n_obs) *n_obs = h->nobs;
  return BA_OK;
}

int ba_debug_run(ba_problem* h, int upto) {
  if (!h || upto < BA_STAGE_LINEARIZE || upto > BA_STAGE_UPDATE)
    return fail(BA_ERR_ARG, "bad arguments");
  CHECK_RC(stage_linearize(h));
  h->linearized = 1;
  if (upto >= BA_STAGE_SCHUR) CHECK_RC(stage_schur(h));
  if (upto >= BA_STAGE_PCG) CHECK_RC(stage_solve(h));
  if (upto >= BA_STAGE_UPDATE) CHECK_RC(stage_update(h));
  CHECK_RC(read_out(h));
  if (h->prof_on) {
    // the step record carries the PCG count only after the update stage
    int iters = h->h_out->pcg_iters;
    if (upto == BA_STAGE_PCG) {
      PcgState st;
      CHECK_RC(d2h(h, &st, h->pcg, sizeof(st)));
      iters = st.iters;
    }
    CHECK_RC(prof_collect(h, iters));
  }
  return BA_OK;
}

int64_t ba_debug_size(const ba_problem* h, int which) {
  if (!h) return BA_ERR_ARG;
  const int64_t nc = h->nc, np = h->np, N = h->nobs, i4 = 4, d8 = 8;
  switch (which) {
    case BA_DBG_PERM_PT: case BA_DBG_PERM_CAM: return N * i4;
    case BA_DBG_PT_PTR: return (np + 1) * i4;
    case BA_DBG_CAM_PTR: return (nc + 1) * i4;
    case BA_DBG_R: return 2 * N * d8;
    case BA_DBG_JC: return 18 * N * d8;
    case BA_DBG_JP: return 6 * N * d8;
    case BA_DBG_W: return N * d8;
    case BA_DBG_B: case BA_DBG_BD: case BA_DBG_M: return 81 * nc * d8;
    case BA_DBG_GC: case BA_DBG_RHS: case BA_DBG_DC: case BA_DBG_CAMS_TRIAL: return 9 * nc * d8;
    case BA_DBG_C: case BA_DBG_CINV: return 9 * np * d8;
    case BA_DBG_GP: case BA_DBG_V: case BA_DBG_DP: case BA_DBG_PTS_TRIAL: return 3 * np * d8;
    case BA_DBG_PCG: return 2 * d8;
    case BA_DBG_TRIAL_COST: return d8;
    case BA_DBG_S: return h->opt.solver == BA_SOLVER_DENSE_SCHUR ? 81 * nc * nc * d8 : BA_ERR_ARG;
    default: return BA_ERR_ARG;
  }
}

int ba_debug_get(ba_problem* h, int which, void* host_out, int64_t bytes) {
  if (!h || !host_out) return fail(BA_ERR_ARG, "bad arguments");
  const int64_t need = ba_debug_size(h, which);
  if (need < 0 || bytes != need) return fail(BA_ERR_ARG, "bad array id or byte count");
  const int64_t nc = h->nc, np = h->np, N = h->nobs;
  const int t = 1 - h->cur;
  switch (which) {
    case BA_DBG_PERM_PT: return d2h(h, host_out, h->perm_pt, bytes);
    case BA_DBG_PERM_CAM: return d2h(h, host_out, h->perm_cam, bytes);
    case BA_DBG_PT_PTR: return d2h(h, host_out, h->pt_ptr, bytes);
    case BA_DBG_CAM_PTR: return d2h(h, host_out, h->cam_ptr, bytes);
    case BA_DBG_R: case BA_DBG_JC: case BA_DBG_JP: case BA_DBG_W: {
      if (N == 0) return BA_OK;
      double* buf = nullptr;
      HIPC(hipMalloc(&buf, sizeof(double) * 27 * N));
      Dev d = make_dev(h);
      launch_debug_obs(d, h->perm_pt, buf, buf + 2 * N, buf + 20 * N, buf + 26 * N, h->stream);
      const size_t off = which == BA_DBG_R ? 0 : which == BA_DBG_JC ? 2 * N : which == BA_DBG_JP ? 20 * N : 26 * N;
      int rc = d2h(h, host_out, buf + off, bytes);
      (void)hipFree(buf);
      return rc;
    }
    case BA_DBG_GC: return d2h(h, host_out, h->gc, bytes);
    case BA_DBG_GP: return d2h(h, host_out, h->gp, bytes);
    case BA_DBG_V:   // v = C~^-1 g_p sits in elements 3..5 of each point record until the PCG
      if (bytes) HIPC(hipMemcpy2DAsync(host_out, 3 * sizeof(double), h->prec + 3, 8 * sizeof(double),
                                       3 * sizeof(double), (size_t)h->np, hipMemcpyDeviceToHost,
                                       h->stream));
      HIPC(hipStreamSynchronize(h->stream));
      return BA_OK;
    case BA_DBG_RHS: return d2h(h, host_out, h->rhs, bytes);
    case BA_DBG_DC: return d2h(h, host_out, h->x, bytes);
    case BA_DBG_DP: return d2h(h, host_out, h->dp, bytes);
    case BA_DBG_CAMS_TRIAL: return d2h(h, host_out, h->cams[t], bytes);
    case BA_DBG_PTS_TRIAL: return d2h(h, host_out, h->pts[t], bytes);
    case BA_DBG_B: case BA_DBG_BD: case BA_DBG_M: {
      std::vector<double> packed(45 * nc);
      const double* src = which == BA_DBG_B ? h->B : which == BA_DBG_BD ? h->Bd : h->Mfull;
      CHECK_RC(d2h(h, packed.data(), src, sizeof(double) * packed.size()));
      expand_sym(packed.data(), 9, nc, static_cast<double*>(host_out));
      return BA_OK;
    }
    case BA_DBG_C: case BA_DBG_CINV: {
      std::vector<double> packed(6 * np);
      CHECK_RC(d2h(h, packed.data(), which == BA_DBG_C ? h->C : h->Cinv, sizeof(double) * packed.size()));
      expand_sym(packed.data(), 3, np, static_cast<double*>(host_out));
      return BA_OK;
    }
    case BA_DBG_PCG: {
      PcgState st;
      CHECK_RC(d2h(h, &st, h->pcg, sizeof(st)));
      double* o = static_cast<double*>(host_out);
      o[0] = st.iters;
      o[1] = st.rhs_norm > 0.0 ? st.res_norm / st.rhs_norm : 0.0;
      return BA_OK;
    }
    case BA_DBG_S: {
      // assembled again from the current state (the solve factors it in place)
      Dev d = make_dev(h);
      launch_ds_runs(d, h->stream);
      launch_ds_fill(d, h->stream);
      launch_ds_assemble(d, h->stream);
      HIPC(hipGetLastError());
      const int64_t n = 9 * nc, ld = h->ds_ld;
      double* o = static_cast<double*>(host_out);
      HIPC(hipMemcpy2DAsync(o, n * sizeof(double), h->ds_S, ld * sizeof(double), n * sizeof(double),
                            (size_t)n, hipMemcpyDeviceToHost, h->stream));
      HIPC(hipStreamSynchronize(h->stream));
      for (int64_t i = 0; i < n; ++i)   // only the lower triangle is assembled
        for (int64_t j = i + 1; j < n; ++j) o[i * n + j] = o[j * n + i];
      return BA_OK;
    }
    case BA_DBG_TRIAL_COST: {
      StepOut so;
      CHECK_RC(d2h(h, &so, h->out, sizeof(so)));
      *static_cast<double*>(host_out) = so.trial_cost;
      return BA_OK;
    }
    default: return fail(BA_ERR_ARG, "bad array id");
  }
}

int ba_profile_enable(ba_problem* h, int kernel_mask, int every) {
  if (!h) return fail(BA_ERR_ARG, "null handle");
  if (every < 1) return fail(BA_ERR_ARG, "every must be >= 1");
  h->prof_on = kernel_mask;
  h->prof_every = every;
  for (int k = 0; k < BA_K_NUM; ++k) h->prof_seen[k] = 0;
  h->prof_recs.clear();
  h->prof_used = 0;
  return BA_OK;
}

int ba_profile_reset(ba_problem* h) {
  if (!h) return fail(BA_ERR_ARG, "null handle");
  for (int k = 0; k < BA_K_NUM; ++k) {
    h->prof_count[k] = 0;
    h->prof_ms[k] = 0.0;
  }
  return BA_OK;
}

int ba_profile_get(ba_problem* h, int kernel, int64_t* launches, double* total_ms) {
  if (!h || kernel < 0 || kernel >= BA_K_NUM) return fail(BA_ERR_ARG, "bad arguments");
  if (launches) *launches = h->prof_count[kernel];
  if (total_ms) *total_ms = h->prof_ms[kernel];
  return BA_OK;
}

const char* ba_kernel_name(int kernel) {
  return (kernel >= 0 && kernel < BA_K_NUM) ? kKernelNames[kernel] : "unknown";
}

const char* ba_status_string(int code) {
  static thread_local std::string msg;
  const char* base = "unknown status";
  switch (code) {
    case BA_OK: base = "ok"; break;
    case BA_ERR_ARG: base = "invalid argument"; break;
    case BA_ERR_NONFINITE: base = "non-finite value"; break;
    case BA_ERR_NOT_SPD: base = "matrix not positive definite"; break;
    case BA_ERR_DEVICE: base = "device error"; break;
    case BA_ERR_ALLOC: base = "allocation failed"; break;
  }
  msg = base;
  if (code != BA_OK && !g_err.empty()) msg += ": " + g_err;
  return msg.c_str();
}

}  // extern "C"
