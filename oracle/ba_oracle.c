/* CPU oracle for one Levenberg-Marquardt iteration of bundle adjustment (fp64).
 *
 * TEST INFRASTRUCTURE ONLY: plain loops, no blocking, no fusion.  Only the test
 * suite, the smoke check and the CPU-baseline leg of the benchmark may load it.
 * It shares no code with the GPU library.
 *
 * Threads: built with -fopenmp, loops whose iterations own their outputs (one
 * observation, camera or point each) are shared out, and every sum over
 * observations is an "owner scan": each thread owns a contiguous range of
 * cameras (or points), walks all observations in index order and adds those
 * of its own, so every accumulator receives its terms in observation order
 * from one thread, as in the plain loop.  The cost is a serial sum of
 * per-observation terms.  Both builds therefore give the same bits (pinned by
 * a test).  Without -fopenmp the pragmas are ignored and a scan is the plain
 * loop over all observations.
 *
 * Pages cited (by title and section):
 *  [BAE]      "Bundle Adjustment in the Eager Mode" (summary article): one residual
 *             per observation depending on one camera and one point; LM with sparse
 *             matmul, diagonal damping, Cholesky for small problems, PCG for large.
 *  [NSLAM]    NeRF-SLAM reproduction notes, sec. 2.2 (project with depth clamped
 *             at 1e-6), sec. 3.1 (H = J^T W J, b = -J^T W r, block structure
 *             [B E; E^T C]), sec. 3.2 (Schur complement, eqs. (1) and (2), dense
 *             reference step with explicit C^-1 and a Cholesky of S).
 *  [F2SLAM]   F^2SLAM article, sec. 5.3 (Huber kernel).
 *  [THESEUS]  Theseus note, "Method and architecture" (cost 1/2 sum |w c|^2,
 *             normal equations, retraction, LM with adaptive damping, Lie groups
 *             with analytic tangent derivatives).
 *
 * Readings where the pages are silent or garbled are stated at each function.
 */
#include "ba_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

struct orc_problem {
  int64_t nc, np, nobs;
  orc_opts opt;
  double *cams, *pts, *uv;
  int32_t *cam_idx, *pt_idx;
  int32_t *perm_pt, *perm_cam, *pt_ptr, *cam_ptr;
  double* terms;   /* per-observation cost terms of orc_cost_at */
  double *r, *Jc, *Jp, *w, *rho;
  double *B, *gc, *C, *gp;
  double *Bd, *Cinv, *v, *rhs, *M, *Mchol;
  double *dc, *dp;
  double *cams_trial, *pts_trial;
  double lambda, cost;
  int linearized;
  /* dogleg: radius, and at the current linearisation (dl_valid) the
   * Gauss-Newton step (in dc, dp) and the scalars of the step's model */
  double radius;
  int dl_valid, dl_iters;
  double dl_rel, dl_gg, dl_nn, dl_gn, dl_JgJg, dl_JgJn, dl_JnJn;
};

/* ------------------------------------------------------------- threads -- */

/* [lo, hi): the calling thread's share of n owned items (all of them outside
 * a parallel region or without OpenMP). */
static void my_range(int64_t n, int64_t* lo, int64_t* hi) {
#ifdef _OPENMP
  const int64_t t = omp_get_thread_num(), T = omp_get_num_threads();
#else
  const int64_t t = 0, T = 1;
#endif
  *lo = n * t / T;
  *hi = n * (t + 1) / T;
}

/* ---------------------------------------------------------------- SO(3) -- */

/* Rotation matrix of an axis-angle vector by the Rodrigues formula
 * R = I + sin(a)/a [w]x + (1 - cos(a))/a^2 [w]x^2, a = |w|; for a < 1e-8 the
 * second-order series I + [w]x + 1/2 [w]x^2.  [THESEUS] closed-form exp map. */
void orc_so3_exp(const double* w, double* R) {
  double a2 = w[0] * w[0] + w[1] * w[1] + w[2] * w[2];
  double a = sqrt(a2);
  double A, Bc;
  if (a < 1e-8) {
    A = 1.0;
    Bc = 0.5;
  } else {
    A = sin(a) / a;
    Bc = (1.0 - cos(a)) / a2;
  }
  double K[9] = {0.0, -w[2], w[1], w[2], 0.0, -w[0], -w[1], w[0], 0.0};
  double K2[9];
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double s = 0.0;
      for (int l = 0; l < 3; l++) s += K[3 * i + l] * K[3 * l + j];
      K2[3 * i + j] = s;
    }
  for (int i = 0; i < 9; i++) R[i] = A * K[i] + Bc * K2[i];
  R[0] += 1.0;
  R[4] += 1.0;
  R[8] += 1.0;
}

/* Unit quaternion (qw, qx, qy, qz) of an axis-angle vector. */
static void quat_from_aa(const double* w, double* q) {
  double a = sqrt(w[0] * w[0] + w[1] * w[1] + w[2] * w[2]);
  double c, s;
  if (a < 1e-8) {
    c = 1.0;
    s = 0.5;
  } else {
    c = cos(0.5 * a);
    s = sin(0.5 * a) / a;
  }
  q[0] = c;
  q[1] = s * w[0];
  q[2] = s * w[1];
  q[3] = s * w[2];
}

/* Hamilton product a (x) b. */
static void quat_mul(const double* a, const double* b, double* o) {
  o[0] = a[0] * b[0] - a[1] * b[1] - a[2] * b[2] - a[3] * b[3];
  o[1] = a[0] * b[1] + a[1] * b[0] + a[2] * b[3] - a[3] * b[2];
  o[2] = a[0] * b[2] - a[1] * b[3] + a[2] * b[0] + a[3] * b[1];
  o[3] = a[0] * b[3] + a[1] * b[2] - a[2] * b[1] + a[3] * b[0];
}

/* Axis-angle of a unit quaternion, taking the hemisphere qw >= 0 so that the
 * returned angle lies in [0, pi]; 2 v / qw for |v| < 1e-12. */
static void aa_from_quat(const double* qin, double* w) {
  double q[4] = {qin[0], qin[1], qin[2], qin[3]};
  if (q[0] < 0.0)
    for (int i = 0; i < 4; i++) q[i] = -q[i];
  double vn = sqrt(q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
  double k;
  if (vn < 1e-12)
    k = 2.0 / q[0];
  else
    k = 2.0 * atan2(vn, q[0]) / vn;
  w[0] = k * q[1];
  w[1] = k * q[2];
  w[2] = k * q[3];
}

/* ------------------------------------------------------ one observation -- */

/* Residual, Jacobians and robust weight of one observation.
 *
 * Camera model (9 parameters, principal point 0): P = R X + t, z = max(P_z, 1e-6)
 * ([NSLAM] sec. 2.2 clamps the depth at 1e-6 before dividing), p = P_xy / z,
 * n = |p|^2, s = 1 + k1 n + k2 n^2, u = f s p, r = u - uv.
 *
 * Jacobians (reading of [THESEUS] "analytic tangent derivatives" and retraction):
 * rotation in the left tangent of SO(3), R <- Exp(dphi) R, so dP/ddphi = -[R X]x;
 * translation, intrinsics and the point additive.  With
 * D = du/dp = f (s I + 2 (k1 + 2 k2 n) p p^T) and Q = dp/dP (zero third column
 * when the clamp is active), A = D Q:
 *   Jc = [A (-[R X]x) | A | s p | f n p | f n^2 p],  Jp = A R.
 *
 * Robust kernel ([F2SLAM] sec. 5.3, whose comparison operator was lost in the
 * page text; read as <= for the quadratic branch) applied to the 2-D norm
 * e = |r| of each observation: rho = e^2 / 2 for e <= delta, else
 * delta (e - delta / 2).  The weight w = rho'(e) / e (1, or delta / e) makes
 * sum w J^T r the exact gradient and sum w J^T J the Gauss-Newton matrix of
 * [NSLAM] sec. 3.1.  Squared loss: rho = e^2 / 2, w = 1. */
int orc_project_one(const double* cam, const double* X, const double* uv, int loss, double delta,
                    double* r, double* Jc, double* Jp, double* w_out, double* rho_out) {
  double R[9];
  orc_so3_exp(cam, R);
  const double* t = cam + 3;
  double f = cam[6], k1 = cam[7], k2 = cam[8];
  double q[3], P[3];
  for (int i = 0; i < 3; i++) {
    q[i] = R[3 * i + 0] * X[0] + R[3 * i + 1] * X[1] + R[3 * i + 2] * X[2];
    P[i] = q[i] + t[i];
  }
  int clamped = P[2] < 1e-6;
  double z = clamped ? 1e-6 : P[2];
  double p[2] = {P[0] / z, P[1] / z};
  double n = p[0] * p[0] + p[1] * p[1];
  double s = 1.0 + k1 * n + k2 * n * n;
  double u[2] = {f * s * p[0], f * s * p[1]};
  r[0] = u[0] - uv[0];
  r[1] = u[1] - uv[1];

  double c = 2.0 * (k1 + 2.0 * k2 * n);
  double D[4] = {f * (s + c * p[0] * p[0]), f * c * p[0] * p[1], f * c * p[1] * p[0],
                 f * (s + c * p[1] * p[1])};
  double Q[6] = {1.0 / z, 0.0, clamped ? 0.0 : -P[0] / (z * z),
                 0.0, 1.0 / z, clamped ? 0.0 : -P[1] / (z * z)};
  double A[6];
  for (int i = 0; i < 2; i++)
    for (int j = 0; j < 3; j++) A[3 * i + j] = D[2 * i + 0] * Q[0 + j] + D[2 * i + 1] * Q[3 + j];

  double mqx[9] = {0.0, q[2], -q[1], -q[2], 0.0, q[0], q[1], -q[0], 0.0}; /* -[q]x */
  for (int i = 0; i < 2; i++) {
    for (int j = 0; j < 3; j++) {
      double s1 = 0.0, s2 = 0.0;
      for (int l = 0; l < 3; l++) {
        s1 += A[3 * i + l] * mqx[3 * l + j];
        s2 += A[3 * i + l] * R[3 * l + j];
      }
      Jc[9 * i + j] = s1;
      Jc[9 * i + 3 + j] = A[3 * i + j];
      Jp[3 * i + j] = s2;
    }
    Jc[9 * i + 6] = s * p[i];
    Jc[9 * i + 7] = f * n * p[i];
    Jc[9 * i + 8] = f * n * n * p[i];
  }

  double e = sqrt(r[0] * r[0] + r[1] * r[1]);
  if (loss == 1 && e > delta) {
    *rho_out = delta * (e - 0.5 * delta);
    *w_out = delta / e;
  } else {
    *rho_out = 0.5 * e * e;
    *w_out = 1.0;
  }
  return clamped;
}

/* Cost of one observation only (same model as above, no derivatives). */
static double obs_cost(const double* cam, const double* X, const double* uv, int loss,
                       double delta) {
  double r[2], Jc[18], Jp[6], w, rho;
  orc_project_one(cam, X, uv, loss, delta, r, Jc, Jp, &w, &rho);
  return rho;
}

/* Camera retraction: rotation by left multiplication, q' = q(dphi) (x) q(w),
 * everything else additive ([THESEUS] retraction onto the manifold; the step
 * solves H delta = -J^T W r as in [NSLAM] sec. 3.1, so the update adds delta). */
int orc_retract_camera(const double* cam, const double* d, double* out) {
  double qa[4], qb[4], qc[4];
  quat_from_aa(d, qa);
  quat_from_aa(cam, qb);
  quat_mul(qa, qb, qc);
  aa_from_quat(qc, out);
  for (int i = 3; i < 9; i++) out[i] = cam[i] + d[i];
  return ORC_OK;
}

/* -------------------------------------------------- small dense algebra -- */

/* In-place lower Cholesky of an n x n row-major SPD matrix; -1 if not SPD. */
static int chol(double* A, int n) {
  for (int j = 0; j < n; j++) {
    double d = A[n * j + j];
    for (int l = 0; l < j; l++) d -= A[n * j + l] * A[n * j + l];
    if (!(d > 0.0) || !isfinite(d)) return -1;
    d = sqrt(d);
    A[n * j + j] = d;
    for (int i = j + 1; i < n; i++) {
      double s = A[n * i + j];
      for (int l = 0; l < j; l++) s -= A[n * i + l] * A[n * j + l];
      A[n * i + j] = s / d;
    }
    for (int i = 0; i < j; i++) A[n * i + j] = 0.0;
  }
  return 0;
}

/* Solve L L^T x = b with the factor from chol(). */
static void chol_solve(const double* L, int n, const double* b, double* x) {
  for (int i = 0; i < n; i++) {
    double s = b[i];
    for (int l = 0; l < i; l++) s -= L[n * i + l] * x[l];
    x[i] = s / L[n * i + i];
  }
  for (int i = n - 1; i >= 0; i--) {
    double s = x[i];
    for (int l = i + 1; l < n; l++) s -= L[n * l + i] * x[l];
    x[i] = s / L[n * i + i];
  }
}

static double dot(const double* a, const double* b, int64_t n) {
  double s = 0.0;
  for (int64_t i = 0; i < n; i++) s += a[i] * b[i];
  return s;
}

/* ----------------------------------------------------------- structure -- */

static const int32_t* g_key1;
static const int32_t* g_key2;
static int cmp_keys(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  if (g_key1[a] != g_key1[b]) return g_key1[a] < g_key1[b] ? -1 : 1;
  if (g_key2[a] != g_key2[b]) return g_key2[a] < g_key2[b] ? -1 : 1;
  return a < b ? -1 : (a > b);
}

/* Observation orderings and CSR offsets.  Index ops fix where the blocks are
 * non-zero ([BAE], sparsity-aware AutoDiff: index ops poses[cidx], points[pidx]);
 * the structure is fixed across iterations, which the pages cache.  Reading: the
 * keys (pt, cam, k) and (cam, pt, k) define a unique order. */
static void build_structure(orc_problem* h) {
  int64_t N = h->nobs;
  for (int64_t k = 0; k < N; k++) h->perm_pt[k] = h->perm_cam[k] = (int32_t)k;
  g_key1 = h->pt_idx;
  g_key2 = h->cam_idx;
  qsort(h->perm_pt, (size_t)N, sizeof(int32_t), cmp_keys);
  g_key1 = h->cam_idx;
  g_key2 = h->pt_idx;
  qsort(h->perm_cam, (size_t)N, sizeof(int32_t), cmp_keys);
  memset(h->pt_ptr, 0, sizeof(int32_t) * (h->np + 1));
  memset(h->cam_ptr, 0, sizeof(int32_t) * (h->nc + 1));
  for (int64_t k = 0; k < N; k++) {
    h->pt_ptr[h->pt_idx[k] + 1]++;
    h->cam_ptr[h->cam_idx[k] + 1]++;
  }
  for (int64_t i = 0; i < h->np; i++) h->pt_ptr[i + 1] += h->pt_ptr[i];
  for (int64_t j = 0; j < h->nc; j++) h->cam_ptr[j + 1] += h->cam_ptr[j];
}

/* ------------------------------------------------------------ lifecycle -- */

int orc_opts_default(orc_opts* o) {
  if (!o) return ORC_ERR_ARG;
  o->loss = 0;
  o->huber_delta = 2.0;
  o->lambda0 = 1e-3;
  o->lambda_up = 10.0;
  o->lambda_down = 10.0;
  o->lambda_min = 1e-16;
  o->lambda_max = 1e16;
  o->diag_floor = 1e-6;
  o->pcg_max_iters = 50;
  o->pcg_rel_tol = 1e-6;
  o->solver = 0;
  o->strategy = 0;
  o->dl_radius0 = 1.0;
  o->dl_gn_damping = 1e-6;
  return ORC_OK;
}

void orc_destroy(orc_problem* h) {
  if (!h) return;
  void* bufs[] = {h->cams, h->pts, h->uv, h->cam_idx, h->pt_idx, h->perm_pt, h->perm_cam,
                  h->pt_ptr, h->cam_ptr, h->terms, h->r, h->Jc, h->Jp, h->w, h->rho, h->B, h->gc,
                  h->C, h->gp, h->Bd, h->Cinv, h->v, h->rhs, h->M, h->Mchol, h->dc, h->dp,
                  h->cams_trial, h->pts_trial};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); i++) free(bufs[i]);
  free(h);
}

int orc_create(const double* cams, int64_t nc, const double* pts, int64_t np,
               const int32_t* cam_idx, const int32_t* pt_idx, const double* uv, int64_t nobs,
               const orc_opts* opts, orc_problem** out) {
  if (!out || !cams || !pts || nc <= 0 || np <= 0 || nobs < 0) return ORC_ERR_ARG;
  if (nobs > 0 && (!cam_idx || !pt_idx || !uv)) return ORC_ERR_ARG;
  for (int64_t k = 0; k < nobs; k++)
    if (cam_idx[k] < 0 || cam_idx[k] >= nc || pt_idx[k] < 0 || pt_idx[k] >= np)
      return ORC_ERR_ARG;
  for (int64_t i = 0; i < 9 * nc; i++)
    if (!isfinite(cams[i])) return ORC_ERR_NONFINITE;
  for (int64_t i = 0; i < 3 * np; i++)
    if (!isfinite(pts[i])) return ORC_ERR_NONFINITE;
  for (int64_t i = 0; i < 2 * nobs; i++)
    if (!isfinite(uv[i])) return ORC_ERR_NONFINITE;

  orc_problem* h = (orc_problem*)calloc(1, sizeof(orc_problem));
  if (!h) return ORC_ERR_ALLOC;
  h->nc = nc;
  h->np = np;
  h->nobs = nobs;
  if (opts)
    h->opt = *opts;
  else
    orc_opts_default(&h->opt);
  size_t N = (size_t)(nobs > 0 ? nobs : 1);
#define ALLOC(p, n, T)                              \
  do {                                              \
    (p) = (T*)calloc((size_t)(n), sizeof(T));       \
    if (!(p)) {                                     \
      orc_destroy(h);                               \
      return ORC_ERR_ALLOC;                         \
    }                                               \
  } while (0)
  ALLOC(h->cams, 9 * nc, double);
  ALLOC(h->pts, 3 * np, double);
  ALLOC(h->uv, 2 * N, double);
  ALLOC(h->cam_idx, N, int32_t);
  ALLOC(h->pt_idx, N, int32_t);
  ALLOC(h->perm_pt, N, int32_t);
  ALLOC(h->perm_cam, N, int32_t);
  ALLOC(h->pt_ptr, np + 1, int32_t);
  ALLOC(h->cam_ptr, nc + 1, int32_t);
  ALLOC(h->terms, N, double);
  ALLOC(h->r, 2 * N, double);
  ALLOC(h->Jc, 18 * N, double);
  ALLOC(h->Jp, 6 * N, double);
  ALLOC(h->w, N, double);
  ALLOC(h->rho, N, double);
  ALLOC(h->B, 81 * nc, double);
  ALLOC(h->gc, 9 * nc, double);
  ALLOC(h->C, 9 * np, double);
  ALLOC(h->gp, 3 * np, double);
  ALLOC(h->Bd, 81 * nc, double);
  ALLOC(h->Cinv, 9 * np, double);
  ALLOC(h->v, 3 * np, double);
  ALLOC(h->rhs, 9 * nc, double);
  ALLOC(h->M, 81 * nc, double);
  ALLOC(h->Mchol, 81 * nc, double);
  ALLOC(h->dc, 9 * nc, double);
  ALLOC(h->dp, 3 * np, double);
  ALLOC(h->cams_trial, 9 * nc, double);
  ALLOC(h->pts_trial, 3 * np, double);
#undef ALLOC
  memcpy(h->cams, cams, sizeof(double) * 9 * nc);
  memcpy(h->pts, pts, sizeof(double) * 3 * np);
  if (nobs > 0) {
    memcpy(h->uv, uv, sizeof(double) * 2 * nobs);
    memcpy(h->cam_idx, cam_idx, sizeof(int32_t) * nobs);
    memcpy(h->pt_idx, pt_idx, sizeof(int32_t) * nobs);
  }
  build_structure(h);
  h->lambda = h->opt.lambda0;
  h->radius = h->opt.dl_radius0;
  h->dl_valid = 0;
  h->linearized = 0;
  orc_cost_at(h, h->cams, h->pts, &h->cost);
  if (!isfinite(h->cost)) {
    orc_destroy(h);
    return ORC_ERR_NONFINITE;
  }
  *out = h;
  return ORC_OK;
}

int64_t orc_array_size(const orc_problem* h, int which) {
  int64_t nc = h->nc, np = h->np, N = h->nobs;
  switch (which) {
    case ORC_CAMS: case ORC_CAMS_TRIAL: case ORC_GC: case ORC_RHS: case ORC_DC: return 9 * nc;
    case ORC_PTS: case ORC_PTS_TRIAL: case ORC_GP: case ORC_V: case ORC_DP: return 3 * np;
    case ORC_PERM_PT: case ORC_PERM_CAM: case ORC_W: case ORC_RHO: return N;
    case ORC_PT_PTR: return np + 1;
    case ORC_CAM_PTR: return nc + 1;
    case ORC_R: return 2 * N;
    case ORC_JC: return 18 * N;
    case ORC_JP: return 6 * N;
    case ORC_B: case ORC_BD: case ORC_M: return 81 * nc;
    case ORC_C: case ORC_CINV: return 9 * np;
    default: return -1;
  }
}

static void* array_ptr(const orc_problem* h, int which) {
  switch (which) {
    case ORC_CAMS: return h->cams;
    case ORC_PTS: return h->pts;
    case ORC_PERM_PT: return h->perm_pt;
    case ORC_PERM_CAM: return h->perm_cam;
    case ORC_PT_PTR: return h->pt_ptr;
    case ORC_CAM_PTR: return h->cam_ptr;
    case ORC_R: return h->r;
    case ORC_JC: return h->Jc;
    case ORC_JP: return h->Jp;
    case ORC_W: return h->w;
    case ORC_RHO: return h->rho;
    case ORC_B: return h->B;
    case ORC_GC: return h->gc;
    case ORC_C: return h->C;
    case ORC_GP: return h->gp;
    case ORC_BD: return h->Bd;
    case ORC_CINV: return h->Cinv;
    case ORC_V: return h->v;
    case ORC_RHS: return h->rhs;
    case ORC_M: return h->M;
    case ORC_DC: return h->dc;
    case ORC_DP: return h->dp;
    case ORC_CAMS_TRIAL: return h->cams_trial;
    case ORC_PTS_TRIAL: return h->pts_trial;
    default: return NULL;
  }
}

static size_t elem_size(int which) {
  return (which == ORC_PERM_PT || which == ORC_PERM_CAM || which == ORC_PT_PTR ||
          which == ORC_CAM_PTR) ? sizeof(int32_t) : sizeof(double);
}

int orc_get(const orc_problem* h, int which, void* out) {
  void* p = array_ptr(h, which);
  if (!p || !out) return ORC_ERR_ARG;
  memcpy(out, p, elem_size(which) * (size_t)orc_array_size(h, which));
  return ORC_OK;
}

int orc_set(orc_problem* h, int which, const void* in) {
  if (which != ORC_CAMS && which != ORC_PTS) return ORC_ERR_ARG;
  memcpy(array_ptr(h, which), in, elem_size(which) * (size_t)orc_array_size(h, which));
  h->linearized = 0;
  h->dl_valid = 0;
  orc_cost_at(h, h->cams, h->pts, &h->cost);
  return ORC_OK;
}

double orc_get_lambda(const orc_problem* h) { return h->lambda; }
double orc_get_radius(const orc_problem* h) { return h->radius; }
void orc_set_radius(orc_problem* h, double radius) { h->radius = radius; }
void orc_set_lambda(orc_problem* h, double lam) { h->lambda = lam; }
double orc_get_cost(const orc_problem* h) { return h->cost; }

/* ---------------------------------------------------------- the LM step -- */

/* Total cost sum_k rho_k, summed in observation order ([THESEUS] cost
 * S = 1/2 sum |w c|^2; with the robust kernel, sum rho). */
int orc_cost_at(const orc_problem* h, const double* cams, const double* pts, double* cost) {
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < h->nobs; k++)
    h->terms[k] = obs_cost(cams + 9 * h->cam_idx[k], pts + 3 * h->pt_idx[k], h->uv + 2 * k,
                           h->opt.loss, h->opt.huber_delta);
  double s = 0.0;
  for (int64_t k = 0; k < h->nobs; k++) s += h->terms[k];
  *cost = s;
  return isfinite(s) ? ORC_OK : ORC_ERR_NONFINITE;
}

/* Linearisation and block assembly ([NSLAM] sec. 3.1: H = J^T W J, b = -J^T W r,
 * with B the 9x9 camera blocks, C the 3x3 point blocks, E the coupling blocks
 * that exist only for observed pairs).  Sums run in observation order. */
int orc_linearize(orc_problem* h) {
  memset(h->B, 0, sizeof(double) * 81 * h->nc);
  memset(h->gc, 0, sizeof(double) * 9 * h->nc);
  memset(h->C, 0, sizeof(double) * 9 * h->np);
  memset(h->gp, 0, sizeof(double) * 3 * h->np);
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < h->nobs; k++) {
    int32_t j = h->cam_idx[k], i = h->pt_idx[k];
    orc_project_one(h->cams + 9 * j, h->pts + 3 * i, h->uv + 2 * k, h->opt.loss,
                    h->opt.huber_delta, h->r + 2 * k, h->Jc + 18 * k, h->Jp + 6 * k, h->w + k,
                    h->rho + k);
  }
#pragma omp parallel
  {
    int64_t j0, j1, i0, i1;
    my_range(h->nc, &j0, &j1);
    my_range(h->np, &i0, &i1);
    for (int64_t k = 0; k < h->nobs; k++) {
      int32_t j = h->cam_idx[k], i = h->pt_idx[k];
      const double* r = h->r + 2 * k;
      const double* Jc = h->Jc + 18 * k;
      const double* Jp = h->Jp + 6 * k;
      double w = h->w[k];
      if (j >= j0 && j < j1) {
        double* B = h->B + 81 * j;
        for (int a = 0; a < 9; a++) {
          for (int b = 0; b < 9; b++) B[9 * a + b] += w * (Jc[a] * Jc[b] + Jc[9 + a] * Jc[9 + b]);
          h->gc[9 * j + a] += w * (Jc[a] * r[0] + Jc[9 + a] * r[1]);
        }
      }
      if (i >= i0 && i < i1) {
        double* C = h->C + 9 * i;
        for (int a = 0; a < 3; a++) {
          for (int b = 0; b < 3; b++) C[3 * a + b] += w * (Jp[a] * Jp[b] + Jp[3 + a] * Jp[3 + b]);
          h->gp[3 * i + a] += w * (Jp[a] * r[0] + Jp[3 + a] * r[1]);
        }
      }
    }
  }
  h->linearized = 1;
  return ORC_OK;
}

/* E_k = w_k Jc_k^T Jp_k (9x3), recomputed from the stored blocks. */
static void E_block(const orc_problem* h, int64_t k, double* E) {
  const double* Jc = h->Jc + 18 * k;
  const double* Jp = h->Jp + 6 * k;
  double w = h->w[k];
  for (int a = 0; a < 9; a++)
    for (int b = 0; b < 3; b++) E[3 * a + b] = w * (Jc[a] * Jp[b] + Jc[9 + a] * Jp[3 + b]);
}

/* LM damping and point-block inverse.  [BAE] lists diagonal damping; [THESEUS]
 * LM with adaptive damping.  Reading (Marquardt): D = diag(J^T W J) floored at
 * diag_floor, H~ = H + lambda D, applied to B and C alike.  The inverse of each
 * damped 3x3 point block is formed explicitly, which [NSLAM] sec. 3.2 allows
 * because the blocks are tiny (via its Cholesky factor).  v_i = C~_i^-1 g_p,i. */
int orc_damp(orc_problem* h) {
  double lam = h->lambda, fl = h->opt.diag_floor;
  int bad = 0;
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < h->nc; j++) {
    double* Bd = h->Bd + 81 * j;
    memcpy(Bd, h->B + 81 * j, sizeof(double) * 81);
    for (int a = 0; a < 9; a++) {
      double d = Bd[10 * a];
      Bd[10 * a] += lam * (d > fl ? d : fl);
    }
  }
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t i = 0; i < h->np; i++) {
    double L[9];
    memcpy(L, h->C + 9 * i, sizeof(double) * 9);
    for (int a = 0; a < 3; a++) {
      double d = L[4 * a];
      L[4 * a] += lam * (d > fl ? d : fl);
    }
    if (chol(L, 3)) {
      bad = 1;
      continue;
    }
    double* Ci = h->Cinv + 9 * i;
    for (int c = 0; c < 3; c++) {
      double e[3] = {0.0, 0.0, 0.0}, x[3];
      e[c] = 1.0;
      chol_solve(L, 3, e, x);
      for (int a = 0; a < 3; a++) Ci[3 * a + c] = x[a];
    }
    for (int a = 0; a < 3; a++)
      h->v[3 * i + a] = Ci[3 * a] * h->gp[3 * i] + Ci[3 * a + 1] * h->gp[3 * i + 1] +
                        Ci[3 * a + 2] * h->gp[3 * i + 2];
  }
  return bad ? ORC_ERR_NOT_SPD : ORC_OK;
}

/* Reduced right-hand side and block-Jacobi preconditioner ([NSLAM] sec. 3.2,
 * eq. (2): (B - E C^-1 E^T) dc = b_c - E C^-1 b_d with b = -g, so
 * rhs = -g_c + E C~^-1 g_p = -g_c + E v).  M_j is the exact diagonal block S_jj:
 * B~_j - sum over (j, i) of Ebar C~_i^-1 Ebar^T, Ebar summing the coupling blocks
 * of repeated (camera, point) observations.  Each M_j is Cholesky factored. */
int orc_schur(orc_problem* h) {
  for (int64_t j = 0; j < h->nc; j++) {
    for (int a = 0; a < 9; a++) h->rhs[9 * j + a] = -h->gc[9 * j + a];
    memcpy(h->M + 81 * j, h->Bd + 81 * j, sizeof(double) * 81);
  }
#pragma omp parallel
  {
    int64_t j0, j1;
    my_range(h->nc, &j0, &j1);
    for (int64_t k = 0; k < h->nobs; k++) {
      int32_t j = h->cam_idx[k], i = h->pt_idx[k];
      if (j < j0 || j >= j1) continue;
      double E[27];
      E_block(h, k, E);
      const double* vi = h->v + 3 * i;
      for (int a = 0; a < 9; a++)
        h->rhs[9 * j + a] += E[3 * a] * vi[0] + E[3 * a + 1] * vi[1] + E[3 * a + 2] * vi[2];
    }
  }
  /* the (camera, point) runs of the (cam, pt, k) order; a camera's runs are
   * contiguous, so each camera's block is formed by one thread in run order */
  int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
  for (int64_t jc = 0; jc < h->nc; jc++) {
  int64_t s = h->cam_ptr[jc];
  while (s < h->cam_ptr[jc + 1]) {
    int32_t k0 = h->perm_cam[s];
    int32_t j = h->cam_idx[k0], i = h->pt_idx[k0];
    double Eb[27] = {0};
    int64_t e = s;
    while (e < h->nobs && h->cam_idx[h->perm_cam[e]] == j && h->pt_idx[h->perm_cam[e]] == i) {
      double E[27];
      E_block(h, h->perm_cam[e], E);
      for (int l = 0; l < 27; l++) Eb[l] += E[l];
      e++;
    }
    const double* Ci = h->Cinv + 9 * i;
    double* M = h->M + 81 * j;
    for (int a = 0; a < 9; a++) {
      double EC[3];
      for (int c = 0; c < 3; c++)
        EC[c] = Eb[3 * a] * Ci[c] + Eb[3 * a + 1] * Ci[3 + c] + Eb[3 * a + 2] * Ci[6 + c];
      for (int b = 0; b < 9; b++)
        M[9 * a + b] -= EC[0] * Eb[3 * b] + EC[1] * Eb[3 * b + 1] + EC[2] * Eb[3 * b + 2];
    }
    s = e;
  }
  memcpy(h->Mchol + 81 * jc, h->M + 81 * jc, sizeof(double) * 81);
  if (chol(h->Mchol + 81 * jc, 9)) bad = 1;
  }
  return bad ? ORC_ERR_NOT_SPD : ORC_OK;
}

/* Implicit Schur product S x = B~ x - E C~^-1 E^T x, without forming S:
 * y_i = sum_{k in i} E_k^T x_cam(k), z_i = C~_i^-1 y_i,
 * (S x)_j = B~_j x_j - sum_{k in j} E_k z_pt(k). */
int orc_schur_matvec(orc_problem* h, const double* x, double* out) {
  double* z = (double*)calloc((size_t)(3 * h->np), sizeof(double));
  double* y = (double*)calloc((size_t)(3 * h->np), sizeof(double));
  if (!z || !y) {
    free(z);
    free(y);
    return ORC_ERR_ALLOC;
  }
#pragma omp parallel
  {
    int64_t i0, i1;
    my_range(h->np, &i0, &i1);
    for (int64_t k = 0; k < h->nobs; k++) {
      if (h->pt_idx[k] < i0 || h->pt_idx[k] >= i1) continue;
      double E[27];
      E_block(h, k, E);
      const double* xc = x + 9 * h->cam_idx[k];
      double* yi = y + 3 * h->pt_idx[k];
      for (int b = 0; b < 3; b++) {
        double s = 0.0;
        for (int a = 0; a < 9; a++) s += E[3 * a + b] * xc[a];
        yi[b] += s;
      }
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < h->np; i++) {
    const double* Ci = h->Cinv + 9 * i;
    for (int a = 0; a < 3; a++)
      z[3 * i + a] = Ci[3 * a] * y[3 * i] + Ci[3 * a + 1] * y[3 * i + 1] + Ci[3 * a + 2] * y[3 * i + 2];
  }
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < h->nc; j++) {
    const double* Bd = h->Bd + 81 * j;
    for (int a = 0; a < 9; a++) {
      double s = 0.0;
      for (int b = 0; b < 9; b++) s += Bd[9 * a + b] * x[9 * j + b];
      out[9 * j + a] = s;
    }
  }
#pragma omp parallel
  {
    int64_t j0, j1;
    my_range(h->nc, &j0, &j1);
    for (int64_t k = 0; k < h->nobs; k++) {
      if (h->cam_idx[k] < j0 || h->cam_idx[k] >= j1) continue;
      double E[27];
      E_block(h, k, E);
      const double* zi = z + 3 * h->pt_idx[k];
      double* o = out + 9 * h->cam_idx[k];
      for (int a = 0; a < 9; a++) o[a] -= E[3 * a] * zi[0] + E[3 * a + 1] * zi[1] + E[3 * a + 2] * zi[2];
    }
  }
  free(z);
  free(y);
  return ORC_OK;
}

/* Preconditioned conjugate gradients on S dc = rhs ([BAE]: PCG for large
 * problems).  x0 = 0, preconditioner M = blockdiag(S_jj) applied through its
 * Cholesky factors.  Reading: stop once |r|_2 <= tol |rhs|_2 after an update, or
 * at max_iters; stop early (keeping x) if p^T S p is not positive and finite. */
int orc_pcg(orc_problem* h, int max_iters, double rel_tol, int* iters_out, double* rel_res_out) {
  int64_t n = 9 * h->nc;
  double* x = h->dc;
  double* r = (double*)malloc(sizeof(double) * n);
  double* z = (double*)malloc(sizeof(double) * n);
  double* p = (double*)malloc(sizeof(double) * n);
  double* q = (double*)malloc(sizeof(double) * n);
  if (!r || !z || !p || !q) {
    free(r);
    free(z);
    free(p);
    free(q);
    return ORC_ERR_ALLOC;
  }
  for (int64_t a = 0; a < n; a++) {
    x[a] = 0.0;
    r[a] = h->rhs[a];
  }
  double rhs_norm = sqrt(dot(r, r, n));
  int it = 0;
  double res = rhs_norm;
  if (rhs_norm > 0.0) {
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < h->nc; j++) chol_solve(h->Mchol + 81 * j, 9, r + 9 * j, z + 9 * j);
    memcpy(p, z, sizeof(double) * n);
    double rz = dot(r, z, n);
    for (int k = 1; k <= max_iters; k++) {
      orc_schur_matvec(h, p, q);
      double pq = dot(p, q, n);
      if (!(pq > 0.0) || !isfinite(pq)) break;
      double alpha = rz / pq;
      for (int64_t a = 0; a < n; a++) {
        x[a] += alpha * p[a];
        r[a] -= alpha * q[a];
      }
      it = k;
      res = sqrt(dot(r, r, n));
      if (res <= rel_tol * rhs_norm) break;
#pragma omp parallel for schedule(static)
      for (int64_t j = 0; j < h->nc; j++) chol_solve(h->Mchol + 81 * j, 9, r + 9 * j, z + 9 * j);
      double rz_new = dot(r, z, n);
      double beta = rz_new / rz;
      rz = rz_new;
      for (int64_t a = 0; a < n; a++) p[a] = z[a] + beta * p[a];
    }
  } else {
    memset(x, 0, sizeof(double) * n);
  }
  if (iters_out) *iters_out = it;
  if (rel_res_out) *rel_res_out = rhs_norm > 0.0 ? res / rhs_norm : 0.0;
  free(r);
  free(z);
  free(p);
  free(q);
  return ORC_OK;
}

/* Dense reduced camera matrix S = B~ - E C~^-1 E^T (9 nc square), formed
 * explicitly for small problems ([NSLAM] sec. 3.2, dense reference step). */
int orc_explicit_S(orc_problem* h, double* S) {
  int64_t n = 9 * h->nc;
  memset(S, 0, sizeof(double) * (size_t)(n * n));
  for (int64_t j = 0; j < h->nc; j++)
    for (int a = 0; a < 9; a++)
      for (int b = 0; b < 9; b++) S[(9 * j + a) * n + 9 * j + b] = h->Bd[81 * j + 9 * a + b];
  for (int64_t i = 0; i < h->np; i++) {
    const double* Ci = h->Cinv + 9 * i;
    for (int32_t s1 = h->pt_ptr[i]; s1 < h->pt_ptr[i + 1]; s1++) {
      int32_t k1 = h->perm_pt[s1];
      double E1[27];
      E_block(h, k1, E1);
      int64_t j1 = h->cam_idx[k1];
      double EC[27];
      for (int a = 0; a < 9; a++)
        for (int c = 0; c < 3; c++)
          EC[3 * a + c] = E1[3 * a] * Ci[c] + E1[3 * a + 1] * Ci[3 + c] + E1[3 * a + 2] * Ci[6 + c];
      for (int32_t s2 = h->pt_ptr[i]; s2 < h->pt_ptr[i + 1]; s2++) {
        int32_t k2 = h->perm_pt[s2];
        double E2[27];
        E_block(h, k2, E2);
        int64_t j2 = h->cam_idx[k2];
        for (int a = 0; a < 9; a++)
          for (int b = 0; b < 9; b++)
            S[(9 * j1 + a) * n + 9 * j2 + b] -=
                EC[3 * a] * E2[3 * b] + EC[3 * a + 1] * E2[3 * b + 1] + EC[3 * a + 2] * E2[3 * b + 2];
      }
    }
  }
  return ORC_OK;
}

/* Camera update by a Cholesky factorisation of the explicit S, as in the dense
 * reference step of [NSLAM] sec. 3.2 (S solved by Cholesky, never inverted). */
int orc_dense_schur_solve(orc_problem* h) {
  int64_t n = 9 * h->nc;
  double* S = (double*)malloc(sizeof(double) * (size_t)(n * n));
  if (!S) return ORC_ERR_ALLOC;
  orc_explicit_S(h, S);
  if (chol(S, (int)n)) {
    free(S);
    return ORC_ERR_NOT_SPD;
  }
  chol_solve(S, (int)n, h->rhs, h->dc);
  free(S);
  return ORC_OK;
}

/* Camera marginal covariance ([NSLAM] sec. 3.2, the dense reference step: the
 * Cholesky factor of S that gives the camera update also gives S^-1 by solving
 * against the identity, column by column; S is never inverted directly).
 * Computed at the current parameters and lambda: linearise, damp, form S~ =
 * B~ - E C~^-1 E^T, factor it, and solve S~ x = e_k for every k.  out receives
 * the 9x9 diagonal blocks of S~^-1 (nc x 81, row-major): each camera's
 * marginal covariance under the damped Gauss-Newton model. */
int orc_covariance(orc_problem* h, double* out) {
  h->dl_valid = 0;
  int rc = orc_linearize(h);
  if (rc) return rc;
  if ((rc = orc_damp(h))) return rc;
  const int64_t n = 9 * h->nc;
  double* S = (double*)malloc(sizeof(double) * (size_t)(n * n));
  double* e = (double*)calloc((size_t)n, sizeof(double));
  double* x = (double*)malloc(sizeof(double) * (size_t)n);
  if (!S || !e || !x) {
    free(S);
    free(e);
    free(x);
    return ORC_ERR_ALLOC;
  }
  orc_explicit_S(h, S);
  rc = chol(S, (int)n) ? ORC_ERR_NOT_SPD : ORC_OK;
  for (int64_t k = 0; k < n && rc == ORC_OK; k++) {
    e[k] = 1.0;
    chol_solve(S, (int)n, e, x);   /* column k of S~^-1 */
    e[k] = 0.0;
    const int64_t j = k / 9;
    const int b = (int)(k % 9);
    for (int a = 0; a < 9; a++) out[81 * j + 9 * a + b] = x[9 * j + a];
  }
  free(S);
  free(e);
  free(x);
  return rc;
}

/* Point back-substitution, [NSLAM] sec. 3.2 eq. (1): dp = C~^-1 (b_d - E^T dc)
 * with b_d = -g_p. */
int orc_backsub(orc_problem* h) {
  double* y = (double*)malloc(sizeof(double) * (size_t)(3 * h->np));
  if (!y) return ORC_ERR_ALLOC;
  for (int64_t i = 0; i < 3 * h->np; i++) y[i] = -h->gp[i];
#pragma omp parallel
  {
    int64_t i0, i1;
    my_range(h->np, &i0, &i1);
    for (int64_t k = 0; k < h->nobs; k++) {
      if (h->pt_idx[k] < i0 || h->pt_idx[k] >= i1) continue;
      double E[27];
      E_block(h, k, E);
      const double* xc = h->dc + 9 * h->cam_idx[k];
      double* yi = y + 3 * h->pt_idx[k];
      for (int b = 0; b < 3; b++) {
        double s = 0.0;
        for (int a = 0; a < 9; a++) s += E[3 * a + b] * xc[a];
        yi[b] -= s;
      }
    }
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < h->np; i++) {
    const double* Ci = h->Cinv + 9 * i;
    for (int a = 0; a < 3; a++)
      h->dp[3 * i + a] = Ci[3 * a] * y[3 * i] + Ci[3 * a + 1] * y[3 * i + 1] + Ci[3 * a + 2] * y[3 * i + 2];
  }
  free(y);
  return ORC_OK;
}

/* Trial parameters x' = x (+) delta: camera retraction, points additive. */
int orc_retract(orc_problem* h) {
#pragma omp parallel for schedule(static)
  for (int64_t j = 0; j < h->nc; j++)
    orc_retract_camera(h->cams + 9 * j, h->dc + 9 * j, h->cams_trial + 9 * j);
  for (int64_t i = 0; i < 3 * h->np; i++) h->pts_trial[i] = h->pts[i] + h->dp[i];
  return ORC_OK;
}

/* One LM iteration ([THESEUS]: linearise, solve the normal equations, retract;
 * LM with adaptive damping).  Reading of the unstated schedule: accept iff the
 * trial cost is strictly lower; accept divides lambda by lambda_down (floor
 * lambda_min), reject multiplies it by lambda_up (cap lambda_max) and keeps x.
 * A rejected iteration still counts. */
int orc_lm_step(orc_problem* h, orc_step_info* info) {
  int rc;
  if (h->opt.strategy == 1) return orc_dogleg_step(h, info);
  if (!h->linearized && (rc = orc_linearize(h))) return rc;
  if ((rc = orc_damp(h))) return rc;
  if ((rc = orc_schur(h))) return rc;
  int iters = 0;
  double rel = 0.0;
  if (h->opt.solver == 1) {
    if ((rc = orc_dense_schur_solve(h))) return rc;
  } else {
    if ((rc = orc_pcg(h, h->opt.pcg_max_iters, h->opt.pcg_rel_tol, &iters, &rel))) return rc;
  }
  if ((rc = orc_backsub(h))) return rc;
  orc_retract(h);
  double trial;
  orc_cost_at(h, h->cams_trial, h->pts_trial, &trial);
  orc_step_info inf;
  memset(&inf, 0, sizeof(inf));
  inf.cost_before = h->cost;
  inf.cost_after = trial;
  inf.lambda = h->lambda;
  inf.pcg_iters = iters;
  inf.pcg_rel_res = rel;
  if (isfinite(trial) && trial < h->cost) {
    inf.accepted = 1;
    memcpy(h->cams, h->cams_trial, sizeof(double) * 9 * h->nc);
    memcpy(h->pts, h->pts_trial, sizeof(double) * 3 * h->np);
    h->cost = trial;
    h->linearized = 0;
    h->lambda = h->lambda / h->opt.lambda_down;
    if (h->lambda < h->opt.lambda_min) h->lambda = h->opt.lambda_min;
  } else {
    inf.accepted = 0;
    h->lambda = h->lambda * h->opt.lambda_up;
    if (h->lambda > h->opt.lambda_max) h->lambda = h->opt.lambda_max;
  }
  if (info) *info = inf;
  return ORC_OK;
}

/* One dogleg iteration ([THESEUS]: LM with adaptive damping, and Dogleg, are
 * offered beside Gauss-Newton; [BAE] names dogleg among the further
 * optimisers).  Powell's dogleg in the trust-region form of Madsen, Nielsen
 * and Tingleff's notes on non-linear least squares, with the quadratic model
 * L(h) = C + g^T h + 1/2 h^T H h, H = J^T W J (the IRLS weights for Huber):
 *   h_sd = -alpha g, alpha = |g|^2 / |J g|_W^2, the model's minimiser along -g;
 *   h_gn from (H + mu D) h = -g by the configured solver (Schur elimination,
 *        PCG or the dense Cholesky of S, back-substitution).  Reading: mu is a
 *        small fixed Marquardt damping (opts.dl_gn_damping, D as for LM),
 *        because H of a BA problem is singular along its gauge;
 *   h = h_gn if |h_gn| <= radius; else -(radius / |g|) g if alpha |g| >=
 *        radius; else -alpha g + beta (h_gn + alpha g) with |h| = radius;
 *   gain ratio rho = (C - C(x + h)) / (L(0) - L(h)); the step is kept iff the
 *        cost is strictly lower (as for LM); radius = max(radius, 3 |h|) when
 *        rho > 0.75, radius / 2 when rho < 0.25.
 * |.| is the Euclidean norm over all parameters in the tangent of the
 * retraction.  h_gn, alpha and the model's scalars are kept while the point
 * of linearisation does not move, so a rejected step costs one trial cost. */
int orc_dogleg_step(orc_problem* h, orc_step_info* info) {
  int rc;
  const int64_t nc = h->nc, np = h->np;
  if (!h->dl_valid) {
    if (!h->linearized && (rc = orc_linearize(h))) return rc;
    const double lam = h->lambda;
    h->lambda = h->opt.dl_gn_damping;
    rc = orc_damp(h);
    if (!rc) rc = orc_schur(h);
    int iters = 0;
    double rel = 0.0;
    if (!rc) {
      if (h->opt.solver == 1) rc = orc_dense_schur_solve(h);
      else rc = orc_pcg(h, h->opt.pcg_max_iters, h->opt.pcg_rel_tol, &iters, &rel);
    }
    if (!rc) rc = orc_backsub(h);
    h->lambda = lam;
    if (rc) return rc;
    double gg = 0.0, nn = 0.0, gn = 0.0;
    for (int64_t e = 0; e < 9 * nc; e++) {
      gg += h->gc[e] * h->gc[e];
      nn += h->dc[e] * h->dc[e];
      gn += h->gc[e] * h->dc[e];
    }
    for (int64_t e = 0; e < 3 * np; e++) {
      gg += h->gp[e] * h->gp[e];
      nn += h->dp[e] * h->dp[e];
      gn += h->gp[e] * h->dp[e];
    }
    double uu = 0.0, uv = 0.0, vv = 0.0;   /* |J g|_W^2, (J g)^T W (J h_gn), |J h_gn|_W^2 */
    for (int64_t k = 0; k < h->nobs; k++) {
      const double* Jc = h->Jc + 18 * k;
      const double* Jp = h->Jp + 6 * k;
      const double* gcj = h->gc + 9 * h->cam_idx[k];
      const double* gpi = h->gp + 3 * h->pt_idx[k];
      const double* dcj = h->dc + 9 * h->cam_idx[k];
      const double* dpi = h->dp + 3 * h->pt_idx[k];
      for (int a = 0; a < 2; a++) {
        double u = 0.0, v = 0.0;
        for (int b = 0; b < 9; b++) {
          u += Jc[9 * a + b] * gcj[b];
          v += Jc[9 * a + b] * dcj[b];
        }
        for (int b = 0; b < 3; b++) {
          u += Jp[3 * a + b] * gpi[b];
          v += Jp[3 * a + b] * dpi[b];
        }
        uu += h->w[k] * u * u;
        uv += h->w[k] * u * v;
        vv += h->w[k] * v * v;
      }
    }
    h->dl_gg = gg;
    h->dl_nn = nn;
    h->dl_gn = gn;
    h->dl_JgJg = uu;
    h->dl_JgJn = uv;
    h->dl_JnJn = vv;
    h->dl_iters = iters;
    h->dl_rel = rel;
    h->dl_valid = 1;
  }
  /* the step as h = s_g g + s_n h_gn */
  const double R = h->radius, gnorm = sqrt(h->dl_gg), nnorm = sqrt(h->dl_nn);
  double s_g = 0.0, s_n = 0.0;
  int kind = 0;
  if (h->dl_gg == 0.0) {
    kind = 0;   /* stationary: no step */
  } else if (nnorm <= R) {
    s_n = 1.0;
    kind = 0;
  } else {
    const double alpha = h->dl_JgJg > 0.0 ? h->dl_gg / h->dl_JgJg : INFINITY;
    if (alpha * gnorm >= R) {
      s_g = -R / gnorm;
      kind = 1;
    } else {
      /* a = -alpha g, b = h_gn: |a + beta (b - a)| = R */
      const double aa = alpha * alpha * h->dl_gg;
      const double c = -alpha * h->dl_gn - aa;                 /* a^T (b - a) */
      const double dd = h->dl_nn + 2.0 * alpha * h->dl_gn + aa;   /* |b - a|^2 */
      const double disc = sqrt(c * c + dd * (R * R - aa));
      const double beta = c <= 0.0 ? (-c + disc) / dd : (R * R - aa) / (c + disc);
      s_g = -alpha * (1.0 - beta);
      s_n = beta;
      kind = 2;
    }
  }
  const double hh = s_g * s_g * h->dl_gg + 2.0 * s_g * s_n * h->dl_gn + s_n * s_n * h->dl_nn;
  const double hnorm = sqrt(hh > 0.0 ? hh : 0.0);
  const double gh = s_g * h->dl_gg + s_n * h->dl_gn;
  const double hHh = s_g * s_g * h->dl_JgJg + 2.0 * s_g * s_n * h->dl_JgJn + s_n * s_n * h->dl_JnJn;
  const double model = -gh - 0.5 * hHh;   /* L(0) - L(h) */
  for (int64_t j = 0; j < nc; j++) {
    double d[9];
    for (int a = 0; a < 9; a++) d[a] = s_g * h->gc[9 * j + a] + s_n * h->dc[9 * j + a];
    orc_retract_camera(h->cams + 9 * j, d, h->cams_trial + 9 * j);
  }
  for (int64_t e = 0; e < 3 * np; e++) h->pts_trial[e] = h->pts[e] + (s_g * h->gp[e] + s_n * h->dp[e]);
  double trial;
  orc_cost_at(h, h->cams_trial, h->pts_trial, &trial);
  const double rho = model > 0.0 ? (h->cost - trial) / model : 0.0;
  orc_step_info inf;
  memset(&inf, 0, sizeof(inf));
  inf.cost_before = h->cost;
  inf.cost_after = trial;
  inf.lambda = h->lambda;
  inf.pcg_iters = h->dl_iters;
  inf.pcg_rel_res = h->dl_rel;
  inf.radius = R;
  inf.gain_ratio = rho;
  inf.step_norm = hnorm;
  inf.step_kind = kind;
  if (rho > 0.75) {
    if (3.0 * hnorm > h->radius) h->radius = 3.0 * hnorm;
  } else if (rho < 0.25) {
    h->radius = 0.5 * h->radius;
  }
  if (isfinite(trial) && trial < h->cost) {
    inf.accepted = 1;
    memcpy(h->cams, h->cams_trial, sizeof(double) * 9 * nc);
    memcpy(h->pts, h->pts_trial, sizeof(double) * 3 * np);
    h->cost = trial;
    h->linearized = 0;
    h->dl_valid = 0;
  } else {
    inf.accepted = 0;
  }
  h->dl_iters = 0;   /* a repeat at this linearisation runs no solve */
  h->dl_rel = 0.0;
  if (info) *info = inf;
  return ORC_OK;
}

/* Implicit backward ([THESEUS], "backward modes", implicit differentiation):
 * with the optimality condition g(theta; u) = grad_theta S = 0, the note gets
 * D_u theta* = -(D_theta g)^-1 D_u g by differentiating one Newton step at the
 * solution, h(theta; u) = theta - [Hess S]^-1_stop grad S, the Hessian held
 * fixed.  Readings: the Hessian is the damped Gauss-Newton matrix of the
 * current LM state, H~ = J^T W J + lambda diag (the damping makes it
 * invertible; the undamped one is singular along the 7-dimensional gauge of a
 * BA problem); u are the observed pixels.  grad S = sum_k J_k^T psi(r_k) with
 * psi(r) = d rho(|r|) / dr and r_k = u^_k(theta) - u_k, so
 * d grad S / d u_k = -J_k^T psi'(r_k) and, for a loss f of the solution with
 * gradient G,
 *   df/du_k = psi'(r_k) J_k H~^-1 G,
 * psi' = I for the squared loss and inside the Huber threshold, and
 * (delta / |r|) (I - r r^T / |r|^2) beyond it.  H~^-1 G is the damped system
 * of an LM step solved with g = -G: Schur complement, the configured solver
 * (PCG, or the dense Cholesky of S), back-substitution.  grad_cams is nc x 9,
 * grad_pts np x 3, out_uv nobs x 2 in the original observation order. */
int orc_backward(orc_problem* h, const double* grad_cams, const double* grad_pts, double* out_uv,
                 int* iters_out, double* rel_res_out) {
  int rc = orc_linearize(h);
  if (rc) return rc;
  for (int64_t e = 0; e < 9 * h->nc; e++) h->gc[e] = -grad_cams[e];
  for (int64_t e = 0; e < 3 * h->np; e++) h->gp[e] = -grad_pts[e];
  h->linearized = 0; /* g no longer holds the gradient of the cost */
  h->dl_valid = 0;
  if ((rc = orc_damp(h))) return rc;
  if ((rc = orc_schur(h))) return rc;
  int iters = 0;
  double rel = 0.0;
  if (h->opt.solver == 1) {
    if ((rc = orc_dense_schur_solve(h))) return rc;
  } else {
    if ((rc = orc_pcg(h, h->opt.pcg_max_iters, h->opt.pcg_rel_tol, &iters, &rel))) return rc;
  }
  if ((rc = orc_backsub(h))) return rc;
#pragma omp parallel for schedule(static)
  for (int64_t k = 0; k < h->nobs; k++) {
    const double* Jc = h->Jc + 18 * k;
    const double* Jp = h->Jp + 6 * k;
    const double* xc = h->dc + 9 * h->cam_idx[k];
    const double* xp = h->dp + 3 * h->pt_idx[k];
    double y[2];
    for (int a = 0; a < 2; a++) {
      double t = 0.0;
      for (int b = 0; b < 9; b++) t += Jc[9 * a + b] * xc[b];
      for (int b = 0; b < 3; b++) t += Jp[3 * a + b] * xp[b];
      y[a] = t;
    }
    const double* r = h->r + 2 * k;
    const double e = sqrt(r[0] * r[0] + r[1] * r[1]);
    if (h->opt.loss == 1 && e > h->opt.huber_delta) {
      const double ry = (r[0] * y[0] + r[1] * y[1]) / (e * e);
      out_uv[2 * k] = h->opt.huber_delta / e * (y[0] - r[0] * ry);
      out_uv[2 * k + 1] = h->opt.huber_delta / e * (y[1] - r[1] * ry);
    } else {
      out_uv[2 * k] = y[0];
      out_uv[2 * k + 1] = y[1];
    }
  }
  if (iters_out) *iters_out = iters;
  if (rel_res_out) *rel_res_out = rel;
  return ORC_OK;
}

int orc_solve(orc_problem* h, int n_iters, orc_step_info* infos) {
  for (int it = 0; it < n_iters; it++) {
    int rc = orc_lm_step(h, infos ? infos + it : NULL);
    if (rc) return rc;
  }
  return ORC_OK;
}

/* Threads the loops above run on (1 without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
