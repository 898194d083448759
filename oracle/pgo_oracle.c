/* CPU oracle for pose-graph optimisation (fp64).
 *
 * TEST INFRASTRUCTURE ONLY: plain loops, no blocking, no threads.  Only the
 * test suite, the smoke check and the CPU-baseline leg of the benchmark may
 * load it.  It shares no code with the GPU library.
 *
 * Pages cited (by title and section):
 *  [BAE]      "Bundle Adjustment in the Eager Mode" (summary article), the pose
 *             graph optimisation paragraph: a set of poses constrained by
 *             relative-pose measurements (odometry, loop closures); indexing
 *             decides which two poses a residual joins, Lie-group operations
 *             give the residual and its Jacobian blocks, sparse LM solves.
 *  [THESEUS]  Theseus note, "Method and architecture": manifold variables with
 *             retraction and analytic tangent derivatives, cost 1/2 sum |w c|^2,
 *             LM with adaptive damping; pose graph optimisation as an
 *             application of the same components.
 *
 * Readings (the pages give no residual formula for PGO):
 *  - pose T = (R, t) maps body to world; an edge (i, j) measures T_i^-1 T_j as
 *    (R_ij, t_ij);
 *  - residual r = [r_R; r_t] with r_R = Log(R_ij^T R_i^T R_j) and
 *    r_t = R_i^T (t_j - t_i) - t_ij, weighted by diag(w_R I3, w_t I3);
 *  - tangent xi = [dphi; dt], retraction R <- R Exp(dphi), t <- t + dt;
 *  - the first n_fixed poses are held (the gauge);
 *  - LM exactly as the bundle-adjustment oracle: Marquardt damping with a
 *    floor, accept iff the cost decreases strictly, lambda / 10 or x 10.
 */
#include "pgo_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

struct porc_problem {
  int64_t n, m;
  int n_fixed;
  porc_opts opt;
  double *poses, *trial;
  int32_t* edges;
  double *meas, *info;
  double *r, *Ji, *Jj, *Hd, *Ho, *g, *dx;
  double lambda, cost;
  int linearized;
};

/* ------------------------------------------------------------- SO(3) --- */

/* Rodrigues: R = I + sin(a)/a [w]x + (1 - cos a)/a^2 [w]x^2 (series below 1e-8). */
void porc_so3_exp(const double* w, double* R) {
  const double a2 = w[0] * w[0] + w[1] * w[1] + w[2] * w[2], a = sqrt(a2);
  double A, B;
  if (a < 1e-8) {
    A = 1.0;
    B = 0.5;
  } else {
    A = sin(a) / a;
    B = (1.0 - cos(a)) / a2;
  }
  const double K[9] = {0.0, -w[2], w[1], w[2], 0.0, -w[0], -w[1], w[0], 0.0};
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double k2 = 0.0;
      for (int l = 0; l < 3; l++) k2 += K[3 * i + l] * K[3 * l + j];
      R[3 * i + j] = (i == j ? 1.0 : 0.0) + A * K[3 * i + j] + B * k2;
    }
}

/* Log through the unit quaternion of R (Shepperd's choice of the largest
 * component): w = 2 atan2(|v|, q_w) v / |v|, q_w >= 0. */
void porc_so3_log(const double* R, double* w) {
  const double tr = R[0] + R[4] + R[8];
  double q[4];   /* w, x, y, z */
  if (tr > R[0] && tr > R[4] && tr > R[8]) {
    const double s = 2.0 * sqrt(1.0 + tr);
    q[0] = 0.25 * s;
    q[1] = (R[7] - R[5]) / s;
    q[2] = (R[2] - R[6]) / s;
    q[3] = (R[3] - R[1]) / s;
  } else if (R[0] >= R[4] && R[0] >= R[8]) {
    const double s = 2.0 * sqrt(1.0 + R[0] - R[4] - R[8]);
    q[0] = (R[7] - R[5]) / s;
    q[1] = 0.25 * s;
    q[2] = (R[1] + R[3]) / s;
    q[3] = (R[2] + R[6]) / s;
  } else if (R[4] >= R[8]) {
    const double s = 2.0 * sqrt(1.0 + R[4] - R[0] - R[8]);
    q[0] = (R[2] - R[6]) / s;
    q[1] = (R[1] + R[3]) / s;
    q[2] = 0.25 * s;
    q[3] = (R[5] + R[7]) / s;
  } else {
    const double s = 2.0 * sqrt(1.0 + R[8] - R[0] - R[4]);
    q[0] = (R[3] - R[1]) / s;
    q[1] = (R[2] + R[6]) / s;
    q[2] = (R[5] + R[7]) / s;
    q[3] = 0.25 * s;
  }
  if (q[0] < 0.0)
    for (int k = 0; k < 4; k++) q[k] = -q[k];
  const double vn = sqrt(q[1] * q[1] + q[2] * q[2] + q[3] * q[3]);
  if (vn < 1e-12) {
    for (int k = 0; k < 3; k++) w[k] = 2.0 * q[k + 1] / q[0];
    return;
  }
  const double ang = 2.0 * atan2(vn, q[0]);
  for (int k = 0; k < 3; k++) w[k] = ang * q[k + 1] / vn;
}

/* Inverse right Jacobian of SO(3): Log(Exp(w) Exp(d)) = w + Jr^-1(w) d + O(d^2),
 * Jr^-1(w) = I + 1/2 [w]x + (1/a^2 - (1 + cos a) / (2 a sin a)) [w]x^2. */
static void so3_jr_inv(const double* w, double* J) {
  const double a2 = w[0] * w[0] + w[1] * w[1] + w[2] * w[2], a = sqrt(a2);
  const double c = a < 1e-4 ? 1.0 / 12.0 + a2 / 720.0 : 1.0 / a2 - (1.0 + cos(a)) / (2.0 * a * sin(a));
  const double K[9] = {0.0, -w[2], w[1], w[2], 0.0, -w[0], -w[1], w[0], 0.0};
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double k2 = 0.0;
      for (int l = 0; l < 3; l++) k2 += K[3 * i + l] * K[3 * l + j];
      J[3 * i + j] = (i == j ? 1.0 : 0.0) + 0.5 * K[3 * i + j] + c * k2;
    }
}

static void matmul3(const double* A, const double* B, double* C) {
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double s = 0.0;
      for (int l = 0; l < 3; l++) s += A[3 * i + l] * B[3 * l + j];
      C[3 * i + j] = s;
    }
}

static void transpose3(const double* A, double* B) {
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) B[3 * j + i] = A[3 * i + j];
}

/* ------------------------------------------------------------ edges --- */

/* r = [Log(R_ij^T R_i^T R_j); R_i^T (t_j - t_i) - t_ij] and its Jacobians in
 * the tangents of pose i and pose j (columns [dphi, dt]):
 *   dr_R/dphi_i = -Jr^-1(r_R) R_j^T R_i,  dr_R/dphi_j = Jr^-1(r_R),
 *   dr_t/dphi_i = [R_i^T (t_j - t_i)]x,   dr_t/dt_i = -R_i^T,  dr_t/dt_j = R_i^T. */
void porc_edge(const double* pi, const double* pj, const double* meas, double* r, double* Ji,
               double* Jj) {
  double Ri[9], Rj[9], Rm[9], RiT[9], RmT[9], A[9], E[9];
  porc_so3_exp(pi, Ri);
  porc_so3_exp(pj, Rj);
  porc_so3_exp(meas, Rm);
  transpose3(Ri, RiT);
  transpose3(Rm, RmT);
  matmul3(RiT, Rj, A);
  matmul3(RmT, A, E);
  porc_so3_log(E, r);
  double d[3] = {pj[3] - pi[3], pj[4] - pi[4], pj[5] - pi[5]};
  double u[3];
  for (int a = 0; a < 3; a++) {
    u[a] = RiT[3 * a] * d[0] + RiT[3 * a + 1] * d[1] + RiT[3 * a + 2] * d[2];
    r[3 + a] = u[a] - meas[3 + a];
  }
  double Jr[9], RjT[9], B[9], C[9];
  so3_jr_inv(r, Jr);
  transpose3(Rj, RjT);
  matmul3(RjT, Ri, B);
  matmul3(Jr, B, C);
  for (int k = 0; k < 36; k++) Ji[k] = Jj[k] = 0.0;
  const double ux[9] = {0.0, -u[2], u[1], u[2], 0.0, -u[0], -u[1], u[0], 0.0};
  for (int a = 0; a < 3; a++)
    for (int b = 0; b < 3; b++) {
      Ji[6 * a + b] = -C[3 * a + b];
      Jj[6 * a + b] = Jr[3 * a + b];
      Ji[6 * (3 + a) + b] = ux[3 * a + b];
      Ji[6 * (3 + a) + 3 + b] = -RiT[3 * a + b];
      Jj[6 * (3 + a) + 3 + b] = RiT[3 * a + b];
    }
}

void porc_retract(const double* pose, const double* xi, double* out) {
  double R[9], D[9], Rn[9];
  porc_so3_exp(pose, R);
  porc_so3_exp(xi, D);
  matmul3(R, D, Rn);
  porc_so3_log(Rn, out);
  for (int a = 0; a < 3; a++) out[3 + a] = pose[3 + a] + xi[3 + a];
}

static double edge_cost(const porc_problem* h, const double* poses, int64_t e) {
  double r[6], Ji[36], Jj[36];
  const int32_t i = h->edges[2 * e], j = h->edges[2 * e + 1];
  porc_edge(poses + 6 * i, poses + 6 * j, h->meas + 6 * e, r, Ji, Jj);
  const double wR = h->info[2 * e], wt = h->info[2 * e + 1];
  return 0.5 * (wR * (r[0] * r[0] + r[1] * r[1] + r[2] * r[2]) +
                wt * (r[3] * r[3] + r[4] * r[4] + r[5] * r[5]));
}

int porc_cost_at(const porc_problem* h, const double* poses, double* cost) {
  double c = 0.0;
  for (int64_t e = 0; e < h->m; e++) c += edge_cost(h, poses, e);
  *cost = c;
  return 0;
}

/* ------------------------------------------------------------ set-up --- */

int porc_opts_default(porc_opts* o) {
  if (!o) return -1;
  o->lambda0 = 1e-3;
  o->lambda_up = 10.0;
  o->lambda_down = 10.0;
  o->lambda_min = 1e-16;
  o->lambda_max = 1e16;
  o->diag_floor = 1e-6;
  o->pcg_max_iters = 200;
  o->pcg_rel_tol = 1e-8;
  o->solver = 0;
  return 0;
}

int porc_create(const double* poses, int64_t n, const int32_t* edges, const double* meas,
                const double* info, int64_t m, int n_fixed, const porc_opts* opts,
                porc_problem** out) {
  *out = NULL;
  if (n <= 0 || m < 0 || n_fixed < 0 || n_fixed > n) return -1;
  for (int64_t e = 0; e < m; e++)
    if (edges[2 * e] < 0 || edges[2 * e] >= n || edges[2 * e + 1] < 0 || edges[2 * e + 1] >= n ||
        edges[2 * e] == edges[2 * e + 1])
      return -1;
  porc_problem* h = (porc_problem*)calloc(1, sizeof(porc_problem));
  h->n = n;
  h->m = m;
  h->n_fixed = n_fixed;
  if (opts) h->opt = *opts;
  else porc_opts_default(&h->opt);
  const size_t m1 = (size_t)(m > 0 ? m : 1);
  h->poses = (double*)malloc(sizeof(double) * 6 * n);
  h->trial = (double*)malloc(sizeof(double) * 6 * n);
  h->edges = (int32_t*)malloc(sizeof(int32_t) * 2 * m1);
  h->meas = (double*)malloc(sizeof(double) * 6 * m1);
  h->info = (double*)malloc(sizeof(double) * 2 * m1);
  h->r = (double*)malloc(sizeof(double) * 6 * m1);
  h->Ji = (double*)malloc(sizeof(double) * 36 * m1);
  h->Jj = (double*)malloc(sizeof(double) * 36 * m1);
  h->Ho = (double*)malloc(sizeof(double) * 36 * m1);
  h->Hd = (double*)malloc(sizeof(double) * 36 * n);
  h->g = (double*)malloc(sizeof(double) * 6 * n);
  h->dx = (double*)calloc(6 * n, sizeof(double));
  memcpy(h->poses, poses, sizeof(double) * 6 * n);
  if (m) {
    memcpy(h->edges, edges, sizeof(int32_t) * 2 * m);
    memcpy(h->meas, meas, sizeof(double) * 6 * m);
    memcpy(h->info, info, sizeof(double) * 2 * m);
  }
  h->lambda = h->opt.lambda0;
  porc_cost_at(h, h->poses, &h->cost);
  *out = h;
  return 0;
}

void porc_destroy(porc_problem* h) {
  if (!h) return;
  free(h->poses);
  free(h->trial);
  free(h->edges);
  free(h->meas);
  free(h->info);
  free(h->r);
  free(h->Ji);
  free(h->Jj);
  free(h->Ho);
  free(h->Hd);
  free(h->g);
  free(h->dx);
  free(h);
}

int64_t porc_array_size(const porc_problem* h, int which) {
  switch (which) {
    case PORC_POSES: case PORC_G: case PORC_DX: return 6 * h->n;
    case PORC_R: return 6 * h->m;
    case PORC_JI: case PORC_JJ: case PORC_HO: return 36 * h->m;
    case PORC_HD: return 36 * h->n;
    default: return -1;
  }
}

int porc_get(const porc_problem* h, int which, double* out) {
  const double* src = NULL;
  switch (which) {
    case PORC_POSES: src = h->poses; break;
    case PORC_R: src = h->r; break;
    case PORC_JI: src = h->Ji; break;
    case PORC_JJ: src = h->Jj; break;
    case PORC_HD: src = h->Hd; break;
    case PORC_HO: src = h->Ho; break;
    case PORC_G: src = h->g; break;
    case PORC_DX: src = h->dx; break;
    default: return -1;
  }
  memcpy(out, src, sizeof(double) * (size_t)porc_array_size(h, which));
  return 0;
}

double porc_get_lambda(const porc_problem* h) { return h->lambda; }
void porc_set_lambda(porc_problem* h, double lam) { h->lambda = lam; }
double porc_get_cost(const porc_problem* h) { return h->cost; }

/* ------------------------------------------------------- linearise --- */

/* H = sum_e J^T Omega J as diagonal 6x6 blocks per pose and one off-diagonal
 * block H_ij = Ji^T Omega Jj per edge; g = sum_e J^T Omega r ([THESEUS]
 * normal equations of 1/2 sum |w c|^2). */
int porc_linearize(porc_problem* h) {
  memset(h->Hd, 0, sizeof(double) * 36 * h->n);
  memset(h->g, 0, sizeof(double) * 6 * h->n);
  for (int64_t e = 0; e < h->m; e++) {
    const int32_t i = h->edges[2 * e], j = h->edges[2 * e + 1];
    double* r = h->r + 6 * e;
    double* Ji = h->Ji + 36 * e;
    double* Jj = h->Jj + 36 * e;
    porc_edge(h->poses + 6 * i, h->poses + 6 * j, h->meas + 6 * e, r, Ji, Jj);
    double om[6];
    for (int a = 0; a < 3; a++) {
      om[a] = h->info[2 * e];
      om[3 + a] = h->info[2 * e + 1];
    }
    for (int a = 0; a < 6; a++) {
      for (int b = 0; b < 6; b++) {
        double sii = 0.0, sjj = 0.0, sij = 0.0;
        for (int k = 0; k < 6; k++) {
          sii += Ji[6 * k + a] * om[k] * Ji[6 * k + b];
          sjj += Jj[6 * k + a] * om[k] * Jj[6 * k + b];
          sij += Ji[6 * k + a] * om[k] * Jj[6 * k + b];
        }
        h->Hd[36 * i + 6 * a + b] += sii;
        h->Hd[36 * j + 6 * a + b] += sjj;
        h->Ho[36 * e + 6 * a + b] = sij;
      }
      double gi = 0.0, gj = 0.0;
      for (int k = 0; k < 6; k++) {
        gi += Ji[6 * k + a] * om[k] * r[k];
        gj += Jj[6 * k + a] * om[k] * r[k];
      }
      h->g[6 * i + a] += gi;
      h->g[6 * j + a] += gj;
    }
  }
  h->linearized = 1;
  return 0;
}

/* --------------------------------------------------------------- solve --- */

/* y = H~ x for the free poses (held poses: identity rows, x = 0 there). */
static void matvec(const porc_problem* h, const double* Hdd, const double* x, double* y) {
  const int64_t n = h->n;
  for (int64_t i = 0; i < n; i++)
    for (int a = 0; a < 6; a++) {
      double s = 0.0;
      for (int b = 0; b < 6; b++) s += Hdd[36 * i + 6 * a + b] * x[6 * i + b];
      y[6 * i + a] = s;
    }
  for (int64_t e = 0; e < h->m; e++) {
    const int32_t i = h->edges[2 * e], j = h->edges[2 * e + 1];
    if (i < h->n_fixed || j < h->n_fixed) continue;
    const double* Hij = h->Ho + 36 * e;
    for (int a = 0; a < 6; a++)
      for (int b = 0; b < 6; b++) {
        y[6 * i + a] += Hij[6 * a + b] * x[6 * j + b];
        y[6 * j + b] += Hij[6 * a + b] * x[6 * i + a];
      }
  }
}

static int chol(double* A, int n) {
  for (int j = 0; j < n; j++) {
    double d = A[j * n + j];
    for (int k = 0; k < j; k++) d -= A[j * n + k] * A[j * n + k];
    if (!(d > 0.0)) return -3;
    d = sqrt(d);
    A[j * n + j] = d;
    for (int i = j + 1; i < n; i++) {
      double s = A[i * n + j];
      for (int k = 0; k < j; k++) s -= A[i * n + k] * A[j * n + k];
      A[i * n + j] = s / d;
    }
  }
  return 0;
}

static void chol_solve(const double* L, int n, const double* b, double* x) {
  for (int i = 0; i < n; i++) {
    double s = b[i];
    for (int k = 0; k < i; k++) s -= L[i * n + k] * x[k];
    x[i] = s / L[i * n + i];
  }
  for (int i = n - 1; i >= 0; i--) {
    double s = x[i];
    for (int k = i + 1; k < n; k++) s -= L[k * n + i] * x[k];
    x[i] = s / L[i * n + i];
  }
}

/* Damped step H~ dx = -g: Marquardt damping H~ = H + lambda diag(max(diag H,
 * floor)) on the free poses, the held poses' rows and columns replaced by the
 * identity (their step is 0).  Solver: dense Cholesky of H~, or PCG from 0
 * with the 6x6 diagonal blocks of H~ as the preconditioner, stopping when
 * |r| <= tol |b| or at the iteration limit, or when p^T H~ p is not positive. */
int porc_solve_step(porc_problem* h, int* iters_out, double* rel_out) {
  const int64_t n = h->n, N = 6 * n;
  double* Hdd = (double*)malloc(sizeof(double) * 36 * n);
  double* b = (double*)malloc(sizeof(double) * N);
  memcpy(Hdd, h->Hd, sizeof(double) * 36 * n);
  for (int64_t i = 0; i < n; i++)
    for (int a = 0; a < 6; a++) {
      double* d = Hdd + 36 * i + 7 * a;
      *d += h->lambda * fmax(*d, h->opt.diag_floor);
      b[6 * i + a] = -h->g[6 * i + a];
    }
  for (int64_t i = 0; i < h->n_fixed; i++) {
    for (int k = 0; k < 36; k++) Hdd[36 * i + k] = (k % 7 == 0) ? 1.0 : 0.0;
    for (int a = 0; a < 6; a++) b[6 * i + a] = 0.0;
  }
  int rc = 0, iters = 0;
  double rel = 0.0;
  if (h->opt.solver == 1) {
    double* A = (double*)calloc((size_t)(N * N), sizeof(double));
    for (int64_t i = 0; i < n; i++)
      for (int a = 0; a < 6; a++)
        for (int c = 0; c < 6; c++) A[(6 * i + a) * N + 6 * i + c] = Hdd[36 * i + 6 * a + c];
    for (int64_t e = 0; e < h->m; e++) {
      const int32_t i = h->edges[2 * e], j = h->edges[2 * e + 1];
      if (i < h->n_fixed || j < h->n_fixed) continue;
      for (int a = 0; a < 6; a++)
        for (int c = 0; c < 6; c++) {
          A[(6 * i + a) * N + 6 * j + c] += h->Ho[36 * e + 6 * a + c];
          A[(6 * j + c) * N + 6 * i + a] += h->Ho[36 * e + 6 * a + c];
        }
    }
    rc = chol(A, (int)N);
    if (!rc) chol_solve(A, (int)N, b, h->dx);
    free(A);
  } else {
    double* Minv = (double*)malloc(sizeof(double) * 36 * n);
    for (int64_t i = 0; i < n && !rc; i++) {
      double L[36];
      memcpy(L, Hdd + 36 * i, sizeof(L));
      rc = chol(L, 6);
      for (int c = 0; c < 6 && !rc; c++) {
        double e[6] = {0, 0, 0, 0, 0, 0}, col[6];
        e[c] = 1.0;
        chol_solve(L, 6, e, col);
        for (int a = 0; a < 6; a++) Minv[36 * i + 6 * a + c] = col[a];
      }
    }
    double *x = h->dx, *r = (double*)malloc(sizeof(double) * N), *z = (double*)malloc(sizeof(double) * N),
           *p = (double*)malloc(sizeof(double) * N), *q = (double*)malloc(sizeof(double) * N);
    double bn = 0.0;
    for (int64_t k = 0; k < N; k++) {
      x[k] = 0.0;
      r[k] = b[k];
      bn += b[k] * b[k];
    }
    bn = sqrt(bn);
    for (int64_t i = 0; i < n; i++)
      for (int a = 0; a < 6; a++) {
        double s = 0.0;
        for (int c = 0; c < 6; c++) s += Minv[36 * i + 6 * a + c] * r[6 * i + c];
        z[6 * i + a] = s;
      }
    double rz = 0.0;
    for (int64_t k = 0; k < N; k++) {
      p[k] = z[k];
      rz += r[k] * z[k];
    }
    double rn = bn;
    while (!rc && bn > 0.0 && iters < h->opt.pcg_max_iters) {
      if (iters >= 1 && rn <= h->opt.pcg_rel_tol * bn) break;
      matvec(h, Hdd, p, q);
      double pq = 0.0;
      for (int64_t k = 0; k < N; k++) pq += p[k] * q[k];
      if (!(pq > 0.0)) break;
      const double alpha = rz / pq;
      rn = 0.0;
      for (int64_t k = 0; k < N; k++) {
        x[k] += alpha * p[k];
        r[k] -= alpha * q[k];
        rn += r[k] * r[k];
      }
      rn = sqrt(rn);
      for (int64_t i = 0; i < n; i++)
        for (int a = 0; a < 6; a++) {
          double s = 0.0;
          for (int c = 0; c < 6; c++) s += Minv[36 * i + 6 * a + c] * r[6 * i + c];
          z[6 * i + a] = s;
        }
      double rz_new = 0.0;
      for (int64_t k = 0; k < N; k++) rz_new += r[k] * z[k];
      const double beta = rz_new / rz;
      rz = rz_new;
      for (int64_t k = 0; k < N; k++) p[k] = z[k] + beta * p[k];
      iters++;
    }
    rel = bn > 0.0 ? rn / bn : 0.0;
    free(Minv);
    free(r);
    free(z);
    free(p);
    free(q);
  }
  free(Hdd);
  free(b);
  if (iters_out) *iters_out = iters;
  if (rel_out) *rel_out = rel;
  return rc;
}

/* One LM iteration: linearise (skipped after a rejected step), damped step,
 * retraction of every free pose, trial cost, accept iff strictly lower. */
int porc_lm_step(porc_problem* h, porc_step_info* info) {
  int rc;
  if (!h->linearized && (rc = porc_linearize(h))) return rc;
  int iters = 0;
  double rel = 0.0;
  if ((rc = porc_solve_step(h, &iters, &rel))) return rc;
  for (int64_t i = 0; i < h->n; i++) {
    if (i < h->n_fixed) memcpy(h->trial + 6 * i, h->poses + 6 * i, sizeof(double) * 6);
    else porc_retract(h->poses + 6 * i, h->dx + 6 * i, h->trial + 6 * i);
  }
  double trial;
  porc_cost_at(h, h->trial, &trial);
  porc_step_info inf;
  inf.cost_before = h->cost;
  inf.cost_after = trial;
  inf.lambda = h->lambda;
  inf.pcg_iters = iters;
  inf.pcg_rel_res = rel;
  if (isfinite(trial) && trial < h->cost) {
    inf.accepted = 1;
    memcpy(h->poses, h->trial, sizeof(double) * 6 * h->n);
    h->cost = trial;
    h->linearized = 0;
    h->lambda = fmax(h->lambda / h->opt.lambda_down, h->opt.lambda_min);
  } else {
    inf.accepted = 0;
    h->lambda = fmin(h->lambda * h->opt.lambda_up, h->opt.lambda_max);
  }
  if (info) *info = inf;
  return 0;
}

int porc_solve(porc_problem* h, int n_iters, porc_step_info* infos) {
  for (int it = 0; it < n_iters; it++) {
    int rc = porc_lm_step(h, infos ? infos + it : NULL);
    if (rc) return rc;
  }
  return 0;
}
