/* CPU oracle for dense frame-graph bundle adjustment (fp64) — TEST
 * INFRASTRUCTURE ONLY; shares no code with the GPU library.
 *
 * Pages cited (by title and section):
 *  [NSLAM] NeRF-SLAM reproduction notes: sec. 2.2 (backproject a pixel with its
 *          inverse depth, the ray divided by the inverse depth clamped at
 *          1e-6; transform by the relative pose T_ij; project with the depth
 *          clamped at 1e-6; the update operator predicts a target and a
 *          confidence weight per pixel), sec. 2.3 (frame graph: frames are
 *          nodes, edges carry dense correspondences), sec. 3.1 (H = J^T W J,
 *          b = -J^T W r; 6x6 pose blocks B, 1x1 inverse-depth blocks C, sparse
 *          coupling E), sec. 3.2 (Schur complement, eqs. (1) and (2); S solved
 *          by Cholesky, never inverted).
 *  [THESEUS] Theseus note, "Method and architecture" (Gauss-Newton, Lie-group
 *          variables with a retraction).
 *
 * Readings where the pages are silent: poses are world-to-camera; the
 * perturbation is on the left, T <- Exp(xi) T with xi = (rho, phi),
 * translation part first; the first n_fixed poses are held fixed (gauge);
 * each weight multiplies the squared residual (cost 1/2 sum w |r|^2, W of
 * sec. 3.1); Gauss-Newton without damping, every step applied.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

typedef struct {
  int n, H, W, E, nf;
  int64_t P;          /* pixels per frame */
  double fx, fy, cx, cy;
  double *R, *t;      /* n x 9, n x 3 */
  double *d;          /* n x P inverse depths */
  int *ei, *ej;       /* E */
  double *tgt, *w;    /* E x P x 2, E x P */
  /* last linearisation / step */
  double *r, *Ji, *Jj, *Jd;   /* E x P x 2, x12, x12, x2 */
  double *B, *gc;             /* (6n)^2, 6n */
  double *C, *gd;             /* n x P */
  double *S, *rhs;            /* (6(n-nf))^2, 6(n-nf) */
  double *dxi, *dd;           /* 6n, n x P */
} dorc;

enum { DORC_R = 0, DORC_JI, DORC_JJ, DORC_JD, DORC_B, DORC_GC, DORC_C, DORC_GD, DORC_S,
       DORC_RHS, DORC_DXI, DORC_DD, DORC_POSES, DORC_DEPTH };

/* ------------------------------------------------------------ SO(3), SE(3) */

static void quat_to_R(const double* q /* x y z w */, double* R) {
  double x = q[0], y = q[1], z = q[2], w = q[3];
  double n = sqrt(x * x + y * y + z * z + w * w);
  x /= n; y /= n; z /= n; w /= n;
  R[0] = 1 - 2 * (y * y + z * z); R[1] = 2 * (x * y - w * z);     R[2] = 2 * (x * z + w * y);
  R[3] = 2 * (x * y + w * z);     R[4] = 1 - 2 * (x * x + z * z); R[5] = 2 * (y * z - w * x);
  R[6] = 2 * (x * z - w * y);     R[7] = 2 * (y * z + w * x);     R[8] = 1 - 2 * (x * x + y * y);
}

/* Quaternion (x y z w, w >= 0) of a rotation matrix (Shepperd's method). */
static void R_to_quat(const double* R, double* q) {
  double tr = R[0] + R[4] + R[8];
  double x, y, z, w;
  if (tr > 0) {
    double s = 2 * sqrt(tr + 1.0);
    w = 0.25 * s; x = (R[7] - R[5]) / s; y = (R[2] - R[6]) / s; z = (R[3] - R[1]) / s;
  } else if (R[0] > R[4] && R[0] > R[8]) {
    double s = 2 * sqrt(1.0 + R[0] - R[4] - R[8]);
    w = (R[7] - R[5]) / s; x = 0.25 * s; y = (R[1] + R[3]) / s; z = (R[2] + R[6]) / s;
  } else if (R[4] > R[8]) {
    double s = 2 * sqrt(1.0 + R[4] - R[0] - R[8]);
    w = (R[2] - R[6]) / s; x = (R[1] + R[3]) / s; y = 0.25 * s; z = (R[5] + R[7]) / s;
  } else {
    double s = 2 * sqrt(1.0 + R[8] - R[0] - R[4]);
    w = (R[3] - R[1]) / s; x = (R[2] + R[6]) / s; y = (R[5] + R[7]) / s; z = 0.25 * s;
  }
  if (w < 0) { x = -x; y = -y; z = -z; w = -w; }
  q[0] = x; q[1] = y; q[2] = z; q[3] = w;
}

/* SE(3) exponential of xi = (rho, phi): rotation by Rodrigues, translation
 * V rho with V = I + (1 - cos a)/a^2 [phi]x + (a - sin a)/a^3 [phi]x^2. */
static void se3_exp(const double* xi, double* R, double* t) {
  const double* rho = xi;
  const double* ph = xi + 3;
  double a2 = ph[0] * ph[0] + ph[1] * ph[1] + ph[2] * ph[2], a = sqrt(a2);
  double A, Bc, Cc;
  if (a < 1e-2) {  /* Taylor series, truncation below 1e-21 */
    A = 1.0 - a2 / 6.0 * (1.0 - a2 / 20.0 * (1.0 - a2 / 42.0));
    Bc = 0.5 - a2 / 24.0 * (1.0 - a2 / 30.0 * (1.0 - a2 / 56.0));
    Cc = 1.0 / 6.0 - a2 / 120.0 * (1.0 - a2 / 42.0 * (1.0 - a2 / 72.0));
  } else {
    double h = sin(0.5 * a);
    A = sin(a) / a;
    Bc = 2.0 * h * h / a2;
    Cc = (a - sin(a)) / (a2 * a);
  }
  double K[9] = {0, -ph[2], ph[1], ph[2], 0, -ph[0], -ph[1], ph[0], 0}, K2[9];
  for (int i = 0; i < 3; i++)
    for (int j = 0; j < 3; j++) {
      double s = 0;
      for (int l = 0; l < 3; l++) s += K[3 * i + l] * K[3 * l + j];
      K2[3 * i + j] = s;
    }
  double V[9];
  for (int i = 0; i < 9; i++) {
    R[i] = A * K[i] + Bc * K2[i];
    V[i] = Bc * K[i] + Cc * K2[i];
  }
  R[0] += 1; R[4] += 1; R[8] += 1;
  V[0] += 1; V[4] += 1; V[8] += 1;
  for (int i = 0; i < 3; i++) t[i] = V[3 * i] * rho[0] + V[3 * i + 1] * rho[1] + V[3 * i + 2] * rho[2];
}

/* --------------------------------------------------------- one residual -- */

/* Residual of pixel (x, y) of frame i, inverse depth d, in frame j, with its
 * Jacobians for the left perturbations of T_i and T_j and for d.
 * [NSLAM] sec. 2.2: X_i = K^-1 [x, y, 1]^T / max(d, 1e-6);
 * X_j = T_j T_i^-1 X_i; p = (fx X/Z + cx, fy Y/Z + cy), Z = max(X_j.z, 1e-6).
 * Derivatives: dX_j/dxi_j = [I | -[X_j]x], dX_j/dxi_i = R_j R_i^T [-I | [X_i]x],
 * dX_j/dd = -R_j R_i^T ray / d^2 (zero when the clamp is active).
 * Returns 1 if a clamp was active. */
int dorc_residual_one(const double* Ti /* R(9) t(3) */, const double* Tj, const double* K,
                      const double* xy, double d, const double* target, double* r,
                      double* Ji, double* Jj, double* Jd) {
  const double *Ri = Ti, *ti = Ti + 9, *Rj = Tj, *tj = Tj + 9;
  double fx = K[0], fy = K[1], cx = K[2], cy = K[3];
  double ray[3] = {(xy[0] - cx) / fx, (xy[1] - cy) / fy, 1.0};
  int dcl = d < 1e-6;
  double dc = dcl ? 1e-6 : d;
  double Xi[3] = {ray[0] / dc, ray[1] / dc, ray[2] / dc};
  double Xw[3], Xj[3], Rij[9];
  for (int a = 0; a < 3; a++)
    Xw[a] = Ri[a] * (Xi[0] - ti[0]) + Ri[3 + a] * (Xi[1] - ti[1]) + Ri[6 + a] * (Xi[2] - ti[2]);
  for (int a = 0; a < 3; a++) Xj[a] = Rj[3 * a] * Xw[0] + Rj[3 * a + 1] * Xw[1] + Rj[3 * a + 2] * Xw[2] + tj[a];
  for (int a = 0; a < 3; a++)
    for (int b = 0; b < 3; b++)
      Rij[3 * a + b] = Rj[3 * a] * Ri[3 * b] + Rj[3 * a + 1] * Ri[3 * b + 1] + Rj[3 * a + 2] * Ri[3 * b + 2];
  int zcl = Xj[2] < 1e-6;
  double Z = zcl ? 1e-6 : Xj[2];
  r[0] = fx * Xj[0] / Z + cx - target[0];
  r[1] = fy * Xj[1] / Z + cy - target[1];
  double P[6] = {fx / Z, 0, zcl ? 0 : -fx * Xj[0] / (Z * Z), 0, fy / Z, zcl ? 0 : -fy * Xj[1] / (Z * Z)};
  double Mj[18] = {1, 0, 0, 0, Xj[2], -Xj[1], 0, 1, 0, -Xj[2], 0, Xj[0], 0, 0, 1, Xj[1], -Xj[0], 0};
  double Mi0[18] = {-1, 0, 0, 0, -Xi[2], Xi[1], 0, -1, 0, Xi[2], 0, -Xi[0], 0, 0, -1, -Xi[1], Xi[0], 0};
  double Mi[18];
  for (int a = 0; a < 3; a++)
    for (int c = 0; c < 6; c++)
      Mi[6 * a + c] = Rij[3 * a] * Mi0[c] + Rij[3 * a + 1] * Mi0[6 + c] + Rij[3 * a + 2] * Mi0[12 + c];
  double dXd[3];
  for (int a = 0; a < 3; a++)
    dXd[a] = dcl ? 0.0 : -(Rij[3 * a] * ray[0] + Rij[3 * a + 1] * ray[1] + Rij[3 * a + 2] * ray[2]) / (dc * dc);
  for (int row = 0; row < 2; row++) {
    for (int c = 0; c < 6; c++) {
      Ji[6 * row + c] = P[3 * row] * Mi[c] + P[3 * row + 1] * Mi[6 + c] + P[3 * row + 2] * Mi[12 + c];
      Jj[6 * row + c] = P[3 * row] * Mj[c] + P[3 * row + 1] * Mj[6 + c] + P[3 * row + 2] * Mj[12 + c];
    }
    Jd[row] = P[3 * row] * dXd[0] + P[3 * row + 1] * dXd[1] + P[3 * row + 2] * dXd[2];
  }
  return dcl || zcl;
}

/* ------------------------------------------------------------ lifecycle -- */

void dorc_destroy(dorc* h) {
  if (!h) return;
  void* b[] = {h->R, h->t, h->d, h->ei, h->ej, h->tgt, h->w, h->r, h->Ji, h->Jj, h->Jd,
               h->B, h->gc, h->C, h->gd, h->S, h->rhs, h->dxi, h->dd};
  for (size_t i = 0; i < sizeof(b) / sizeof(b[0]); i++) free(b[i]);
  free(h);
}

int dorc_create(const float* poses /* n x 7: t(3) q(4, x y z w) */, const float* depth, int n,
                int H, int W, const float* K, const int32_t* edges /* E x 2 */, int E,
                const float* targets /* E x HW x 2 */, const float* weights, int n_fixed,
                dorc** out) {
  if (!out || n <= 0 || H <= 0 || W <= 0 || E < 0 || n_fixed < 0 || n_fixed > n) return -1;
  dorc* h = (dorc*)calloc(1, sizeof(dorc));
  h->n = n; h->H = H; h->W = W; h->E = E; h->nf = n_fixed;
  h->P = (int64_t)H * W;
  h->fx = K[0]; h->fy = K[1]; h->cx = K[2]; h->cy = K[3];
  int64_t P = h->P, nv = 6 * (int64_t)(n - n_fixed), E1 = E > 0 ? E : 1;
  h->R = calloc(9 * n, 8); h->t = calloc(3 * n, 8); h->d = calloc(n * P, 8);
  h->ei = calloc(E1, 4); h->ej = calloc(E1, 4);
  h->tgt = calloc(E1 * P * 2, 8); h->w = calloc(E1 * P, 8);
  h->r = calloc(E1 * P * 2, 8); h->Ji = calloc(E1 * P * 12, 8); h->Jj = calloc(E1 * P * 12, 8);
  h->Jd = calloc(E1 * P * 2, 8);
  h->B = calloc(36 * (int64_t)n * n, 8); h->gc = calloc(6 * n, 8);
  h->C = calloc(n * P, 8); h->gd = calloc(n * P, 8);
  h->S = calloc(nv * nv + 1, 8); h->rhs = calloc(nv + 1, 8);
  h->dxi = calloc(6 * n, 8); h->dd = calloc(n * P, 8);
  for (int i = 0; i < n; i++) {
    double q[4] = {poses[7 * i + 3], poses[7 * i + 4], poses[7 * i + 5], poses[7 * i + 6]};
    quat_to_R(q, h->R + 9 * i);
    for (int a = 0; a < 3; a++) h->t[3 * i + a] = poses[7 * i + a];
  }
  for (int64_t k = 0; k < n * P; k++) h->d[k] = depth[k];
  for (int e = 0; e < E; e++) {
    if (edges[2 * e] < 0 || edges[2 * e] >= n || edges[2 * e + 1] < 0 || edges[2 * e + 1] >= n) {
      dorc_destroy(h);
      return -1;
    }
    h->ei[e] = edges[2 * e];
    h->ej[e] = edges[2 * e + 1];
  }
  for (int64_t k = 0; k < E * P * 2; k++) h->tgt[k] = targets[k];
  for (int64_t k = 0; k < E * P; k++) h->w[k] = weights[k];
  *out = h;
  return 0;
}

static void pose_of(const dorc* h, int i, double* T) {
  memcpy(T, h->R + 9 * i, 9 * 8);
  memcpy(T + 9, h->t + 3 * i, 3 * 8);
}

/* Cost 1/2 sum w |r|^2 over all edges and pixels, in edge then pixel order. */
double dorc_cost_value(const dorc* h) {
  double K[4] = {h->fx, h->fy, h->cx, h->cy}, s = 0.0;
  for (int e = 0; e < h->E; e++) {
    double Ti[12], Tj[12];
    pose_of(h, h->ei[e], Ti);
    pose_of(h, h->ej[e], Tj);
    for (int64_t p = 0; p < h->P; p++) {
      double xy[2] = {(double)(p % h->W), (double)(p / h->W)}, r[2], Ji[12], Jj[12], Jd[2];
      dorc_residual_one(Ti, Tj, K, xy, h->d[h->ei[e] * h->P + p], h->tgt + 2 * (e * h->P + p), r,
                        Ji, Jj, Jd);
      s += 0.5 * h->w[e * h->P + p] * (r[0] * r[0] + r[1] * r[1]);
    }
  }
  return s;
}

int dorc_cost(dorc* h, double* c) {
  *c = dorc_cost_value(h);
  return isfinite(*c) ? 0 : -2;
}

static int chol(double* A, int n) {
  for (int j = 0; j < n; j++) {
    double d = A[n * j + j];
    for (int l = 0; l < j; l++) d -= A[n * j + l] * A[n * j + l];
    if (!(d > 0.0)) return -1;
    d = sqrt(d);
    A[n * j + j] = d;
    for (int i = j + 1; i < n; i++) {
      double s = A[n * i + j];
      for (int l = 0; l < j; l++) s -= A[n * i + l] * A[n * j + l];
      A[n * i + j] = s / d;
    }
  }
  return 0;
}

/* One Gauss-Newton step ([THESEUS] linearise, solve, retract) with the depths
 * eliminated by the Schur complement ([NSLAM] sec. 3.2).  The step is applied
 * unconditionally.  cost_before / cost_after may be NULL. */
/* Linearisation, B, g_c, C, g_d, and the reduced pose system S, rhs at the
 * current state (the first part of a Gauss-Newton step). */
static void dorc_assemble(dorc* h) {
  int n = h->n, nf = h->nf;
  int64_t P = h->P, N6 = 6 * (int64_t)n, nv = 6 * (int64_t)(n - nf);
  double K[4] = {h->fx, h->fy, h->cx, h->cy};
  memset(h->B, 0, 8 * N6 * N6);
  memset(h->gc, 0, 8 * N6);
  memset(h->C, 0, 8 * n * P);
  memset(h->gd, 0, 8 * n * P);
  /* linearise and assemble B, g_c, C, g_d ([NSLAM] sec. 3.1) */
  for (int e = 0; e < h->E; e++) {
    int i = h->ei[e], j = h->ej[e];
    double Ti[12], Tj[12];
    pose_of(h, i, Ti);
    pose_of(h, j, Tj);
    for (int64_t p = 0; p < P; p++) {
      int64_t k = e * P + p;
      double xy[2] = {(double)(p % h->W), (double)(p / h->W)};
      double* r = h->r + 2 * k;
      double* Ji = h->Ji + 12 * k;
      double* Jj = h->Jj + 12 * k;
      double* Jd = h->Jd + 2 * k;
      dorc_residual_one(Ti, Tj, K, xy, h->d[i * P + p], h->tgt + 2 * k, r, Ji, Jj, Jd);
      double w = h->w[k];
      for (int a = 0; a < 6; a++) {
        for (int b = 0; b < 6; b++) {
          double ii = Ji[a] * Ji[b] + Ji[6 + a] * Ji[6 + b];
          double jj = Jj[a] * Jj[b] + Jj[6 + a] * Jj[6 + b];
          double ij = Ji[a] * Jj[b] + Ji[6 + a] * Jj[6 + b];
          h->B[(6 * i + a) * N6 + 6 * i + b] += w * ii;
          h->B[(6 * j + a) * N6 + 6 * j + b] += w * jj;
          h->B[(6 * i + a) * N6 + 6 * j + b] += w * ij;
          h->B[(6 * j + b) * N6 + 6 * i + a] += w * ij;
        }
        h->gc[6 * i + a] += w * (Ji[a] * r[0] + Ji[6 + a] * r[1]);
        h->gc[6 * j + a] += w * (Jj[a] * r[0] + Jj[6 + a] * r[1]);
      }
      h->C[i * P + p] += w * (Jd[0] * Jd[0] + Jd[1] * Jd[1]);
      h->gd[i * P + p] += w * (Jd[0] * r[0] + Jd[1] * r[1]);
    }
  }
  /* Schur complement on the free poses ([NSLAM] sec. 3.2 eq. (2)):
   * S = B - E C^-1 E^T, rhs = -g_c + E C^-1 g_d, E column of depth (i, p)
   * summed over the edges leaving frame i. */
  for (int64_t a = 0; a < nv; a++) {
    for (int64_t b = 0; b < nv; b++) h->S[a * nv + b] = h->B[(6 * nf + a) * N6 + 6 * nf + b];
    h->rhs[a] = -h->gc[6 * nf + a];
  }
  double* col = (double*)calloc(N6, 8);
  for (int i = 0; i < n; i++) {
    for (int64_t p = 0; p < P; p++) {
      memset(col, 0, 8 * N6);
      for (int e = 0; e < h->E; e++) {
        if (h->ei[e] != i) continue;
        int64_t k = e * P + p;
        double w = h->w[k], *Ji = h->Ji + 12 * k, *Jj = h->Jj + 12 * k, *Jd = h->Jd + 2 * k;
        for (int a = 0; a < 6; a++) {
          col[6 * i + a] += w * (Ji[a] * Jd[0] + Ji[6 + a] * Jd[1]);
          col[6 * h->ej[e] + a] += w * (Jj[a] * Jd[0] + Jj[6 + a] * Jd[1]);
        }
      }
      double c = h->C[i * P + p];
      if (!(c > 0.0)) continue;   /* depth unobserved by any edge: no coupling */
      double v = h->gd[i * P + p] / c;
      for (int64_t a = 0; a < nv; a++) {
        double ea = col[6 * nf + a];
        if (ea == 0.0) continue;
        h->rhs[a] += ea * v;
        for (int64_t b = 0; b < nv; b++) h->S[a * nv + b] -= ea * col[6 * nf + b] / c;
      }
    }
  }
  free(col);
}

/* Pose marginal covariance, the notes' cov_cam ([NSLAM] sec. 3.2, the dense
 * reference step): S factored by Cholesky and S^-1 obtained by solving
 * against the identity, column by column (S is never inverted directly).
 * At the current state; out is nv x nv (nv = 6 free poses), row-major. */
int dorc_covariance(dorc* h, double* out) {
  dorc_assemble(h);
  const int64_t nv = 6 * (int64_t)(h->n - h->nf);
  double* L = (double*)malloc(8 * (nv * nv + 1));
  double* y = (double*)calloc(nv + 1, 8);
  memcpy(L, h->S, 8 * nv * nv);
  int rc = chol(L, (int)nv);
  for (int64_t c = 0; c < nv && rc == 0; c++) {
    for (int64_t a = 0; a < nv; a++) {
      double s = a == c ? 1.0 : 0.0;
      for (int64_t l = 0; l < a; l++) s -= L[a * nv + l] * y[l];
      y[a] = s / L[a * nv + a];
    }
    for (int64_t a = nv - 1; a >= 0; a--) {
      double s = y[a];
      for (int64_t l = a + 1; l < nv; l++) s -= L[l * nv + a] * y[l];
      y[a] = s / L[a * nv + a];
    }
    for (int64_t a = 0; a < nv; a++) out[a * nv + c] = y[a];
  }
  free(L);
  free(y);
  return rc == 0 ? 0 : -3;
}

int dorc_gn_step(dorc* h, double* cost_before, double* cost_after) {
  int n = h->n, nf = h->nf;
  int64_t P = h->P, N6 = 6 * (int64_t)n, nv = 6 * (int64_t)(n - nf);
  if (cost_before) *cost_before = dorc_cost_value(h);
  dorc_assemble(h);
  /* dense Cholesky of S and the camera step */
  double* L = (double*)malloc(8 * (nv * nv + 1));
  memcpy(L, h->S, 8 * nv * nv);
  int rc = chol(L, (int)nv);
  memset(h->dxi, 0, 8 * N6);
  if (rc == 0) {
    double* y = (double*)calloc(nv + 1, 8);
    for (int64_t a = 0; a < nv; a++) {
      double s = h->rhs[a];
      for (int64_t l = 0; l < a; l++) s -= L[a * nv + l] * y[l];
      y[a] = s / L[a * nv + a];
    }
    for (int64_t a = nv - 1; a >= 0; a--) {
      double s = y[a];
      for (int64_t l = a + 1; l < nv; l++) s -= L[l * nv + a] * y[l];
      y[a] = s / L[a * nv + a];
    }
    for (int64_t a = 0; a < nv; a++) h->dxi[6 * nf + a] = y[a];
    free(y);
  }
  free(L);
  if (rc != 0) return -3;
  /* depth back-substitution ([NSLAM] sec. 3.2 eq. (1)): dd = (-g_d - E^T dxi) / C */
  for (int i = 0; i < n; i++) {
    for (int64_t p = 0; p < P; p++) {
      double s = -h->gd[i * P + p];
      for (int e = 0; e < h->E; e++) {
        if (h->ei[e] != i) continue;
        int64_t k = e * P + p;
        double w = h->w[k], *Ji = h->Ji + 12 * k, *Jj = h->Jj + 12 * k, *Jd = h->Jd + 2 * k;
        for (int a = 0; a < 6; a++) {
          s -= w * (Ji[a] * Jd[0] + Ji[6 + a] * Jd[1]) * h->dxi[6 * i + a];
          s -= w * (Jj[a] * Jd[0] + Jj[6 + a] * Jd[1]) * h->dxi[6 * h->ej[e] + a];
        }
      }
      double c = h->C[i * P + p];
      h->dd[i * P + p] = c > 0.0 ? s / c : 0.0;
    }
  }
  /* retraction: T <- Exp(xi) T for the free poses, depths additive */
  for (int i = nf; i < n; i++) {
    double Re[9], te[3], Rn[9], tn[3];
    se3_exp(h->dxi + 6 * i, Re, te);
    double* R = h->R + 9 * i;
    double* t = h->t + 3 * i;
    for (int a = 0; a < 3; a++) {
      for (int b = 0; b < 3; b++) Rn[3 * a + b] = Re[3 * a] * R[b] + Re[3 * a + 1] * R[3 + b] + Re[3 * a + 2] * R[6 + b];
      tn[a] = Re[3 * a] * t[0] + Re[3 * a + 1] * t[1] + Re[3 * a + 2] * t[2] + te[a];
    }
    memcpy(R, Rn, 72);
    memcpy(t, tn, 24);
  }
  for (int64_t k = 0; k < n * P; k++) h->d[k] += h->dd[k];
  if (cost_after) *cost_after = dorc_cost_value(h);
  return 0;
}

int64_t dorc_size(const dorc* h, int which) {
  int64_t n = h->n, P = h->P, E = h->E, nv = 6 * (int64_t)(h->n - h->nf);
  switch (which) {
    case DORC_R: return 2 * E * P;
    case DORC_JI: case DORC_JJ: return 12 * E * P;
    case DORC_JD: return 2 * E * P;
    case DORC_B: return 36 * n * n;
    case DORC_GC: case DORC_DXI: return 6 * n;
    case DORC_C: case DORC_GD: case DORC_DD: case DORC_DEPTH: return n * P;
    case DORC_S: return nv * nv;
    case DORC_RHS: return nv;
    case DORC_POSES: return 7 * n;
    default: return -1;
  }
}

int dorc_get(const dorc* h, int which, void* out) {
  double* o = (double*)out;
  int64_t n = dorc_size(h, which);
  const double* src = NULL;
  switch (which) {
    case DORC_R: src = h->r; break;
    case DORC_JI: src = h->Ji; break;
    case DORC_JJ: src = h->Jj; break;
    case DORC_JD: src = h->Jd; break;
    case DORC_B: src = h->B; break;
    case DORC_GC: src = h->gc; break;
    case DORC_C: src = h->C; break;
    case DORC_GD: src = h->gd; break;
    case DORC_S: src = h->S; break;
    case DORC_RHS: src = h->rhs; break;
    case DORC_DXI: src = h->dxi; break;
    case DORC_DD: src = h->dd; break;
    case DORC_DEPTH: src = h->d; break;
    case DORC_POSES:
      for (int i = 0; i < h->n; i++) {
        memcpy(o + 7 * i, h->t + 3 * i, 24);
        R_to_quat(h->R + 9 * i, o + 7 * i + 3);
      }
      return 0;
    default: return -1;
  }
  memcpy(o, src, 8 * n);
  return 0;
}

/* Pose as R(9) t(3) for the residual entry point (tests). */
int dorc_pose_matrix(const dorc* h, int i, double* T) {
  if (i < 0 || i >= h->n) return -1;
  pose_of(h, i, T);
  return 0;
}

int dorc_se3_exp(const double* xi, double* R, double* t) {
  se3_exp(xi, R, t);
  return 0;
}
