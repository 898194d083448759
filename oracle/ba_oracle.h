/* CPU oracle for one Levenberg-Marquardt iteration of bundle adjustment (fp64).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the CPU
 * baseline leg of the benchmark load this code; the GPU library never does and
 * shares no code with it.
 *
 * Problem: cameras x_c (9 parameters: axis-angle w, translation t, focal f,
 * radial k1, k2), points X (3), observations k = (cam(k), pt(k), uv_k).
 * Cost C = sum_k rho(|r_k|), r_k = predicted pixel - observed pixel
 * ("Bundle Adjustment in the Eager Mode" summary page: reprojection error of 3-D
 * points against image observations; Theseus note, "Method and architecture":
 * S(theta) = 1/2 sum |w_i c_i|^2).
 *
 * Sources for each step are cited beside the functions in ba_oracle.c.
 */
#ifndef BA_ORACLE_H
#define BA_ORACLE_H
#include <stdint.h>

typedef struct {
  int loss;            /* 0 squared, 1 Huber on the 2-D residual norm          */
  double huber_delta;  /* pixels                                               */
  double lambda0, lambda_up, lambda_down, lambda_min, lambda_max;
  double diag_floor;   /* floor on diag(J^T W J) used for the damping diagonal */
  int pcg_max_iters;
  double pcg_rel_tol;
  int solver;          /* 0 Schur + PCG, 1 Schur + dense Cholesky of S          */
  int strategy;        /* 0 Levenberg-Marquardt, 1 dogleg trust region          */
  double dl_radius0;   /* dogleg: initial trust radius                          */
  double dl_gn_damping;/* dogleg: Marquardt damping of its Gauss-Newton step     */
} orc_opts;

typedef struct {
  double cost_before, cost_after, lambda, pcg_rel_res;
  int accepted, pcg_iters;
  /* dogleg only: trust radius used, gain ratio, |h|, 0 Gauss-Newton step,
   * 1 steepest-descent step cut at the radius, 2 blend */
  double radius, gain_ratio, step_norm;
  int step_kind;
} orc_step_info;

typedef struct orc_problem orc_problem;

enum {
  ORC_OK = 0, ORC_ERR_ARG = -1, ORC_ERR_NONFINITE = -2, ORC_ERR_NOT_SPD = -3, ORC_ERR_ALLOC = -4
};

/* Array ids for orc_get / orc_set (sizes in elements in the comment). */
enum {
  ORC_CAMS = 0,      /* nc*9  current cameras                           */
  ORC_PTS,           /* np*3  current points                            */
  ORC_PERM_PT,       /* nobs int32: observations sorted by (pt, cam, k) */
  ORC_PERM_CAM,      /* nobs int32: observations sorted by (cam, pt, k) */
  ORC_PT_PTR,        /* np+1 int32                                      */
  ORC_CAM_PTR,       /* nc+1 int32                                      */
  ORC_R,             /* nobs*2 residual (unweighted), original order    */
  ORC_JC,            /* nobs*18 camera Jacobian, row-major 2x9          */
  ORC_JP,            /* nobs*6 point Jacobian, row-major 2x3            */
  ORC_W,             /* nobs robust weight                              */
  ORC_RHO,           /* nobs robust cost                                */
  ORC_B,             /* nc*81  B_j = sum w Jc^T Jc                      */
  ORC_GC,            /* nc*9   g_c = sum w Jc^T r                       */
  ORC_C,             /* np*9   C_i = sum w Jp^T Jp                      */
  ORC_GP,            /* np*3   g_p = sum w Jp^T r                       */
  ORC_BD,            /* nc*81  damped B                                 */
  ORC_CINV,          /* np*9   inverse of the damped C_i                */
  ORC_V,             /* np*3   Cinv g_p                                 */
  ORC_RHS,           /* nc*9   reduced right-hand side                  */
  ORC_M,             /* nc*81  exact diagonal blocks S_jj               */
  ORC_DC,            /* nc*9   camera update                            */
  ORC_DP,            /* np*3   point update                             */
  ORC_CAMS_TRIAL,    /* nc*9                                            */
  ORC_PTS_TRIAL,     /* np*3                                            */
  ORC_NUM_ARRAYS
};

int orc_opts_default(orc_opts* o);
int orc_create(const double* cams, int64_t nc, const double* pts, int64_t np,
               const int32_t* cam_idx, const int32_t* pt_idx, const double* uv, int64_t nobs,
               const orc_opts* opts, orc_problem** out);
void orc_destroy(orc_problem* h);
int64_t orc_array_size(const orc_problem* h, int which);
int orc_get(const orc_problem* h, int which, void* out);
int orc_set(orc_problem* h, int which, const void* in);

int orc_linearize(orc_problem* h);
int orc_damp(orc_problem* h);
int orc_schur(orc_problem* h);
int orc_pcg(orc_problem* h, int max_iters, double rel_tol, int* iters, double* rel_res);
int orc_dense_schur_solve(orc_problem* h);
/* Camera marginal covariance: the 9x9 diagonal blocks of S~^-1 at the current
 * parameters and lambda (out: nc x 81). */
int orc_covariance(orc_problem* h, double* out);
int orc_backsub(orc_problem* h);
int orc_retract(orc_problem* h);
int orc_cost_at(const orc_problem* h, const double* cams, const double* pts, double* cost);
int orc_lm_step(orc_problem* h, orc_step_info* info);
/* One dogleg iteration (orc_lm_step calls it when opts.strategy is 1). */
int orc_dogleg_step(orc_problem* h, orc_step_info* info);
double orc_get_radius(const orc_problem* h);
void orc_set_radius(orc_problem* h, double radius);
int orc_solve(orc_problem* h, int n_iters, orc_step_info* infos);
/* df/du (nobs x 2) for a loss f of the LM solution with gradient
 * (grad_cams, grad_pts), by implicit differentiation of one damped
 * Gauss-Newton step at the current parameters and lambda. */
int orc_backward(orc_problem* h, const double* grad_cams, const double* grad_pts, double* out_uv,
                 int* iters, double* rel_res);

double orc_get_lambda(const orc_problem* h);
void orc_set_lambda(orc_problem* h, double lam);
double orc_get_cost(const orc_problem* h);

int orc_schur_matvec(orc_problem* h, const double* x, double* out);
int orc_explicit_S(orc_problem* h, double* S);

int orc_project_one(const double* cam, const double* X, const double* uv, int loss, double delta,
                    double* r, double* Jc, double* Jp, double* w, double* rho);
int orc_retract_camera(const double* cam, const double* delta, double* out);
void orc_so3_exp(const double* w, double* R);
/* Threads the oracle's loops run on: 1 for the plain build, OpenMP's maximum
 * for the -fopenmp build. */
int orc_num_threads(void);

#endif
