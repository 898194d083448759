/* CPU oracle for pose-graph optimisation (fp64).  TEST INFRASTRUCTURE ONLY:
 * only the tests, the smoke check and the CPU-baseline leg of the benchmark
 * load it; it shares no code with the GPU library. */
#ifndef PGO_ORACLE_H
#define PGO_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  double lambda0, lambda_up, lambda_down, lambda_min, lambda_max;
  double diag_floor;   /* floor on diag(H) in the damping term          */
  int pcg_max_iters;
  double pcg_rel_tol;
  int solver;          /* 0 PCG with 6x6 block-Jacobi, 1 dense Cholesky */
} porc_opts;

typedef struct {
  double cost_before, cost_after, lambda, pcg_rel_res;
  int accepted, pcg_iters;
} porc_step_info;

typedef struct porc_problem porc_problem;

/* Array ids for porc_get. */
enum {
  PORC_POSES = 0,  /* n*6   current poses [w, t]                        */
  PORC_R,          /* m*6   residual [r_R, r_t] per edge                 */
  PORC_JI,         /* m*36  d r / d xi_i, row-major 6x6                   */
  PORC_JJ,         /* m*36  d r / d xi_j                                  */
  PORC_HD,         /* n*36  diagonal blocks of H = sum J^T Omega J        */
  PORC_HO,         /* m*36  off-diagonal block H_ij of each edge          */
  PORC_G,          /* n*6   g = sum J^T Omega r                          */
  PORC_DX,         /* n*6   step                                          */
  PORC_NUM
};

int porc_opts_default(porc_opts* o);
int porc_create(const double* poses, int64_t n, const int32_t* edges, const double* meas,
                const double* info, int64_t m, int n_fixed, const porc_opts* opts,
                porc_problem** out);
void porc_destroy(porc_problem* h);
int64_t porc_array_size(const porc_problem* h, int which);
int porc_get(const porc_problem* h, int which, double* out);
int porc_linearize(porc_problem* h);
int porc_solve_step(porc_problem* h, int* iters, double* rel_res);
int porc_cost_at(const porc_problem* h, const double* poses, double* cost);
int porc_lm_step(porc_problem* h, porc_step_info* info);
int porc_solve(porc_problem* h, int n_iters, porc_step_info* infos);
double porc_get_lambda(const porc_problem* h);
void porc_set_lambda(porc_problem* h, double lam);
double porc_get_cost(const porc_problem* h);
/* Residual and both Jacobians of one edge, for the finite-difference pins. */
void porc_edge(const double* pose_i, const double* pose_j, const double* meas, double* r,
               double* Ji, double* Jj);
/* Pose retraction x (+) xi: R <- R Exp(dphi), t <- t + dt. */
void porc_retract(const double* pose, const double* xi, double* out);
void porc_so3_log(const double* R, double* w);
void porc_so3_exp(const double* w, double* R);

#ifdef __cplusplus
}
#endif

#endif
