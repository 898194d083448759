/* libpgo: pose-graph optimisation on one MI355X (gfx950), fp64.
 *
 * A set of SE(3) poses constrained by relative-pose measurements (odometry
 * and loop closures), solved by Levenberg-Marquardt: the pose graph
 * optimisation of the eager-mode BA summary (indexing decides which two poses
 * a residual joins, Lie-group operations give the residual and its Jacobian
 * blocks, a sparse LM solves), with the manifold variables, retraction and
 * adaptive damping of the Theseus note.
 *
 * Model (the pages give no residual formula; this is the reading):
 *   pose i: [w_i (axis-angle of R_i), t_i], body to world (x_w = R_i x + t_i);
 *   edge e = (i, j) measures T_i^-1 T_j as [w_e, t_e] (R_e = Exp(w_e));
 *   residual r_e = [Log(R_e^T R_i^T R_j); R_i^T (t_j - t_i) - t_e];
 *   cost 1/2 sum_e (w_R |r_R|^2 + w_t |r_t|^2), info_e = [w_R, w_t];
 *   tangent [dphi, dt], retraction R <- R Exp(dphi), t <- t + dt;
 *   the first n_fixed poses are held (the gauge).
 * Each LM step linearises (analytic 6x6 Jacobian blocks with the inverse
 * right Jacobian of SO(3)), assembles H = sum J^T Omega J as per-pose 6x6
 * blocks and one block per edge, damps it (Marquardt, diag floored), solves
 * H~ dx = -g by PCG with the 6x6 block-Jacobi preconditioner, retracts,
 * evaluates the trial cost and accepts iff it is strictly lower (lambda / 10
 * on accept, x 10 on reject).  Reductions have a fixed order: runs are
 * bitwise reproducible.
 *
 * Errors: every function returns PGO_OK (0) or a negative code; nothing is
 * thrown across the ABI.  A rejected step is not an error.
 */
#ifndef LIBPGO_PGO_H
#define LIBPGO_PGO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  PGO_OK = 0,
  PGO_ERR_ARG = -1,       /* null pointer, bad size, edge index out of range or a self-loop */
  PGO_ERR_NONFINITE = -2, /* non-finite input or cost                                    */
  PGO_ERR_NOT_SPD = -3,   /* a damped 6x6 block failed to factor                          */
  PGO_ERR_DEVICE = -4,    /* HIP runtime error                                            */
  PGO_ERR_ALLOC = -5      /* allocation failed                                            */
};

enum { PGO_MEM_HOST = 0, PGO_MEM_DEVICE = 1 };

typedef struct {
  double lambda0;        /* initial damping (1e-3)                          */
  double lambda_up;      /* factor on a rejected step (10)                  */
  double lambda_down;    /* divisor on an accepted step (10)                */
  double lambda_min;     /* 1e-16                                           */
  double lambda_max;     /* 1e16                                            */
  double diag_floor;     /* floor on diag(H) in the damping term (1e-6)     */
  int pcg_max_iters;     /* 200                                             */
  double pcg_rel_tol;    /* stop when |r|_2 <= tol |b|_2 (1e-8)             */
  int mem;               /* PGO_MEM_HOST / PGO_MEM_DEVICE: where pgo_create's
                            inputs live                                     */
  void* stream;          /* hipStream_t or NULL                             */
} pgo_options;

typedef struct {
  double cost_before, cost_after, lambda, pcg_rel_res;
  int accepted, pcg_iters;
} pgo_step_info;

typedef struct pgo_problem pgo_problem;

/* Fills *o with the defaults above.  PGO_ERR_ARG if o is NULL. */
int pgo_options_default(pgo_options* o);

/* Copies the inputs to the device and validates them: poses n x 6 [w, t],
 * edges m x 2 int32 (i != j, both in [0, n)), meas m x 6 [w_e, t_e],
 * info m x 2 [w_R, w_t] (positive), 0 <= n_fixed <= n.  Builds the per-pose
 * lists of incident edges once.  opts may be NULL (defaults); the caller may
 * free its inputs when this returns.  On error *out is left NULL. */
int pgo_create(const double* poses, int64_t n, const int32_t* edges, const double* meas,
               const double* info, int64_t m, int n_fixed, const pgo_options* opts,
               pgo_problem** out);

/* One LM iteration; info may be NULL. */
int pgo_lm_step(pgo_problem* h, pgo_step_info* info);

/* Exactly n_iters LM iterations; infos (nullable) receives n_iters records. */
int pgo_solve(pgo_problem* h, int n_iters, pgo_step_info* infos);

/* Cost at the current poses, recomputed on the device. */
int pgo_cost(pgo_problem* h, double* cost_out);

/* Current poses into caller-owned host memory (n x 6). */
int pgo_get_poses(pgo_problem* h, double* poses_out);

/* Damping for the next step, and its current value. */
int pgo_set_lambda(pgo_problem* h, double lambda);
int pgo_get_lambda(const pgo_problem* h, double* lambda_out);

/* ---- inspection for the parity tests ------------------------------------ */

enum { PGO_STAGE_LINEARIZE = 1, PGO_STAGE_STEP = 2 };
/* Runs linearisation and the per-pose sums of H and g (and, for
 * PGO_STAGE_STEP, damping and the PCG step) at the current poses and lambda,
 * without retraction or decision. */
int pgo_debug_run(pgo_problem* h, int upto);

enum {
  PGO_DBG_R = 0,   /* m x 6 residual [r_R, r_t]                      */
  PGO_DBG_JI,      /* m x 36 dr/dxi_i, row-major 6 x 6               */
  PGO_DBG_JJ,      /* m x 36 dr/dxi_j                                */
  PGO_DBG_HD,      /* n x 36 diagonal blocks of H (undamped)         */
  PGO_DBG_HO,      /* m x 36 off-diagonal block J_i^T Omega J_j      */
  PGO_DBG_G,       /* n x 6 gradient J^T Omega r                     */
  PGO_DBG_DX,      /* n x 6 step (0 on held poses)                   */
  PGO_DBG_PCG,     /* 2: PCG iterations, relative residual           */
  PGO_DBG_NUM
};
/* r, J_i and J_j are stored only by pgo_debug_run (LM steps do not keep
 * them); the other arrays hold the last step's values.
 * Number of doubles of one debug array (negative PGO_ERR_ARG for a bad id). */
int64_t pgo_debug_size(const pgo_problem* h, int which);
/* Copies it to caller-owned host memory; count must equal pgo_debug_size. */
int pgo_debug_get(pgo_problem* h, int which, double* out, int64_t count);

/* ---- kernel timing for the benchmark ------------------------------------ */

enum {
  PGO_K_PREP = 0,   /* per pose: R and t tables                           */
  PGO_K_EDGE,       /* per edge: residual, Jacobians, block products, cost */
  PGO_K_POSE,       /* per pose: H and g sums, damping, block-Jacobi inverse */
  PGO_K_PCG_A,      /* PCG: stop test, H~ z, p and q = H~ p by recurrence  */
  PGO_K_PCG_B,      /* PCG: x, r, z = M^-1 r                              */
  PGO_K_RETRACT,    /* trial poses                                        */
  PGO_K_COST,       /* trial cost per edge                                */
  PGO_K_NUM
};
/* Bit k of kernel_mask times kernel k with HIP events recorded by its own
 * dispatch, every every-th launch; 0 turns timing off. */
int pgo_profile_enable(pgo_problem* h, int kernel_mask, int every);
/* Launch count and summed duration (ms) of kernel `kernel`. */
int pgo_profile_get(pgo_problem* h, int kernel, int64_t* launches, double* total_ms);

void pgo_destroy(pgo_problem* h);
const char* pgo_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* LIBPGO_PGO_H */
