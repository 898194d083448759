/* libdba — Gauss-Newton iterations of dense frame-graph bundle adjustment
 * (per-pixel inverse depth, SE(3) keyframe poses) on an AMD Instinct MI355X
 * (gfx950), fp32, behind a plain C ABI.
 *
 * The problem (NeRF-SLAM reproduction notes, sec. 2.2 and 2.3): keyframes are
 * the nodes of a frame graph; every pixel of frame i carries an inverse depth
 * d; every edge (i, j) carries, per pixel of frame i, a 2-D target where that
 * pixel should land in frame j and a confidence weight.
 *
 *   poses     n_frames x 7 floats [tx ty tz qx qy qz qw]: world-to-camera
 *             T = [R(q) | t]; q need not be normalised (it is on input).
 *   depths    n_frames x height x width inverse depths, row-major per frame.
 *   K         4 floats fx, fy, cx, cy (pixel (x, y) = column, row).
 *   edges     n_edges x 2 int32 (i, j), 0 <= i, j < n_frames.
 *   targets   n_edges x height x width x 2 floats (x, y) in frame j.
 *   weights   n_edges x height x width floats, finite and >= 0.
 *
 *   residual  X_i = K^-1 [x, y, 1]^T / max(d, 1e-6),  X_j = T_j T_i^-1 X_i,
 *             r = (fx X_j.x / Z + cx, fy X_j.y / Z + cy) - target,
 *             Z = max(X_j.z, 1e-6) (sec. 2.2: both clamps at 1e-6).
 *   cost      C = 1/2 sum w |r|^2 (the weights are W in H = J^T W J, sec. 3.1).
 *   step      Gauss-Newton: H = J^T W J, b = -J^T W r with 6x6 pose blocks,
 *             1x1 inverse-depth blocks and their coupling (sec. 3.1); depths
 *             eliminated by the Schur complement, S = B - E C^-1 E^T,
 *             S dxi = b_c - E C^-1 b_d solved by Cholesky, never by an
 *             explicit inverse; dd = C^-1 (b_d - E^T dxi) (sec. 3.2, eqs. (1)
 *             and (2)).  Poses move by the left SE(3) exponential
 *             T <- Exp(xi) T, xi = (rho, phi) (Theseus note, retraction on Lie
 *             groups); depths additively.  The first n_fixed poses stay
 *             fixed (gauge); every step is applied (no damping).
 *
 * Conventions
 *   - Every function returns DBA_OK (0) or a negative DBA_ERR_* code; nothing
 *     is thrown across the ABI.  dba_status_string() gives a message.
 *   - A handle owns its device memory, sized once in dba_create; no iteration
 *     allocates.
 *   - A handle is not thread-safe.  Device work is enqueued on
 *     options.stream (hipStream_t, NULL = default stream); calls that return
 *     host values synchronise that stream.
 *   - Limits (DBA_ERR_LIMIT): at most 8 out-edges per frame (edges sharing
 *     the source frame i are linearised together), at most 24 free frames.
 */
#ifndef LIBDBA_DBA_H
#define LIBDBA_DBA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  DBA_OK = 0,
  DBA_ERR_ARG = -1,        /* null pointer, bad size or index, bad option            */
  DBA_ERR_NONFINITE = -2,  /* NaN/Inf or a negative weight in an input               */
  DBA_ERR_NOT_SPD = -3,    /* the reduced pose system failed to factor                */
  DBA_ERR_DEVICE = -4,     /* HIP runtime error                                       */
  DBA_ERR_ALLOC = -5,      /* device or pinned-host allocation failed                 */
  DBA_ERR_LIMIT = -6       /* out-degree or free-frame count above the compiled limit */
};

enum { DBA_MEM_HOST = 0, DBA_MEM_DEVICE = 1 };

typedef struct {
  int mem;        /* DBA_MEM_HOST / DBA_MEM_DEVICE: where the input pointers live */
  void* stream;   /* hipStream_t or NULL                                          */
} dba_options;

typedef struct {
  float cost_before;   /* cost at the start of the step      */
  float cost_after;    /* cost after the step was applied    */
} dba_step_info;

typedef struct dba_problem dba_problem;

int dba_options_default(dba_options* o);

/* Copies the inputs to the device, validates them (DBA_ERR_ARG for edge
 * indices, DBA_ERR_NONFINITE for NaN/Inf, negative weights or a zero
 * quaternion), groups the edges by source frame and plans the work.  opts may
 * be NULL.  On error *out is left NULL. */
int dba_create(const float* poses, const float* inv_depth, int n_frames, int height, int width,
               const float* intrinsics, const int32_t* edges, int n_edges,
               const float* targets, const float* weights, int n_fixed,
               const dba_options* opts, dba_problem** out);

/* One Gauss-Newton step (linearise, assemble, eliminate depths, Cholesky of
 * the reduced pose system, back-substitute, retract).  info may be NULL. */
int dba_gn_step(dba_problem* h, dba_step_info* info);

/* n_iters steps with no host synchronisation between them.  costs (may be
 * NULL) receives n_iters + 1 values: the cost before each step and after the
 * last.  Same results, bit for bit, as n_iters calls of dba_gn_step. */
int dba_solve(dba_problem* h, int n_iters, float* costs);

/* Cost at the current state. */
int dba_cost(dba_problem* h, float* cost);

/* Pose marginal covariance at the current state: S^-1, the inverse of the
 * reduced pose system after the depths are eliminated (NeRF-SLAM
 * reproduction notes, sec. 3.2, the cov_cam output of the dense step).  One
 * workgroup factors S by Cholesky in LDS and solves against the identity, in
 * fp32.  cov: caller-owned HOST buffer of nv x nv floats, row-major, nv =
 * 6 (n_frames - n_fixed) (nothing is written when nv is 0).  The state does
 * not change; the inspection arrays S, rhs, C and g_d then hold this
 * linearisation.  DBA_ERR_NOT_SPD (cov untouched) when S is not positive
 * definite; the first call allocates an nv x nv device buffer that the handle
 * keeps. */
int dba_covariance(dba_problem* h, float* cov);

/* Current state to caller-owned host buffers (either may be NULL); poses are
 * normalised with qw >= 0. */
int dba_get_state(dba_problem* h, float* poses, float* inv_depth);

/* Replaces the state from host or device memory per options.mem (either
 * pointer may be NULL to keep that part).  DBA_ERR_NONFINITE if a new depth
 * or pose is non-finite or a quaternion is zero; the handle then keeps its
 * previous state. */
int dba_set_state(dba_problem* h, const float* poses, const float* inv_depth);

int dba_get_sizes(const dba_problem* h, int* n_frames, int* n_pixels, int* n_edges, int* n_fixed);

/* ---- inspection entry points used by the parity tests ------------------- */

enum {
  DBA_STAGE_ASSEMBLE = 1,  /* linearise and assemble WITHOUT eliminating the depths:
                              DBA_DBG_S then holds B on the free poses and DBA_DBG_RHS -g_c */
  DBA_STAGE_JACOBIANS = 2  /* per-residual r, J_i, J_j, J_d at the current state         */
};
int dba_debug_run(dba_problem* h, int stage);

enum {
  DBA_DBG_S = 0,   /* float nv x nv (nv = 6 (n_frames - n_fixed)), reduced matrix of the last step */
  DBA_DBG_RHS,     /* float nv                                                                   */
  DBA_DBG_DXI,     /* float n_frames x 6 pose step (rho, phi) of the last step, 0 when fixed     */
  DBA_DBG_DD,      /* float n_frames x P depth step of the last step                             */
  DBA_DBG_C,       /* float n_frames x P depth block C of the last linearisation (0 if no edge)  */
  DBA_DBG_GD,      /* float n_frames x P depth gradient g_d = sum w J_d r                        */
  DBA_DBG_R,       /* float n_edges x P x 2 (after DBA_STAGE_JACOBIANS)                           */
  DBA_DBG_JI,      /* float n_edges x P x 12, row-major 2 x 6, left perturbation of T_i          */
  DBA_DBG_JJ,      /* float n_edges x P x 12                                                     */
  DBA_DBG_JD,      /* float n_edges x P x 2                                                      */
  DBA_DBG_NUM
};
int64_t dba_debug_size(const dba_problem* h, int which);
int dba_debug_get(dba_problem* h, int which, void* host_out, int64_t bytes);

/* ---- kernel timing for the benchmark ------------------------------------ */

enum {
  DBA_K_LIN = 0,   /* back-substitution of the previous step, linearisation, Schur partials */
  DBA_K_ASSEMBLE,  /* reduced pose system and right-hand side from the partials, cost       */
  DBA_K_SOLVE,     /* Cholesky, triangular solves, retraction                                */
  DBA_K_COST,      /* back-substitution of the last step and cost                            */
  DBA_K_NUM
};
/* kernel_mask bit k set (k = DBA_K_*): launches of kernel k are bracketed by
 * HIP events recorded by the kernel's own dispatch on the handle's stream;
 * per-kernel totals accumulate until dba_profile_reset; 0 turns timing off.
 * every >= 1 times only every every-th launch of each such kernel (a timed
 * dispatch cannot overlap its neighbours).  DBA_ERR_ARG for a null handle or
 * every < 1. */
int dba_profile_enable(dba_problem* h, int kernel_mask, int every);
int dba_profile_reset(dba_problem* h);
int dba_profile_get(dba_problem* h, int kernel, int64_t* launches, double* total_ms);
const char* dba_kernel_name(int kernel);

void dba_destroy(dba_problem* h);
const char* dba_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* LIBDBA_DBA_H */
