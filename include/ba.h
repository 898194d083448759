/* libba — one Levenberg-Marquardt iteration of large-scale bundle adjustment on
 * an AMD Instinct MI355X (gfx950), fp64, behind a plain C ABI.
 *
 * The problem ("Bundle Adjustment in the Eager Mode" summary article: adjust
 * cameras and 3-D points so that projected points line up with their image
 * observations; every residual depends on exactly one camera and one point):
 *
 *   cameras   n_cams x 9 doubles, row-major: [w0 w1 w2 t0 t1 t2 f k1 k2]
 *             w = axis-angle of the world-to-camera rotation R (P = R X + t),
 *             f focal length in pixels, k1, k2 radial distortion on the
 *             normalised coordinates; principal point 0.
 *   points    n_pts x 3 doubles, row-major world coordinates.
 *   obs       n_obs entries: obs_cam_idx[k] in [0, n_cams), obs_pt_idx[k] in
 *             [0, n_pts), obs_uv[2k..2k+1] observed pixel.  Repeated
 *             (camera, point) pairs are allowed (each is its own residual);
 *             cameras or points with no observation are allowed.
 *
 *   residual  r_k = f (1 + k1 n + k2 n^2) p - uv_k,  p = P_xy / max(P_z, 1e-6),
 *             n = |p|^2 (NeRF-SLAM reproduction notes, sec. 2.2: depth clamped
 *             at 1e-6 before the division).
 *   cost      C = sum_k rho(|r_k|): rho(e) = e^2/2, or Huber with threshold
 *             delta (F^2SLAM article, sec. 5.3) applied to the 2-D norm.
 *   step      Gauss-Newton normal equations H delta = -g with H = J^T W J,
 *             g = J^T W r (NeRF-SLAM notes, sec. 3.1), Marquardt damping
 *             H + lambda diag(max(diag H, floor)) ("Bundle Adjustment in the
 *             Eager Mode": diagonal damping; Theseus note: LM with adaptive
 *             damping), points eliminated by the Schur complement and the
 *             reduced camera system (B - E C^-1 E^T) dc = -g_c + E C^-1 g_p
 *             solved by block-Jacobi preconditioned conjugate gradients
 *             without forming it (NeRF-SLAM notes, sec. 3.2, eqs. (1), (2);
 *             "Bundle Adjustment in the Eager Mode": PCG for large problems),
 *             point back-substitution dp = C^-1 (-g_p - E^T dc), retraction
 *             R <- Exp(dphi) R and additive updates elsewhere (Theseus note,
 *             retraction), accepted iff the cost strictly decreases.
 *
 * Conventions
 *   - Every function returns BA_OK (0) or a negative BA_ERR_* code; nothing is
 *     thrown across the ABI.  ba_status_string() gives a message; for
 *     BA_ERR_DEVICE the last HIP error text is kept and appended.
 *   - A handle owns all of its device memory (one arena sized once from
 *     n_cams, n_pts, n_obs in ba_create); no LM call allocates.
 *   - A handle is not thread-safe.  All device work is enqueued on
 *     options.stream (a hipStream_t, NULL = the default stream).  Calls that
 *     return host values synchronise that stream.
 *   - Host output buffers are caller-owned.
 */
#ifndef LIBBA_BA_H
#define LIBBA_BA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  BA_OK = 0,
  BA_ERR_ARG = -1,        /* null pointer, size <= 0, index out of range, bad option  */
  BA_ERR_NONFINITE = -2,  /* NaN/Inf in an input, or a non-finite cost                */
  BA_ERR_NOT_SPD = -3,    /* a damped point block or camera block failed to factor   */
  BA_ERR_DEVICE = -4,     /* HIP runtime error                                        */
  BA_ERR_ALLOC = -5       /* device or pinned-host allocation failed                  */
};

enum { BA_MEM_HOST = 0, BA_MEM_DEVICE = 1 };
/* Solver of the reduced camera system S dc = rhs (the Schur complement of the
 * point blocks, eq. (2) of the NeRF-SLAM reproduction notes, sec. 3.2):
 *   BA_SOLVER_PCG          implicit S, block-Jacobi PCG (any size);
 *   BA_SOLVER_DENSE_SCHUR  explicit S and a Cholesky factorisation on the
 *                          device, the direct solver that the eager-mode BA
 *                          summary uses for small and medium problems; up to
 *                          BA_DENSE_MAX_CAMS cameras (S takes (9 n_cams)^2
 *                          doubles of device memory). */
enum { BA_SOLVER_PCG = 0, BA_SOLVER_DENSE_SCHUR = 1 };
#define BA_DENSE_MAX_CAMS 1536
enum { BA_LOSS_SQUARED = 0, BA_LOSS_HUBER = 1 };
/* Step strategy of ba_lm_step / ba_solve (the Theseus note offers LM with
 * adaptive damping and Dogleg):
 *   BA_STRATEGY_LM      Levenberg-Marquardt (default);
 *   BA_STRATEGY_DOGLEG  Powell's dogleg trust region: the Gauss-Newton step
 *                       (the damped system with the small fixed damping
 *                       dl_gn_damping, which keeps the gauge-singular BA
 *                       system solvable), the Cauchy point -alpha g with
 *                       alpha = |g|^2 / |J g|_W^2, and their blend at the
 *                       trust radius; gain ratio against the quadratic model
 *                       C + g^T h + 1/2 h^T J^T W J h; the radius becomes
 *                       max(radius, 3 |h|) when the ratio exceeds 0.75 and is
 *                       halved below 0.25; a step is kept iff the cost is
 *                       strictly lower.  |.| is the Euclidean norm over all
 *                       parameters in the tangent of the retraction.  While
 *                       the point of linearisation stays, the Gauss-Newton
 *                       step is kept, so a rejected step costs one trial
 *                       cost. */
enum { BA_STRATEGY_LM = 0, BA_STRATEGY_DOGLEG = 1 };

typedef struct {
  int loss;              /* BA_LOSS_SQUARED or BA_LOSS_HUBER                     */
  double huber_delta;    /* pixels (default 2.0)                                 */
  double lambda0;        /* initial damping (1e-3)                               */
  double lambda_up;      /* factor on a rejected step (10)                       */
  double lambda_down;    /* divisor on an accepted step (10)                     */
  double lambda_min;     /* 1e-16                                                */
  double lambda_max;     /* 1e16                                                 */
  double diag_floor;     /* floor on diag(J^T W J) in the damping term (1e-6)    */
  int pcg_max_iters;     /* 50                                                   */
  double pcg_rel_tol;    /* stop when |r|_2 <= tol |rhs|_2 (1e-6)                */
  int mem;               /* BA_MEM_HOST / BA_MEM_DEVICE: where ba_create inputs
                            and ba_set_params inputs live                       */
  void* stream;          /* hipStream_t or NULL                                  */
  int solver;            /* BA_SOLVER_PCG (default) or BA_SOLVER_DENSE_SCHUR;
                            with the dense solver, pcg_iters and pcg_rel_res
                            of the step information are 0                       */
  int strategy;          /* BA_STRATEGY_LM (default) or BA_STRATEGY_DOGLEG       */
  double dl_radius0;     /* dogleg: initial trust radius (1.0)                   */
  double dl_gn_damping;  /* dogleg: Marquardt damping of its Gauss-Newton step,
                            also used by ba_backward and ba_covariance on a
                            dogleg handle (1e-6)                                */
} ba_options;

typedef struct {
  double cost_before;    /* cost at the parameters the step started from       */
  double cost_after;     /* cost at the trial parameters                        */
  double lambda;         /* damping used for this step                          */
  double pcg_rel_res;    /* |r|_2 / |rhs|_2 when PCG stopped                     */
  int accepted;          /* 1 if the trial parameters were kept                 */
  int pcg_iters;         /* PCG iterations run                                  */
  double radius;         /* dogleg: trust radius of this step (0 for LM)        */
  double gain_ratio;     /* dogleg: cost decrease / model decrease              */
  double step_norm;      /* dogleg: |h|                                         */
  int step_kind;         /* dogleg: 0 Gauss-Newton, 1 steepest descent cut at
                            the radius, 2 blend of the two                     */
} ba_step_info;

typedef struct {
  double initial_cost, final_cost, lambda;
  int iterations, accepted, pcg_iters_total;
} ba_summary;

typedef struct {
  double lambda;         /* damping for the next step                           */
  double cost;           /* cost at the current parameters                      */
  int64_t iteration;     /* LM steps taken so far                               */
  double radius;         /* dogleg trust radius; ba_set_state leaves it as it is
                            when this is 0                                      */
} ba_state;

typedef struct ba_problem ba_problem;

/* Fills *o with the defaults listed above.  BA_ERR_ARG if o is NULL. */
int ba_options_default(ba_options* o);

/* Largest sizes ba_create accepts (the kernels index observations and points
 * with 32-bit products below these). */
#define BA_MAX_OBS ((int64_t)1 << 30)
#define BA_MAX_PTS ((int64_t)1 << 28)
#define BA_MAX_CAMS ((int64_t)1 << 24)

/* Copies the inputs to the device (H2D, or D2D when opts->mem == BA_MEM_DEVICE),
 * validates them on the device (index range, finiteness), sorts the
 * observations by (point, camera, k) and by (camera, point, k) with a stable
 * device radix sort (the sparsity pattern is fixed across iterations, the
 * reason the eager-mode BA page caches its symbolic structure), builds the
 * CSR offsets and work partitions, allocates the whole arena and evaluates
 * the initial cost.  The caller may free its inputs when this returns.
 * opts may be NULL (defaults).  On error *out is left NULL.
 * The point passes keep camera data in each compute unit's LDS by size: up
 * to 1,076 cameras whole rows (geometry and the PCG's 9-vector), up to 2,240
 * cameras only the 9-vectors of the PCG and back-substitution passes with the
 * geometry read from memory, past that nothing (everything read from memory).
 * The environment variables BA_NO_LDS_CAMERAS=1 (memory) and
 * BA_SPLIT_LDS_CAMERAS=1 (vectors, where they fit) at creation select another
 * layout.  All layouts compute the same arithmetic in the same order, so they
 * give the same bits. */
int ba_create(const double* cams, int64_t n_cams, const double* points, int64_t n_pts,
              const int32_t* obs_cam_idx, const int32_t* obs_pt_idx, const double* obs_uv,
              int64_t n_obs, const ba_options* opts, ba_problem** out);

/* One LM iteration: linearise (skipped when the previous step was rejected,
 * the parameters being unchanged), damp, eliminate points, PCG, back-substitute,
 * retract, evaluate the trial cost, accept iff it is strictly lower.  info may
 * be NULL.  A rejected step is not an error. */
int ba_lm_step(ba_problem* h, ba_step_info* info);

/* Exactly n_iters LM iterations (no early exit).  s may be NULL.  With the LM
 * strategy the iterations are queued on the handle's stream without reading
 * each one back: the accept/reject decision and the damping update are taken
 * on the device, with the same comparisons and arithmetic as ba_lm_step, so
 * the result equals n_iters calls of ba_lm_step.  The call returns after the
 * last iteration has finished.  A damped block that is not positive definite
 * stops the changes at that iteration: BA_ERR_NOT_SPD is returned and the
 * handle keeps the state after the last good iteration (s is not written),
 * as a loop of ba_lm_step calls would leave it.  The per-iteration records
 * take 48 bytes per iteration of device memory, allocated by the first call
 * that needs more. */
int ba_solve(ba_problem* h, int n_iters, ba_summary* s);

/* Cost at the current parameters, recomputed on the device. */
int ba_cost(ba_problem* h, double* cost_out);

/* Implicit backward through the LM solution, the implicit mode of the Theseus
 * note: one Newton step at the current parameters, h(theta; u) = theta -
 * H~^-1 grad S(theta; u), is differentiated with H~ held fixed, H~ being the
 * damped Gauss-Newton matrix of the current LM state (lambda as the next step
 * would use it; the undamped matrix is singular along the gauge of a BA
 * problem), u the observed pixels.  Given the gradient G of a loss f with
 * respect to the parameters (grad_cams n_cams x 9 in the tangent of the
 * forward step, grad_points n_pts x 3), writes for every observation, in the
 * original order, grad_uv (n_obs x 2):
 *   df/du_k = psi'(r_k) J_k H~^-1 G,
 * with psi(r) = d rho(|r|)/dr: psi' = I for the squared loss and inside the
 * Huber threshold, (delta/|r|)(I - r r^T/|r|^2) beyond it.  H~^-1 G is solved
 * like an LM step (Schur elimination, the handle's solver and tolerance,
 * back-substitution).  The three arrays live where opts.mem says (host or
 * device).  pcg_iters (nullable) receives the PCG iterations (0 with the dense
 * solver).  The parameters and lambda are unchanged; the next LM step
 * linearises again.  BA_ERR_ARG for null arrays, BA_ERR_NOT_SPD if a damped
 * block fails to factor. */
int ba_backward(ba_problem* h, const double* grad_cams, const double* grad_points, double* grad_uv,
                int* pcg_iters);

/* Camera marginal covariance, as in the NeRF-SLAM notes' dense step (sec.
 * 3.2): the Cholesky factor of the reduced camera matrix S gives S^-1 by
 * solves against the identity; S is never inverted directly.  At the current
 * parameters and lambda this linearises, damps, eliminates the points,
 * assembles and factors S~ = L L^T (as an LM step with the dense solver
 * would) while forming Z = L^-T by 32 x 32 tiles in the same launches (fp64
 * MFMA updates), and writes each camera's 9x9 diagonal block of
 * S~^-1 = Z Z^T to cov_out (n_cams x 81,
 * row-major; host memory for BA_MEM_HOST handles, device memory for
 * BA_MEM_DEVICE ones).  The blocks are the cameras' marginal covariances
 * under the damped Gauss-Newton model (S~ includes lambda's damping; at
 * lambda = 0 the reduced matrix of a BA problem is singular along its gauge).
 * Needs opts.solver == BA_SOLVER_DENSE_SCHUR, whose storage holds the factor
 * (BA_ERR_ARG otherwise); BA_ERR_NOT_SPD if S~ fails to factor.  Parameters,
 * lambda and cost are unchanged. */
int ba_covariance(ba_problem* h, double* cov_out);

/* Current parameters to caller-owned host buffers (n_cams x 9, n_pts x 3);
 * either pointer may be NULL. */
int ba_get_params(ba_problem* h, double* cams_out, double* points_out);

/* Replaces the parameters (host or device pointers per options.mem; either may
 * be NULL to keep that part), forces a re-linearisation, recomputes the cost.
 * BA_ERR_NONFINITE if a new parameter or the new cost is not finite; the
 * handle then keeps its previous parameters, cost and linearisation. */
int ba_set_params(ba_problem* h, const double* cams, const double* points);

int ba_get_state(const ba_problem* h, ba_state* st);
int ba_set_state(ba_problem* h, const ba_state* st);

/* Sizes. */
int ba_get_sizes(const ba_problem* h, int64_t* n_cams, int64_t* n_pts, int64_t* n_obs);

/* ---- cost without allocation ---------------------------------------------
 *
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * cost as ba_cost (sum over observations of rho(|r_k|), squared or Huber
 * loss, the same camera model and per-observation arithmetic), but with no
 * handle: every array is caller-owned DEVICE memory in the layout of
 * ba_create (cams n_cams x 9, points n_pts x 3, obs_cam_idx / obs_pt_idx
 * n_obs int32, obs_uv n_obs x 2), and the result is written to cost_out, one
 * double in device memory.  All work is enqueued on `stream` (a hipStream_t,
 * NULL = the default stream); nothing synchronises, so the call can be
 * captured into a graph.  It calls no hipMalloc, hipFree or allocating
 * library routine: its scratch (camera table and per-block partial sums,
 * 768 KiB) is a static device array that each GPU holds until the process
 * ends.  Every call on a GPU shares that array, so calls that overlap on one
 * GPU (on different streams or host threads) race; calls queued on one
 * stream do not.  The per-block partials are added in a fixed order, so
 * equal inputs give equal bits.
 *
 * Returns BA_ERR_ARG for null pointers, n_cams or n_pts <= 0, n_obs < 0,
 * n_cams > BA_NOALLOC_MAX_CAMS, n_obs > BA_NOALLOC_MAX_OBS, a bad loss or a
 * huber_delta that is not positive, all before any device work.  An
 * observation index out of range is not read: the kernel writes NaN to
 * cost_out instead (as it does for non-finite inputs). */
#define BA_NOALLOC_MAX_CAMS 4096
#define BA_NOALLOC_MAX_OBS (16384 * 1024)
int ba_cost_noalloc(const double* cams, int64_t n_cams, const double* points, int64_t n_pts,
                    const int32_t* obs_cam_idx, const int32_t* obs_pt_idx, const double* obs_uv,
                    int64_t n_obs, int loss, double huber_delta, double* cost_out, void* stream);

/* ---- inspection entry points used by the parity tests ------------------- */

enum {
  BA_STAGE_LINEARIZE = 1,  /* residuals, Jacobians, B, g_c, C, g_p at the current parameters */
  BA_STAGE_SCHUR = 2,      /* damping with the current lambda, C~^-1, v, rhs, S_jj, Cholesky */
  BA_STAGE_PCG = 3,        /* camera step dc (PCG, or the dense solve when selected)          */
  BA_STAGE_UPDATE = 4      /* dp, trial parameters, trial cost                                */
};

/* Runs the stages 1..upto of one LM iteration at the current parameters and
 * lambda without taking the accept/reject decision. */
int ba_debug_run(ba_problem* h, int upto);

enum {
  BA_DBG_PERM_PT = 0,   /* int32 n_obs: original index of the k-th observation in (pt, cam, k) order */
  BA_DBG_PERM_CAM,      /* int32 n_obs: same for (cam, pt, k) order                                 */
  BA_DBG_PT_PTR,        /* int32 n_pts + 1                                                          */
  BA_DBG_CAM_PTR,       /* int32 n_cams + 1                                                         */
  BA_DBG_R,             /* double n_obs x 2   residual, original observation order, current params */
  BA_DBG_JC,            /* double n_obs x 18  camera Jacobian (row-major 2 x 9)                    */
  BA_DBG_JP,            /* double n_obs x 6   point Jacobian (row-major 2 x 3)                     */
  BA_DBG_W,             /* double n_obs       robust weight                                        */
  BA_DBG_B,             /* double n_cams x 81                                                      */
  BA_DBG_GC,            /* double n_cams x 9                                                       */
  BA_DBG_C,             /* double n_pts x 9                                                        */
  BA_DBG_GP,            /* double n_pts x 3                                                        */
  BA_DBG_BD,            /* double n_cams x 81 damped B                                             */
  BA_DBG_CINV,          /* double n_pts x 9   inverse of the damped point block                    */
  BA_DBG_V,             /* double n_pts x 3; valid after BA_STAGE_SCHUR, until a PCG stage runs    */
  BA_DBG_RHS,           /* double n_cams x 9                                                       */
  BA_DBG_M,             /* double n_cams x 81 exact diagonal blocks S_jj                           */
  BA_DBG_DC,            /* double n_cams x 9                                                       */
  BA_DBG_DP,            /* double n_pts x 3                                                        */
  BA_DBG_CAMS_TRIAL,    /* double n_cams x 9                                                       */
  BA_DBG_PTS_TRIAL,     /* double n_pts x 3                                                        */
  BA_DBG_PCG,           /* double 2: iterations, relative residual                                 */
  BA_DBG_TRIAL_COST,    /* double 1                                                                */
  BA_DBG_S,             /* double (9 n_cams)^2: the explicit reduced camera matrix S, row-major,
                           assembled on the device from the state after BA_STAGE_SCHUR (the dense
                           solver only; BA_ERR_ARG otherwise)                                      */
  BA_DBG_NUM
};

/* Byte size of one debug array (negative BA_ERR_ARG for a bad id). */
int64_t ba_debug_size(const ba_problem* h, int which);

/* Copies one array to caller-owned host memory; bytes must equal
 * ba_debug_size(h, which). */
int ba_debug_get(ba_problem* h, int which, void* host_out, int64_t bytes);

/* ---- kernel timing for the benchmark ------------------------------------ */

enum {
  BA_K_LIN_PT = 0,   /* point-order linearisation, C and g_p                       */
  BA_K_LIN_CAM,      /* camera-order linearisation, chunk partials of B and g_c    */
  BA_K_DAMP_PT,      /* damped point blocks, their inverses, v                     */
  BA_K_SCHUR_CAM,    /* camera-order E v and Ebar C~^-1 Ebar^T partials            */
  BA_K_PRECOND,      /* per camera B~, rhs, S_jj and its Cholesky factor           */
  BA_K_PCG_INIT,     /* PCG start: r = rhs, z = M^-1 r (no launches of its own: it
                        runs in the BA_K_PRECOND launch)                            */
  BA_K_PCG_PT,       /* PCG point pass: stop test, C~^-1 E^T z                      */
  BA_K_PCG_CAM,      /* PCG camera pass: chunk partials of E C~^-1 E^T z            */
  BA_K_PCG_Q,        /* PCG p, q = S p, p.q: no launches of its own (the
                        BA_K_PCG_XR launch forms them by recurrence); kept so that
                        the ids after it keep their values                        */
  BA_K_PCG_XR,       /* PCG update of x, r, z, with p, q and p.q                   */
  BA_K_BACKSUB,      /* point back-substitution and trial points                   */
  BA_K_RETRACT,      /* trial cameras (no launches of its own in an LM step:
                        BA_K_BACKSUB forms them; the dogleg launches it)           */
  BA_K_COST,         /* trial cost                                                 */
  BA_K_DS_RUNS,      /* dense solver: F = Ebar chol(C~^-1) per (point, camera) run  */
  BA_K_DS_FILL,      /* dense solver: S cleared, padding, rhs row                  */
  BA_K_DS_ASSEMBLE,  /* dense solver: lower 9x9 blocks of S                        */
  BA_K_DS_PANEL,     /* dense solver: the first tile column (factor and solves)     */
  BA_K_DS_UPDATE,    /* dense solver: one launch per later tile column, the trailing
                        update after the previous column (fp64 MFMA) fused with
                        this column's diagonal factor and tile solves             */
  BA_K_DS_BACKSOLVE, /* dense solver: L^T dc = L^-1 rhs                            */
  BA_K_COV_ZERO,     /* covariance: zeros in the strictly upper tiles of S, which
                        then receive Z = L^-T (its diagonal tiles are kept apart):
                        its tiles are solved and updated (fp64 MFMA) within the
                        BA_K_DS_PANEL / BA_K_DS_UPDATE launches of the
                        factorisation                                           */
  BA_K_COV_BLOCKS,   /* covariance: per camera, the 9x9 block of Z Z^T              */
  BA_K_DL_OBS,       /* dogleg: |J g|^2, (J g).(J h_gn), |J h_gn|^2 partials        */
  BA_K_DL_STEP,      /* dogleg: the step's camera part and the trial points         */
  BA_K_NUM
};

/* kernel_mask bit k set (k = BA_K_*): launches of kernel k are bracketed by
 * HIP events, recorded by the kernel's own dispatch on the handle's stream, and
 * per-kernel totals accumulate until ba_profile_reset; 0 turns timing off.
 * every >= 1 times only every every-th launch of each such kernel (a timed
 * dispatch cannot overlap its neighbours, so sparse sampling keeps the cost of
 * timing out of the throughput being timed).  PCG launches queued past the
 * iteration at which the solve stopped exit at once and are not counted.
 * Returns BA_ERR_ARG for a null handle or every < 1. */
int ba_profile_enable(ba_problem* h, int kernel_mask, int every);
int ba_profile_reset(ba_problem* h);
/* Launch count and summed duration (ms) of kernel `kernel` (BA_K_*). */
int ba_profile_get(ba_problem* h, int kernel, int64_t* launches, double* total_ms);
const char* ba_kernel_name(int kernel);

void ba_destroy(ba_problem* h);
const char* ba_status_string(int code);

#ifdef __cplusplus
}
#endif

#endif /* LIBBA_BA_H */
