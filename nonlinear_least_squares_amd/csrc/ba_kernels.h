// Kernel launchers for the gfx950 bundle-adjustment LM iteration (fp64).
//
// Data layout in HBM (all structure-of-arrays, sized once per handle):
//   point order  : observations sorted by (point, camera, k); o_cam, o_pt
//                  (int32), o_uv (2 doubles), w_pt (robust weight)
//   camera order : observations sorted by (camera, point, k); c_pt (int32),
//                  c_uv, w_cam, run_len (length of a repeated (camera, point)
//                  run at its first element, 0 elsewhere)
//   per point    : X (3), C (6, packed upper), g_p (3), C~^-1 (6), v (3),
//                  z (3), dp (3)
//   per camera   : parameters (9), CamT table (16), B (45), g_c (9), B~ (45),
//                  rhs (9), S_jj^-1 (45, packed), PCG vectors (9 each)
//   partitions   : point-order ranges of whole points, one per wavefront of
//                  the persistent point-pass blocks; camera chunks: the
//                  observations of one camera whose points lie in one of
//                  kPointBands equal point-index bands, cut into pieces of
//                  <= kChunk
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

#include "ba_model.h"

namespace ba {

constexpr int kWave = 64;         // wavefront width on gfx950
constexpr int kLdsBlock = 1024;   // threads of the persistent LDS-camera-table kernels
constexpr int kCamLdsStride = 19; // doubles per camera in the LDS table: q (4), t, f, k1, k2, vector (9)
constexpr int kCamLdsFill = 20;   // table elements per thread in the copy (>= 19 * max cameras / kLdsBlock)
// cameras whose whole rows fit: 160 KiB of LDS less 256 bytes for the
// kernels' own LDS variables (and their alignment)
constexpr int kCamLdsMaxCams = (160 * 1024 - 256) / (8 * kCamLdsStride);   // 1,076
static_assert(kCamLdsStride * kCamLdsMaxCams <= kCamLdsFill * 1024, "the copy covers the table");
constexpr int kCostLdsFill = (10 * kCamLdsMaxCams + 1023) / 1024;   // geometry elements per thread
// Where the point passes find the camera data.
constexpr int kCamRows = 0;      // whole rows in LDS (up to kCamLdsMaxCams cameras)
constexpr int kCamVectors = 1;   // the PCG's 9-vectors in LDS, geometry in memory (up to kZLdsMaxCams)
constexpr int kCamMemory = 2;    // the camera table and vectors in memory (any number)
constexpr int kZLdsStride = 9;   // doubles per camera in the vectors layout's LDS table
constexpr int kZLdsMaxCams = 2240;   // 9 * 2240 <= kCamLdsFill * kLdsBlock, 161 KB of LDS
static_assert(kZLdsStride * kZLdsMaxCams <= kCamLdsFill * 1024, "the copy covers the table");
// the largest dynamic LDS any point pass takes
constexpr int kMaxCamLdsBytes = 8 * (kCamLdsStride * kCamLdsMaxCams > kZLdsStride * kZLdsMaxCams
                                         ? kCamLdsStride * kCamLdsMaxCams : kZLdsStride * kZLdsMaxCams);
constexpr int kChunkLoads = 8;   // a camera's chunk partials loaded together in the per-camera sums
constexpr int kChunk = 1024;      // observations per camera chunk (one wavefront)
constexpr int kPointBands = 4;    // point-index bands of the camera chunks (block b: band b % 4,
                                  // on dies b % 8: two dies' L2 per band)
constexpr int kUpdBlock = 1024;   // threads of the single-block cost reduction
constexpr int kLinCamVals = 54;   // B (45) + g_c (9)
constexpr int kSchurVals = 54;    // E v (9) + Ebar C~^-1 Ebar^T (45)

// Keeps msg as the text ba_status_string() appends to `code`; returns code.
int set_error(int code, const std::string& msg);

struct PcgState {     // outcome of the solve, written once when it stops
  double rhs_norm;   // |rhs|_2
  double res_norm;   // |r|_2 after the last update
  int iters;
  int done;
  int breakdown;
  int pad;
};

struct StepOut {     // everything the host reads back after a step
  double trial_cost;
  double pcg_rel_res;
  int pcg_iters;
  int nonfinite;
  int not_spd;
  int pad;
};

// LM state on the device while ba_solve queues its steps without reading
// each one back: the decision after each step (accept if the trial cost is
// finite and lower, then lower the damping, else raise it) is taken by the
// cost reduction kernel, and an accepted trial is copied into the current
// parameters.
struct LmDev {
  double cost;       // cost at the current parameters
  double lambda;     // damping of the next step
  int relin;         // the last step was accepted: linearise again before the next
  int halted;        // a damped block was not positive definite: nothing more is applied
  int pad[2];
};

struct LmLog {       // one record per queued step, read back after the last
  double cost_before, cost_after, lambda, pcg_rel_res;
  int pcg_iters, accepted, not_spd, pad;
};

struct Dev {
  int64_t nc, np, nobs;
  int n_chunks;
  int n_chunk_blocks;    // blocks of the camera passes (blk_chunk entries)
  int lds_blocks, cam_lds_bytes;  // LDS camera-table kernels (bytes 0: not used)
  int loss;
  double delta, diag_floor, lambda, tol;
  // parameters (current and trial)
  const double* cams;
  const double* pts;
  const CamT* tab;
  const double* camq;    // unit quaternion of each camera (4), R = quat_to_R(camq)
  double* cams_trial;
  double* pts_trial;
  CamT* tab_trial;
  double* camq_trial;
  // structure
  const int32_t* o_cam;
  const int32_t* o_pt;
  const double* o_uv;
  const int32_t* c_pt;
  const double* c_uv;
  const int32_t* run_len;
  const int32_t* pt_ptr;
  const int32_t* wave_begin;     // point-order range of each wavefront of the LDS kernels
  const int32_t* cam_chunk_ptr;  // chunks of each camera, in order
  const int4* blk_chunk;         // per block of the camera passes: chunk begin, end, camera,
                                 // chunk id (band = block % kPointBands; id -1: no chunk)
  // linearisation
  double* w_pt;
  double* w_cam;
  double* C;
  double* gp;
  double* B;
  double* gc;
  double* lin_part;
  // elimination
  double* Cinv;
  double* Bd;
  double* rhs;
  double* Minv;
  double* Mfull;     // undamped-by-Cholesky copy of S_jj (packed) for inspection
  double* schur_part;
  // PCG
  double* x;
  double* r;
  double* zc;
  double* pbuf;      // search direction p, 9 nc
  double* q;
  double* prec;      // per-point 64-byte record: X (3), z = C~^-1 E^T p (3), pad (2)
  double* pcg_part;
  double* red_part;  // per-block partial sums of the camera-vector kernels, 8 x red_nb, then 2
  double* pt_dot;    // per-block partials of z^T E C~^-1 E^T z from the LDS point pass
  double* cam_rows;  // LDS point pass, PCG: the camera table rows (kCamLdsStride doubles:
                     // q, t, f, k1, k2, z) padded to kCamLdsFill * kLdsBlock, copied as is
  int cam_layout;    // kCamRows, kCamVectors or kCamMemory (the point passes' camera data)
  int red_nb;        // blocks of the camera-vector kernels
  long long* host_done;  // host-mapped, tagged with pcg_seq in the upper 32 bits: [0] the
                         // solve stopped (low bits: its iteration count), [1] the last
                         // iteration whose stop test found it still running (the host's pacing)
  long long pcg_seq;     // number of this PCG solve on the handle (from 1)
  PcgState* pcg;
  // update
  double* dp;
  double* cost_part;
  StepOut* out;
  int* flags;        // [0] non-finite seen, [1] not SPD
  // queued LM steps (null otherwise): the state, the per-step records and the
  // damping update factors and bounds
  LmDev* lm;
  LmLog* lm_log;
  double lm_up, lm_down, lm_min, lm_max;
  // dense reduced-camera solve (ba_dense.hip), when selected
  int ds_n;          // 9 nc
  int ds_ld;         // ds_n rounded up to the tile order: order and row stride of S
  int ds_T;          // ds_ld / tile order; tile row ds_T holds the right-hand side
  int ds_nruns;      // (point, camera) runs in point order
  int ds_nblk;       // lower 9x9 blocks of S that are assembled (all diagonal ones included)
  const int32_t* ds_run;      // point-order start of each run, ds_nruns + 1
  const int2* ds_blk;         // per block: camera of the block row (x) and column (y), x >= y
  const int32_t* ds_blk_ptr;  // run pairs of each block, ds_nblk + 1
  const int2* ds_pair;        // (run of camera x, run of camera y) of one point
  double* ds_F;      // per run: Ebar L, 9 x 3 row-major, L L^T = C~^-1 of its point
  double* ds_S;      // (ds_ld + tile) x ds_ld row-major: S, factored in place below the
                     // diagonal tiles; rhs row at ds_ld
  double* ds_diag;   // ds_T tiles of tile^2: the factor's diagonal tiles (lower, row-major)
  double* ds_diagT;  // the same tiles transposed
  double* ds_dinv;   // ds_ld: reciprocals of the factor's diagonal
  double* ds_v;      // 2 ds_ld: the back-substitution's right-hand side v, then x
};

// Damping of the step: the LM state's when steps are queued, else the launch's.
__device__ __forceinline__ double step_damping(const Dev& d) {
  return d.lm ? d.lm->lambda : d.lambda;
}
// Queued LM steps launch the linearisation every step; it runs only after an
// accepted step.
__device__ __forceinline__ bool lin_skipped(const Dev& d) {
  return d.lm != nullptr && d.lm->relin == 0;
}

// Events that the next kernel dispatch records at its start and end (set by
// the profiler before a timed launch, consumed by that launch; null when not
// timing).  Recorded by the dispatch itself, so they time the kernel alone.
struct DispatchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
DispatchEvents& dispatch_events();

// Allows the LDS-camera-table kernels `bytes` of dynamic LDS.
// Allows the point passes kMaxCamLdsBytes of dynamic LDS (a per-process
// attribute of the kernels; idempotent, so every handle may call it).
hipError_t set_lds_camera_limit();

void launch_cam_prep(const double* cams, CamT* tab, double* camq, int64_t nc, hipStream_t s);
void launch_lin_pt(const Dev& d, hipStream_t s);
void launch_lin_cam(const Dev& d, hipStream_t s);
// with_lin_final: the same launch also runs k_lin_final's work (extra blocks).
void launch_damp_pt(const Dev& d, hipStream_t s, bool with_lin_final = false);
void launch_schur_cam(const Dev& d, hipStream_t s);
void launch_lin_final(const Dev& d, hipStream_t s);
// with_pcg_init: the same launch also starts the PCG (r = rhs, x = 0, z = M^-1 r,
// the first partial sums, the camera rows of the LDS point pass).
void launch_precond(const Dev& d, hipStream_t s, bool with_pcg_init = false);
void launch_pcg_pt(const Dev& d, int it, hipStream_t s);
void launch_pcg_cam(const Dev& d, hipStream_t s);
// With the LDS point pass, k_pcg_step replaces k_pcg_q and k_pcg_xr.
void launch_pcg_step(const Dev& d, int it, hipStream_t s);
void launch_pcg_final(const Dev& d, int iters, hipStream_t s);
int pcg_red_blocks(int64_t nc);   // blocks of the camera-vector kernels
// pcg_iters >= 0: also k_pcg_final's record of a solve capped at pcg_iters;
// with_retract: also the trial cameras (k_retract's work).
void launch_backsub(const Dev& d, hipStream_t s, int pcg_iters = -1, bool with_retract = false);
void launch_retract(const Dev& d, hipStream_t s);
// Trial cost and the step record; with step >= 0 and d.lm set, also the LM
// decision for queued step `step` (its record goes to d.lm_log[step]).
void launch_cost(const Dev& d, const double* pts, const CamT* tab, const double* camq,
                 hipStream_t s, int step = -1);
// Queued LM steps: the trial parameters become the current ones if the
// decision accepted them.
void launch_lm_commit(const Dev& d, hipStream_t s);
void launch_debug_obs(const Dev& d, const int32_t* perm_pt, double* r, double* Jc, double* Jp,
                      double* w, hipStream_t s);

// Dense reduced-camera solve: runs' F blocks, S and its rhs row, Cholesky by
// tile columns (first diagonal tile; then per column the panel solves and the
// trailing MFMA update, which factors the next diagonal tile),
// back-substitution into x.
int ds_tile();
void launch_ds_runs(const Dev& d, hipStream_t s);
void launch_ds_fill(const Dev& d, hipStream_t s);
void launch_ds_assemble(const Dev& d, hipStream_t s);
// One launch per tile column for the camera solve: update after column k fused
// with the panel of column k + 1 (k = -1: the first panel alone).
void launch_ds_step(const Dev& d, int k, int cov, hipStream_t s);
hipError_t ds_backsolve_limit(int ld);
void launch_ds_backsolve(const Dev& d, hipStream_t s);
// Dogleg (ba_dogleg.hip): the six sums of the step's model, and the trial
// points with the step's camera part for the retraction.
int dl_vec_blocks(int64_t nc, int64_t np);
void launch_dl_vec(const Dev& d, double* vpart, hipStream_t s);
void launch_dl_obs(const Dev& d, double* opart, hipStream_t s);
void launch_dl_final(const Dev& d, const double* vpart, const double* opart, double* out, hipStream_t s);
void launch_dl_step(const Dev& d, double s_g, double s_n, double* hc, hipStream_t s);
// Camera marginal covariance from the dense factor (ba_dense.hip).
// (its tiles of Z = L^-T ride on the factorisation's panel and update
// launches when their `cov` flag is set)
void launch_cov_zero(const Dev& d, hipStream_t s);
void launch_cov_blocks(const Dev& d, double* out, int64_t n_cams, hipStream_t s);

// Implicit backward: a <- -a; per observation psi'(r) (Jc x_cam + Jp dp_pt) to
// out[2 perm_cam[s] ..], s the camera-order slot.
void launch_negate(double* a, int64_t n, hipStream_t s);
void launch_vjp_obs(const Dev& d, const int32_t* perm_cam, double* out, hipStream_t s);

// Structure build helpers.
void launch_validate(const int32_t* cam_idx, const int32_t* pt_idx, const double* uv, int64_t n,
                     const double* cams, int64_t nc, const double* pts, int64_t np, int* flags,
                     hipStream_t s);
void launch_make_keys(const int32_t* major, const int32_t* minor, int64_t n_minor, int64_t n,
                      uint64_t* keys, int32_t* vals, hipStream_t s);
void launch_gather_obs(const int32_t* perm, const int32_t* cam_idx, const int32_t* pt_idx,
                       const double* uv, int64_t n, int32_t* out_cam, int32_t* out_pt,
                       double* out_uv, hipStream_t s);
void launch_seg_ptr(const int32_t* sorted_key, int64_t n, int64_t n_seg, int32_t* ptr,
                    hipStream_t s);
void launch_run_len(const int32_t* c_cam, const int32_t* c_pt, int64_t n, int32_t* run_len,
                    hipStream_t s);

}  // namespace ba
