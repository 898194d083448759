// Kernel launchers of libpgo (pose-graph optimisation, gfx950, fp64).
//
// Layout (structure of arrays, sized once per handle; n poses, m edges):
//   per pose : [w, t] (current and trial), table R (9) and t (3), diagonal
//              block of H (36) undamped and damped, block-Jacobi inverse (36),
//              g (6), PCG vectors x r z p q (6 each)
//   per edge : (i, j), measured R_e (9) and t_e (3), info [w_R, w_t],
//              residual (6), Jacobians (36 + 36), cost, and H_ij in kCoupVals
//              doubles: with R_i^T R_i = I its lower-left 3x3 block is zero and
//              its lower-right one is -w_t I, so it is kept as the upper-left
//              block (9), the upper-right block (9), -w_t, and a 0
//   per pose : the damped diagonal block and its inverse are symmetric and
//              kept as their upper triangles, row by row (kSymVals)
//   per half edge (2m, side 0 = the edge's i, side 1 = its j): that end's
//              contribution to its diagonal block (36) and to g (6), side-major
//              (row side m + e); each
//              pose lists its half edges in edge order (CSR) as pairs (half
//              edge id 2 e + side, pose at the other end), so every sum has a
//              fixed order and the product's gathers depend on one load
//   PCG scalars: per-block partials of r.r (two parities), r.z (two), b.b and
//              p.q, at most kMaxPcgBlocks of each; every block adds them all
//              in a fixed order
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

namespace pgo {

constexpr int kHalfVals = 42;   // 6x6 block + 6-vector
constexpr int kCoupVals = 20;   // H_ij: two 3x3 blocks, -w_t, 0
constexpr int kSymVals = 21;    // upper triangle of a symmetric 6x6 block
constexpr int kPosesPerWave = 10;
// PCG blocks: kBigPcgWaves wavefronts when the graph fills kMaxPcgBlocks
// such blocks, else kSmallPcgWaves; a chunk is ten poses per wavefront.
constexpr int kBigPcgWaves = 16;
constexpr int kSmallPcgWaves = 4;
constexpr int kMaxPcgBlocks = 256;   // one per compute unit
// Indices of the partial-sum arrays.
enum { kRR0 = 0, kRR1 = 1, kRZ0 = 2, kRZ1 = 3, kBB = 4, kPQ = 5, kNumSums = 6 };

struct PcgState {
  double rhs_norm, res_norm;
  int iters, done, breakdown, pad;
};

struct StepOut {
  double trial_cost, pcg_rel_res;
  int pcg_iters, nonfinite, not_spd, pad;
};

struct Dev {
  int64_t n, m;
  int n_fixed;
  double lambda, diag_floor, tol;
  const double* poses;     // current [w, t]
  double* trial;           // trial [w, t]
  double* tab;             // current R (9), t (3)
  double* tab_trial;
  const int2* edges;
  const double* meas_tab;  // R_e (9), t_e (3)
  const double* info;      // [w_R, w_t]
  const int32_t* half_ptr; // n + 1
  const int2* nbr;         // 2m (half-edge id 2 e + side, other pose), grouped by pose
  double* r;               // m x 6
  double* Ji;              // m x 36
  double* Jj;              // m x 36
  double* Hc;              // m x kCoupVals
  double* half;            // 2m x kHalfVals, side-major
  double* cost_part;       // per edge-kernel block
  int n_cost_parts;
  double* Hd;              // n x 36 undamped
  double* Hdd;             // n x kSymVals damped, identity on held poses
  double* Minv;            // n x kSymVals block-Jacobi inverse
  double* g;               // n x 6
  double *x, *rv, *z, *p, *q;   // PCG vectors, 6n each
  double* red;             // per-block partials, kNumSums arrays of red_nb
  int red_nb;              // PCG blocks
  int64_t n_chunks;        // PCG chunks of pcg_waves(n) x 10 poses
  PcgState* pcg;
  int* host_done;
  StepOut* out;
  int* flags;              // [0] non-finite, [1] not SPD
};

struct DispatchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
DispatchEvents& dispatch_events();

int pcg_waves(int64_t n);
int red_blocks(int64_t n);
int64_t pcg_chunks(int64_t n);
int edge_blocks(int64_t m);
void launch_prep(const double* poses, double* tab, int64_t n, hipStream_t s);
void launch_meas_prep(const double* meas, double* meas_tab, int64_t m, hipStream_t s);
// jac: also store r, J_i and J_j (for inspection).
void launch_edge(const Dev& d, bool jac, hipStream_t s);
void launch_pose(const Dev& d, hipStream_t s);
void launch_pcg_init(const Dev& d, hipStream_t s);

void launch_pcg_a(const Dev& d, int it, hipStream_t s);
void launch_pcg_b(const Dev& d, int it, hipStream_t s);
void launch_pcg_final(const Dev& d, int iters, hipStream_t s);
void launch_retract(const Dev& d, hipStream_t s);
void launch_cost(const Dev& d, const double* tab, hipStream_t s);
void launch_cost_final(const Dev& d, hipStream_t s);
void launch_validate(const Dev& d, const double* meas, int* flags, hipStream_t s);
// Full 6x6 H_ij blocks (m x 36) from the compact ones, for inspection.
void launch_expand_coupling(const Dev& d, double* out, hipStream_t s);

}  // namespace pgo
