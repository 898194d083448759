// Pose-graph optimisation kernels (gfx950, fp64).
//
// Pose T = (R, t) maps body to world; an edge (i, j) measures T_i^-1 T_j as
// (R_e, t_e).  Residual r = [r_R; r_t], r_R = Log(R_e^T R_i^T R_j),
// r_t = R_i^T (t_j - t_i) - t_e, weighted by Omega = diag(w_R I, w_t I);
// tangent [dphi; dt] with R <- R Exp(dphi), t <- t + dt.  With
// u = R_i^T (t_j - t_i), Q = R_i^T, J = Jr^-1(r_R) (inverse right Jacobian of
// SO(3)) and A = -J R_j^T R_i, the Jacobian blocks are
//   dr/dxi_i = [[A, 0], [[u]x, -Q]],   dr/dxi_j = [[J, 0], [0, Q]],
// so J^T Omega J splits into 3x3 products (the eager-mode BA summary's pose
// graph: Lie-group operations give each residual and its Jacobian blocks;
// the Theseus note's retraction and analytic tangent derivatives).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pgo_kernels.h"
#include "ba_model.h"   // quat_from_rotvec, quat_to_R

namespace pgo {
namespace {

using ba::quat_from_rotvec;
using ba::quat_to_R;

__device__ __forceinline__ void mat3_tmul(const double* A, const double* B, double* C) {   // A^T B
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) C[3 * i + j] = A[i] * B[j] + A[3 + i] * B[3 + j] + A[6 + i] * B[6 + j];
}

__device__ __forceinline__ void mat3_mul(const double* A, const double* B, double* C) {
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
      C[3 * i + j] = A[3 * i] * B[j] + A[3 * i + 1] * B[3 + j] + A[3 * i + 2] * B[6 + j];
}

// Log of a rotation matrix through its unit quaternion (largest-component
// branch), 2 atan2(|v|, q_w) v / |v| with q_w >= 0.
__device__ __forceinline__ void so3_log(const double* R, double* w) {
  const double tr = R[0] + R[4] + R[8];
  double q0, q1, q2, q3;
  if (tr > R[0] && tr > R[4] && tr > R[8]) {
    const double s = 2.0 * sqrt(1.0 + tr);
    q0 = 0.25 * s;
    q1 = (R[7] - R[5]) / s;
    q2 = (R[2] - R[6]) / s;
    q3 = (R[3] - R[1]) / s;
  } else if (R[0] >= R[4] && R[0] >= R[8]) {
    const double s = 2.0 * sqrt(1.0 + R[0] - R[4] - R[8]);
    q0 = (R[7] - R[5]) / s;
    q1 = 0.25 * s;
    q2 = (R[1] + R[3]) / s;
    q3 = (R[2] + R[6]) / s;
  } else if (R[4] >= R[8]) {
    const double s = 2.0 * sqrt(1.0 + R[4] - R[0] - R[8]);
    q0 = (R[2] - R[6]) / s;
    q1 = (R[1] + R[3]) / s;
    q2 = 0.25 * s;
    q3 = (R[5] + R[7]) / s;
  } else {
    const double s = 2.0 * sqrt(1.0 + R[8] - R[0] - R[4]);
    q0 = (R[3] - R[1]) / s;
    q1 = (R[2] + R[6]) / s;
    q2 = (R[5] + R[7]) / s;
    q3 = 0.25 * s;
  }
  if (q0 < 0.0) {
    q0 = -q0;
    q1 = -q1;
    q2 = -q2;
    q3 = -q3;
  }
  const double vn = sqrt(q1 * q1 + q2 * q2 + q3 * q3);
  const double k = vn < 1e-12 ? 2.0 / q0 : 2.0 * atan2(vn, q0) / vn;
  w[0] = k * q1;
  w[1] = k * q2;
  w[2] = k * q3;
}

// Inverse right Jacobian of SO(3): I + [w]x / 2 + c(a) [w]x^2,
// c = 1/a^2 - (1 + cos a) / (2 a sin a), its series 1/12 + a^2/720 near 0.
__device__ __forceinline__ void so3_jr_inv(const double* w, double* J) {
  const double a2 = w[0] * w[0] + w[1] * w[1] + w[2] * w[2], a = sqrt(a2);
  const double c = a < 1e-4 ? 1.0 / 12.0 + a2 / 720.0 : 1.0 / a2 - (1.0 + cos(a)) / (2.0 * a * sin(a));
  const double K[9] = {0.0, -w[2], w[1], w[2], 0.0, -w[0], -w[1], w[0], 0.0};
#pragma unroll
  for (int i = 0; i < 3; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const double k2 = K[3 * i] * K[j] + K[3 * i + 1] * K[3 + j] + K[3 * i + 2] * K[6 + j];
      J[3 * i + j] = (i == j ? 1.0 : 0.0) + 0.5 * K[3 * i + j] + c * k2;
    }
}

// Per pose (or measurement): R (9) and t (3) from [w, t].
__global__ void k_prep(const double* __restrict__ x, double* __restrict__ tab, int64_t n) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= n) return;
  double q[4], R[9];
  quat_from_rotvec(x[6 * i], x[6 * i + 1], x[6 * i + 2], q);
  quat_to_R(q, R);
#pragma unroll
  for (int k = 0; k < 9; ++k) tab[12 * i + k] = R[k];
#pragma unroll
  for (int k = 0; k < 3; ++k) tab[12 * i + 9 + k] = x[6 * i + 3 + k];
}

// Residual of one edge, and when J is set the Jacobian pieces of the header.
__device__ __forceinline__ double edge_eval(const Dev& d, const double* tab, int64_t e, double* r,
                                            double* Jr, double* A, double* u, double* Q) {
  const int2 ij = d.edges[e];
  const double* Ti = tab + 12 * (int64_t)ij.x;
  const double* Tj = tab + 12 * (int64_t)ij.y;
  const double* Me = d.meas_tab + 12 * e;
  double Rel[9], E[9];
  mat3_tmul(Ti, Tj, Rel);   // R_i^T R_j
  mat3_tmul(Me, Rel, E);    // R_e^T R_i^T R_j
  so3_log(E, r);
  const double dt0 = Tj[9] - Ti[9], dt1 = Tj[10] - Ti[10], dt2 = Tj[11] - Ti[11];
#pragma unroll
  for (int a = 0; a < 3; ++a) {
    u[a] = Ti[a] * dt0 + Ti[3 + a] * dt1 + Ti[6 + a] * dt2;
    r[3 + a] = u[a] - Me[9 + a];
  }
  const double wR = d.info[2 * e], wt = d.info[2 * e + 1];
  const double c = 0.5 * (wR * (r[0] * r[0] + r[1] * r[1] + r[2] * r[2]) +
                          wt * (r[3] * r[3] + r[4] * r[4] + r[5] * r[5]));
  if (Jr) {
    so3_jr_inv(r, Jr);
    double B[9];
    mat3_tmul(Tj, Ti, B);   // R_j^T R_i
    mat3_mul(Jr, B, A);
#pragma unroll
    for (int k = 0; k < 9; ++k) A[k] = -A[k];
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int b = 0; b < 3; ++b) Q[3 * a + b] = Ti[3 * b + a];   // R_i^T
  }
  return c;
}

__device__ __forceinline__ double block_sum(double v, double* s_buf) {
  // fixed-order sum over a 256-thread block
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) s_buf[w] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0)
    for (int k = 0; k < (int)(blockDim.x >> 6); ++k) t += s_buf[k];
  return t;
}

// Per edge: residual, Jacobians, the three blocks of J^T Omega J, both ends'
// g parts, and a per-block partial of the cost.  The residual and the
// Jacobian blocks are stored only for inspection (kJac); the products are
// written as 16-byte pieces, the ends' shares side-major (all side-0 rows in
// edge order, then all side-1 rows).
template <bool kJac>
__global__ __launch_bounds__(256) void k_edge(Dev d) {
  __shared__ double s_buf[4];
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  double c = 0.0;
  if (e < d.m) {
    double r[6], Jr[9], A[9], u[3], Q[9];
    c = edge_eval(d, d.tab, e, r, Jr, A, u, Q);
    const double wR = d.info[2 * e], wt = d.info[2 * e + 1];
    const double U[9] = {0.0, -u[2], u[1], u[2], 0.0, -u[0], -u[1], u[0], 0.0};
    if (kJac) {
      // Jacobians, row-major 6x6
      double* Ji = d.Ji + 36 * e;
      double* Jj = d.Jj + 36 * e;
#pragma unroll
      for (int a = 0; a < 3; ++a)
#pragma unroll
        for (int b = 0; b < 3; ++b) {
          Ji[6 * a + b] = A[3 * a + b];
          Ji[6 * a + 3 + b] = 0.0;
          Ji[6 * (3 + a) + b] = U[3 * a + b];
          Ji[6 * (3 + a) + 3 + b] = -Q[3 * a + b];
          Jj[6 * a + b] = Jr[3 * a + b];
          Jj[6 * a + 3 + b] = 0.0;
          Jj[6 * (3 + a) + b] = 0.0;
          Jj[6 * (3 + a) + 3 + b] = Q[3 * a + b];
        }
#pragma unroll
      for (int k = 0; k < 6; ++k) d.r[6 * e + k] = r[k];
    }
    double AtA[9], UtU[9], UtQ[9], QtQ[9], JtJ[9], AtJ[9];
    mat3_tmul(A, A, AtA);
    mat3_tmul(U, U, UtU);
    mat3_tmul(U, Q, UtQ);
    mat3_tmul(Q, Q, QtQ);
    mat3_tmul(Jr, Jr, JtJ);
    mat3_tmul(A, Jr, AtJ);
    double Hi[kHalfVals], Hj[kHalfVals], Hc[kCoupVals];
#pragma unroll
    for (int a = 0; a < 3; ++a)
#pragma unroll
      for (int b = 0; b < 3; ++b) {
        Hi[6 * a + b] = wR * AtA[3 * a + b] + wt * UtU[3 * a + b];
        Hi[6 * a + 3 + b] = -wt * UtQ[3 * a + b];
        Hi[6 * (3 + a) + b] = -wt * UtQ[3 * b + a];
        Hi[6 * (3 + a) + 3 + b] = wt * QtQ[3 * a + b];
        Hj[6 * a + b] = wR * JtJ[3 * a + b];
        Hj[6 * a + 3 + b] = 0.0;
        Hj[6 * (3 + a) + b] = 0.0;
        Hj[6 * (3 + a) + 3 + b] = wt * QtQ[3 * a + b];
        Hc[3 * a + b] = wR * AtJ[3 * a + b];
        Hc[9 + 3 * a + b] = wt * UtQ[3 * a + b];
      }
    Hc[18] = -wt;
    Hc[19] = 0.0;
#pragma unroll
    for (int a = 0; a < 3; ++a) {
      const double aR = A[a] * r[0] + A[3 + a] * r[1] + A[6 + a] * r[2];
      const double uT = U[a] * r[3] + U[3 + a] * r[4] + U[6 + a] * r[5];
      const double qT = Q[a] * r[3] + Q[3 + a] * r[4] + Q[6 + a] * r[5];
      const double jR = Jr[a] * r[0] + Jr[3 + a] * r[1] + Jr[6 + a] * r[2];
      Hi[36 + a] = wR * aR + wt * uT;
      Hi[39 + a] = -wt * qT;
      Hj[36 + a] = wR * jR;
      Hj[39 + a] = wt * qT;
    }
    double2* hi = reinterpret_cast<double2*>(d.half + kHalfVals * e);
    double2* hj = reinterpret_cast<double2*>(d.half + kHalfVals * (d.m + e));
    double2* hc = reinterpret_cast<double2*>(d.Hc + kCoupVals * e);
#pragma unroll
    for (int k = 0; k < kHalfVals / 2; ++k) {
      hi[k] = make_double2(Hi[2 * k], Hi[2 * k + 1]);
      hj[k] = make_double2(Hj[2 * k], Hj[2 * k + 1]);
    }
#pragma unroll
    for (int k = 0; k < kCoupVals / 2; ++k) hc[k] = make_double2(Hc[2 * k], Hc[2 * k + 1]);
  }
  const double t = block_sum(c, s_buf);
  if (threadIdx.x == 0) d.cost_part[blockIdx.x] = t;
}

// 6x6 SPD inverse by Cholesky (row-major in and out); false if a pivot fails.
__device__ __forceinline__ bool inv6(const double* H, double* Mi) {
  double L[36];
#pragma unroll
  for (int k = 0; k < 36; ++k) L[k] = H[k];
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    double s = L[7 * j];
#pragma unroll
    for (int k = 0; k < j; ++k) s -= L[6 * j + k] * L[6 * j + k];
    if (!(s > 0.0) || !isfinite(s)) return false;
    const double dj = sqrt(s);
    L[7 * j] = dj;
#pragma unroll
    for (int i = j + 1; i < 6; ++i) {
      double t = L[6 * i + j];
#pragma unroll
      for (int k = 0; k < j; ++k) t -= L[6 * i + k] * L[6 * j + k];
      L[6 * i + j] = t / dj;
    }
  }
#pragma unroll
  for (int c = 0; c < 6; ++c) {
    double y[6];
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      double s = i == c ? 1.0 : 0.0;
#pragma unroll
      for (int k = 0; k < i; ++k) s -= L[6 * i + k] * y[k];
      y[i] = s / L[7 * i];
    }
#pragma unroll
    for (int i = 5; i >= 0; --i) {
      double s = y[i];
#pragma unroll
      for (int k = i + 1; k < 6; ++k) s -= L[6 * k + i] * y[k];
      y[i] = s / L[7 * i];
    }
#pragma unroll
    for (int i = 0; i < 6; ++i) Mi[6 * i + c] = y[i];
  }
  return true;
}

// Per pose: H and g summed over its half edges in list order, Marquardt
// damping of the diagonal (floored), identity on held poses, block-Jacobi
// inverse.
__global__ __launch_bounds__(128) void k_pose(Dev d) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= d.n) return;
  double H[36], g[6];
#pragma unroll
  for (int k = 0; k < 36; ++k) H[k] = 0.0;
#pragma unroll
  for (int k = 0; k < 6; ++k) g[k] = 0.0;
  for (int h = d.half_ptr[i]; h < d.half_ptr[i + 1]; ++h) {
    const int hid = d.nbr[h].x;   // 2 e + side; rows are side-major
    const double2* src =
        reinterpret_cast<const double2*>(d.half + kHalfVals * ((hid & 1) * d.m + (hid >> 1)));
#pragma unroll
    for (int k = 0; k < 18; ++k) {
      const double2 v = src[k];
      H[2 * k] += v.x;
      H[2 * k + 1] += v.y;
    }
#pragma unroll
    for (int k = 0; k < 3; ++k) {
      const double2 v = src[18 + k];
      g[2 * k] += v.x;
      g[2 * k + 1] += v.y;
    }
  }
#pragma unroll
  for (int k = 0; k < 36; ++k) d.Hd[36 * i + k] = H[k];
#pragma unroll
  for (int k = 0; k < 6; ++k) d.g[6 * i + k] = g[k];
  if (i < d.n_fixed) {
#pragma unroll
    for (int k = 0; k < 36; ++k) H[k] = (k % 7 == 0) ? 1.0 : 0.0;
  } else {
#pragma unroll
    for (int a = 0; a < 6; ++a) H[7 * a] += d.lambda * fmax(H[7 * a], d.diag_floor);
  }
  double Mi[36];
  if (!inv6(H, Mi)) d.flags[1] = 1;
  int k = 0;
#pragma unroll
  for (int a = 0; a < 6; ++a)
#pragma unroll
    for (int b = a; b < 6; ++b, ++k) {
      d.Hdd[kSymVals * i + k] = H[6 * a + b];
      d.Minv[kSymVals * i + k] = Mi[6 * a + b];
    }
}

// Index of entry (a, b) of a symmetric 6x6 block kept as its upper triangle.
__device__ __forceinline__ int sym_idx(int a, int b) {
  const int i = min(a, b), j = max(a, b);
  return i * (11 - i) / 2 + j;
}

// ---- PCG on H~ dx = -g: six lanes per pose, ten poses per wavefront ---------
//
// As in the bundle-adjustment solve, the product is applied to z, and
// p = z + beta p and q = H~ p = H~ z + beta q follow by recurrence, so one
// kernel does the product, the stop test and the recurrences and a second the
// update of x, r and z.  The poses are cut into chunks of W x 10 (ten per
// wavefront of a block of W); at most kMaxPcgBlocks blocks each take a fixed
// set of chunks, so each block leaves one partial per sum and every block can
// add all the partials itself, in a fixed order, to get the same totals.
// Large graphs use blocks of 16 wavefronts (one per compute unit), smaller
// ones blocks of 4, so that they still spread over many compute units.

struct Lane {
  int64_t i;   // pose (clamped on idle lanes)
  int a;       // row 0..5
  int base;    // first lane of the pose's group
  bool on;
};

// The chunks of this block.  Blocks are handed to the eight XCDs in turn
// (block b to XCD b mod 8); each XCD takes one contiguous range of chunks,
// in proportion to its blocks, and its blocks take that range's chunks in
// turn, so a pose's graph neighbours, whose z and H_ij it gathers, mostly sit
// in the same XCD's L2.
struct Chunks {
  int64_t first, end;
  int step;
};

__device__ __forceinline__ Chunks my_chunks(int64_t n_chunks) {
  const int G = gridDim.x, b = blockIdx.x, x = b % 8, l = b / 8;
  const int per = G / 8, rem = G % 8;
  const int bx = per + (x < rem ? 1 : 0);
  const int sx = x * per + min(x, rem);
  const int64_t cb = n_chunks * sx / G, ce = n_chunks * (sx + bx) / G;
  return {cb + l, ce, bx};
}

template <int W>
__device__ __forceinline__ Lane pose_lane(int64_t chunk, int64_t n) {
  const int lane = threadIdx.x & 63;
  Lane l;
  const int64_t i = chunk * (W * kPosesPerWave) + (threadIdx.x >> 6) * kPosesPerWave + lane / 6;
  l.on = lane < 6 * kPosesPerWave && i < n;
  l.i = l.on ? i : 0;
  l.a = lane % 6;
  l.base = lane - lane % 6;
  if (lane >= 6 * kPosesPerWave) {
    l.a = 0;
    l.base = 0;
  }
  return l;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return __shfl(v, 0, 64);
}

// Sum over the block's W wavefronts in wave order (every thread gets it).
template <int W>
__device__ __forceinline__ double block_waves_sum(double v, double* s_buf) {
  v = wave_sum(v);
  if ((threadIdx.x & 63) == 0) s_buf[threadIdx.x >> 6] = v;
  __syncthreads();
  double t = 0.0;
#pragma unroll
  for (int w = 0; w < W; ++w) t += s_buf[w];
  return t;
}

__device__ __forceinline__ double partial_sum(const double* a, int n) {
  const int lane = threadIdx.x & 63;
  double v = 0.0;
  for (int k = lane; k < n; k += 64) v += a[k];
  return wave_sum(v);
}

__device__ __forceinline__ double* red_arr(const Dev& d, int k) { return d.red + k * d.red_nb; }

// Total of partial array k, the same in every block.
__device__ __forceinline__ double total(const Dev& d, int k) {
  return partial_sum(red_arr(d, k), d.red_nb);
}

// row a of (M v) for the pose of this lane group, M symmetric (upper triangle)
__device__ __forceinline__ double apply_sym6(const double* M, const Lane& l, double v) {
  double s = 0.0;
#pragma unroll
  for (int b = 0; b < 6; ++b) s += M[sym_idx(l.a, b)] * __shfl(v, l.base + b, 64);
  return s;
}

__device__ __forceinline__ void stop_pcg(const Dev& d, int iters, double res, double rhs,
                                         int breakdown) {
  d.pcg->done = 1;
  d.pcg->iters = iters;
  d.pcg->res_norm = res;
  d.pcg->rhs_norm = rhs;
  d.pcg->breakdown = breakdown;
  *d.host_done = 1;
  __threadfence_system();
}

template <int W>
__global__ __launch_bounds__(64 * W) void k_pcg_init(Dev d) {
  __shared__ double s_rr[W], s_rz[W];
  double rr = 0.0, rz = 0.0;
  const Chunks ch = my_chunks(d.n_chunks);
  for (int64_t c = ch.first; c < ch.end; c += ch.step) {
    const Lane l = pose_lane<W>(c, d.n);
    const int64_t e = 6 * l.i + l.a;
    const double b = (l.on && l.i >= d.n_fixed) ? -d.g[e] : 0.0;
    const double z = apply_sym6(d.Minv + kSymVals * l.i, l, b);
    if (l.on) {
      d.x[e] = 0.0;
      d.rv[e] = b;
      d.z[e] = z;
      rr += b * b;
      rz += b * z;
    }
  }
  rr = block_waves_sum<W>(rr, s_rr);
  rz = block_waves_sum<W>(rz, s_rz);
  if (threadIdx.x == 0) {
    red_arr(d, kRR0)[blockIdx.x] = rr;
    red_arr(d, kRZ0)[blockIdx.x] = rz;
    red_arr(d, kBB)[blockIdx.x] = rr;
    if (blockIdx.x == 0) {
      d.pcg->done = 0;
      d.pcg->iters = 0;
      d.pcg->breakdown = 0;
    }
  }
}

// Entry of the compact H_ij that multiplies z_other[b] in row a of this
// pose's product: side 0 (this pose is the edge's i) takes row a of H_ij,
// side 1 (it is the edge's j) row a of H_ij^T.  With H_ij = [[M, N], [0, -w I]]
// held as M (0..8), N (9..17), -w (18), 0 (19):
//   side 0, a < 3: M[a][b] (b < 3), N[a][b-3];   a >= 3: -w if b == a
//   side 1, a < 3: M[b][a] (b < 3), 0;           a >= 3: N[b][a-3] (b < 3), -w if b == a
__device__ __forceinline__ int coup_idx(int side, int a, int b) {
  if (side == 0) {
    if (a < 3) return b < 3 ? 3 * a + b : 9 + 3 * a + (b - 3);
    return b == a ? 18 : 19;
  }
  if (a < 3) return b < 3 ? 3 * b + a : 19;
  return b < 3 ? 9 + 3 * b + (a - 3) : (b == a ? 18 : 19);
}

template <int W>
__global__ __launch_bounds__(64 * W) void k_pcg_a(Dev d, int it) {
  __shared__ double s_buf[W];
  __shared__ double s_coup[W][4 * kPosesPerWave * kCoupVals];   // 4 slots x 10 poses
  __shared__ double s_hdd[W][kPosesPerWave * kSymVals];          // 10 damped blocks
  if (d.pcg->done) return;
  const double rhs = sqrt(total(d, kBB));
  if (it == 0) {
    if (rhs == 0.0) {
      if (blockIdx.x == 0 && threadIdx.x == 0) stop_pcg(d, 0, 0.0, 0.0, 0);
      return;
    }
  } else {
    const double res = sqrt(total(d, kRR0 + (it & 1)));
    if (res <= d.tol * rhs) {
      if (blockIdx.x == 0 && threadIdx.x == 0) stop_pcg(d, it, res, rhs, 0);
      return;
    }
  }
  const double beta = it > 0 ? total(d, kRZ0 + (it & 1)) / total(d, kRZ0 + ((it + 1) & 1)) : 0.0;
  const int lane = threadIdx.x & 63, grp = lane / 6;
  double* s_c = s_coup[threadIdx.x >> 6];
  double* s_h = s_hdd[threadIdx.x >> 6] + min(grp, kPosesPerWave - 1) * kSymVals;
  double pq = 0.0;
  const Chunks ch = my_chunks(d.n_chunks);
  for (int64_t c = ch.first; c < ch.end; c += ch.step) {
    const Lane l = pose_lane<W>(c, d.n);
    const int64_t e = 6 * l.i + l.a;
    // the pose's 21 damped-block values are fetched once by its six lanes
    // (a, a + 6, a + 12, a + 18) and passed through LDS
    const double zi = d.z[e];
    double hv4[4];
    {
      const double* Hp = d.Hdd + kSymVals * l.i;
#pragma unroll
      for (int u = 0; u < 3; ++u) hv4[u] = Hp[6 * u + l.a];
      hv4[3] = l.a < 3 ? Hp[18 + l.a] : 0.0;
    }
    const bool free_pose = l.on && l.i >= d.n_fixed;
    const int h0 = d.half_ptr[l.i], h1 = free_pose ? d.half_ptr[l.i + 1] : h0;
    const double pe = d.p[e], qe = d.q[e];
    if (lane < 6 * kPosesPerWave) {
#pragma unroll
      for (int u = 0; u < 3; ++u) s_h[6 * u + l.a] = hv4[u];
      if (l.a < 3) s_h[18 + l.a] = hv4[3];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    double w = 0.0;
#pragma unroll
    for (int b = 0; b < 6; ++b) w += s_h[sym_idx(l.a, b)] * __shfl(zi, l.base + b, 64);
    // Half edges four at a time, so that their gathers are in flight
    // together.  Past the end of the list the last entry is loaded again and
    // its terms are zeroed (w + 0 * z is w), so the terms still add up in list
    // order.  The six lanes of a pose share the loads: lane a fetches element
    // a of the other end's z, passed to the group by shuffles, and 16-byte
    // pieces a and a + 6 of the 20-double coupling block, staged in the
    // wavefront's LDS rows, from which each lane reads its six coefficients.
    for (int h = h0; h < h1; h += 4) {
      int2 nb[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) nb[k] = d.nbr[min(h + k, h1 - 1)];
      double2 c0[4], c1[4];
      double zk[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double2* src = reinterpret_cast<const double2*>(d.Hc + kCoupVals * (int64_t)(nb[k].x >> 1));
        c0[k] = src[l.a];
        c1[k] = l.a < 4 ? src[6 + l.a] : make_double2(0.0, 0.0);
        zk[k] = d.z[6 * (int64_t)nb[k].y + l.a];
      }
      if (lane < 6 * kPosesPerWave) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          double* row = s_c + (k * kPosesPerWave + grp) * kCoupVals;
          row[2 * l.a] = c0[k].x;
          row[2 * l.a + 1] = c0[k].y;
          if (l.a < 4) {
            row[12 + 2 * l.a] = c1[k].x;
            row[13 + 2 * l.a] = c1[k].y;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const double* row = s_c + (k * kPosesPerWave + min(grp, kPosesPerWave - 1)) * kCoupVals;
        const bool live = h + k < h1;
        const int side = nb[k].x & 1;
#pragma unroll
        for (int b = 0; b < 6; ++b) {
          const double v = row[coup_idx(side, l.a, b)];
          w += (live ? v : 0.0) * __shfl(zk[k], l.base + b, 64);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (l.on) {
      double pn = zi, qn = w;
      if (it > 0) {
        pn = zi + beta * pe;
        qn = w + beta * qe;
      }
      d.p[e] = pn;
      d.q[e] = qn;
      pq += pn * qn;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  pq = block_waves_sum<W>(pq, s_buf);
  if (threadIdx.x == 0) red_arr(d, kPQ)[blockIdx.x] = pq;
}

template <int W>
__global__ __launch_bounds__(64 * W) void k_pcg_b(Dev d, int it) {
  __shared__ double s_rr[W], s_rz[W];
  if (d.pcg->done) return;
  const double pq = total(d, kPQ);
  if (!(pq > 0.0) || !isfinite(pq)) {
    // every block reads its totals before block 0 stops the solve
    const double rhs = sqrt(total(d, kBB)), res = sqrt(total(d, kRR0 + (it & 1)));
    if (blockIdx.x == 0 && threadIdx.x == 0) stop_pcg(d, it, res, rhs, 1);
    return;
  }
  const double alpha = total(d, kRZ0 + (it & 1)) / pq;
  double rr = 0.0, rz = 0.0;
  const Chunks ch = my_chunks(d.n_chunks);
  for (int64_t c = ch.first; c < ch.end; c += ch.step) {
    const Lane l = pose_lane<W>(c, d.n);
    const int64_t e = 6 * l.i + l.a;
    double mrow[6];
#pragma unroll
    for (int b = 0; b < 6; ++b) mrow[b] = d.Minv[kSymVals * l.i + sym_idx(l.a, b)];
    const double xe = d.x[e], re = d.rv[e], pe = d.p[e], qe = d.q[e];
    double r = 0.0;
    if (l.on) {
      d.x[e] = xe + alpha * pe;
      r = re - alpha * qe;
      d.rv[e] = r;
    }
    double z = 0.0;
#pragma unroll
    for (int b = 0; b < 6; ++b) z += mrow[b] * __shfl(r, l.base + b, 64);
    if (l.on) {
      d.z[e] = z;
      rr += r * r;
      rz += r * z;
    }
  }
  rr = block_waves_sum<W>(rr, s_rr);
  rz = block_waves_sum<W>(rz, s_rz);
  if (threadIdx.x == 0) {
    red_arr(d, kRR0 + ((it + 1) & 1))[blockIdx.x] = rr;
    red_arr(d, kRZ0 + ((it + 1) & 1))[blockIdx.x] = rz;
  }
}

__global__ __launch_bounds__(64) void k_pcg_final(Dev d, int iters) {
  if (d.pcg->done) return;
  const double rhs = sqrt(total(d, kBB));
  const double res = iters == 0 ? rhs : sqrt(total(d, kRR0 + (iters & 1)));
  if (threadIdx.x == 0) stop_pcg(d, iters, res, rhs, 0);
}

// Trial poses: q(R) (x) q(dphi) in the hemisphere q_w >= 0, back to axis-angle
// by 2 atan2(|v|, q_w) v / |v|; t + dt.  Held poses are copied.
__global__ void k_retract(Dev d) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i >= d.n) return;
  const double* x = d.poses + 6 * i;
  double* o = d.trial + 6 * i;
  if (i < d.n_fixed) {
#pragma unroll
    for (int k = 0; k < 6; ++k) o[k] = x[k];
    return;
  }
  const double* dx = d.x + 6 * i;
  double a[4], b[4];
  quat_from_rotvec(x[0], x[1], x[2], a);
  quat_from_rotvec(dx[0], dx[1], dx[2], b);
  double q0 = a[0] * b[0] - a[1] * b[1] - a[2] * b[2] - a[3] * b[3];
  double q1 = a[0] * b[1] + a[1] * b[0] + a[2] * b[3] - a[3] * b[2];
  double q2 = a[0] * b[2] - a[1] * b[3] + a[2] * b[0] + a[3] * b[1];
  double q3 = a[0] * b[3] + a[1] * b[2] - a[2] * b[1] + a[3] * b[0];
  if (q0 < 0.0) {
    q0 = -q0;
    q1 = -q1;
    q2 = -q2;
    q3 = -q3;
  }
  const double vn = sqrt(q1 * q1 + q2 * q2 + q3 * q3);
  const double k = vn < 1e-12 ? 2.0 / q0 : 2.0 * atan2(vn, q0) / vn;
  o[0] = k * q1;
  o[1] = k * q2;
  o[2] = k * q3;
#pragma unroll
  for (int c = 0; c < 3; ++c) o[3 + c] = x[3 + c] + dx[3 + c];
}

__global__ __launch_bounds__(256) void k_cost(Dev d, const double* tab) {
  __shared__ double s_buf[4];
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  double c = 0.0;
  if (e < d.m) {
    double r[6], u[3];
    c = edge_eval(d, tab, e, r, nullptr, nullptr, u, nullptr);
  }
  const double t = block_sum(c, s_buf);
  if (threadIdx.x == 0) d.cost_part[blockIdx.x] = t;
}

__global__ __launch_bounds__(256) void k_cost_final(Dev d) {
  __shared__ double s_buf[4];
  double v = 0.0;
  for (int k = threadIdx.x; k < d.n_cost_parts; k += 256) v += d.cost_part[k];
  const double t = block_sum(v, s_buf);
  if (threadIdx.x == 0) {
    d.out->trial_cost = t;
    d.out->pcg_iters = d.pcg->iters;
    d.out->pcg_rel_res = d.pcg->rhs_norm > 0.0 ? d.pcg->res_norm / d.pcg->rhs_norm : 0.0;
    d.out->nonfinite = isfinite(t) ? 0 : 1;
    d.out->not_spd = d.flags[1];
  }
}

// Inputs: edge indices in range and distinct, values finite, weights positive.
__global__ void k_validate(Dev d, const double* meas, int* flags) {
  const int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k < d.m) {
    const int2 ij = d.edges[k];
    if (ij.x < 0 || ij.x >= d.n || ij.y < 0 || ij.y >= d.n || ij.x == ij.y) flags[1] = 1;
    for (int c = 0; c < 6; ++c)
      if (!isfinite(meas[6 * k + c])) flags[0] = 1;
    if (!(d.info[2 * k] > 0.0) || !(d.info[2 * k + 1] > 0.0) || !isfinite(d.info[2 * k]) ||
        !isfinite(d.info[2 * k + 1]))
      flags[1] = 1;
  }
  if (k < d.n)
    for (int c = 0; c < 6; ++c)
      if (!isfinite(d.poses[6 * k + c])) flags[0] = 1;
}

__global__ void k_expand_coupling(Dev d, double* out) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= d.m) return;
  const double* Hc = d.Hc + kCoupVals * e;
#pragma unroll
  for (int a = 0; a < 6; ++a)
#pragma unroll
    for (int b = 0; b < 6; ++b) out[36 * e + 6 * a + b] = Hc[coup_idx(0, a, b)];
}

template <typename... KArgs, typename... Args>
void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, Args... args) {
  DispatchEvents& ev = dispatch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, 0u, s, ev.start, ev.stop, 0u,
                        static_cast<KArgs>(args)...);
  if (ev.start) {
    ev.used = true;
    ev.start = ev.stop = nullptr;
  }
}

unsigned blocks(int64_t n, int t) { return (unsigned)((n + t - 1) / t); }

}  // namespace

DispatchEvents& dispatch_events() {
  thread_local DispatchEvents ev;
  return ev;
}

int pcg_waves(int64_t n) {
  return (n + kBigPcgWaves * kPosesPerWave - 1) / (kBigPcgWaves * kPosesPerWave) >= kMaxPcgBlocks
             ? kBigPcgWaves : kSmallPcgWaves;
}
int64_t pcg_chunks(int64_t n) {
  const int64_t c = (int64_t)pcg_waves(n) * kPosesPerWave;
  return (n + c - 1) / c;
}
int red_blocks(int64_t n) { return (int)std::max<int64_t>(std::min<int64_t>(pcg_chunks(n), kMaxPcgBlocks), 1); }
int edge_blocks(int64_t m) { return (int)std::max<int64_t>((m + 255) / 256, 1); }

void launch_prep(const double* poses, double* tab, int64_t n, hipStream_t s) {
  if (n > 0) launch(k_prep, dim3(blocks(n, 256)), dim3(256), s, poses, tab, n);
}
void launch_meas_prep(const double* meas, double* meas_tab, int64_t m, hipStream_t s) {
  if (m > 0) launch(k_prep, dim3(blocks(m, 256)), dim3(256), s, meas, meas_tab, m);
}
void launch_edge(const Dev& d, bool jac, hipStream_t s) {
  if (jac) launch(k_edge<true>, dim3(edge_blocks(d.m)), dim3(256), s, d);
  else launch(k_edge<false>, dim3(edge_blocks(d.m)), dim3(256), s, d);
}
void launch_pose(const Dev& d, hipStream_t s) { launch(k_pose, dim3(blocks(d.n, 128)), dim3(128), s, d); }
void launch_pcg_init(const Dev& d, hipStream_t s) {
  if (pcg_waves(d.n) == kBigPcgWaves)
    launch(k_pcg_init<kBigPcgWaves>, dim3(d.red_nb), dim3(64 * kBigPcgWaves), s, d);
  else
    launch(k_pcg_init<kSmallPcgWaves>, dim3(d.red_nb), dim3(64 * kSmallPcgWaves), s, d);
}
void launch_pcg_a(const Dev& d, int it, hipStream_t s) {
  if (pcg_waves(d.n) == kBigPcgWaves)
    launch(k_pcg_a<kBigPcgWaves>, dim3(d.red_nb), dim3(64 * kBigPcgWaves), s, d, it);
  else
    launch(k_pcg_a<kSmallPcgWaves>, dim3(d.red_nb), dim3(64 * kSmallPcgWaves), s, d, it);
}
void launch_pcg_b(const Dev& d, int it, hipStream_t s) {
  if (pcg_waves(d.n) == kBigPcgWaves)
    launch(k_pcg_b<kBigPcgWaves>, dim3(d.red_nb), dim3(64 * kBigPcgWaves), s, d, it);
  else
    launch(k_pcg_b<kSmallPcgWaves>, dim3(d.red_nb), dim3(64 * kSmallPcgWaves), s, d, it);
}
void launch_pcg_final(const Dev& d, int iters, hipStream_t s) {
  launch(k_pcg_final, dim3(1), dim3(64), s, d, iters);
}
void launch_retract(const Dev& d, hipStream_t s) { launch(k_retract, dim3(blocks(d.n, 256)), dim3(256), s, d); }
void launch_cost(const Dev& d, const double* tab, hipStream_t s) {
  launch(k_cost, dim3(edge_blocks(d.m)), dim3(256), s, d, tab);
}
void launch_cost_final(const Dev& d, hipStream_t s) { launch(k_cost_final, dim3(1), dim3(256), s, d); }
void launch_expand_coupling(const Dev& d, double* out, hipStream_t s) {
  if (d.m > 0) launch(k_expand_coupling, dim3(blocks(d.m, 256)), dim3(256), s, d, out);
}
void launch_validate(const Dev& d, const double* meas, int* flags, hipStream_t s) {
  const int64_t n = std::max<int64_t>(std::max<int64_t>(d.n, d.m), 1);
  launch(k_validate, dim3(blocks(n, 256)), dim3(256), s, d, meas, flags);
}

}  // namespace pgo
