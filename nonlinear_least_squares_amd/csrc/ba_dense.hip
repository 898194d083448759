// Dense reduced-camera solve for small and medium scenes (gfx950, fp64).
//
// The camera system S dc = rhs of the Schur elimination (the NeRF-SLAM
// reproduction notes, sec. 3.2, eq. (2); the eager-mode BA summary names a
// Cholesky direct solver for small and medium problems) is formed explicitly,
//   S = B~ - sum_i Ebar_i C~_i^-1 Ebar_i^T,
// and factored S = L L^T in place.  Per (point, camera) run r the 9x3 block
// F_r = Ebar_r L_i, with L_i L_i^T = C~_i^-1, turns every point's
// contribution into outer products: S_{j2 j1} -= sum_i F_{i,j2} F_{i,j1}^T.
// Each lower 9x9 block of S is summed by one workgroup over a fixed list of
// run pairs, with fp64 MFMA (no atomics, so the result is the same bits on
// every run).
//
// Storage: S is row-major with leading dimension N_p = 9 n_c rounded up to a
// multiple of 32 (padding: identity on the diagonal, zeros elsewhere).  Row
// N_p holds the right-hand side, and rows N_p + 1 .. N_p + 31 are zero, so the
// right-hand side is one more 32-row tile row of the factorisation: a
// Cholesky factorisation of [[S, b], [b^T, .]] leaves y = L^-1 b in that row.
// Only the lower triangle is read or written after assembly.
//
// Factorisation, right-looking by 32 x 32 tiles, two launches per tile
// column k:
//   panel   one wavefront per tile row i > k (and the rhs row) solves its
//           tile against the factored diagonal tile, L_ik = A_ik L_kk^-T;
//   update  one wavefront per trailing tile (i, j), k < j <= i:
//           A_ij -= L_ik L_jk^T with fp64 MFMA (16x16x4), the one dense
//           contraction of the bundle-adjustment pages' methods; the
//           wavefront of tile (k + 1, k + 1) then factors it (lane r holds
//           row r, column values move by readlane), so the next panel starts
//           from a factored diagonal tile.
// The factor's diagonal tiles are kept apart (ds_diag); the back-substitution
// L^T dc = y runs in one workgroup, tile by tile.
#include <hip/hip_runtime.h>

#include "ba_launch.h"

namespace ba {
namespace {

typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kT = 32;            // tile order of the factorisation
constexpr int kSolveThreads = 1024;
static_assert(kT * kT == kSolveThreads, "the back-substitution loads one diagonal tile per thread");

__device__ __forceinline__ double lane_bcast(double x, int l) {
  const int lo = __builtin_amdgcn_readlane(__double2loint(x), l);
  const int hi = __builtin_amdgcn_readlane(__double2hiint(x), l);
  return __hiloint2double(hi, lo);
}

__device__ __forceinline__ void cam_from_table(const CamT* tab, int j, CamG& c) {
  const CamT& t = tab[j];
#pragma unroll
  for (int k = 0; k < 9; ++k) c.R[k] = t.R[k];
#pragma unroll
  for (int k = 0; k < 3; ++k) c.t[k] = t.t[k];
  c.f = t.f;
  c.k1 = t.k1;
  c.k2 = t.k2;
}

// Per run r (consecutive point-order observations of one point and one
// camera, which share their Jacobians): Ebar = W Jc^T Jp with W the sum of the
// run's robust weights, L = chol(C~^-1) of the point, F = Ebar L.
__global__ void k_ds_runs(Dev d) {
  const int r = blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= d.ds_nruns) return;
  const int b = d.ds_run[r], e = d.ds_run[r + 1];
  const int j = d.o_cam[b], i = d.o_pt[b];
  double W = 0.0;
  for (int s = b; s < e; ++s) W += d.w_pt[s];
  CamG c;
  cam_from_table(d.tab, j, c);
  Geo g;
  geo_eval(c, d.pts[3 * (int64_t)i], d.pts[3 * (int64_t)i + 1], d.pts[3 * (int64_t)i + 2], g);
  double Jc[18], Jp[6];
  jc_rows(g, c.f, Jc);
  jp_rows(g, c.R, Jp);
  // C~^-1 (packed upper: 00 01 02 11 12 22) = L L^T, L lower
  const double* Ci = d.Cinv + 6 * (int64_t)i;
  const double l00 = sqrt(Ci[0]);
  const double l10 = Ci[1] / l00, l20 = Ci[2] / l00;
  const double l11 = sqrt(Ci[3] - l10 * l10);
  const double l21 = (Ci[4] - l20 * l10) / l11;
  const double l22 = sqrt(Ci[5] - l20 * l20 - l21 * l21);
  double* F = d.ds_F + 27 * (int64_t)r;
#pragma unroll
  for (int a = 0; a < 9; ++a) {
    const double e0 = W * (Jc[a] * Jp[0] + Jc[9 + a] * Jp[3]);
    const double e1 = W * (Jc[a] * Jp[1] + Jc[9 + a] * Jp[4]);
    const double e2 = W * (Jc[a] * Jp[2] + Jc[9 + a] * Jp[5]);
    F[3 * a] = e0 * l00 + e1 * l10 + e2 * l20;
    F[3 * a + 1] = e1 * l11 + e2 * l21;
    F[3 * a + 2] = e2 * l22;
  }
}

// S and the rhs rows: zeros, identity on the padded diagonal, rhs in row N_p.
__global__ void k_ds_fill(Dev d) {
  const int64_t ld = d.ds_ld;
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= (ld + kT) * ld) return;
  const int64_t row = e / ld, col = e - row * ld;
  double v = 0.0;
  if (row < ld && row == col && row >= d.ds_n) v = 1.0;
  if (row == ld && col < d.ds_n) v = d.rhs[col];
  d.ds_S[e] = v;
}

// One lower 9x9 block (j2, j1) of S per workgroup: B~ on the diagonal minus
// sum over the block's run pairs (a, b) of F_a F_b^T.  That sum is a product
// of a 9 x 3p and a 3p x 9 matrix, done with fp64 MFMA (16x16x4): one pair per
// instruction, the 9 x 3 blocks padded to 16 x 4 (lane l supplies row l % 16,
// column l / 16 of F_a and of F_b).  The block's pairs are split into
// kAsmWaves contiguous shares, one per wavefront, 16 pairs in flight; the
// wavefronts' sums are added in wavefront order, so the result does not
// depend on timing.
constexpr int kAsmWaves = 4;
__global__ __launch_bounds__(64 * kAsmWaves) void k_ds_assemble(Dev d) {
  __shared__ double s_acc[kAsmWaves][4][64];
  const int blk = blockIdx.x;
  const int2 jj = d.ds_blk[blk];   // x = j2 (row block), y = j1 (column block), j2 >= j1
  const int p0 = d.ds_blk_ptr[blk], p1 = d.ds_blk_ptr[blk + 1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int m = lane & 15, kk = lane >> 4;
  const bool act = m < 9 && kk < 3;
  const int off = act ? 3 * m + kk : 0;
  const int q0 = p0 + (int)(((int64_t)(p1 - p0) * w) / kAsmWaves);
  const int q1 = p0 + (int)(((int64_t)(p1 - p0) * (w + 1)) / kAsmWaves);
  const double* F = d.ds_F;
  v4d acc = {0.0, 0.0, 0.0, 0.0};
  for (int pb = q0; pb < q1; pb += 16) {
    const int nb = min(16, q1 - pb);
    const int2 pr = d.ds_pair[pb + min(lane, nb - 1)];
    double av[16], bv[16];
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int ra = __builtin_amdgcn_readlane(pr.x, q), rb = __builtin_amdgcn_readlane(pr.y, q);
      av[q] = F[27 * (int64_t)ra + off];
      bv[q] = F[27 * (int64_t)rb + off];
    }
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const bool on = act && q < nb;
      acc = __builtin_amdgcn_mfma_f64_16x16x4f64(on ? av[q] : 0.0, on ? bv[q] : 0.0, acc, 0, 0, 0);
    }
  }
#pragma unroll
  for (int v = 0; v < 4; ++v) s_acc[w][v][lane] = acc[v];
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    double tot = 0.0;
#pragma unroll
    for (int u = 0; u < kAsmWaves; ++u) tot += s_acc[u][v][lane];
    const int al = 4 * v + kk, be = m;   // element v of lane l: row 4 v + l / 16, column l % 16
    if (al < 9 && be < 9) {
      double val = -tot;
      if (jj.x == jj.y) val += d.Bd[45 * (int64_t)jj.x + (al <= be ? sym_idx(9, al, be) : sym_idx(9, be, al))];
      d.ds_S[(9 * (int64_t)jj.x + al) * d.ds_ld + 9 * (int64_t)jj.y + be] = val;
    }
  }
}

// 1 / sqrt(x) for x > 0: the hardware estimate and two Newton steps
// y <- y (3 - x y^2) / 2, each doubling the correct bits of an estimate good
// to about 2^-23.
__device__ __forceinline__ double rsqrt_newton(double x) {
  double y = __builtin_amdgcn_rsq(x);
  y = y * fma(-0.5 * x, y * y, 1.5);
  return y * fma(-0.5 * x, y * y, 1.5);
}

// Factor one 32 x 32 diagonal tile held as rows src[r * stride + c] (lane r
// holds row r) into ds_diag (L, row-major, zeros above the diagonal),
// ds_diagT (its transpose) and ds_dinv (1 / L(c, c)).  Column c's values move
// to every lane by readlane.  One wavefront; lanes 32..63 repeat lanes 0..31
// and store nothing.  A pivot that is not positive and finite sets the not-SPD
// flag (and is taken as 1).
__device__ __forceinline__ void factor_diag_tile(const Dev& d, int kt, const double* src,
                                                 int64_t stride) {
  const int r = threadIdx.x & (kT - 1);
  double a[kT];
#pragma unroll
  for (int c = 0; c < kT; ++c) a[c] = src[r * stride + c];
  bool bad = false;
  double myinv = 0.0;
#pragma unroll
  for (int c = 0; c < kT; ++c) {
    double piv = lane_bcast(a[c], c);
    if (!(piv > 0.0) || !isfinite(piv)) {
      bad = true;
      piv = 1.0;
    }
    const double inv = rsqrt_newton(piv);
    a[c] = r == c ? piv * inv : a[c] * inv;   // L(r, c) for r >= c
    if (r == c) myinv = inv;
#pragma unroll
    for (int j = c + 1; j < kT; ++j) a[j] -= a[c] * lane_bcast(a[c], j);   // L(j, c)
  }
  if (bad && threadIdx.x == 0) d.flags[1] = 1;
  if (threadIdx.x >= kT) return;
  double* L = d.ds_diag + (int64_t)kt * kT * kT;
  double* LT = d.ds_diagT + (int64_t)kt * kT * kT;
#pragma unroll
  for (int c = 0; c < kT; ++c) {
    const double v = c <= r ? a[c] : 0.0;
    L[kT * r + c] = v;
    LT[kT * c + r] = v;
  }
  d.ds_dinv[kT * kt + r] = myinv;
}

// The first diagonal tile (the update kernel factors each later one).
__global__ __launch_bounds__(64) void k_ds_diag0(Dev d) {
  factor_diag_tile(d, 0, d.ds_S, d.ds_ld);
}

// Tile column k, its diagonal tile already factored: one wavefront per tile
// row i = k + 1 .. T (T: the rhs tile row) solves L_ik L_kk^T = A_ik in place,
// lane r taking row r.  The factor's columns and pivot reciprocals are staged
// in LDS and read at wavefront-uniform addresses (broadcasts).
// Row r (lane r & 31) of one tile at `row` (stride ld) solved in place
// against the factored diagonal tile k, X L_kk^T = A: the factor's columns and
// pivot reciprocals are staged in LDS (s_l, kT * kT + kT doubles) and read at
// wavefront-uniform addresses (broadcasts).
// With `ident` the tile starts as the identity instead of being read.
__device__ __forceinline__ void panel_solve(const Dev& d, int k, double* row, double* s_l,
                                            bool ident) {
  const double* LT = d.ds_diagT + (int64_t)k * kT * kT;
  const int r = threadIdx.x & (kT - 1);
  double b[kT];
#pragma unroll
  for (int c = 0; c < kT; ++c) b[c] = ident ? (c == r ? 1.0 : 0.0) : row[c];
  double lt[kT * kT / 64];
#pragma unroll
  for (int u = 0; u < kT * kT / 64; ++u) lt[u] = LT[threadIdx.x + 64 * u];
#pragma unroll
  for (int u = 0; u < kT * kT / 64; ++u) s_l[threadIdx.x + 64 * u] = lt[u];
  if (threadIdx.x < kT) s_l[kT * kT + threadIdx.x] = d.ds_dinv[kT * k + threadIdx.x];
  __syncthreads();
#pragma unroll
  for (int c = 0; c < kT; ++c) {
    b[c] *= s_l[kT * kT + c];
#pragma unroll
    for (int j = c + 1; j < kT; ++j) b[j] -= b[c] * s_l[kT * c + j];   // L(j, c)
  }
  if (threadIdx.x >= kT) return;
#pragma unroll
  for (int c = 0; c < kT; ++c) row[c] = b[c];
}

// Tile column k, its diagonal tile already factored: one wavefront per tile
// row i = k + 1 .. T (T: the rhs tile row) solves L_ik L_kk^T = A_ik in place,
// lane r taking row r.  With `cov`, k + 1 more wavefronts solve the tiles
// Z_jk (j <= k) of Z = L^-T against the same L_kk^T (Z_kk from the identity).
__global__ __launch_bounds__(64) void k_ds_panel(Dev d, int k, int cov) {
  __shared__ double s_l[kT * kT + kT];
  const int nds = d.ds_T - k;
  const int b = blockIdx.x;
  const int r = threadIdx.x & (kT - 1);
  const int row_tile = b < nds ? k + 1 + b : b - nds;
  panel_solve(d, k, d.ds_S + (int64_t)(kT * row_tile + r) * d.ds_ld + kT * k, s_l,
              b >= nds && row_tile == k);
}

// C -= A B^T for 32 x 32 tiles of S (leading dimension ld) as 2 x 2 MFMA
// tiles of 16 x 16 over K = 32 in steps of 4; the accumulators are left in acc.
// Operand layout of v_mfma_f64_16x16x4_f64 (lane l): A(m, kk) with m = l % 16,
// kk = l / 16; B(kk, n) with n = l % 16; accumulator element v (0..3) is row
// 4 v + l / 16 of column l % 16.
__device__ __forceinline__ void tile_sub_abt(double* C, const double* A, const double* B,
                                             int64_t ld, v4d (&acc)[2][2]) {
  const int l = threadIdx.x;
  const int lr = l & 15, lk = l >> 4;
  double av[2][8], bv[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      av[h][s] = -A[(int64_t)(16 * h + lr) * ld + 4 * s + lk];
      bv[h][s] = B[(int64_t)(16 * h + lr) * ld + 4 * s + lk];
    }
  }
#pragma unroll
  for (int mh = 0; mh < 2; ++mh)
#pragma unroll
    for (int nh = 0; nh < 2; ++nh)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[mh][nh][v] = C[(int64_t)(16 * mh + 4 * v + lk) * ld + 16 * nh + lr];
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int mh = 0; mh < 2; ++mh)
#pragma unroll
      for (int nh = 0; nh < 2; ++nh)
        acc[mh][nh] = __builtin_amdgcn_mfma_f64_16x16x4f64(av[mh][s], bv[nh][s], acc[mh][nh], 0, 0, 0);
#pragma unroll
  for (int mh = 0; mh < 2; ++mh)
#pragma unroll
    for (int nh = 0; nh < 2; ++nh)
#pragma unroll
      for (int v = 0; v < 4; ++v) C[(int64_t)(16 * mh + 4 * v + lk) * ld + 16 * nh + lr] = acc[mh][nh][v];
}

// Trailing update after tile column k: one wavefront per tile (i, j) with
// k < j <= i < T, then the rhs tile row (T, j): A_ij -= L_ik L_jk^T.  The
// wavefront of tile (k + 1, k + 1) then factors that tile for the next panel.
// With `cov`, one more wavefront per tile Z_ji, j <= k < i: Z_ji -= Z_jk L_ik^T.
__global__ __launch_bounds__(64) void k_ds_update(Dev d, int k, int cov) {
  const int m = d.ds_T - k - 1;          // trailing tile columns
  const int tri = m * (m + 1) / 2;
  const int id = blockIdx.x;
  if (id >= tri + m) {
    const int cid = id - (tri + m);
    const int j = cid % (k + 1), i = k + 1 + cid / (k + 1);
    const int64_t ld = d.ds_ld;
    double* S = d.ds_S;
    v4d acc[2][2];
    tile_sub_abt(S + (int64_t)(kT * j) * ld + kT * i, S + (int64_t)(kT * j) * ld + kT * k,
                 S + (int64_t)(kT * i) * ld + kT * k, ld, acc);
    return;
  }
  int i, j;
  if (id < tri) {
    int ii = (int)((sqrt(8.0 * id + 1.0) - 1.0) * 0.5);
    while ((ii + 1) * (ii + 2) / 2 <= id) ++ii;
    while (ii * (ii + 1) / 2 > id) --ii;
    i = k + 1 + ii;
    j = k + 1 + (id - ii * (ii + 1) / 2);
  } else {
    i = d.ds_T;
    j = k + 1 + (id - tri);
  }
  const int l = threadIdx.x;
  const int lr = l & 15, lk = l >> 4;
  const int64_t ld = d.ds_ld;
  double* S = d.ds_S;
  v4d acc[2][2];
  tile_sub_abt(S + (int64_t)(kT * i) * ld + kT * j, S + (int64_t)(kT * i) * ld + kT * k,
               S + (int64_t)(kT * j) * ld + kT * k, ld, acc);
  if (id == 0) {
    // tile (k + 1, k + 1) is final now: factor it for the next panel, its
    // rows passed through LDS
    __shared__ double s_t[kT * kT];
#pragma unroll
    for (int mh = 0; mh < 2; ++mh)
#pragma unroll
      for (int nh = 0; nh < 2; ++nh)
#pragma unroll
        for (int v = 0; v < 4; ++v) s_t[(16 * mh + 4 * v + lk) * kT + 16 * nh + lr] = acc[mh][nh][v];
    __syncthreads();
    factor_diag_tile(d, k + 1, s_t, kT);
  }
}

// ---- camera marginal covariance: blocks of S^-1 = L^-T L^-1 ---------------
//
// Z = L^-T (upper triangular) is formed by tiles in the strictly upper tiles
// of S, which the factorisation never reads, and in its diagonal tiles once
// they are factored (the factor's diagonal tiles live in ds_diag).  Z L^T = I
// gives, tile by tile,
//   Z_jk L_kk^T = delta_jk I - sum_{m < k} Z_jm L_km^T,
// so the factorisation's launches carry it along: the panel of tile column k
// also solves the tiles Z_jk, j <= k, against L_kk^T, and the update after it
// also takes them out of the later columns, Z_ji -= Z_jk L_ik^T for j <= k < i.
// Each camera's 9x9 block of S^-1 = Z Z^T is then the 45 dot products of its
// 9 rows of Z.

// Zeros in the strictly upper tiles of S (the assembly may have written the
// upper part of a diagonal 9x9 block there), before the factorisation.
__global__ void k_cov_zero(Dev d) {
  const int64_t ld = d.ds_ld;
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e >= ld * ld) return;
  const int64_t row = e / ld, col = e - row * ld;
  if (col / kT > row / kT) d.ds_S[e] = 0.0;
}

// One workgroup per camera c: rows r_a = 9 c + a of Z (a < 9), each nonzero
// from its own tile's first column on; cov_c[a][b] = sum over columns of
// Z[r_a] Z[r_b].  Thread t takes columns t, t + 256, ...; the 45 sums are
// reduced across the wavefront, then over the four wavefronts in order.
__global__ __launch_bounds__(256) void k_cov_blocks(Dev d, double* out) {
  __shared__ double s_part[4][45];
  const int c = blockIdx.x;
  const int64_t ld = d.ds_ld, n = d.ds_n;
  const int64_t r0 = 9 * (int64_t)c;
  const double* Z = d.ds_S;
  int64_t start[9];
#pragma unroll
  for (int a = 0; a < 9; ++a) start[a] = (r0 + a) / kT * kT;
  double acc[45];
#pragma unroll
  for (int q = 0; q < 45; ++q) acc[q] = 0.0;
  for (int64_t col = start[0] + threadIdx.x; col < n; col += 256) {
    double z[9];
#pragma unroll
    for (int a = 0; a < 9; ++a) z[a] = col >= start[a] ? Z[(r0 + a) * ld + col] : 0.0;
    int q = 0;
#pragma unroll
    for (int a = 0; a < 9; ++a)
#pragma unroll
      for (int b = a; b < 9; ++b, ++q) acc[q] += z[a] * z[b];
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 45; ++q) {
    double v = acc[q];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    if (lane == 0) s_part[w][q] = v;
  }
  __syncthreads();
  if (threadIdx.x < 45) {
    const int q = threadIdx.x;
    const double v = ((s_part[0][q] + s_part[1][q]) + s_part[2][q]) + s_part[3][q];
    int a = 0, rem = q;
    while (rem >= 9 - a) {
      rem -= 9 - a;
      ++a;
    }
    const int b = a + rem;
    out[81 * (int64_t)c + 9 * a + b] = v;
    out[81 * (int64_t)c + 9 * b + a] = v;
  }
}

// L^T dc = y by tile columns from the last, right-looking: v starts as y (in
// LDS); for each tile column kt, one wavefront solves the 32 x 32 triangle
// L_kk^T x_kt = v_kt (lane c holds column c of L_kk; the pivots' reciprocals
// are formed up front, so each of the 32 dependent steps is a broadcast and a
// multiply-add), then all threads take x_kt out of the unknowns above it,
// v_j -= sum_e L(32 kt + e, j) x_e for j < 32 kt, reading tile row kt of L
// row by row (coalesced; 32 loads in flight per column).  The next diagonal
// tile is loaded one step ahead.  Writes dc and the solver state.
__global__ __launch_bounds__(kSolveThreads) void k_ds_backsolve(Dev d) {
  extern __shared__ double s_v[];               // N_p: y, then x where solved
  __shared__ double s_diag[kT * kT];
  const int64_t ld = d.ds_ld;
  const double* S = d.ds_S;
  const double* y = S + ld * ld;                // the rhs row after the factorisation
  const int t = threadIdx.x, c = t & (kT - 1);
  for (int64_t j = t; j < ld; j += kSolveThreads) s_v[j] = y[j];
  s_diag[t] = d.ds_diag[(int64_t)(d.ds_T - 1) * kT * kT + t];   // kT * kT == kSolveThreads
  __syncthreads();
  for (int kt = d.ds_T - 1; kt >= 0; --kt) {
    const double dg_next = d.ds_diag[(int64_t)max(kt - 1, 0) * kT * kT + t];
    if (t < 64) {
      double col[kT];
#pragma unroll
      for (int e = 0; e < kT; ++e) col[e] = s_diag[kT * e + c];   // L(e, c)
      double dsel = col[0];
#pragma unroll
      for (int e = 1; e < kT; ++e)
        if (c == e) dsel = col[e];
      const double inv = 1.0 / dsel;
      double v = s_v[kT * kt + c];
      double xm = 0.0;
#pragma unroll
      for (int e = kT - 1; e >= 0; --e) {
        const double xe = lane_bcast(v * inv, e);
        if (c == e) xm = xe;
        if (c < e) v -= col[e] * xe;
      }
      if (t < kT) s_v[kT * kt + c] = xm;
    }
    __syncthreads();
    s_diag[t] = dg_next;
    const double* Lrow = S + (int64_t)(kT * kt) * ld;
    for (int64_t j = t; j < kT * (int64_t)kt; j += kSolveThreads) {
      double lv[kT];
#pragma unroll
      for (int e = 0; e < kT; ++e) lv[e] = Lrow[e * ld + j];
      double acc = 0.0;
#pragma unroll
      for (int e = 0; e < kT; ++e) acc += lv[e] * s_v[kT * kt + e];
      s_v[j] -= acc;
    }
    __syncthreads();
  }
  for (int e = t; e < d.ds_n; e += kSolveThreads) d.x[e] = s_v[e];
  if (t == 0) {
    d.pcg->done = 1;
    d.pcg->iters = 0;
    d.pcg->res_norm = 0.0;
    d.pcg->rhs_norm = 0.0;
    d.pcg->breakdown = 0;
  }
}

}  // namespace

int ds_tile() { return kT; }

void launch_cov_zero(const Dev& d, hipStream_t s) {
  const int64_t n = (int64_t)d.ds_ld * d.ds_ld;
  launch_timed(k_cov_zero, dim3((unsigned)((n + 255) / 256)), dim3(256), s, 0u, d);
}
int cov_update_tiles(const Dev& d, int k) { return (k + 1) * (d.ds_T - k - 1); }
void launch_cov_blocks(const Dev& d, double* out, int64_t n_cams, hipStream_t s) {
  if (n_cams > 0) launch_timed(k_cov_blocks, dim3((unsigned)n_cams), dim3(256), s, 0u, d, out);
}

void launch_ds_runs(const Dev& d, hipStream_t s) {
  if (d.ds_nruns > 0) launch_timed(k_ds_runs, dim3((d.ds_nruns + 255) / 256), dim3(256), s, 0u, d);
}
void launch_ds_fill(const Dev& d, hipStream_t s) {
  const int64_t n = ((int64_t)d.ds_ld + kT) * d.ds_ld;
  launch_timed(k_ds_fill, dim3((unsigned)((n + 255) / 256)), dim3(256), s, 0u, d);
}
void launch_ds_assemble(const Dev& d, hipStream_t s) {
  if (d.ds_nblk > 0) launch_timed(k_ds_assemble, dim3(d.ds_nblk), dim3(64 * kAsmWaves), s, 0u, d);
}
void launch_ds_diag0(const Dev& d, hipStream_t s) { launch_timed(k_ds_diag0, dim3(1), dim3(64), s, 0u, d); }
void launch_ds_panel(const Dev& d, int k, int cov, hipStream_t s) {
  launch_timed(k_ds_panel, dim3(d.ds_T - k + (cov ? k + 1 : 0)), dim3(64), s, 0u, d, k, cov);
}
int ds_update_tiles(const Dev& d, int k) {
  const int m = d.ds_T - k - 1;
  return m * (m + 1) / 2 + m;
}
void launch_ds_update(const Dev& d, int k, int cov, hipStream_t s) {
  const int n = ds_update_tiles(d, k) + (cov ? cov_update_tiles(d, k) : 0);
  if (n > 0) launch_timed(k_ds_update, dim3(n), dim3(64), s, 0u, d, k, cov);
}
hipError_t ds_backsolve_limit(int ld) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ds_backsolve),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)(8 * ld));
}
void launch_ds_backsolve(const Dev& d, hipStream_t s) {
  launch_timed(k_ds_backsolve, dim3(1), dim3(kSolveThreads), s, (uint32_t)(8 * d.ds_ld), d);
}

}  // namespace ba
