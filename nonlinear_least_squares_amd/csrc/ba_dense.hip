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
// run pairs (no atomics, so the result is the same bits on every run).
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
//   panel   one wavefront per tile row i >= k (and the rhs row): the diagonal
//           tile is factored in registers (lane r holds row r; column values
//           move by readlane), redundantly in every wavefront, and the row's
//           tile is solved against it, L_ik = A_ik L_kk^-T;
//   update  one wavefront per trailing tile (i, j), k < j <= i:
//           A_ij -= L_ik L_jk^T with fp64 MFMA (16x16x4), the one dense
//           contraction of the bundle-adjustment pages' methods.
// The factor's diagonal tiles are kept apart (ds_diag); the back-substitution
// L^T dc = y runs in one workgroup, tile by tile.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "ba_kernels.h"

namespace ba {
namespace {

typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kT = 32;            // tile order of the factorisation
constexpr int kAsmThreads = 128;  // threads of an assembly block (81 used)
constexpr int kAsmBatch = 16;     // run pairs staged in LDS at a time
constexpr int kSolveThreads = 1024;

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
// the sum over the block's run pairs of F_a F_b^T, in list order.
__global__ __launch_bounds__(kAsmThreads) void k_ds_assemble(Dev d) {
  __shared__ double s_f[kAsmBatch][54];
  const int blk = blockIdx.x;
  const int2 jj = d.ds_blk[blk];   // x = j2 (row block), y = j1 (column block), j2 >= j1
  const int p0 = d.ds_blk_ptr[blk], p1 = d.ds_blk_ptr[blk + 1];
  const int t = threadIdx.x;
  const int al = t / 9, be = t - 9 * (t / 9);
  double acc = 0.0;
  for (int pb = p0; pb < p1; pb += kAsmBatch) {
    const int np = min(kAsmBatch, p1 - pb);
    for (int e = t; e < np * 54; e += kAsmThreads) {
      const int p = e / 54, k = e - 54 * p;
      const int2 pr = d.ds_pair[pb + p];
      s_f[p][k] = k < 27 ? d.ds_F[27 * (int64_t)pr.x + k] : d.ds_F[27 * (int64_t)pr.y + (k - 27)];
    }
    __syncthreads();
    if (t < 81) {
      for (int p = 0; p < np; ++p) {
        const double* fa = s_f[p] + 3 * al;
        const double* fb = s_f[p] + 27 + 3 * be;
        acc += fa[0] * fb[0] + fa[1] * fb[1] + fa[2] * fb[2];
      }
    }
    __syncthreads();
  }
  if (t < 81) {
    double v = -acc;
    if (jj.x == jj.y) v += d.Bd[45 * (int64_t)jj.x + (al <= be ? sym_idx(9, al, be) : sym_idx(9, be, al))];
    d.ds_S[(9 * (int64_t)jj.x + al) * d.ds_ld + 9 * (int64_t)jj.y + be] = v;
  }
}

// Tile column k: wavefront b factors the diagonal tile and then handles tile
// row k + b (the diagonal tile itself for b = 0; the rhs tile row for
// k + b = T).  Every wavefront reads the diagonal tile, so its factor goes to
// a separate array (ds_diag) rather than back in place.  Lanes 32..63 repeat
// lanes 0..31 and store nothing.
__global__ __launch_bounds__(64) void k_ds_panel(Dev d, int k) {
  const int i = k + blockIdx.x;
  const int r = threadIdx.x & (kT - 1);
  const int64_t ld = d.ds_ld;
  double* S = d.ds_S;
  double a[kT], b[kT];
  const double* arow = S + (int64_t)(kT * k + r) * ld + kT * k;
  const double* brow = S + (int64_t)(kT * i + r) * ld + kT * k;
#pragma unroll
  for (int c = 0; c < kT; ++c) {
    a[c] = arow[c];
    b[c] = brow[c];
  }
  bool bad = false;
#pragma unroll
  for (int c = 0; c < kT; ++c) {
    double piv = lane_bcast(a[c], c);
    if (!(piv > 0.0) || !isfinite(piv)) {
      bad = true;
      piv = 1.0;
    }
    const double lc = sqrt(piv), inv = 1.0 / lc;
    a[c] = r == c ? lc : a[c] * inv;   // L(r, c) for r >= c
    b[c] *= inv;                        // x_c of this row
#pragma unroll
    for (int j = c + 1; j < kT; ++j) {
      const double ljc = lane_bcast(a[c], j);   // L(j, c)
      a[j] -= a[c] * ljc;
      b[j] -= b[c] * ljc;
    }
  }
  if (bad && blockIdx.x == 0 && threadIdx.x == 0) d.flags[1] = 1;
  if (threadIdx.x >= kT) return;
  if (i == k) {
    double* out = d.ds_diag + (int64_t)k * kT * kT + kT * r;
#pragma unroll
    for (int c = 0; c < kT; ++c) out[c] = c <= r ? a[c] : 0.0;
  } else {
    double* out = S + (int64_t)(kT * i + r) * ld + kT * k;
#pragma unroll
    for (int c = 0; c < kT; ++c) out[c] = b[c];
  }
}

// Trailing update after tile column k: one wavefront per tile (i, j) with
// k < j <= i < T, then the rhs tile row (T, j).  A_ij -= L_ik L_jk^T as 2 x 2
// MFMA tiles of 16 x 16 over K = 32 in steps of 4.  Operand layout of
// v_mfma_f64_16x16x4_f64 (lane l): A(m, kk) with m = l % 16, kk = l / 16;
// B(kk, n) with n = l % 16; accumulator element v (0..3) is row 4 v + l / 16
// of column l % 16.
__global__ __launch_bounds__(64) void k_ds_update(Dev d, int k) {
  const int m = d.ds_T - k - 1;          // trailing tile columns
  const int tri = m * (m + 1) / 2;
  const int id = blockIdx.x;
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
  const double* Li = S + (int64_t)(kT * i) * ld + kT * k;
  const double* Lj = S + (int64_t)(kT * j) * ld + kT * k;
  double* C = S + (int64_t)(kT * i) * ld + kT * j;
  double av[2][8], bv[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      av[h][s] = -Li[(int64_t)(16 * h + lr) * ld + 4 * s + lk];
      bv[h][s] = Lj[(int64_t)(16 * h + lr) * ld + 4 * s + lk];
    }
  }
  v4d acc[2][2];
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

// L^T dc = y by tile columns from the last: the contribution of the solved
// unknowns below the tile (a 32-column GEMV over those rows, 32 row groups of
// 32 threads, summed in group order), then the 32 x 32 triangular solve by
// one wavefront holding the tile's columns.  Writes dc and the solver state.
__global__ __launch_bounds__(kSolveThreads) void k_ds_backsolve(Dev d) {
  extern __shared__ double s_x[];               // N_p unknowns
  __shared__ double s_part[kT][kT + 1];
  const int64_t ld = d.ds_ld;
  const double* S = d.ds_S;
  const double* y = S + ld * ld;                // the rhs row after the factorisation
  const int t = threadIdx.x, c = t & (kT - 1), g = t / kT;
  for (int kt = d.ds_T - 1; kt >= 0; --kt) {
    double acc = 0.0;
    for (int64_t row = kT * (int64_t)(kt + 1) + g; row < ld; row += kSolveThreads / kT)
      acc += S[row * ld + kT * kt + c] * s_x[row];
    s_part[g][c] = acc;
    __syncthreads();
    if (t < 64) {
      double col[kT];
#pragma unroll
      for (int e = 0; e < kT; ++e) col[e] = d.ds_diag[(int64_t)kt * kT * kT + kT * e + c];   // L(e, c)
      double v = y[kT * kt + c];
      for (int gg = 0; gg < kSolveThreads / kT; ++gg) v -= s_part[gg][c];
      double xm = 0.0;
#pragma unroll
      for (int e = kT - 1; e >= 0; --e) {
        const double xe = lane_bcast(v, e) / lane_bcast(col[e], e);
        if (c == e) xm = xe;
        if (c < e) v -= col[e] * xe;
      }
      if (t < kT) s_x[kT * kt + c] = xm;
    }
    __syncthreads();
  }
  for (int e = t; e < d.ds_n; e += kSolveThreads) d.x[e] = s_x[e];
  if (t == 0) {
    d.pcg->done = 1;
    d.pcg->iters = 0;
    d.pcg->res_norm = 0.0;
    d.pcg->rhs_norm = 0.0;
    d.pcg->breakdown = 0;
  }
}

template <typename... KArgs, typename... Args>
void launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, uint32_t shmem,
            Args... args) {
  DispatchEvents& ev = dispatch_events();
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0u,
                        static_cast<KArgs>(args)...);
  if (ev.start) {
    ev.used = true;
    ev.start = ev.stop = nullptr;
  }
}

}  // namespace

int ds_tile() { return kT; }

void launch_ds_runs(const Dev& d, hipStream_t s) {
  if (d.ds_nruns > 0) launch(k_ds_runs, dim3((d.ds_nruns + 255) / 256), dim3(256), s, 0u, d);
}
void launch_ds_fill(const Dev& d, hipStream_t s) {
  const int64_t n = ((int64_t)d.ds_ld + kT) * d.ds_ld;
  launch(k_ds_fill, dim3((unsigned)((n + 255) / 256)), dim3(256), s, 0u, d);
}
void launch_ds_assemble(const Dev& d, hipStream_t s) {
  if (d.ds_nblk > 0) launch(k_ds_assemble, dim3(d.ds_nblk), dim3(kAsmThreads), s, 0u, d);
}
void launch_ds_panel(const Dev& d, int k, hipStream_t s) {
  launch(k_ds_panel, dim3(d.ds_T - k + 1), dim3(64), s, 0u, d, k);
}
int ds_update_tiles(const Dev& d, int k) {
  const int m = d.ds_T - k - 1;
  return m * (m + 1) / 2 + m;
}
void launch_ds_update(const Dev& d, int k, hipStream_t s) {
  const int n = ds_update_tiles(d, k);
  if (n > 0) launch(k_ds_update, dim3(n), dim3(64), s, 0u, d, k);
}
hipError_t ds_backsolve_limit(int ld) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ds_backsolve),
                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)(8 * ld));
}
void launch_ds_backsolve(const Dev& d, hipStream_t s) {
  launch(k_ds_backsolve, dim3(1), dim3(kSolveThreads), s, (uint32_t)(8 * d.ds_ld), d);
}

}  // namespace ba
