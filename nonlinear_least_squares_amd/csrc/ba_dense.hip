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
// Factorisation, right-looking by 32 x 32 tiles, one launch per tile column
// (k_ds_step): the trailing update after column k, A_ij -= L_ik L_jk^T with
// fp64 MFMA (16x16x4), the one dense contraction of the bundle-adjustment
// pages' methods, fused with the panel of column k + 1: the blocks of that
// column form and factor its diagonal tile themselves and solve their own
// tiles against it, L_ik = A_ik L_kk^-T.  The covariance's tiles of Z = L^-T
// ride in the same launches.  The factor's diagonal tiles are kept apart
// (ds_diag); the back-substitution L^T dc = y runs by 128-row blocks over
// many workgroups (k_ds_bsolve).
#include <hip/hip_runtime.h>

#include "ba_launch.h"

namespace ba {
namespace {

typedef double v4d __attribute__((ext_vector_type(4)));

constexpr int kT = 32;            // tile order of the factorisation

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

constexpr int kH = kT / 2;                       // half a tile
constexpr int kFactorScratch = 2 * kH * kH + kT;   // LDS doubles factor_tile uses

// Factor in place the 32 x 32 tile whose row r lane r holds in a[] (lanes
// 32..63 repeat lanes 0..31): afterwards a[c] = L(r, c) for c <= r (the
// entries above the diagonal are left meaningless) and s_x[2 kH^2 + c] =
// 1 / L(c, c).  Blocked by halves: the first 16 columns by rows, each column's
// entries moving to every lane by readlane and only the first 16 columns
// updated; then the trailing block A22 - L21 L21^T with fp64 MFMA
// (16x16x4), its operands and result passed through LDS (s_x, kFactorScratch
// doubles); then its 16 columns as the first.  Readlane throughput bounds the
// unblocked form, and the blocking halves the broadcasts (272 for 528).  A
// pivot that is not positive and finite sets `bad` and is taken as 1.  Every
// caller runs the same instructions on the same data, so each holds the same
// bits.
__device__ __forceinline__ void factor_tile(double (&a)[kT], double* s_x, bool& bad) {
  const int r = threadIdx.x & (kT - 1);
  double* s_p = s_x;                  // L21, rows 16..31 of the tile, 16 x 16
  double* s_q = s_x + kH * kH;        // A22
  double* s_inv = s_x + 2 * kH * kH;
  bad = false;
#pragma unroll
  for (int c = 0; c < kT; ++c) {
    if (c == kH) {
      if (r >= kH) {
#pragma unroll
        for (int u = 0; u < kH; ++u) {
          s_p[kH * (r - kH) + u] = a[u];
          s_q[kH * (r - kH) + u] = a[kH + u];
        }
      }
      __syncthreads();
      // acc(m, n) = A22(m, n) - sum_k L21(m, k) L21(n, k); both operands take
      // L21(l % 16, 4 s + l / 16) (see tile_sub_abt for the layout)
      const int l = threadIdx.x;
      const int lr = l & 15, lk = l >> 4;
      v4d acc;
      double pv[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[v] = s_q[kH * (4 * v + lk) + lr];
#pragma unroll
      for (int st = 0; st < 4; ++st) pv[st] = s_p[kH * lr + 4 * st + lk];
#pragma unroll
      for (int st = 0; st < 4; ++st) acc = __builtin_amdgcn_mfma_f64_16x16x4f64(-pv[st], pv[st], acc, 0, 0, 0);
      // each lane writes back the elements it read
#pragma unroll
      for (int v = 0; v < 4; ++v) s_q[kH * (4 * v + lk) + lr] = acc[v];
      __syncthreads();
      // lanes of rows 0..15 take a row of it too, into entries they never use
#pragma unroll
      for (int u = 0; u < kH; ++u) a[kH + u] = s_q[kH * (r & (kH - 1)) + u];
    }
    double piv = lane_bcast(a[c], c);
    if (!(piv > 0.0) || !isfinite(piv)) {
      bad = true;
      piv = 1.0;
    }
    const double inv = rsqrt_newton(piv);
    a[c] *= inv;   // L(r, c); on lane c, piv * inv
    s_inv[c] = inv;   // the same value from every lane
    const int e = c < kH ? kH : kT;
#pragma unroll
    for (int j = c + 1; j < e; ++j) a[j] -= a[c] * lane_bcast(a[c], j);   // L(j, c)
  }
  __syncthreads();
}

// C -= A B^T for 32 x 32 tiles of S (leading dimension ld) as 2 x 2 MFMA
// tiles of 16 x 16 over K = 32 in steps of 4; the accumulators are left in acc.
// Operand layout of v_mfma_f64_16x16x4_f64 (lane l): A(m, kk) with m = l % 16,
// kk = l / 16; B(kk, n) with n = l % 16; accumulator element v (0..3) is row
// 4 v + l / 16 of column l % 16.
__device__ __forceinline__ void tile_sub_abt(double* C, const double* A, const double* B,
                                             int64_t ld, v4d (&acc)[2][2], int64_t lda = 0) {
  const int64_t la = lda ? lda : ld;
  const int l = threadIdx.x;
  const int lr = l & 15, lk = l >> 4;
  double av[2][8], bv[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      av[h][s] = -A[(int64_t)(16 * h + lr) * la + 4 * s + lk];
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

// The diagonal tile and one tile of the same tile column after the update,
// accd = Cd - B B^T and acco = Co - Ao B^T (no subtraction without `sub`),
// with every load issued before the first product: B (the tile column's
// block of the previous column, L_dk) serves as both operands of the first
// and as the right operand of the second.
__device__ __forceinline__ void tile_abt_pair(const double* Cd, const double* Co, const double* Ao,
                                              const double* B, int64_t ld, bool sub,
                                              v4d (&accd)[2][2], v4d (&acco)[2][2], int64_t ldco = 0,
                                              int64_t ldao = 0) {
  const int64_t lc = ldco ? ldco : ld, la = ldao ? ldao : ld;
  const int l = threadIdx.x;
  const int lr = l & 15, lk = l >> 4;
  // the diagonal tile is accumulated negated, -(Cd) + B B^T, and negated
  // back (exact), so that both products take B as it is loaded
#pragma unroll
  for (int mh = 0; mh < 2; ++mh)
#pragma unroll
    for (int nh = 0; nh < 2; ++nh)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int64_t o = (int64_t)(16 * mh + 4 * v + lk) * ld + 16 * nh + lr;
        accd[mh][nh][v] = -Cd[o];
        acco[mh][nh][v] = Co[(int64_t)(16 * mh + 4 * v + lk) * lc + 16 * nh + lr];
      }
  if (sub) {
  double bv[2][8], ao[2][8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      bv[h][s] = B[(int64_t)(16 * h + lr) * ld + 4 * s + lk];
      ao[h][s] = -Ao[(int64_t)(16 * h + lr) * la + 4 * s + lk];
    }
  }
#pragma unroll
  for (int s = 0; s < 8; ++s)
#pragma unroll
    for (int mh = 0; mh < 2; ++mh)
#pragma unroll
      for (int nh = 0; nh < 2; ++nh) {
        accd[mh][nh] = __builtin_amdgcn_mfma_f64_16x16x4f64(bv[mh][s], bv[nh][s], accd[mh][nh], 0, 0, 0);
        acco[mh][nh] = __builtin_amdgcn_mfma_f64_16x16x4f64(ao[mh][s], bv[nh][s], acco[mh][nh], 0, 0, 0);
      }
  }
#pragma unroll
  for (int mh = 0; mh < 2; ++mh)
#pragma unroll
    for (int nh = 0; nh < 2; ++nh) accd[mh][nh] = -accd[mh][nh];
}

// The accumulator tile as rows of s_t (kT x kT, row-major).
__device__ __forceinline__ void acc_to_rows(const v4d (&acc)[2][2], double* s_t) {
  const int l = threadIdx.x;
  const int lr = l & 15, lk = l >> 4;
#pragma unroll
  for (int mh = 0; mh < 2; ++mh)
#pragma unroll
    for (int nh = 0; nh < 2; ++nh)
#pragma unroll
      for (int v = 0; v < 4; ++v) s_t[(16 * mh + 4 * v + lk) * kT + 16 * nh + lr] = acc[mh][nh][v];
}

// Factor the diagonal tile whose row r lane r holds in a[] (lanes 32..63
// repeat lanes 0..31) with factor_tile, s_l serving as its scratch, leaving
// its transpose and the pivot reciprocals in s_l (the layout solve_rows
// reads) and, with `to_global`, in ds_diag, ds_dinv and (with `write_lt`)
// ds_diagT.
__device__ __forceinline__ void factor_rows(const Dev& d, int kt, double (&a)[kT], double* s_l,
                                            bool to_global, bool write_lt = true) {
  const int r = threadIdx.x & (kT - 1);
  bool bad;
  factor_tile(a, s_l, bad);
  const double myinv = s_l[2 * kH * kH + r];
  __syncthreads();
  if (threadIdx.x >= kT) return;
#pragma unroll
  for (int c = 0; c < kT; ++c) s_l[kT * c + r] = c <= r ? a[c] : 0.0;
  s_l[kT * kT + r] = myinv;
  if (!to_global) return;
  if (bad) d.flags[1] = 1;
  double* L = d.ds_diag + (int64_t)kt * kT * kT;
  double* LT = d.ds_diagT + (int64_t)kt * kT * kT;
#pragma unroll
  for (int c = 0; c < kT; ++c) {
    const double v = c <= r ? a[c] : 0.0;
    L[kT * r + c] = v;
    if (write_lt) LT[kT * c + r] = v;
  }
  d.ds_dinv[kT * kt + r] = myinv;
}

// Row r (lane r) of the tile held as rows of s_t solved against the factor
// in s_l, X L^T = A, and stored to dst (stride ld).
__device__ __forceinline__ void solve_rows(const double* s_t, const double* s_l, double* dst,
                                           int64_t ld) {
  const int r = threadIdx.x & (kT - 1);
  double b[kT];
#pragma unroll
  for (int c = 0; c < kT; ++c) b[c] = s_t[r * kT + c];
#pragma unroll
  for (int c = 0; c < kT; ++c) {
    b[c] *= s_l[kT * kT + c];
#pragma unroll
    for (int j = c + 1; j < kT; ++j) b[j] -= b[c] * s_l[kT * c + j];   // L(j, c)
  }
  if (threadIdx.x >= kT) return;
#pragma unroll
  for (int c = 0; c < kT; ++c) dst[(int64_t)r * ld + c] = b[c];
}

// One step of the factorisation: the trailing update after tile column k
// (none for k = -1) and the panel of tile column kc = k + 1 in one launch, so
// that the chain is one launch per tile column.  With m = T - kc, block
// b < m takes tile (kc + b, kc) and block m the rhs tile (T, kc): each forms
// the diagonal tile A_dd - L_dk L_dk^T of column kc and factors it (the same
// instructions on the same data in every block, so the same bits; block 0
// also stores the factor), then updates its own tile and solves it in place,
// L_ikc = (A_ikc - L_ik L_kck^T) L_dd^-T.  No block writes the diagonal tile
// of S, so each reads it before its update.  With `cov` (the covariance),
// kc + 1 more blocks do the same for the tiles Z_jkc (j <= kc) of Z = L^-T,
// Z_jkc L_dd^T = delta_jkc I - Z_jk L_kck^T, which keep Z's earlier updates
// in the strictly upper tiles of S; Z_kckc, which starts as the identity, goes
// to ds_diagT (the diagonal tile of S is still being read in this launch).
// The remaining blocks, after a short sleep, take the other trailing tiles
// (i, j), kc < j <= i < T, and rhs tiles (T, j), j > kc, and only update them,
// and with `cov` the tiles Z_ji -= Z_jk L_ik^T, j <= k < kc < i.  The column
// blocks come first, so their longer chains start in the first round.
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_ds_step(Dev d, int k, int cov) {
  __shared__ double s_t[kT * kT];
  __shared__ double s_l[kT * kT + kT];
  const int T = d.ds_T, kc = k + 1, m = T - kc;
  const int k0 = max(k, 0);
  const bool sub = k >= 0;
  const int64_t ld = d.ds_ld;
  double* S = d.ds_S;
  double* Zd = d.ds_diagT;   // Z's diagonal tiles, with `cov`
  const int id = blockIdx.x;
  const int ncol = m + 1, nzp = cov ? kc + 1 : 0;
  v4d acc[2][2];
  if (id >= ncol + nzp) {
    // Column kc's blocks start the chain the next launch waits on; about
    // 1.7 us of sleep here lets their loads reach memory ahead of the
    // trailing tiles' (1.61 -> 1.54 ms per medium LM step; more was slower).
    __builtin_amdgcn_s_sleep(32);
    __builtin_amdgcn_s_sleep(32);
    const int rid = id - ncol - nzp;
    const int ntr = (m - 1) * m / 2, nts = ntr + m - 1;
    if (rid < nts) {
      int i, j;
      if (rid < ntr) {
        int ii = (int)((sqrt(8.0 * rid + 1.0) - 1.0) * 0.5);
        while ((ii + 1) * (ii + 2) / 2 <= rid) ++ii;
        while (ii * (ii + 1) / 2 > rid) --ii;
        i = kc + 1 + ii;
        j = kc + 1 + (rid - ii * (ii + 1) / 2);
      } else {
        i = T;
        j = kc + 1 + (rid - ntr);
      }
      tile_sub_abt(S + (int64_t)(kT * i) * ld + kT * j, S + (int64_t)(kT * i) * ld + kT * k0,
                   S + (int64_t)(kT * j) * ld + kT * k0, ld, acc);
    } else {
      const int zid = rid - nts;
      const int j = zid % (k + 1), i = kc + 1 + zid / (k + 1);
      const double* Zjk = j == k ? Zd + (int64_t)k * kT * kT : S + (int64_t)(kT * j) * ld + kT * k;
      tile_sub_abt(S + (int64_t)(kT * j) * ld + kT * i, Zjk, S + (int64_t)(kT * i) * ld + kT * k, ld, acc,
                   j == k ? kT : ld);
    }
    return;
  }
  const bool zt = id >= ncol;
  const int j = id - ncol;
  const bool ident = zt && j == kc;
  const double* Ld = S + (int64_t)(kT * kc) * ld + kT * k0;
  const double* Cd = S + (int64_t)(kT * kc) * ld + kT * kc;
  double* own;
  const double* Ao;
  int64_t ldo, ldao;
  if (!zt) {
    const int i = id < m ? kc + id : T;
    own = S + (int64_t)(kT * i) * ld + kT * kc;
    Ao = S + (int64_t)(kT * i) * ld + kT * k0;
    ldo = ld;
    ldao = ld;
  } else if (!ident) {
    own = S + (int64_t)(kT * j) * ld + kT * kc;
    Ao = j == k ? Zd + (int64_t)k * kT * kT : S + (int64_t)(kT * j) * ld + kT * k0;
    ldo = ld;
    ldao = j == k ? kT : ld;
  } else {
    own = Zd + (int64_t)kc * kT * kT;
    Ao = Ld;   // not used: the tile starts as the identity
    ldo = kT;
    ldao = ld;
  }
  v4d acco[2][2];
  tile_abt_pair(Cd, ident ? Cd : own, Ao, Ld, ld, sub, acc, acco, ident ? ld : ldo, ldao);
  // the diagonal tile's rows go to the lanes through s_t, which then takes
  // the block's own tile (so that its accumulators are not held through the
  // factorisation)
  acc_to_rows(acc, s_t);
  __syncthreads();
  const int r = threadIdx.x & (kT - 1);
  double a[kT];
#pragma unroll
  for (int c = 0; c < kT; ++c) a[c] = s_t[r * kT + c];
  __syncthreads();
  if (id != 0) {
    if (ident) {
#pragma unroll
      for (int c = 0; c < kT; ++c) s_t[r * kT + c] = c == r ? 1.0 : 0.0;
    } else {
      acc_to_rows(acco, s_t);
    }
  }
  factor_rows(d, kc, a, s_l, id == 0, !cov);
  __syncthreads();
  if (id == 0) return;
  solve_rows(s_t, s_l, own, ldo);
}

// ---- camera marginal covariance: blocks of S^-1 = L^-T L^-1 ---------------
//
// Z = L^-T (upper triangular) is formed by tiles in the strictly upper tiles
// of S, which the factorisation never reads, and its diagonal tiles in
// ds_diagT (the factor's diagonal tiles live in ds_diag).  Z L^T = I gives,
// tile by tile,
//   Z_jk L_kk^T = delta_jk I - sum_{m < k} Z_jm L_km^T,
// so the factorisation's launches carry it along (k_ds_step with `cov`): the
// launch of tile column k also solves the tiles Z_jk, j <= k, against L_kk^T,
// and takes the tiles of column k - 1 out of the later columns,
// Z_ji -= Z_j,k-1 L_i,k-1^T for j <= k - 1 < k < i.
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
    for (int a = 0; a < 9; ++a)
      z[a] = col < start[a] ? 0.0
           : (col < start[a] + kT ? d.ds_diagT[start[a] * kT + (r0 + a - start[a]) * kT + (col - start[a])]
                                  : Z[(r0 + a) * ld + col]);
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

// Back-substitution L^T x = y by blocks of kBsTiles tiles (128 rows) from the
// last, one launch per block b = B - 1 .. 0 (B = ceil(T / kBsTiles)), with
// v (y with the solved blocks' contributions taken out) and x in ds_v:
//   workgroup 0 stages the block's ten tiles in LDS (its diagonal tiles of
//   the factor from ds_diag, the six below them from S, each a contiguous
//   32 x 32 slot), takes x_{b+1}, which the previous launch solved, out of
//   its own block, v_b -= L_{b+1,b}^T x_{b+1}, then solves L_bb^T x_b = v_b
//   tile by tile from the bottom: each 32 x 32 triangle by one wavefront
//   (lane c holds column c of the diagonal tile with its pivot set apart, so
//   each of the 32 steps is a broadcast and a multiply-add on every lane),
//   then the tile's x taken out of the block's rows above it.
//   The other workgroups take x_{b+1} out of the rows above block b, 64
//   columns each, v_j -= sum_e L(r_e, j) x_{b+1}(e), four quarters of the
//   rows summed in a fixed order; in the first launch (no x_{b+1}) they copy
//   y into v.
// Row and column indices past the matrix are clamped to real ones and their
// products multiplied by zero, so every load is issued unconditionally.
constexpr int kBsTiles = 4;
constexpr int kBsRows = kBsTiles * kT;   // 128
constexpr int kBsSlots = kBsTiles + kBsTiles * (kBsTiles - 1) / 2;   // 10 tiles
constexpr int kBsThreads = 256;

// Slot of block-local tile (i, j), j <= i: diagonal tiles first, then the
// tiles below the diagonal in row order.
__host__ __device__ constexpr int bs_slot(int i, int j) {
  return i == j ? i : kBsTiles + i * (i - 1) / 2 + j;
}

__global__ __launch_bounds__(kBsThreads) void k_ds_bsolve(Dev d, int b) {
  extern __shared__ double s_L[];                 // kBsSlots tiles of kT x kT (workgroup 0)
  __shared__ double s_v[kBsRows], s_x1[kBsRows];
  __shared__ double s_p[4][64];
  const int T = d.ds_T, B = (T + kBsTiles - 1) / kBsTiles;
  const int64_t ld = d.ds_ld;
  const double* S = d.ds_S;
  const double* y = S + ld * ld;
  double* v = d.ds_v;
  double* xs = d.ds_v + ld;
  const int t = threadIdx.x;
  const int t0 = kBsTiles * b, nb = min(kBsTiles, T - t0), nr = kT * nb;
  const int r0 = kT * t0, r1 = r0 + nr;                                   // rows of block b
  const int n1 = b + 1 < B ? kT * min(kBsTiles, T - t0 - kBsTiles) : 0;   // rows of block b + 1
  if (blockIdx.x > 0) {
    const int j = 64 * (blockIdx.x - 1) + (t & 63);
    const int q = t >> 6;
    if (n1 == 0) {   // first launch: v = y above the last block
      if (q == 0 && j < r0) v[j] = y[j];
      return;
    }
    const int jc = min(j, r0 - 1);
    double lv[kT], xv[kT];
#pragma unroll
    for (int e = 0; e < kT; ++e) {
      const int row = kT * q + e;
      const int rc = min(row, n1 - 1);
      lv[e] = S[(int64_t)(r1 + rc) * ld + jc];
      xv[e] = row < n1 ? xs[r1 + rc] : 0.0;
    }
    double part = 0.0;
#pragma unroll
    for (int e = 0; e < kT; ++e) part = fma(lv[e], xv[e], part);
    s_p[q][t & 63] = part;
    __syncthreads();
    if (q == 0 && j < r0) v[j] -= (s_p[0][t] + s_p[1][t]) + (s_p[2][t] + s_p[3][t]);
    return;
  }
  // Workgroup 0.  All loads first: the ten tiles (40 doubles per thread; a
  // tile outside a short last block is a clamped copy of a real one, never
  // read), v_b, x_{b+1}, and for the elimination of x_{b+1} column c = t & 127
  // of the next block's rows, half h = t >> 7 of them.
  const int c = t & (kBsRows - 1), h = t >> 7;
  {
    double lt[kBsSlots * 4];
#pragma unroll
    for (int u = 0; u < kBsSlots * 4; ++u) {
      const int slot = u >> 2, e = t + kBsThreads * (u & 3);
      const int rr = e >> 5, cc = e & (kT - 1);
      int ti = slot, tj = slot;
      if (slot >= kBsTiles) {
        const int q = slot - kBsTiles;
        ti = q < 1 ? 1 : (q < 3 ? 2 : 3);
        tj = q - ti * (ti - 1) / 2;
      }
      ti = min(ti, nb - 1);
      tj = min(tj, nb - 1);
      lt[u] = slot < kBsTiles ? d.ds_diag[(int64_t)(t0 + ti) * kT * kT + e]
                              : S[(int64_t)(r0 + kT * ti + rr) * ld + r0 + kT * tj + cc];
    }
    double nv[kBsRows / 2];
    const int cc = min(c, nr - 1);
#pragma unroll
    for (int u = 0; u < kBsRows / 2; ++u) {
      const int e = kBsRows / 2 * h + u;
      nv[u] = n1 > 0 ? S[(int64_t)(r1 + min(e, n1 - 1)) * ld + r0 + cc] : 0.0;
    }
    if (t < nr) s_v[t] = n1 == 0 ? y[r0 + t] : v[r0 + t];
    if (t < n1) s_x1[t] = xs[r1 + t];
#pragma unroll
    for (int u = 0; u < kBsSlots * 4; ++u) s_L[(u >> 2) * kT * kT + t + kBsThreads * (u & 3)] = lt[u];
    __syncthreads();
    if (n1 > 0) {
      // x_{b+1} out of block b: each half's sum, then half 0 + half 1
      double part = 0.0;
#pragma unroll
      for (int u = 0; u < kBsRows / 2; ++u) {
        const int e = kBsRows / 2 * h + u;
        part = fma(nv[u], e < n1 ? s_x1[e] : 0.0, part);
      }
      __syncthreads();
      if (h == 1) s_x1[c] = part;   // s_x1's values are all in the sums now
      __syncthreads();
      if (h == 0 && c < nr) s_v[c] -= part + s_x1[c];
      __syncthreads();
    }
  }
  // the triangles of the block from the bottom
  for (int p = nb - 1; p >= 0; --p) {
    const int o = kT * p;
    if (t < 64) {
      const int cl = t & (kT - 1);
      const double* Lt = s_L + bs_slot(p, p) * kT * kT;
      double col[kT];
#pragma unroll
      for (int e = 0; e < kT; ++e) col[e] = e == cl ? 0.0 : Lt[e * kT + cl];   // L(e, cl), pivot apart
      const double inv = 1.0 / Lt[cl * kT + cl];
      double vv = s_v[o + cl];
#pragma unroll
      for (int e = kT - 1; e >= 0; --e) vv = fma(-col[e], lane_bcast(vv * inv, e), vv);
      if (t < kT) s_v[o + cl] = vv * inv;
    }
    __syncthreads();
    // x of tile p out of the block's rows above it (block-local columns < o)
    if (t < o) {
      const double* Lr = s_L + bs_slot(p, t >> 5) * kT * kT + (t & (kT - 1));
      double acc = 0.0;
#pragma unroll
      for (int e = 0; e < kT; ++e) acc = fma(Lr[e * kT], s_v[o + e], acc);
      s_v[t] -= acc;
    }
    __syncthreads();
  }
  if (t < nr) {
    xs[r0 + t] = s_v[t];
    if (r0 + t < d.ds_n) d.x[r0 + t] = s_v[t];
  }
  if (b == 0 && t == 0) {
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
int ds_step_blocks(const Dev& d, int k, int cov) {
  const int kc = k + 1, m = d.ds_T - kc;
  int n = m + 1 + (cov ? kc + 1 : 0);
  if (k >= 0) n += (m - 1) * m / 2 + (m - 1) + (cov ? (k + 1) * (m - 1) : 0);
  return n;
}
void launch_ds_step(const Dev& d, int k, int cov, hipStream_t s) {
  launch_timed(k_ds_step, dim3(ds_step_blocks(d, k, cov)), dim3(64), s, 0u, d, k, cov);
}
hipError_t ds_backsolve_limit(int ld) {
  (void)ld;
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&k_ds_bsolve),
                             hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)(8 * kBsSlots * kT * kT));
}
void launch_ds_backsolve(const Dev& d, hipStream_t s) {
  const int B = (d.ds_T + kBsTiles - 1) / kBsTiles;
  for (int b = B - 1; b >= 0; --b) {
    const int nw = 1 + (kT * kBsTiles * b + 63) / 64;   // workgroup 0 + 64 columns each above
    launch_timed(k_ds_bsolve, dim3(nw), dim3(kBsThreads), s, (uint32_t)(8 * kBsSlots * kT * kT), d, b);
  }
}

}  // namespace ba
