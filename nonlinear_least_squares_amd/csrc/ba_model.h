// Per-observation camera model, Jacobian products and small dense algebra for
// the gfx950 bundle-adjustment kernels (fp64).
//
// Camera: P = R X + t, p = P_xy / max(P_z, 1e-6) (depth clamp as in the
// NeRF-SLAM reproduction notes, sec. 2.2), n = |p|^2, s = 1 + k1 n + k2 n^2,
// u = f s p.  Rotation in the left tangent (R <- Exp(dphi) R), everything
// else additive, which gives with A = du/dP (2x3) and q = R X:
//   Jc x = A (dphi x q + dt) + p (s df + f n dk1 + f n^2 dk2)
//   Jc^T y = [q x a, a, s p.y, f n p.y, f n^2 p.y],  a = A^T y
//   Jp x = A (R x),  Jp^T y = R^T a
// so the 2x9 and 2x3 blocks never need to be stored for the matrix-free
// Schur products; explicit rows exist only for block assembly.
#pragma once
#include <hip/hip_runtime.h>

namespace ba {

// Per-camera table derived from the 9 parameters once per parameter change:
// 16 doubles = one 128-byte line.
struct alignas(128) CamT {
  double R[9];
  double t[3];
  double f, k1, k2, pad;
};

// Geometry part of a camera table entry, as the kernels hold it in registers.
struct CamG {
  double R[9];
  double t[3];
  double f, k1, k2;
};

// Geometry of one observation at the current parameters.
// 1/x for x >= 1e-6: the hardware estimate refined by two Newton steps, each
// r <- r + r (1 - x r), which doubles the correct bits of an estimate good to
// about 2^-23; the result is within an ulp or so of the rounded quotient.
__device__ __forceinline__ double recip(double x) {
  double r = __builtin_amdgcn_rcp(x);
  double e = fma(-x, r, 1.0);
  r = fma(r, e, r);
  e = fma(-x, r, 1.0);
  return fma(r, e, r);
}

struct Geo {
  double q0, q1, q2;                     // R X
  double p0, p1, n, s;                   // normalised coordinates, |p|^2, radial factor
  double a00, a01, a02, a10, a11, a12;   // A = du/dP
  double u0, u1;                         // predicted pixel
};

__device__ __forceinline__ void geo_eval(const CamG& c, double X0, double X1, double X2, Geo& g) {
  g.q0 = c.R[0] * X0 + c.R[1] * X1 + c.R[2] * X2;
  g.q1 = c.R[3] * X0 + c.R[4] * X1 + c.R[5] * X2;
  g.q2 = c.R[6] * X0 + c.R[7] * X1 + c.R[8] * X2;
  const double P0 = g.q0 + c.t[0], P1 = g.q1 + c.t[1], P2 = g.q2 + c.t[2];
  const bool clamped = P2 < 1e-6;
  const double iz = recip(clamped ? 1e-6 : P2);
  g.p0 = P0 * iz;
  g.p1 = P1 * iz;
  g.n = g.p0 * g.p0 + g.p1 * g.p1;
  g.s = 1.0 + g.n * (c.k1 + c.k2 * g.n);
  const double fs = c.f * g.s;
  g.u0 = fs * g.p0;
  g.u1 = fs * g.p1;
  // du/dp = f (s I + 2 (k1 + 2 k2 n) p p^T); dp/dP = iz [I | -p] (third column 0 when clamped)
  const double fc = 2.0 * c.f * (c.k1 + 2.0 * c.k2 * g.n);
  const double d00 = fs + fc * g.p0 * g.p0, d01 = fc * g.p0 * g.p1, d11 = fs + fc * g.p1 * g.p1;
  g.a00 = d00 * iz;
  g.a01 = d01 * iz;
  g.a10 = d01 * iz;
  g.a11 = d11 * iz;
  g.a02 = clamped ? 0.0 : -(g.a00 * g.p0 + g.a01 * g.p1);
  g.a12 = clamped ? 0.0 : -(g.a10 * g.p0 + g.a11 * g.p1);
}

// Explicit camera Jacobian rows (2 x 9, row-major).
__device__ __forceinline__ void jc_rows(const Geo& g, double f, double J[18]) {
  J[0] = g.a02 * g.q1 - g.a01 * g.q2;
  J[1] = g.a00 * g.q2 - g.a02 * g.q0;
  J[2] = g.a01 * g.q0 - g.a00 * g.q1;
  J[3] = g.a00;
  J[4] = g.a01;
  J[5] = g.a02;
  J[6] = g.s * g.p0;
  J[7] = f * g.n * g.p0;
  J[8] = f * g.n * g.n * g.p0;
  J[9] = g.a12 * g.q1 - g.a11 * g.q2;
  J[10] = g.a10 * g.q2 - g.a12 * g.q0;
  J[11] = g.a11 * g.q0 - g.a10 * g.q1;
  J[12] = g.a10;
  J[13] = g.a11;
  J[14] = g.a12;
  J[15] = g.s * g.p1;
  J[16] = f * g.n * g.p1;
  J[17] = f * g.n * g.n * g.p1;
}

// Explicit point Jacobian rows Jp = A R (2 x 3, row-major).
__device__ __forceinline__ void jp_rows(const Geo& g, const double* R, double J[6]) {
  for (int j = 0; j < 3; ++j) {
    J[j] = g.a00 * R[j] + g.a01 * R[3 + j] + g.a02 * R[6 + j];
    J[3 + j] = g.a10 * R[j] + g.a11 * R[3 + j] + g.a12 * R[6 + j];
  }
}

// o = Jc x for a camera step x = (dphi, dt, df, dk1, dk2).
__device__ __forceinline__ void jc_apply(const Geo& g, double f, const double* x, double& o0,
                                         double& o1) {
  const double c0 = x[1] * g.q2 - x[2] * g.q1 + x[3];
  const double c1 = x[2] * g.q0 - x[0] * g.q2 + x[4];
  const double c2 = x[0] * g.q1 - x[1] * g.q0 + x[5];
  const double m = g.s * x[6] + f * g.n * (x[7] + g.n * x[8]);
  o0 = g.a00 * c0 + g.a01 * c1 + g.a02 * c2 + g.p0 * m;
  o1 = g.a10 * c0 + g.a11 * c1 + g.a12 * c2 + g.p1 * m;
}

// o += wt * Jc^T y.
__device__ __forceinline__ void jct_acc(const Geo& g, double f, double y0, double y1, double* o) {
  const double a0 = g.a00 * y0 + g.a10 * y1;
  const double a1 = g.a01 * y0 + g.a11 * y1;
  const double a2 = g.a02 * y0 + g.a12 * y1;
  const double py = g.p0 * y0 + g.p1 * y1;
  o[0] += g.q1 * a2 - g.q2 * a1;
  o[1] += g.q2 * a0 - g.q0 * a2;
  o[2] += g.q0 * a1 - g.q1 * a0;
  o[3] += a0;
  o[4] += a1;
  o[5] += a2;
  o[6] += g.s * py;
  o[7] += f * g.n * py;
  o[8] += f * g.n * g.n * py;
}

// Jp x = A (R x).
__device__ __forceinline__ void jp_apply(const Geo& g, const double* R, double x0, double x1,
                                         double x2, double& o0, double& o1) {
  const double y0 = R[0] * x0 + R[1] * x1 + R[2] * x2;
  const double y1 = R[3] * x0 + R[4] * x1 + R[5] * x2;
  const double y2 = R[6] * x0 + R[7] * x1 + R[8] * x2;
  o0 = g.a00 * y0 + g.a01 * y1 + g.a02 * y2;
  o1 = g.a10 * y0 + g.a11 * y1 + g.a12 * y2;
}

// Jp^T y = R^T (A^T y).
__device__ __forceinline__ void jpt_apply(const Geo& g, const double* R, double y0, double y1,
                                          double& o0, double& o1, double& o2) {
  const double a0 = g.a00 * y0 + g.a10 * y1;
  const double a1 = g.a01 * y0 + g.a11 * y1;
  const double a2 = g.a02 * y0 + g.a12 * y1;
  o0 = R[0] * a0 + R[3] * a1 + R[6] * a2;
  o1 = R[1] * a0 + R[4] * a1 + R[7] * a2;
  o2 = R[2] * a0 + R[5] * a1 + R[8] * a2;
}

// Huber weight (rho'(e)/e) and cost on the 2-D residual norm, the quadratic
// branch taken for e <= delta (F^2SLAM article, sec. 5.3).
__device__ __forceinline__ void robust(double r0, double r1, int loss, double delta, double& w,
                                       double& rho) {
  const double e2 = r0 * r0 + r1 * r1;
  const double e = sqrt(e2);
  if (loss == 1 && e > delta) {
    w = delta / e;
    rho = delta * (e - 0.5 * delta);
  } else {
    w = 1.0;
    rho = 0.5 * e2;
  }
}

// Unit quaternion (w, x, y, z), w >= 0, of the rotation vector (w0, w1, w2):
// (cos(th/2), sin(th/2) w / th), and (1, w / 2) below th = 1e-8.
__device__ __forceinline__ void quat_from_rotvec(double w0, double w1, double w2, double* q) {
  const double th = sqrt(w0 * w0 + w1 * w1 + w2 * w2);
  const double h = th < 1e-8 ? 0.5 : sin(0.5 * th) / th;
  q[0] = th < 1e-8 ? 1.0 : cos(0.5 * th);
  q[1] = h * w0;
  q[2] = h * w1;
  q[3] = h * w2;
}

// Rotation matrix (row-major) of a unit quaternion: I + 2 w [v]x + 2 [v]x^2.
// Every kernel that needs a camera's R forms it with this function from the
// same quaternion, so all of them see the same bits.
__device__ __forceinline__ void quat_to_R(const double* q, double* R) {
  const double w = q[0], x = q[1], y = q[2], z = q[3];
  const double x2 = x + x, y2 = y + y, z2 = z + z;
  const double xx = x * x2, yy = y * y2, zz = z * z2;
  const double xy = x * y2, xz = x * z2, yz = y * z2;
  const double wx = w * x2, wy = w * y2, wz = w * z2;
  R[0] = 1.0 - (yy + zz);
  R[1] = xy - wz;
  R[2] = xz + wy;
  R[3] = xy + wz;
  R[4] = 1.0 - (xx + zz);
  R[5] = yz - wx;
  R[6] = xz - wy;
  R[7] = yz + wx;
  R[8] = 1.0 - (xx + yy);
}

// Packed symmetric storage: upper triangle row by row, index of (i, j), i <= j.
__host__ __device__ constexpr int sym_idx(int n, int i, int j) {
  return i * n - (i * (i - 1)) / 2 + (j - i);
}

// In-place Cholesky of a packed 9x9 SPD matrix into a packed lower factor
// stored in the same upper-triangle layout (L(j, i) at sym_idx(i, j)).
// Returns false if a pivot is not positive and finite.
template <int N>
__device__ __forceinline__ bool chol_packed(double* A) {
#pragma unroll
  for (int j = 0; j < N; ++j) {
    double d = A[sym_idx(N, j, j)];
#pragma unroll
    for (int l = 0; l < j; ++l) d -= A[sym_idx(N, l, j)] * A[sym_idx(N, l, j)];
    if (!(d > 0.0) || !isfinite(d)) return false;
    d = sqrt(d);
    A[sym_idx(N, j, j)] = d;
    const double id = 1.0 / d;
#pragma unroll
    for (int i = j + 1; i < N; ++i) {
      double s = A[sym_idx(N, j, i)];
#pragma unroll
      for (int l = 0; l < j; ++l) s -= A[sym_idx(N, l, i)] * A[sym_idx(N, l, j)];
      A[sym_idx(N, j, i)] = s * id;
    }
  }
  return true;
}

// Solve L L^T x = b with the packed factor from chol_packed.
template <int N>
__device__ __forceinline__ void chol_solve_packed(const double* L, const double* b, double* x) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    double s = b[i];
#pragma unroll
    for (int l = 0; l < i; ++l) s -= L[sym_idx(N, l, i)] * x[l];
    x[i] = s / L[sym_idx(N, i, i)];
  }
#pragma unroll
  for (int i = N - 1; i >= 0; --i) {
    double s = x[i];
#pragma unroll
    for (int l = i + 1; l < N; ++l) s -= L[sym_idx(N, i, l)] * x[l];
    x[i] = s / L[sym_idx(N, i, i)];
  }
}

}  // namespace ba
