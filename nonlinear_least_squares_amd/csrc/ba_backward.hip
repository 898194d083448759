// Implicit backward through the LM solution (gfx950, fp64).
//
// The Theseus note's implicit mode differentiates one Newton step at the
// solution, h(theta; u) = theta - [Hess S]^-1_stop grad S, with the Hessian
// held fixed.  Here the Hessian is the damped Gauss-Newton matrix H~ of the
// current LM state (the undamped one is singular along the gauge of a BA
// problem), and u are the observed pixels.  Since grad S = sum_k J_k^T psi(r_k)
// with r_k = u^_k(theta) - u_k and psi(r) = d rho(|r|) / dr, a loss f of the
// solution with gradient G has
//   df/du_k = psi'(r_k) J_k H~^-1 G,
// psi' = I for the squared loss and inside the Huber threshold delta,
// (delta / |r|)(I - r r^T / |r|^2) beyond it.  H~^-1 G is the damped system of
// an LM step with g = -G, solved by the same Schur elimination, solver and
// back-substitution as the forward step (ba_capi.hip); the kernels here set
// g = -G and apply psi'(r_k) J_k to the solution per observation.
#include <hip/hip_runtime.h>

#include "ba_launch.h"

namespace ba {
namespace {

__global__ void k_negate(double* a, int64_t n) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e < n) a[e] = -a[e];
}

// One thread per point-order observation s; the result goes to the
// observation's original index perm_pt[s].  x holds the camera part of
// H~^-1 G, dp its point part.
__global__ void k_vjp_obs(Dev d, const int32_t* __restrict__ perm_pt, double* __restrict__ out) {
  const int64_t s = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (s >= d.nobs) return;
  const int j = d.o_cam[s], i = d.o_pt[s];
  const CamT& t = d.tab[j];
  CamG c;
#pragma unroll
  for (int k = 0; k < 9; ++k) c.R[k] = t.R[k];
#pragma unroll
  for (int k = 0; k < 3; ++k) c.t[k] = t.t[k];
  c.f = t.f;
  c.k1 = t.k1;
  c.k2 = t.k2;
  Geo g;
  geo_eval(c, d.pts[3 * (int64_t)i], d.pts[3 * (int64_t)i + 1], d.pts[3 * (int64_t)i + 2], g);
  const double r0 = g.u0 - d.o_uv[2 * s], r1 = g.u1 - d.o_uv[2 * s + 1];
  double y0, y1, t0, t1;
  jc_apply(g, c.f, d.x + 9 * (int64_t)j, y0, y1);
  jp_apply(g, c.R, d.dp[3 * (int64_t)i], d.dp[3 * (int64_t)i + 1], d.dp[3 * (int64_t)i + 2], t0, t1);
  y0 += t0;
  y1 += t1;
  const double e = sqrt(r0 * r0 + r1 * r1);
  if (d.loss == 1 && e > d.delta) {
    const double ry = (r0 * y0 + r1 * y1) / (e * e), sc = d.delta / e;
    y0 = sc * (y0 - r0 * ry);
    y1 = sc * (y1 - r1 * ry);
  }
  const int64_t k = perm_pt[s];
  out[2 * k] = y0;
  out[2 * k + 1] = y1;
}

}  // namespace

void launch_negate(double* a, int64_t n, hipStream_t s) {
  if (n > 0) launch_timed(k_negate, dim3((unsigned)((n + 255) / 256)), dim3(256), s, 0u, a, n);
}

void launch_vjp_obs(const Dev& d, const int32_t* perm_pt, double* out, hipStream_t s) {
  if (d.nobs > 0)
    launch_timed(k_vjp_obs, dim3((unsigned)((d.nobs + 255) / 256)), dim3(256), s, 0u, d, perm_pt, out);
}

}  // namespace ba
