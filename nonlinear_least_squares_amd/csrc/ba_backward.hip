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
// g = -G and apply psi'(r_k) J_k to the solution per observation, in camera
// order (camera chunks, the camera's data uniform across a wavefront).
#include <hip/hip_runtime.h>

#include "ba_launch.h"

namespace ba {
namespace {

__global__ void k_negate(double* a, int64_t n) {
  const int64_t e = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (e < n) a[e] = -a[e];
}

// One wavefront per camera chunk (the camera passes' blocks): the camera and
// its part of H~^-1 G (x) are uniform across the wavefront; per observation
// the point, its part dp and the observed pixel are read, and the result goes
// to the observation's original index perm_cam[s].
__global__ __launch_bounds__(64) void k_vjp_cam(Dev d, const int32_t* __restrict__ perm_cam,
                                                double* __restrict__ out) {
  const int4 bi = d.blk_chunk[blockIdx.x];
  const int cb = bi.x, ce = bi.y, j = bi.z;
  if (bi.w < 0) return;
  const CamT& t = d.tab[j];
  CamG c;
#pragma unroll
  for (int k = 0; k < 9; ++k) c.R[k] = t.R[k];
#pragma unroll
  for (int k = 0; k < 3; ++k) c.t[k] = t.t[k];
  c.f = t.f;
  c.k1 = t.k1;
  c.k2 = t.k2;
  double xc[9];
#pragma unroll
  for (int k = 0; k < 9; ++k) xc[k] = d.x[9 * (int64_t)j + k];
  for (int s = cb + (int)threadIdx.x; s < ce; s += 64) {
    const int64_t i = d.c_pt[s];
    Geo g;
    geo_eval(c, d.pts[3 * i], d.pts[3 * i + 1], d.pts[3 * i + 2], g);
    const double r0 = g.u0 - d.c_uv[2 * (int64_t)s], r1 = g.u1 - d.c_uv[2 * (int64_t)s + 1];
    double y0, y1, t0, t1;
    jc_apply(g, c.f, xc, y0, y1);
    jp_apply(g, c.R, d.dp[3 * i], d.dp[3 * i + 1], d.dp[3 * i + 2], t0, t1);
    y0 += t0;
    y1 += t1;
    const double e = sqrt(r0 * r0 + r1 * r1);
    if (d.loss == 1 && e > d.delta) {
      const double ry = (r0 * y0 + r1 * y1) / (e * e), sc = d.delta / e;
      y0 = sc * (y0 - r0 * ry);
      y1 = sc * (y1 - r1 * ry);
    }
    const int64_t k = perm_cam[s];
    out[2 * k] = y0;
    out[2 * k + 1] = y1;
  }
}

}  // namespace

void launch_negate(double* a, int64_t n, hipStream_t s) {
  if (n > 0) launch_timed(k_negate, dim3((unsigned)((n + 255) / 256)), dim3(256), s, 0u, a, n);
}

void launch_vjp_obs(const Dev& d, const int32_t* perm_cam, double* out, hipStream_t s) {
  if (d.n_chunk_blocks > 0)
    launch_timed(k_vjp_cam, dim3(d.n_chunk_blocks), dim3(64), s, 0u, d, perm_cam, out);
}

}  // namespace ba
