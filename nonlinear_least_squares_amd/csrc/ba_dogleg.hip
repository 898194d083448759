// Dogleg trust-region iteration of bundle adjustment (gfx950, fp64).
//
// The Theseus note offers Dogleg beside LM with adaptive damping.  Powell's
// dogleg, in the trust-region form of Madsen, Nielsen and Tingleff's notes on
// non-linear least squares, works on the quadratic model
//   L(h) = C + g^T h + 1/2 h^T H h,   H = J^T W J,
// with the Cauchy point -alpha g (alpha = |g|^2 / |J g|_W^2) and a
// Gauss-Newton step h_gn.  Here h_gn comes from the LM machinery with a small
// fixed Marquardt damping (H of a BA problem is singular along its gauge):
// Schur elimination, the configured solver, back-substitution.  Every step
// the host then picks is h = s_g g + s_n h_gn, so the model needs only six
// sums, taken once per point of linearisation:
//   |g|^2, |h_gn|^2, g^T h_gn      over the parameters, and
//   |J g|_W^2, (J g)^T W (J h_gn), |J h_gn|_W^2   over the observations.
// The kernels here form those sums (per-block partials, then one block adds
// them in a fixed order) and the trial parameters for given (s_g, s_n).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ba_launch.h"

namespace ba {
namespace {

constexpr int kVecBlock = 256;

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return __shfl(v, 0, 64);
}

// One wavefront per camera chunk (the camera passes' blocks): the camera, its
// gradient and its part of h_gn are uniform across the wavefront; per
// observation u = J_k [g_c; g_p] and v = J_k [dc; dp], and the wavefront's
// sums of w u.u, w u.v, w v.v become the block's partials.
__global__ __launch_bounds__(64) void k_dl_obs(Dev d, double* __restrict__ part) {
  const int4 bi = d.blk_chunk[blockIdx.x];
  const int cb = bi.x, ce = bi.y, j = bi.z;
  double uu = 0.0, uv = 0.0, vv = 0.0;
  if (bi.w >= 0) {
    const CamT& t = d.tab[j];
    CamG c;
#pragma unroll
    for (int k = 0; k < 9; ++k) c.R[k] = t.R[k];
#pragma unroll
    for (int k = 0; k < 3; ++k) c.t[k] = t.t[k];
    c.f = t.f;
    c.k1 = t.k1;
    c.k2 = t.k2;
    double gcj[9], dcj[9];
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      gcj[k] = d.gc[9 * (int64_t)j + k];
      dcj[k] = d.x[9 * (int64_t)j + k];
    }
    for (int s = cb + (int)threadIdx.x; s < ce; s += 64) {
      const int64_t i = d.c_pt[s];
      Geo g;
      geo_eval(c, d.pts[3 * i], d.pts[3 * i + 1], d.pts[3 * i + 2], g);
      double u0, u1, v0, v1, t0, t1;
      jc_apply(g, c.f, gcj, u0, u1);
      jp_apply(g, c.R, d.gp[3 * i], d.gp[3 * i + 1], d.gp[3 * i + 2], t0, t1);
      u0 += t0;
      u1 += t1;
      jc_apply(g, c.f, dcj, v0, v1);
      jp_apply(g, c.R, d.dp[3 * i], d.dp[3 * i + 1], d.dp[3 * i + 2], t0, t1);
      v0 += t0;
      v1 += t1;
      const double w = d.w_cam[s];
      uu += w * (u0 * u0 + u1 * u1);
      uv += w * (u0 * v0 + u1 * v1);
      vv += w * (v0 * v0 + v1 * v1);
    }
  }
  uu = wave_sum(uu);
  uv = wave_sum(uv);
  vv = wave_sum(vv);
  if (threadIdx.x == 0) {
    part[3 * (int64_t)blockIdx.x] = uu;
    part[3 * (int64_t)blockIdx.x + 1] = uv;
    part[3 * (int64_t)blockIdx.x + 2] = vv;
  }
}

// Over the 9 nc camera and 3 np point entries: partials of g.g, h_gn.h_gn and
// g.h_gn, one triple per block (wavefronts added in order).
__global__ __launch_bounds__(kVecBlock) void k_dl_vec(Dev d, double* __restrict__ part) {
  __shared__ double s_p[3][kVecBlock / 64];
  const int64_t nc9 = 9 * d.nc, n = nc9 + 3 * d.np;
  const int64_t e = blockIdx.x * (int64_t)kVecBlock + threadIdx.x;
  double gg = 0.0, nn = 0.0, gn = 0.0;
  if (e < n) {
    const double a = e < nc9 ? d.gc[e] : d.gp[e - nc9];
    const double b = e < nc9 ? d.x[e] : d.dp[e - nc9];
    gg = a * a;
    nn = b * b;
    gn = a * b;
  }
  gg = wave_sum(gg);
  nn = wave_sum(nn);
  gn = wave_sum(gn);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    s_p[0][w] = gg;
    s_p[1][w] = nn;
    s_p[2][w] = gn;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    double t = 0.0;
#pragma unroll
    for (int k = 0; k < kVecBlock / 64; ++k) t += s_p[threadIdx.x][k];
    part[3 * (int64_t)blockIdx.x + threadIdx.x] = t;
  }
}

// One block: out = [g.g, h_gn.h_gn, g.h_gn, |Jg|^2, (Jg).(Jh_gn), |Jh_gn|^2],
// each the sum of its partials in block order (thread t takes blocks t,
// t + 256, ..., then a fixed tree).
__global__ __launch_bounds__(256) void k_dl_final(const double* __restrict__ vpart, int nv,
                                                  const double* __restrict__ opart, int no,
                                                  double* __restrict__ out) {
  __shared__ double s_p[6][4];
  double acc[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
  for (int b = threadIdx.x; b < nv; b += 256)
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[q] += vpart[3 * (int64_t)b + q];
  for (int b = threadIdx.x; b < no; b += 256)
#pragma unroll
    for (int q = 0; q < 3; ++q) acc[3 + q] += opart[3 * (int64_t)b + q];
  const int w = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < 6; ++q) {
    const double v = wave_sum(acc[q]);
    if ((threadIdx.x & 63) == 0) s_p[q][w] = v;
  }
  __syncthreads();
  if (threadIdx.x < 6) out[threadIdx.x] = ((s_p[threadIdx.x][0] + s_p[threadIdx.x][1]) +
                                           s_p[threadIdx.x][2]) + s_p[threadIdx.x][3];
}

// The step's camera part, hc = s_g g_c + s_n dc (the retraction reads it), and
// the trial points, X + s_g g_p + s_n dp.
__global__ __launch_bounds__(kVecBlock) void k_dl_step(Dev d, double s_g, double s_n,
                                                       double* __restrict__ hc) {
  const int64_t nc9 = 9 * d.nc, n = nc9 + 3 * d.np;
  const int64_t e = blockIdx.x * (int64_t)kVecBlock + threadIdx.x;
  if (e >= n) return;
  if (e < nc9) {
    hc[e] = s_g * d.gc[e] + s_n * d.x[e];
  } else {
    const int64_t p = e - nc9;
    d.pts_trial[p] = d.pts[p] + (s_g * d.gp[p] + s_n * d.dp[p]);
  }
}

}  // namespace

int dl_vec_blocks(int64_t nc, int64_t np) {
  return (int)std::max<int64_t>((9 * nc + 3 * np + kVecBlock - 1) / kVecBlock, 1);
}

void launch_dl_vec(const Dev& d, double* vpart, hipStream_t s) {
  launch_timed(k_dl_vec, dim3(dl_vec_blocks(d.nc, d.np)), dim3(kVecBlock), s, 0u, d, vpart);
}
void launch_dl_obs(const Dev& d, double* opart, hipStream_t s) {
  if (d.n_chunk_blocks > 0) launch_timed(k_dl_obs, dim3(d.n_chunk_blocks), dim3(64), s, 0u, d, opart);
}
void launch_dl_final(const Dev& d, const double* vpart, const double* opart, double* out, hipStream_t s) {
  launch_timed(k_dl_final, dim3(1), dim3(256), s, 0u, vpart, dl_vec_blocks(d.nc, d.np), opart,
               d.n_chunk_blocks, out);
}

void launch_dl_step(const Dev& d, double s_g, double s_n, double* hc, hipStream_t s) {
  launch_timed(k_dl_step, dim3(dl_vec_blocks(d.nc, d.np)), dim3(kVecBlock), s, 0u, d, s_g, s_n, hc);
}

}  // namespace ba
