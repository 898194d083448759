// ba_cost_noalloc: the bundle-adjustment cost with no handle and no device
// allocation, for callers that cannot allocate (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  Declared in
// include/ba.h.
//
// The scratch memory (per-camera geometry table and per-block partial sums)
// is one file-scope device array.  In host code its name is only a host-side
// stand-in, so the entry point looks up the array's device address once per
// device with hipGetSymbolAddress and passes that address to the kernels.
#include <hip/hip_runtime.h>

#include <cmath>
#include <mutex>
#include <string>

#include "../../include/ba.h"
#include "ba_kernels.h"

namespace ba {
namespace {

constexpr int kNaBlockObs = 1024;                          // observations per partial sum
constexpr int kNaThreads = 256;                            // threads of the partial-sum kernel
constexpr int kNaFinalThreads = 1024;                      // threads of the final sum
constexpr int64_t kNaMaxParts = BA_NOALLOC_MAX_OBS / kNaBlockObs;
constexpr size_t kNaTabBytes = sizeof(CamT) * BA_NOALLOC_MAX_CAMS;        // 512 KiB
constexpr size_t kNaQuatBytes = 4 * sizeof(double) * BA_NOALLOC_MAX_CAMS; // 128 KiB
constexpr size_t kNaPartBytes = sizeof(double) * kNaMaxParts;             // 128 KiB
constexpr size_t kNaScratchBytes = kNaTabBytes + kNaQuatBytes + kNaPartBytes;
static_assert(BA_NOALLOC_MAX_OBS % kNaBlockObs == 0, "whole blocks");
static_assert(kNaTabBytes % 256 == 0 && kNaQuatBytes % 256 == 0, "aligned pieces");

}  // namespace
}  // namespace ba

// Scratch of ba_cost_noalloc, one copy per GPU, held until the process ends.
static __device__ __align__(256) unsigned char scratch[ba::kNaScratchBytes];

namespace ba {
namespace {

// Fixed-order sum of one value per thread of a block of NT threads: a
// butterfly inside each wavefront, then the wavefront totals in order.
template <int NT>
__device__ __forceinline__ double na_block_sum(double v) {
  __shared__ double s_w[NT / kWave];
#pragma unroll
  for (int off = kWave / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  if ((threadIdx.x & (kWave - 1)) == 0) s_w[threadIdx.x / kWave] = v;
  __syncthreads();
  double t = 0.0;
  if (threadIdx.x == 0) {
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) t += s_w[w];
  }
  return t;
}

// Partial cost of observations [b * kNaBlockObs, (b + 1) * kNaBlockObs) in
// the caller's order.  An index out of range is never used for a load: the
// observation contributes NaN instead.
__global__ __launch_bounds__(kNaThreads) void k_na_cost(
    const CamT* __restrict__ tab, int64_t nc, const double* __restrict__ pts, int64_t np,
    const int32_t* __restrict__ cam_idx, const int32_t* __restrict__ pt_idx,
    const double* __restrict__ uv, int64_t n, int loss, double delta, double* __restrict__ part) {
  const int64_t b0 = (int64_t)blockIdx.x * kNaBlockObs;
  const int64_t b1 = b0 + kNaBlockObs < n ? b0 + kNaBlockObs : n;
  double acc = 0.0;
  for (int64_t k = b0 + threadIdx.x; k < b1; k += kNaThreads) {
    const int32_t j = cam_idx[k], i = pt_idx[k];
    if (j < 0 || j >= nc || i < 0 || i >= np) {
      acc += NAN;
      continue;
    }
    const CamT& t = tab[j];
    CamG c;
#pragma unroll
    for (int a = 0; a < 9; ++a) c.R[a] = t.R[a];
    c.t[0] = t.t[0];
    c.t[1] = t.t[1];
    c.t[2] = t.t[2];
    c.f = t.f;
    c.k1 = t.k1;
    c.k2 = t.k2;
    Geo g;
    geo_eval(c, pts[3 * (int64_t)i], pts[3 * (int64_t)i + 1], pts[3 * (int64_t)i + 2], g);
    double w, rho;
    robust(g.u0 - uv[2 * k], g.u1 - uv[2 * k + 1], loss, delta, w, rho);
    acc += rho;
  }
  const double s = na_block_sum<kNaThreads>(acc);
  if (threadIdx.x == 0) part[blockIdx.x] = s;
}

// The partials in block order by one block; the total to out.
__global__ __launch_bounds__(kNaFinalThreads) void k_na_final(const double* __restrict__ part,
                                                             int n_parts, double* __restrict__ out) {
  double acc = 0.0;
  for (int b = threadIdx.x; b < n_parts; b += kNaFinalThreads) acc += part[b];
  const double s = na_block_sum<kNaFinalThreads>(acc);
  if (threadIdx.x == 0) *out = s;
}

// Device address of `scratch` on each device, looked up once per device with
// that device current.
constexpr int kNaMaxDevices = 64;
std::mutex g_na_mu;
void* g_na_scratch[kNaMaxDevices] = {};

int na_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(BA_ERR_DEVICE, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kNaMaxDevices) return set_error(BA_ERR_DEVICE, "device ordinal out of range");
  std::lock_guard<std::mutex> lock(g_na_mu);
  if (!g_na_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return set_error(BA_ERR_DEVICE, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_na_scratch[dev] = p;
  }
  *out = g_na_scratch[dev];
  return BA_OK;
}

}  // namespace
}  // namespace ba

extern "C" int ba_cost_noalloc(const double* cams, int64_t n_cams, const double* points,
                               int64_t n_pts, const int32_t* obs_cam_idx, const int32_t* obs_pt_idx,
                               const double* obs_uv, int64_t n_obs, int loss, double huber_delta,
                               double* cost_out, void* stream) {
  using namespace ba;
  if (!cams || !points || !cost_out || (n_obs > 0 && (!obs_cam_idx || !obs_pt_idx || !obs_uv)))
    return set_error(BA_ERR_ARG, "null pointer");
  if (n_cams <= 0 || n_pts <= 0 || n_obs < 0) return set_error(BA_ERR_ARG, "non-positive sizes");
  if (n_cams > BA_NOALLOC_MAX_CAMS)
    return set_error(BA_ERR_ARG, "n_cams exceeds BA_NOALLOC_MAX_CAMS (4096)");
  if (n_obs > BA_NOALLOC_MAX_OBS)
    return set_error(BA_ERR_ARG, "n_obs exceeds BA_NOALLOC_MAX_OBS (16,777,216)");
  if (n_pts >= ((int64_t)1 << 31)) return set_error(BA_ERR_ARG, "n_pts must be below 2^31");
  if (loss != BA_LOSS_SQUARED && loss != BA_LOSS_HUBER) return set_error(BA_ERR_ARG, "bad loss");
  if (!(huber_delta > 0.0)) return set_error(BA_ERR_ARG, "huber_delta must be > 0");
  void* base = nullptr;
  int rc = na_scratch(&base);
  if (rc != BA_OK) return rc;
  unsigned char* sp = static_cast<unsigned char*>(base);
  CamT* tab = reinterpret_cast<CamT*>(sp);
  double* camq = reinterpret_cast<double*>(sp + kNaTabBytes);
  double* part = reinterpret_cast<double*>(sp + kNaTabBytes + kNaQuatBytes);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  launch_cam_prep(cams, tab, camq, n_cams, s);
  const int n_parts = (int)((n_obs + kNaBlockObs - 1) / kNaBlockObs);
  if (n_parts > 0)
    hipLaunchKernelGGL(k_na_cost, dim3(n_parts), dim3(kNaThreads), 0, s, tab, n_cams, points,
                       n_pts, obs_cam_idx, obs_pt_idx, obs_uv, n_obs, loss, huber_delta, part);
  hipLaunchKernelGGL(k_na_final, dim3(1), dim3(kNaFinalThreads), 0, s, part, n_parts, cost_out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(BA_ERR_DEVICE, std::string("launch: ") + hipGetErrorString(e));
  return BA_OK;
}
