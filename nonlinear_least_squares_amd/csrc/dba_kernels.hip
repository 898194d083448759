// libdba: Gauss-Newton iterations of dense frame-graph bundle adjustment on
// gfx950 in fp32 — kernels and the C ABI declared in include/dba.h.
//
// Problem and notation follow the NeRF-SLAM reproduction notes: the image
// model of sec. 2.2 (inverse depth clamped at 1e-6, depth clamped at 1e-6
// before the division), the frame graph of sec. 2.3, the block structure of
// H = J^T W J of sec. 3.1 (6x6 pose blocks B, 1x1 inverse-depth blocks C,
// coupling E) and the Schur elimination of sec. 3.2 (eqs. (1), (2); S solved
// by Cholesky).  Poses move by the left SE(3) exponential (Theseus note,
// retraction on Lie groups).
//
// Work layout.  Edges are grouped by their source frame i: every residual of
// pixel p of frame i depends on the same inverse depth d_ip, so the Schur
// column of d_ip touches only the poses of i and of the targets of i's edges
// ("slots" 0 = i, 1 + l = target of edge l).  One block takes a pixel range
// of one group; per 64-pixel sub-tile it
//   phase 0  applies the previous step's depth update (optional),
//   phase 1  evaluates r, J_i, J_j, J_d for every (pixel, edge) and writes
//            sqrt(w)-scaled rows to LDS, field-major (one float per pixel),
//   phase 1b sums C, g_d and the Schur column over the pixel's edges and
//            scales it by C^-1/2, so that B - E C^-1 E^T becomes a sum of
//            outer products x y^T of LDS rows (negative for the Schur rows),
//   phase 2  accumulates 6x6 outer-product blocks ("tasks") with one pixel
//            per lane and a fixed set of tasks per wave, in registers.
// At the end the lanes' accumulators are summed through LDS in a fixed order
// into one partial record per (block, task); a second kernel sums the
// records over a group's blocks; a single-workgroup kernel assembles the
// reduced pose system, factors it, solves and retracts.  No floating-point
// atomics: every sum has a fixed order, so results are bitwise reproducible.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/dba.h"

namespace {

constexpr int kSub = 64;                  // pixels per sub-tile (one per lane in phase 2)
constexpr int kThreads = 256;             // threads of the linearisation block
constexpr int kWaves = kThreads / 64;
constexpr int kMaxDeg = 8;                // out-edges per frame
constexpr int kTPW = 4;                   // tasks per wave per pass
constexpr int kMaxTasks = 1 + 2 * kMaxDeg + kMaxDeg * (kMaxDeg - 1) / 2;
constexpr int kMaxPairs = 2 * kMaxDeg + 1;
constexpr int kMaxPasses = (kMaxTasks + kWaves * kTPW - 1) / (kWaves * kTPW);
constexpr int kRec = 36;                  // floats per task record
constexpr int kRedPitch = 65;
constexpr int kMaxFree = 24;
constexpr int kSolveThreads = 1024;
constexpr int kCostCap = 4096;            // cost slots per dba_solve chunk
constexpr int kTargetBlocks = 512;

// LDS field layout of one sub-tile for a group of out-degree d.
__host__ __device__ constexpr int f_a(int l) { return 26 * l; }        // sqrt(w) J_i, 2 x 6
__host__ __device__ constexpr int f_b(int l) { return 26 * l + 12; }   // sqrt(w) J_j, 2 x 6
__host__ __device__ constexpr int f_sr(int l) { return 26 * l + 24; }  // sqrt(w) r, 2
__host__ __device__ constexpr int f_s(int d, int slot) { return 26 * d + 6 * slot; }  // Schur column
__host__ __device__ constexpr int f_t(int d) { return 32 * d + 6; }   // g_d C^-1/2
__host__ __device__ constexpr int f_scr(int d, int l) { return 32 * d + 7 + 8 * l; }  // C, g_d, col_i parts
__host__ __device__ constexpr int n_fields(int d) { return 40 * d + 7; }
__host__ __device__ constexpr int sym6(int i, int j) { return i * 6 - (i * (i - 1)) / 2 + (j - i); }

// Pair encoding: x | y << 9 | z << 18, bit 27 negates the outer product,
// bit 28 negates the right-hand-side term, bit 29 marks a Schur pair.
constexpr int kNegM = 1 << 27, kNegR = 1 << 28, kSchurPair = 1 << 29;

struct Group {
  int frame, deg, n_tasks, n_passes;
  int task_begin, unit_begin, n_units, rec_begin;
  int edge[kMaxDeg];
  int slot_frame[kMaxDeg + 1];
  signed char sched[kMaxPasses][kWaves][kTPW];
};

struct Task {
  int diag, npairs;
  int pair[kMaxPairs];
};

struct Unit {
  int group, pix_begin, pix_end, rec_begin;
};

struct LinArgs {
  const Group* groups;
  const Task* tasks;
  const Unit* units;
  const float* poseRt;   // n x 16: R (row-major), t
  const float* dxi;      // n x 6
  float* depth;          // n x P
  float* dd_out;         // n x P
  const float* targets;  // E x P x 2
  const float* weights;  // E x P
  float* fstore;         // n x 8 x P: C, g_d, col_i (6)
  float* estore;         // E x 6 x P: col_j of each edge
  float* partial;        // records x 36
  float* cost_part;      // units: sum of w |r|^2
  const int* status;     // non-zero after a failed solve: no depth update
  float fx, fy, cx, cy, ifx, ify;
  int P, W, schur;
};

// ---------------------------------------------------------------- device --

// Relative pose T_ij = T_j T_i^-1: R_ij = R_j R_i^T, t_ij = t_j - R_ij t_i.
__device__ __forceinline__ void rel_pose(const float* Ti, const float* Tj, float* o) {
  for (int r = 0; r < 3; ++r)
    for (int c = 0; c < 3; ++c)
      o[3 * r + c] = Tj[3 * r] * Ti[3 * c] + Tj[3 * r + 1] * Ti[3 * c + 1] + Tj[3 * r + 2] * Ti[3 * c + 2];
  for (int r = 0; r < 3; ++r)
    o[9 + r] = Tj[9 + r] - (o[3 * r] * Ti[9] + o[3 * r + 1] * Ti[10] + o[3 * r + 2] * Ti[11]);
}

// Hardware reciprocal, square root and reciprocal square root (about 1 ulp,
// against several times the latency for the correctly rounded forms).
__device__ __forceinline__ float frcp(float x) { return __builtin_amdgcn_rcpf(x); }
__device__ __forceinline__ float fsqrt(float x) { return __builtin_amdgcn_sqrtf(x); }
__device__ __forceinline__ float frsq(float x) { return __builtin_amdgcn_rsqf(x); }

struct PixOut {
  float r0, r1;
  float ji[12], jj[12], jd[2];
};

// Residual of pixel (x, y) with inverse depth d under T_ij, and with JAC its
// Jacobians: with P = d(proj)/dX_j (third column 0 when the depth clamp is
// active), J_j row k = [P_k, X_j x P_k] (left perturbation of T_j),
// Q_k = P_k R_ij, J_i row k = [-Q_k, Q_k x X_i] (left perturbation of T_i),
// J_d = -Q ray / d^2 (0 when the inverse-depth clamp is active).
template <bool JAC>
__device__ __forceinline__ void pix_eval(const float* T, float fx, float fy, float cx, float cy,
                                         float ifx, float ify, float x, float y, float d,
                                         float tx, float ty, PixOut& o) {
  const float ray0 = (x - cx) * ifx, ray1 = (y - cy) * ify;
  const bool dcl = d < 1e-6f;
  const float id = frcp(dcl ? 1e-6f : d);
  const float X0 = ray0 * id, X1 = ray1 * id, X2 = id;
  const float Y0 = T[0] * X0 + T[1] * X1 + T[2] * X2 + T[9];
  const float Y1 = T[3] * X0 + T[4] * X1 + T[5] * X2 + T[10];
  const float Y2 = T[6] * X0 + T[7] * X1 + T[8] * X2 + T[11];
  const bool zcl = Y2 < 1e-6f;
  const float iz = frcp(zcl ? 1e-6f : Y2);
  o.r0 = fx * (Y0 * iz) + cx - tx;
  o.r1 = fy * (Y1 * iz) + cy - ty;
  if constexpr (JAC) {
    const float p00 = fx * iz, p11 = fy * iz;
    const float p02 = zcl ? 0.0f : -p00 * Y0 * iz;
    const float p12 = zcl ? 0.0f : -p11 * Y1 * iz;
    // J_j
    o.jj[0] = p00; o.jj[1] = 0.0f; o.jj[2] = p02;
    o.jj[3] = Y1 * p02; o.jj[4] = Y2 * p00 - Y0 * p02; o.jj[5] = -Y1 * p00;
    o.jj[6] = 0.0f; o.jj[7] = p11; o.jj[8] = p12;
    o.jj[9] = Y1 * p12 - Y2 * p11; o.jj[10] = -Y0 * p12; o.jj[11] = Y0 * p11;
    // Q = P R
    float q0[3], q1[3];
    for (int c = 0; c < 3; ++c) {
      q0[c] = p00 * T[c] + p02 * T[6 + c];
      q1[c] = p11 * T[3 + c] + p12 * T[6 + c];
    }
    o.ji[0] = -q0[0]; o.ji[1] = -q0[1]; o.ji[2] = -q0[2];
    o.ji[3] = q0[1] * X2 - q0[2] * X1; o.ji[4] = q0[2] * X0 - q0[0] * X2; o.ji[5] = q0[0] * X1 - q0[1] * X0;
    o.ji[6] = -q1[0]; o.ji[7] = -q1[1]; o.ji[8] = -q1[2];
    o.ji[9] = q1[1] * X2 - q1[2] * X1; o.ji[10] = q1[2] * X0 - q1[0] * X2; o.ji[11] = q1[0] * X1 - q1[1] * X0;
    const float id2 = dcl ? 0.0f : id * id;
    o.jd[0] = -(q0[0] * ray0 + q0[1] * ray1 + q0[2]) * id2;
    o.jd[1] = -(q1[0] * ray0 + q1[1] * ray1 + q1[2]) * id2;
  }
}

// Wave-uniform copy of a value (the compiler cannot see that tid >> 6 is).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float xor_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}

// Fixed-order sum of n partials by one wave (all 64 lanes must call it).
__device__ __forceinline__ float wave_sum_parts(const float* parts, int n) {
  const int lane = threadIdx.x & 63;
  float s = 0.0f;
  for (int i = lane; i < n; i += 64) s += parts[i];
  return xor_sum(s);
}

// Items of one sub-tile: (slot, pixel) for the depth back-substitution
// (slot 0 = the frame's own coupling C, g_d, col_i; slot 1 + l = col_j of
// edge l) and (edge, pixel) for the linearisation, 64 pixels per slot.
constexpr int kBsItems = (kMaxDeg + 1) * kSub / kThreads + ((kMaxDeg + 1) * kSub % kThreads ? 1 : 0);
constexpr int kLinItems = kMaxDeg * kSub / kThreads;

template <bool BACKSUB, bool LIN>
__global__ __launch_bounds__(kThreads) void k_lin(LinArgs a) {
  extern __shared__ float sm[];
  const Unit u = a.units[blockIdx.x];
  const Group& g = a.groups[u.group];
  const int d = g.deg, frame = g.frame;
  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int64_t P = a.P;
  const int fac_size = LIN ? max(n_fields(d) * kSub, kWaves * kRec * kRedPitch) : 0;
  float* fac = sm;
  float* rel = sm + fac_size;                 // kMaxDeg x 12
  float* dx = rel + kMaxDeg * 12;             // (kMaxDeg + 1) x 6
  float* bs = dx + (kMaxDeg + 1) * 6;         // (kMaxDeg + 2) x kSub: C, slot parts, old depth
  float* wsum = bs + (kMaxDeg + 3) * kSub;    // kWaves

  if (tid < d) {
    rel_pose(a.poseRt + 16 * frame, a.poseRt + 16 * g.slot_frame[1 + tid], rel + 12 * tid);
  }
  if (BACKSUB && tid < 6 * (d + 1)) dx[tid] = a.dxi[6 * g.slot_frame[tid / 6] + tid % 6];
  const bool apply = BACKSUB && *a.status == 0;
  __syncthreads();
  float* bsC = bs;                     // C of each pixel
  float* bsD = bs + kSub;              // depth before the update
  float* bsS = bs + 2 * kSub;          // slot parts of g_d + col . dxi

  float cost = 0.0f;
  float acc[kTPW][kRec];
  const int passes = LIN ? g.n_passes : 1;
  for (int pass = 0; pass < passes; ++pass) {
    if constexpr (LIN) {
#pragma unroll
      for (int k = 0; k < kTPW; ++k)
#pragma unroll
        for (int e = 0; e < kRec; ++e) acc[k][e] = 0.0f;
    }
    const bool upd = apply && pass == 0;
    for (int sub = u.pix_begin; sub < u.pix_end; sub += kSub) {
      const int npx = min(kSub, u.pix_end - sub);
      // every global load of the sub-tile first: targets and weights of the
      // (edge, pixel) items, then depths and stored coupling of the slots
      float2 tgv[kLinItems];
      float wv[kLinItems];
#pragma unroll
      for (int m = 0; m < kLinItems; ++m) {
        const int it = tid + m * kThreads, l = it >> 6, pl = it & 63;
        tgv[m] = make_float2(0.0f, 0.0f);
        wv[m] = 0.0f;
        if (l < d && pl < npx) {
          const int64_t ep = (int64_t)g.edge[l] * P + sub + pl;
          tgv[m] = reinterpret_cast<const float2*>(a.targets)[ep];
          wv[m] = a.weights[ep];
        }
      }
#pragma unroll
      for (int m = 0; m < kBsItems; ++m) {
        const int it = tid + m * kThreads, sl = it >> 6, pl = it & 63;
        if (sl > d || pl >= npx) continue;
        const int p = sub + pl;
        if (sl == 0) {
          bsD[pl] = a.depth[(int64_t)frame * P + p];
          if (upd) {
            const float* fs = a.fstore + (int64_t)frame * 8 * P + p;
            bsC[pl] = fs[0];
            float v = fs[P];
#pragma unroll
            for (int c = 0; c < 6; ++c) v += fs[(2 + c) * P] * dx[c];
            bsS[pl] = v;
          }
        } else if (upd) {
          const float* es = a.estore + (int64_t)g.edge[sl - 1] * 6 * P + p;
          float v = 0.0f;
#pragma unroll
          for (int c = 0; c < 6; ++c) v += es[c * P] * dx[6 * sl + c];
          bsS[sl * kSub + pl] = v;
        }
      }
      __syncthreads();
      // phase 1: depth after the previous step (redundantly per edge, same
      // arithmetic everywhere), then one (edge, pixel) item per thread
#pragma unroll
      for (int m = 0; m < kLinItems; ++m) {
        const int it = tid + m * kThreads, l = uniform(it >> 6), pl = it & 63;
        if (l >= d) continue;
        if (pl < npx) {
          const int p = sub + pl;
          float dv = bsD[pl];
          if (upd) {
            float sv = bsS[pl];
            for (int s2 = 1; s2 <= d; ++s2) sv += bsS[s2 * kSub + pl];
            const float C = bsC[pl];
            const float step = C > 0.0f ? -sv * frcp(C) : 0.0f;
            dv = dv + step;
            if (l == 0) {
              const int64_t idx = (int64_t)frame * P + p;
              a.depth[idx] = dv;
              a.dd_out[idx] = step;
            }
          }
          PixOut o;
          pix_eval<LIN>(rel + 12 * l, a.fx, a.fy, a.cx, a.cy, a.ifx, a.ify, (float)(p % a.W),
                        (float)(p / a.W), dv, tgv[m].x, tgv[m].y, o);
          const float sw = fsqrt(wv[m]);
          const float sr0 = sw * o.r0, sr1 = sw * o.r1;
          if (pass == 0) cost += sr0 * sr0 + sr1 * sr1;
          if constexpr (LIN) {
            float av[12], bv[12];
#pragma unroll
            for (int k = 0; k < 12; ++k) {
              av[k] = sw * o.ji[k];
              bv[k] = sw * o.jj[k];
            }
            const float sd0 = sw * o.jd[0], sd1 = sw * o.jd[1];
#pragma unroll
            for (int k = 0; k < 12; ++k) {
              fac[(f_a(l) + k) * kSub + pl] = av[k];
              fac[(f_b(l) + k) * kSub + pl] = bv[k];
            }
            fac[(f_sr(l) + 0) * kSub + pl] = sr0;
            fac[(f_sr(l) + 1) * kSub + pl] = sr1;
            const int sc = f_scr(d, l);
            fac[(sc + 0) * kSub + pl] = sd0 * sd0 + sd1 * sd1;
            fac[(sc + 1) * kSub + pl] = sd0 * sr0 + sd1 * sr1;
#pragma unroll
            for (int c = 0; c < 6; ++c) {
              fac[(sc + 2 + c) * kSub + pl] = av[c] * sd0 + av[6 + c] * sd1;
              fac[(f_s(d, 1 + l) + c) * kSub + pl] = bv[c] * sd0 + bv[6 + c] * sd1;
            }
          }
        } else if constexpr (LIN) {
#pragma unroll
          for (int k = 0; k < 26; ++k) fac[(f_a(l) + k) * kSub + pl] = 0.0f;
#pragma unroll
          for (int k = 0; k < 8; ++k) fac[(f_scr(d, l) + k) * kSub + pl] = 0.0f;
#pragma unroll
          for (int c = 0; c < 6; ++c) fac[(f_s(d, 1 + l) + c) * kSub + pl] = 0.0f;
        }
      }
      __syncthreads();
      if constexpr (LIN) {
        // phase 1b: C, g_d and the Schur column of each pixel, scaled by C^-1/2
        if (tid < kSub) {
          const int pl = tid;
          float C = 0.0f, gd = 0.0f, col[6] = {0, 0, 0, 0, 0, 0};
          for (int l = 0; l < d; ++l) {
            const int sc = f_scr(d, l);
            C += fac[(sc + 0) * kSub + pl];
            gd += fac[(sc + 1) * kSub + pl];
#pragma unroll
            for (int c = 0; c < 6; ++c) col[c] += fac[(sc + 2 + c) * kSub + pl];
          }
          if (pass == 0 && pl < npx) {
            const int p = sub + pl;
            float* fs = a.fstore + (int64_t)frame * 8 * P + p;
            fs[0] = C;
            fs[P] = gd;
#pragma unroll
            for (int c = 0; c < 6; ++c) fs[(2 + c) * P] = col[c];
            for (int l = 0; l < d; ++l) {
              float* es = a.estore + (int64_t)g.edge[l] * 6 * P + p;
#pragma unroll
              for (int c = 0; c < 6; ++c) es[c * P] = fac[(f_s(d, 1 + l) + c) * kSub + pl];
            }
          }
          const float inv = C > 0.0f ? frsq(C) : 0.0f;
#pragma unroll
          for (int c = 0; c < 6; ++c) fac[(f_s(d, 0) + c) * kSub + pl] = col[c] * inv;
          for (int l = 0; l < d; ++l)
#pragma unroll
            for (int c = 0; c < 6; ++c) fac[(f_s(d, 1 + l) + c) * kSub + pl] *= inv;
          fac[f_t(d) * kSub + pl] = gd * inv;
        }
        __syncthreads();
        // phase 2: outer-product blocks, one pixel per lane
#pragma unroll
        for (int k = 0; k < kTPW; ++k) {
          const int tl = g.sched[pass][wave][k];
          if (tl < 0) continue;
          const Task& T = a.tasks[g.task_begin + tl];
          const bool diag = T.diag != 0;
          for (int q = 0; q < T.npairs; ++q) {
            const int pk = T.pair[q];
            if (!a.schur && (pk & kSchurPair)) continue;
            const int xo = pk & 511, yo = (pk >> 9) & 511;
            float xv[6], yv[6];
#pragma unroll
            for (int c = 0; c < 6; ++c) {
              xv[c] = fac[(xo + c) * kSub + lane];
              yv[c] = fac[(yo + c) * kSub + lane];
            }
            const float ms = (pk & kNegM) ? -1.0f : 1.0f;
            if (diag) {
              const float zv = fac[((pk >> 18) & 511) * kSub + lane] * ((pk & kNegR) ? -1.0f : 1.0f);
#pragma unroll
              for (int r = 0; r < 6; ++r) {
                const float xm = ms * xv[r];
#pragma unroll
                for (int c = r; c < 6; ++c) acc[k][sym6(r, c)] += xm * yv[c];
                acc[k][21 + r] += xv[r] * zv;
              }
            } else {
#pragma unroll
              for (int r = 0; r < 6; ++r) {
                const float xm = ms * xv[r];
#pragma unroll
                for (int c = 0; c < 6; ++c) acc[k][6 * r + c] += xm * yv[c];
              }
            }
          }
        }
        __syncthreads();
      }
    }
    if constexpr (LIN) {
      // lanes -> one record per task, summed in lane order
      float* rw = fac + wave * kRec * kRedPitch;
#pragma unroll
      for (int k = 0; k < kTPW; ++k) {
        const int tl = g.sched[pass][wave][k];
#pragma unroll
        for (int e = 0; e < kRec; ++e) rw[e * kRedPitch + lane] = acc[k][e];
        __syncthreads();
        if (tl >= 0 && lane < kRec) {
          // four interleaved chains, then a fixed tree
          const float* row = rw + lane * kRedPitch;
          float s0 = 0.0f, s1 = 0.0f, s2 = 0.0f, s3 = 0.0f;
#pragma unroll
          for (int j = 0; j < 64; j += 4) {
            s0 += row[j];
            s1 += row[j + 1];
            s2 += row[j + 2];
            s3 += row[j + 3];
          }
          a.partial[(int64_t)(u.rec_begin + tl) * kRec + lane] = (s0 + s1) + (s2 + s3);
        }
        __syncthreads();
      }
    }
  }
  // block cost: lanes by xor butterfly, waves in order
  const float wsv = xor_sum(cost);
  if (lane == 0) wsum[wave] = wsv;
  __syncthreads();
  if (tid == 0) {
    float s = 0.0f;
    for (int w = 0; w < kWaves; ++w) s += wsum[w];
    a.cost_part[blockIdx.x] = s;
  }
}

// One contribution of a task to an entry of the reduced system: the task's
// record of pixel-range block u sits at partial[(rec0 + u * stride) * 36].
struct Contrib {
  int rec0, stride, mode, pad;   // mode: 0 as is, 1 transposed, 2 plus transpose, 3 packed symmetric
};

constexpr int kAsmLanes = 32;

struct AsmArgs {
  const float* partial;
  const int* blk_ab;       // upper 6x6 blocks (A, B), A <= B, of the reduced system
  const int* blk_ptr;      // contributions of each block
  const Contrib* blk_ent;
  const int* rhs_ptr;      // contributions to each free frame's right-hand side (entries 21..26)
  const Contrib* rhs_ent;
  const float* cost_part;
  float* S;                // nv x nv, both triangles
  float* rhs;              // nv
  float* costs;
  int n_upper, nv, n_units, units_per_group, cost_slot;
};

// Reduced system from the blocks' partial records.  32 lanes share one
// entry (of an upper 6x6 block, then of the right-hand side): lane j takes
// the (contribution, pixel-range block) pairs j, j + 32, ... and the lanes'
// sums meet in a fixed butterfly.  The last block's first wave sums the cost
// partials.
__global__ void k_assemble(AsmArgs a) {
  if (blockIdx.x == gridDim.x - 1) {
    if (a.cost_slot >= 0 && threadIdx.x < 64) {
      const float c = wave_sum_parts(a.cost_part, a.n_units);
      if (threadIdx.x == 0) a.costs[a.cost_slot] = 0.5f * c;
    }
    return;
  }
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const int item = gid / kAsmLanes, ln = gid % kAsmLanes;
  const int NU = a.units_per_group;
  const bool is_blk = item < a.n_upper * kRec;
  const int k = item - a.n_upper * kRec;
  if (!is_blk && k >= a.nv) return;   // whole 32-lane groups leave together
  int q0, q1, i0, i1 = -1, A, B, r, c;
  const Contrib* ents;
  if (is_blk) {
    const int bi = item / kRec, e = item % kRec;
    r = e / 6;
    c = e % 6;
    A = a.blk_ab[2 * bi];
    B = a.blk_ab[2 * bi + 1];
    q0 = a.blk_ptr[bi];
    q1 = a.blk_ptr[bi + 1];
    ents = a.blk_ent;
  } else {
    A = k / 6;
    r = k % 6;
    B = c = 0;
    q0 = a.rhs_ptr[A];
    q1 = a.rhs_ptr[A + 1];
    ents = a.rhs_ent;
  }
  float v = 0.0f;
  for (int pidx = ln; pidx < (q1 - q0) * NU; pidx += kAsmLanes) {
    const Contrib ct = ents[q0 + pidx / NU];
    const float* rec = a.partial + (int64_t)(ct.rec0 + (pidx % NU) * ct.stride) * kRec;
    if (!is_blk) {
      v += rec[21 + r];
      continue;
    }
    switch (ct.mode) {
      case 0: i0 = 6 * r + c; break;
      case 1: i0 = 6 * c + r; break;
      case 2: i0 = 6 * r + c; i1 = 6 * c + r; break;
      default: i0 = sym6(min(r, c), max(r, c)); break;
    }
    v += ct.mode == 2 ? rec[i0] + rec[i1] : rec[i0];
  }
#pragma unroll
  for (int m = kAsmLanes / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kAsmLanes);
  if (ln != 0) return;
  if (is_blk) {
    a.S[(6 * A + r) * a.nv + 6 * B + c] = v;
    if (A != B) a.S[(6 * B + c) * a.nv + 6 * A + r] = v;
  } else {
    a.rhs[k] = v;
  }
}

__global__ void k_cost_final(const float* cost_part, int n_units, float* costs, int slot) {
  const float s = wave_sum_parts(cost_part, n_units);
  if (threadIdx.x == 0) costs[slot] = 0.5f * s;
}

// SE(3) left update of pose (t, q): T <- Exp(xi) T with xi = (rho, phi).
// Coefficients sin(a)/a, (1 - cos a)/a^2, (a - sin a)/a^3 and sin(a/2)/a by
// their Taylor series below a = 0.5 (truncation under 2e-8 relative), where
// the closed forms lose digits in fp32.
__device__ void se3_left_update(const float* xi, float* t, float* q) {
  const float r0 = xi[0], r1 = xi[1], r2 = xi[2], w0 = xi[3], w1 = xi[4], w2 = xi[5];
  const float a2 = w0 * w0 + w1 * w1 + w2 * w2, a = sqrtf(a2);
  float A, Bc, Cc, hs;
  if (a < 0.5f) {
    A = 1.0f - a2 / 6.0f * (1.0f - a2 / 20.0f * (1.0f - a2 / 42.0f));
    Bc = 0.5f - a2 / 24.0f * (1.0f - a2 / 30.0f * (1.0f - a2 / 56.0f));
    Cc = 1.0f / 6.0f - a2 / 120.0f * (1.0f - a2 / 42.0f * (1.0f - a2 / 72.0f));
    hs = 0.5f * (1.0f - a2 / 24.0f * (1.0f - a2 / 80.0f * (1.0f - a2 / 168.0f)));
  } else {
    const float s = sinf(a), h = sinf(0.5f * a);
    A = s / a;
    Bc = 2.0f * h * h / a2;
    Cc = (a - s) / (a2 * a);
    hs = h / a;
  }
  const float hc = cosf(0.5f * a);
  // w x t, w x (w x t), and the same for rho
  const float k0 = w1 * t[2] - w2 * t[1], k1 = w2 * t[0] - w0 * t[2], k2 = w0 * t[1] - w1 * t[0];
  const float kk0 = w1 * k2 - w2 * k1, kk1 = w2 * k0 - w0 * k2, kk2 = w0 * k1 - w1 * k0;
  const float m0 = w1 * r2 - w2 * r1, m1 = w2 * r0 - w0 * r2, m2 = w0 * r1 - w1 * r0;
  const float mm0 = w1 * m2 - w2 * m1, mm1 = w2 * m0 - w0 * m2, mm2 = w0 * m1 - w1 * m0;
  const float nt0 = t[0] + A * k0 + Bc * kk0 + r0 + Bc * m0 + Cc * mm0;
  const float nt1 = t[1] + A * k1 + Bc * kk1 + r1 + Bc * m1 + Cc * mm1;
  const float nt2 = t[2] + A * k2 + Bc * kk2 + r2 + Bc * m2 + Cc * mm2;
  t[0] = nt0; t[1] = nt1; t[2] = nt2;
  // q <- q(Exp(phi)) * q (Hamilton product, [x y z w])
  const float ex = hs * w0, ey = hs * w1, ez = hs * w2, ew = hc;
  const float x = q[0], y = q[1], z = q[2], w = q[3];
  float nx = ew * x + w * ex + (ey * z - ez * y);
  float ny = ew * y + w * ey + (ez * x - ex * z);
  float nz = ew * z + w * ez + (ex * y - ey * x);
  float nw = ew * w - (ex * x + ey * y + ez * z);
  float inv = 1.0f / sqrtf(nx * nx + ny * ny + nz * nz + nw * nw);
  if (nw < 0.0f) inv = -inv;
  q[0] = nx * inv; q[1] = ny * inv; q[2] = nz * inv; q[3] = nw * inv;
}

__device__ void quat_to_rt(const float* t, const float* q, float* o) {
  const float x = q[0], y = q[1], z = q[2], w = q[3];
  o[0] = 1.0f - 2.0f * (y * y + z * z); o[1] = 2.0f * (x * y - w * z); o[2] = 2.0f * (x * z + w * y);
  o[3] = 2.0f * (x * y + w * z); o[4] = 1.0f - 2.0f * (x * x + z * z); o[5] = 2.0f * (y * z - w * x);
  o[6] = 2.0f * (x * z - w * y); o[7] = 2.0f * (y * z + w * x); o[8] = 1.0f - 2.0f * (x * x + y * y);
  o[9] = t[0]; o[10] = t[1]; o[11] = t[2];
  o[12] = o[13] = o[14] = o[15] = 0.0f;
}

// Input poses: normalise q (hemisphere qw >= 0) and derive R, t.
__global__ void k_pose_prep(float* pose7, float* poseRt, int n, int* flags) {
  const int f = blockIdx.x * blockDim.x + threadIdx.x;
  if (f >= n) return;
  float* p = pose7 + 8 * f;
  bool ok = true;
  for (int k = 0; k < 7; ++k) ok = ok && isfinite(p[k]);
  const float nn = p[3] * p[3] + p[4] * p[4] + p[5] * p[5] + p[6] * p[6];
  if (!ok || !(nn > 0.0f) || !isfinite(nn)) {
    atomicOr(flags, 1);
    return;
  }
  float inv = 1.0f / sqrtf(nn);
  if (p[6] < 0.0f) inv = -inv;
  for (int k = 3; k < 7; ++k) p[k] *= inv;
  p[7] = 0.0f;
  quat_to_rt(p, p + 3, poseRt + 16 * f);
}

// flags bit 1: non-finite depth or target, bit 2: bad weight.
__global__ void k_validate(const float* depth, int64_t nd, const float* targets, int64_t nt,
                           const float* weights, int64_t nw, int* flags) {
  int bad = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nd; i += stride)
    if (!isfinite(depth[i])) bad |= 2;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nt; i += stride)
    if (!isfinite(targets[i])) bad |= 2;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nw; i += stride)
    if (!(weights[i] >= 0.0f) || !isfinite(weights[i])) bad |= 4;
  if (bad) atomicOr(flags, bad);
}

struct SolveArgs {
  const float* S;       // nv x nv
  const float* rhs;     // nv
  float* dxi;
  float* pose7;
  float* poseRt;
  int* status;
  int n, nf, nv;
};

__host__ __device__ constexpr int tri6(int i, int j) { return i * (i + 1) / 2 + j; }

constexpr int kMaxNv = 6 * kMaxFree;
constexpr int kSolveLoads = (kMaxNv * kMaxNv + kSolveThreads - 1) / kSolveThreads;

// Cholesky of the 6x6 diagonal block at (k0, k0) in place (lower triangle),
// reciprocals of its diagonal to Ld; *flag = 1 if a pivot is not positive.
// One thread.
__device__ void factor6(float* S, int pitch, int k0, float* Ld, int* flag) {
  float L[21], id[6];
#pragma unroll
  for (int i = 0; i < 6; ++i)
#pragma unroll
    for (int j = 0; j <= i; ++j) L[tri6(i, j)] = S[(k0 + i) * pitch + k0 + j];
  bool ok = true;
#pragma unroll
  for (int j = 0; j < 6; ++j) {
    float dj = L[tri6(j, j)];
#pragma unroll
    for (int l = 0; l < j; ++l) dj -= L[tri6(j, l)] * L[tri6(j, l)];
    ok = ok && dj > 0.0f && isfinite(dj);
    id[j] = frsq(dj);    // 1 / L_jj
    L[tri6(j, j)] = dj * id[j];
#pragma unroll
    for (int i = j + 1; i < 6; ++i) {
      float t = L[tri6(i, j)];
#pragma unroll
      for (int l = 0; l < j; ++l) t -= L[tri6(i, l)] * L[tri6(j, l)];
      L[tri6(i, j)] = t * id[j];
    }
  }
#pragma unroll
  for (int i = 0; i < 6; ++i) {
#pragma unroll
    for (int j = 0; j <= i; ++j) S[(k0 + i) * pitch + k0 + j] = L[tri6(i, j)];
    Ld[k0 + i] = id[i];
  }
  if (!ok) *flag = 1;
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Cholesky of the reduced pose system in LDS by 6x6 blocks (one pose per
// block) with the right-hand side as an extra row, so that the factor's last
// row is L^-1 rhs (the forward solve).  Per block column K: each row below
// solves its 6 panel entries against L_KK, then waves 1.. update the
// trailing matrix while wave 0 updates and factors the next diagonal block
// (look-ahead); two barriers per block column.  The backward solve
// L^T x = y goes block by block (every thread forms x_K, one barrier each).
// Then the retraction of the free poses.
__global__ __launch_bounds__(kSolveThreads) void k_solve(SolveArgs a) {
  extern __shared__ float sm[];
  const int nv = a.nv, pitch = nv + 1, nb = nv / 6;
  const int tid = threadIdx.x, bd = blockDim.x, lane = tid & 63, wave = tid >> 6;
  float* S = sm;                          // (nv + 1) x pitch, row nv = rhs
  float* Pn = S + (nv + 1) * pitch;       // (nv - 5) x 6 panel
  float* Ld = Pn + 6 * max(nv - 5, 0);    // nv reciprocals of the factor's diagonal
  float* xs = Ld + nv;                    // nv
  float* xo = xs + nv;                    // nv
  int* flag = reinterpret_cast<int*>(xo + nv);

  {
    float v[kSolveLoads];
#pragma unroll
    for (int m = 0; m < kSolveLoads; ++m) {
      const int e = tid + m * kSolveThreads;
      v[m] = e < nv * nv ? a.S[e] : 0.0f;
    }
    const float rv = tid < nv ? a.rhs[tid] : 0.0f;
#pragma unroll
    for (int m = 0; m < kSolveLoads; ++m) {
      const int e = tid + m * kSolveThreads;
      if (e < nv * nv) S[(e / nv) * pitch + e % nv] = v[m];
    }
    if (tid < nv) S[nv * pitch + tid] = rv;
  }
  if (tid == 0) *flag = 0;
  __syncthreads();
  const bool prior_fail = *a.status != 0;
  if (!prior_fail && nb > 0) {
    if (tid == 0) factor6(S, pitch, 0, Ld, flag);
    __syncthreads();
    for (int K = 0; K < nb; ++K) {
      if (*flag) break;
      const int k0 = 6 * K, m = nv - k0 - 6, mr = m + 1;   // rows below, with the rhs row
      for (int t = tid; t < mr; t += bd) {
        const float* ar = S + (k0 + 6 + t) * pitch + k0;
        float l[6];
#pragma unroll
        for (int c = 0; c < 6; ++c) {
          float v = ar[c];
#pragma unroll
          for (int q = 0; q < c; ++q) v -= l[q] * S[(k0 + c) * pitch + k0 + q];
          l[c] = v * Ld[k0 + c];
        }
#pragma unroll
        for (int c = 0; c < 6; ++c) Pn[6 * t + c] = l[c];
      }
      __syncthreads();
      if (wave == 0) {
        if (K + 1 < nb) {
          if (lane < 21) {
            int r = 0;
            while (tri6(r + 1, 0) <= lane) ++r;
            const int c = lane - tri6(r, 0);
            float* sp = S + (k0 + 6 + r) * pitch + k0 + 6 + c;
            float v = *sp;
#pragma unroll
            for (int q = 0; q < 6; ++q) v -= Pn[6 * r + q] * Pn[6 * c + q];
            *sp = v;
          }
          wave_lds_sync();
          if (lane == 0) factor6(S, pitch, k0 + 6, Ld, flag);
        }
      } else {
        const int w = tid - 64, ty = w >> 5, tx = w & 31, nty = (bd - 64) >> 5;
        for (int t = w; t < 6 * mr; t += bd - 64) S[(k0 + 6 + t / 6) * pitch + k0 + t % 6] = Pn[t];
        for (int ii = ty; ii < mr; ii += nty) {
          const float* pi = Pn + 6 * ii;
          for (int jj = tx; jj <= ii && jj < m; jj += 32) {
            if (ii < 6) continue;    // next diagonal block: wave 0
            const float* pj = Pn + 6 * jj;
            float* sp = S + (k0 + 6 + ii) * pitch + k0 + 6 + jj;
            float v = *sp;
#pragma unroll
            for (int c = 0; c < 6; ++c) v -= pi[c] * pj[c];
            *sp = v;
          }
        }
      }
      __syncthreads();
    }
  }
  const bool failed = prior_fail || *flag != 0;
  if (!failed) {
    for (int t = tid; t < nv; t += bd) xs[t] = S[nv * pitch + t];
    __syncthreads();
    for (int K = nb - 1; K >= 0; --K) {
      const int k0 = 6 * K;
      float x[6];
#pragma unroll
      for (int c = 5; c >= 0; --c) {
        float v = xs[k0 + c];
#pragma unroll
        for (int q = c + 1; q < 6; ++q) v -= S[(k0 + q) * pitch + k0 + c] * x[q];
        x[c] = v * Ld[k0 + c];
      }
      for (int t = tid; t < k0; t += bd) {
        float v = xs[t];
#pragma unroll
        for (int c = 0; c < 6; ++c) v -= S[(k0 + c) * pitch + t] * x[c];
        xs[t] = v;
      }
      if (tid < 6) xo[k0 + tid] = x[tid];
      __syncthreads();
    }
  }
  __syncthreads();
  if (tid == 0 && failed && !prior_fail) *a.status = DBA_ERR_NOT_SPD;
  for (int f = tid; f < a.n; f += bd) {
    float xi[6] = {0, 0, 0, 0, 0, 0};
    if (!failed && f >= a.nf)
      for (int c = 0; c < 6; ++c) xi[c] = xo[6 * (f - a.nf) + c];
    for (int c = 0; c < 6; ++c) a.dxi[6 * f + c] = xi[c];
    if (!failed && f >= a.nf) {
      float* p = a.pose7 + 8 * f;
      float t[3] = {p[0], p[1], p[2]}, q[4] = {p[3], p[4], p[5], p[6]};
      se3_left_update(xi, t, q);
      for (int c = 0; c < 3; ++c) p[c] = t[c];
      for (int c = 0; c < 4; ++c) p[3 + c] = q[c];
      quat_to_rt(t, q, a.poseRt + 16 * f);
    }
  }
}

// Pose marginal covariance S^-1 of the free poses (the NeRF-SLAM notes'
// cov_cam, sec. 3.2): one workgroup.  Right-looking Cholesky of S in LDS, a
// column per step (scale the column, barrier, update the trailing lower
// triangle, barrier), then thread c solves L L^T x = e_c for column c of the
// inverse, in place in the output (row-major nv x nv, column c written by
// thread c only).  A prior failure or a pivot that is not positive sets
// *status and leaves out untouched.
__global__ __launch_bounds__(kSolveThreads) void k_cov(const float* S_in, int* status,
                                                       float* out, int nv) {
  extern __shared__ float sm[];
  const int pitch = nv + 1, tid = threadIdx.x, bd = blockDim.x;
  float* L = sm;                 // nv x pitch, lower triangle used
  float* Ld = L + nv * pitch;    // nv reciprocals of the factor's diagonal
  for (int e = tid; e < nv * nv; e += bd) L[(e / nv) * pitch + e % nv] = S_in[e];
  const bool prior_fail = *status != 0;
  __syncthreads();
  bool ok = !prior_fail;
  for (int j = 0; j < nv && ok; ++j) {
    const float djj = L[j * pitch + j];        // every thread reads the same value
    ok = djj > 0.0f && isfinite(djj);
    if (!ok) break;
    const float inv = 1.0f / sqrtf(djj);
    for (int i = j + 1 + tid; i < nv; i += bd) L[i * pitch + j] *= inv;
    if (tid == 0) Ld[j] = inv;   // the diagonal itself stays: other waves may still read it
    __syncthreads();
    const int m = nv - j - 1, ty = tid >> 5, tx = tid & 31, nty = bd >> 5;
    for (int ii = ty; ii < m; ii += nty) {
      const int i = j + 1 + ii;
      const float lij = L[i * pitch + j];
      for (int k = j + 1 + tx; k <= i; k += 32) L[i * pitch + k] -= lij * L[k * pitch + j];
    }
    __syncthreads();
  }
  if (!ok) {
    if (tid == 0 && !prior_fail) *status = DBA_ERR_NOT_SPD;
    return;
  }
  const int c = tid;
  if (c >= nv) return;
  // forward: y = L^-1 e_c (zero above row c)
  for (int a = 0; a < c; ++a) out[(int64_t)a * nv + c] = 0.0f;
  out[(int64_t)c * nv + c] = Ld[c];
  for (int a = c + 1; a < nv; ++a) {
    float s = 0.0f;
    for (int l = c; l < a; ++l) s -= L[a * pitch + l] * out[(int64_t)l * nv + c];
    out[(int64_t)a * nv + c] = s * Ld[a];
  }
  // backward: x = L^-T y
  for (int a = nv - 1; a >= 0; --a) {
    float s = out[(int64_t)a * nv + c];
    for (int l = a + 1; l < nv; ++l) s -= L[l * pitch + a] * out[(int64_t)l * nv + c];
    out[(int64_t)a * nv + c] = s * Ld[a];
  }
}

// Per-residual values for inspection, same device function as the solver.
__global__ void k_debug_jac(const float* poseRt, const int* edge_i, const int* edge_j,
                            const float* depth, const float* targets, int E, int P, int W,
                            float fx, float fy, float cx, float cy, float ifx, float ify,
                            float* r, float* Ji, float* Jj, float* Jd) {
  const int64_t k = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (k >= (int64_t)E * P) return;
  const int e = (int)(k / P), p = (int)(k % P);
  const int i = edge_i[e], j = edge_j[e];
  float T[12];
  rel_pose(poseRt + 16 * i, poseRt + 16 * j, T);
  PixOut o;
  pix_eval<true>(T, fx, fy, cx, cy, ifx, ify, (float)(p % W), (float)(p / W),
                 depth[(int64_t)i * P + p], targets[2 * k], targets[2 * k + 1], o);
  r[2 * k] = o.r0;
  r[2 * k + 1] = o.r1;
  for (int c = 0; c < 12; ++c) {
    Ji[12 * k + c] = o.ji[c];
    Jj[12 * k + c] = o.jj[c];
  }
  Jd[2 * k] = o.jd[0];
  Jd[2 * k + 1] = o.jd[1];
}

// ------------------------------------------------------------------ host --

thread_local std::string g_err;

int fail(int code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIPC(expr)                                                   \
  do {                                                               \
    hipError_t e_ = (expr);                                          \
    if (e_ != hipSuccess) {                                          \
      g_err = std::string(#expr) + ": " + hipGetErrorString(e_);     \
      return DBA_ERR_DEVICE;                                         \
    }                                                                \
  } while (0)

#define CHECK_RC(expr)              \
  do {                              \
    int rc_ = (expr);               \
    if (rc_ != DBA_OK) return rc_;  \
  } while (0)

struct Arena {
  char* base = nullptr;
  std::vector<std::pair<void**, size_t>> plan;
  template <class T>
  void add(T*& p, int64_t count) {
    plan.emplace_back(reinterpret_cast<void**>(&p), sizeof(T) * (size_t)std::max<int64_t>(count, 1));
  }
  int commit(hipStream_t s) {
    size_t total = 0;
    for (auto& e : plan) total += (e.second + 255) & ~size_t(255);
    if (hipMalloc(&base, total) != hipSuccess) {
      base = nullptr;
      return fail(DBA_ERR_ALLOC, "hipMalloc of the device arena failed");
    }
    size_t off = 0;
    for (auto& e : plan) {
      *e.first = base + off;
      off += (e.second + 255) & ~size_t(255);
    }
    HIPC(hipMemsetAsync(base, 0, total, s));
    return DBA_OK;
  }
};

struct ProfRec {
  int kernel;
  hipEvent_t a, b;
};

}  // namespace

struct dba_problem {
  dba_options opt{};
  hipStream_t stream = nullptr;
  int n = 0, H = 0, W = 0, E = 0, nf = 0, nv = 0;
  int64_t P = 0;
  float K[4] = {0, 0, 0, 0};
  std::vector<int> h_ei, h_ej;
  int n_groups = 0, n_tasks = 0, n_units = 0, n_records = 0, max_deg = 0, n_upper = 0;
  size_t lin_lds = 0, solve_lds = 0;
  Arena arena;
  float *pose7 = nullptr, *poseRt = nullptr, *dxi = nullptr, *depth = nullptr, *dd = nullptr;
  float *pose7_stage = nullptr, *poseRt_stage = nullptr;   // dba_set_state checks new poses here
  float *targets = nullptr, *weights = nullptr, *fstore = nullptr, *estore = nullptr;
  float *partial = nullptr, *cost_part = nullptr, *costs = nullptr;
  float *S_dbg = nullptr, *rhs_dbg = nullptr;
  int* status = nullptr;
  int* flags = nullptr;
  Group* groups = nullptr;
  Task* tasks = nullptr;
  Unit* units = nullptr;
  int *task_group = nullptr, *blk_ab = nullptr, *blk_ptr = nullptr, *rhs_ptr = nullptr,
      *edge_i = nullptr, *edge_j = nullptr;
  Contrib *blk_ent = nullptr, *rhs_ent = nullptr;
  int units_per_group = 0;
  float* h_pin = nullptr;   // pinned: costs + status
  // per-residual inspection buffers (allocated on first use)
  float *dbg_r = nullptr, *dbg_ji = nullptr, *dbg_jj = nullptr, *dbg_jd = nullptr;
  float* cov_buf = nullptr;   // nv x nv pose covariance (allocated on first use)
  // profiling
  int prof_on = 0;
  int prof_every = 1;
  int64_t prof_seen[DBA_K_NUM] = {0, 0, 0, 0};
  std::vector<ProfRec> prof_recs;
  std::vector<hipEvent_t> prof_pool;
  size_t prof_used = 0;
  int64_t prof_count[DBA_K_NUM] = {0, 0, 0, 0};
  double prof_ms[DBA_K_NUM] = {0, 0, 0, 0};
};

namespace {

int prof_collect(dba_problem* h) {
  for (auto& r : h->prof_recs) {
    float ms = 0.0f;
    HIPC(hipEventElapsedTime(&ms, r.a, r.b));
    h->prof_ms[r.kernel] += ms;
    h->prof_count[r.kernel] += 1;
  }
  h->prof_recs.clear();
  h->prof_used = 0;
  return DBA_OK;
}

// Launch on the handle's stream; when kernel `kid` is being timed, the
// dispatch itself records a pair of pool events at its start and end.
template <typename... KArgs, typename... Args>
int timed_launch(dba_problem* h, int kid, void (*kernel)(KArgs...), dim3 grid, dim3 block,
                 uint32_t shmem, Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (((h->prof_on >> kid) & 1) && h->prof_seen[kid]++ % h->prof_every == 0) {
    if (h->prof_used + 2 > h->prof_pool.size()) {
      for (int i = 0; i < 64; ++i) {
        hipEvent_t e;
        HIPC(hipEventCreate(&e));
        h->prof_pool.push_back(e);
      }
    }
    a = h->prof_pool[h->prof_used++];
    b = h->prof_pool[h->prof_used++];
    h->prof_recs.push_back({kid, a, b});
  }
  hipExtLaunchKernelGGL(kernel, grid, block, shmem, h->stream, a, b, 0u, static_cast<KArgs>(args)...);
  HIPC(hipGetLastError());
  return DBA_OK;
}

LinArgs lin_args(dba_problem* h, int schur) {
  LinArgs a;
  a.groups = h->groups;
  a.tasks = h->tasks;
  a.units = h->units;
  a.poseRt = h->poseRt;
  a.dxi = h->dxi;
  a.depth = h->depth;
  a.dd_out = h->dd;
  a.targets = h->targets;
  a.weights = h->weights;
  a.fstore = h->fstore;
  a.estore = h->estore;
  a.partial = h->partial;
  a.cost_part = h->cost_part;
  a.status = h->status;
  a.fx = h->K[0];
  a.fy = h->K[1];
  a.cx = h->K[2];
  a.cy = h->K[3];
  a.ifx = 1.0f / h->K[0];
  a.ify = 1.0f / h->K[1];
  a.P = (int)h->P;
  a.W = h->W;
  a.schur = schur;
  return a;
}

size_t cost_lds() {
  return (size_t)(kMaxDeg * 12 + (kMaxDeg + 1) * 6 + (kMaxDeg + 3) * kSub + kWaves) * sizeof(float);
}

// Linearisation (LIN) or cost (!LIN) pass, with the previous step's depth
// update applied first when BACKSUB.
template <bool BACKSUB, bool LIN>
int launch_lin(dba_problem* h, int schur) {
  if (h->n_units == 0) return DBA_OK;
  const size_t lds = LIN ? h->lin_lds : cost_lds();
  return timed_launch(h, LIN ? DBA_K_LIN : DBA_K_COST, &k_lin<BACKSUB, LIN>, dim3(h->n_units),
                      dim3(kThreads), (uint32_t)lds, lin_args(h, schur));
}

// Reduced system, right-hand side and (slot >= 0) the cost at the
// linearisation point from the blocks' partials.
int launch_assemble(dba_problem* h, int slot) {
  AsmArgs a;
  a.partial = h->partial;
  a.blk_ab = h->blk_ab;
  a.blk_ptr = h->blk_ptr;
  a.blk_ent = h->blk_ent;
  a.rhs_ptr = h->rhs_ptr;
  a.rhs_ent = h->rhs_ent;
  a.cost_part = h->cost_part;
  a.S = h->S_dbg;
  a.rhs = h->rhs_dbg;
  a.costs = h->costs;
  a.n_upper = h->n_upper;
  a.nv = h->nv;
  a.n_units = h->n_units;
  a.units_per_group = h->units_per_group;
  a.cost_slot = slot;
  const int64_t n = (int64_t)(h->n_upper * kRec + h->nv) * kAsmLanes;
  return timed_launch(h, DBA_K_ASSEMBLE, &k_assemble, dim3((unsigned)((n + 255) / 256) + 1),
                      dim3(256), 0u, a);
}

int launch_solve(dba_problem* h) {
  SolveArgs a;
  a.S = h->S_dbg;
  a.rhs = h->rhs_dbg;
  a.dxi = h->dxi;
  a.pose7 = h->pose7;
  a.poseRt = h->poseRt;
  a.status = h->status;
  a.n = h->n;
  a.nf = h->nf;
  a.nv = h->nv;
  return timed_launch(h, DBA_K_SOLVE, &k_solve, dim3(1), dim3(kSolveThreads),
                      (uint32_t)h->solve_lds, a);
}

int launch_cost_final(dba_problem* h, int slot) {
  hipLaunchKernelGGL(k_cost_final, dim3(1), dim3(64), 0, h->stream, h->cost_part, h->n_units,
                     h->costs, slot);
  HIPC(hipGetLastError());
  return DBA_OK;
}

// Reads costs[0..n_costs) and the status word; synchronises the stream.
int fetch(dba_problem* h, int n_costs, float* out) {
  int* st = reinterpret_cast<int*>(h->h_pin + kCostCap);
  if (n_costs > 0)
    HIPC(hipMemcpyAsync(h->h_pin, h->costs, sizeof(float) * n_costs, hipMemcpyDeviceToHost, h->stream));
  HIPC(hipMemcpyAsync(st, h->status, sizeof(int), hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  if (h->prof_on) CHECK_RC(prof_collect(h));
  if (out)
    for (int i = 0; i < n_costs; ++i) out[i] = h->h_pin[i];
  if (*st != 0) {
    HIPC(hipMemsetAsync(h->status, 0, sizeof(int), h->stream));
    return fail(*st, "the reduced pose system is not positive definite");
  }
  for (int i = 0; i < n_costs; ++i)
    if (!std::isfinite(h->h_pin[i])) return fail(DBA_ERR_NONFINITE, "non-finite cost");
  return DBA_OK;
}

// ---- planning (host, once) -------------------------------------------------

int pack_pair(int x, int y, int z, int flags) { return x | (y << 9) | (z << 18) | flags; }

int build_plan(dba_problem* h, std::vector<Group>& groups, std::vector<Task>& tasks,
               std::vector<Unit>& units, std::vector<int>& task_group, std::vector<int>& blk_ab,
               std::vector<int>& blk_ptr, std::vector<Contrib>& blk_ent, std::vector<int>& rhs_ptr,
               std::vector<Contrib>& rhs_ent) {
  const int n = h->n, nf = h->nf, nfree = n - nf;
  std::vector<std::vector<int>> out(n);
  for (int e = 0; e < h->E; ++e) out[h->h_ei[e]].push_back(e);
  struct TaskInfo {
    int fa, fb, diag;
  };
  std::vector<TaskInfo> tinfo;
  int total_sub = 0;
  for (int i = 0; i < n; ++i)
    if (!out[i].empty()) total_sub += (int)((h->P + kSub - 1) / kSub);
  int n_grp = 0;
  for (int i = 0; i < n; ++i) n_grp += !out[i].empty();
  const int sub_per_unit = n_grp ? std::max(1, (int)std::lround((double)total_sub / kTargetBlocks)) : 1;
  int rec = 0;
  for (int i = 0; i < n; ++i) {
    const int d = (int)out[i].size();
    if (d == 0) continue;
    if (d > kMaxDeg)
      return fail(DBA_ERR_LIMIT, "frame " + std::to_string(i) + " has " + std::to_string(d) +
                                     " out-edges; the limit is " + std::to_string(kMaxDeg));
    h->max_deg = std::max(h->max_deg, d);
    Group g;
    std::memset(&g, 0, sizeof(g));
    g.frame = i;
    g.deg = d;
    g.slot_frame[0] = i;
    for (int l = 0; l < d; ++l) {
      g.edge[l] = out[i][l];
      g.slot_frame[1 + l] = h->h_ej[out[i][l]];
    }
    g.task_begin = (int)tasks.size();
    // tasks in a fixed order; frames by slot
    std::vector<std::pair<Task, std::pair<int, int>>> tl;
    auto add = [&](int sa, int sb, int diag, std::vector<int> pairs) {
      Task t;
      std::memset(&t, 0, sizeof(t));
      t.diag = diag;
      t.npairs = (int)pairs.size();
      for (size_t q = 0; q < pairs.size(); ++q) t.pair[q] = pairs[q];
      tl.push_back({t, {sa, sb}});
    };
    {
      std::vector<int> p00;
      for (int l = 0; l < d; ++l) {
        p00.push_back(pack_pair(f_a(l), f_a(l), f_sr(l), kNegR));
        p00.push_back(pack_pair(f_a(l) + 6, f_a(l) + 6, f_sr(l) + 1, kNegR));
      }
      p00.push_back(pack_pair(f_s(d, 0), f_s(d, 0), f_t(d), kNegM | kSchurPair));
      add(0, 0, 1, p00);
    }
    for (int l = 0; l < d; ++l)
      add(0, 1 + l, 0, {pack_pair(f_a(l), f_b(l), 0, 0), pack_pair(f_a(l) + 6, f_b(l) + 6, 0, 0),
                        pack_pair(f_s(d, 0), f_s(d, 1 + l), 0, kNegM | kSchurPair)});
    for (int l = 0; l < d; ++l)
      add(1 + l, 1 + l, 1, {pack_pair(f_b(l), f_b(l), f_sr(l), kNegR),
                            pack_pair(f_b(l) + 6, f_b(l) + 6, f_sr(l) + 1, kNegR),
                            pack_pair(f_s(d, 1 + l), f_s(d, 1 + l), f_t(d), kNegM | kSchurPair)});
    for (int l = 0; l < d; ++l)
      for (int m = l + 1; m < d; ++m)
        add(1 + l, 1 + m, 0, {pack_pair(f_s(d, 1 + l), f_s(d, 1 + m), 0, kNegM | kSchurPair)});
    g.n_tasks = (int)tl.size();
    // schedule: longest task first into the (pass, wave) bin with the fewest pairs
    const int bins_per_pass = kWaves;
    g.n_passes = (g.n_tasks + kWaves * kTPW - 1) / (kWaves * kTPW);
    std::memset(g.sched, -1, sizeof(g.sched));
    std::vector<int> order(g.n_tasks);
    for (int t = 0; t < g.n_tasks; ++t) order[t] = t;
    std::stable_sort(order.begin(), order.end(),
                     [&](int x, int y) { return tl[x].first.npairs > tl[y].first.npairs; });
    const int nbins = g.n_passes * bins_per_pass;
    std::vector<int> load(nbins, 0), cnt(nbins, 0);
    for (int t : order) {
      int best = -1;
      for (int b = 0; b < nbins; ++b)
        if (cnt[b] < kTPW && (best < 0 || load[b] < load[best])) best = b;
      g.sched[best / kWaves][best % kWaves][cnt[best]] = (signed char)t;
      load[best] += tl[t].first.npairs;
      cnt[best] += 1;
    }
    for (auto& t : tl) {
      tasks.push_back(t.first);
      tinfo.push_back({g.slot_frame[t.second.first], g.slot_frame[t.second.second], t.first.diag});
      task_group.push_back((int)groups.size());
    }
    // pixel ranges
    const int nsub = (int)((h->P + kSub - 1) / kSub);
    const int nu = (nsub + sub_per_unit - 1) / sub_per_unit;
    g.unit_begin = (int)units.size();
    g.n_units = nu;
    h->units_per_group = nu;
    g.rec_begin = rec;
    for (int k = 0; k < nu; ++k) {
      Unit u;
      u.group = (int)groups.size();
      u.pix_begin = k * sub_per_unit * kSub;
      u.pix_end = (int)std::min<int64_t>(h->P, (int64_t)(k + 1) * sub_per_unit * kSub);
      u.rec_begin = rec + k * g.n_tasks;
      units.push_back(u);
    }
    rec += nu * g.n_tasks;
    groups.push_back(g);
  }
  h->n_records = rec;
  // assembly lists over the free frames: upper 6x6 blocks in row order
  std::vector<std::vector<int>> blk(std::max(1, nfree * nfree)), rl(std::max(1, nfree));
  for (size_t t = 0; t < tinfo.size(); ++t) {
    const int A = tinfo[t].fa - nf, B = tinfo[t].fb - nf;
    if (A < 0 || B < 0) continue;
    const int tt = (int)t << 2;
    if (tinfo[t].diag) {
      blk[A * nfree + A].push_back(tt | 3);
      rl[A].push_back((int)t);
    } else if (A == B) {
      blk[A * nfree + A].push_back(tt | 2);
    } else if (A < B) {
      blk[A * nfree + B].push_back(tt | 0);
    } else {
      blk[B * nfree + A].push_back(tt | 1);
    }
  }
  auto contrib = [&](int x) {
    const int t = x >> 2;
    const Group& g = groups[task_group[t]];
    return Contrib{g.rec_begin + (t - g.task_begin), g.n_tasks, x & 3, 0};
  };
  blk_ptr.assign(1, 0);
  for (int A = 0; A < nfree; ++A)
    for (int B = A; B < nfree; ++B) {
      blk_ab.push_back(A);
      blk_ab.push_back(B);
      for (int x : blk[A * nfree + B]) blk_ent.push_back(contrib(x));
      blk_ptr.push_back((int)blk_ent.size());
    }
  rhs_ptr.assign(1, 0);
  for (int A = 0; A < nfree; ++A) {
    for (int x : rl[A]) rhs_ent.push_back(contrib(x << 2));
    rhs_ptr.push_back((int)rhs_ent.size());
  }
  return DBA_OK;
}

template <class T>
int upload(dba_problem* h, T* dst, const std::vector<T>& src) {
  if (!src.empty())
    HIPC(hipMemcpyAsync(dst, src.data(), sizeof(T) * src.size(), hipMemcpyHostToDevice, h->stream));
  return DBA_OK;
}

int copy_in(dba_problem* h, void* dst, const void* src, size_t bytes) {
  if (bytes == 0) return DBA_OK;
  HIPC(hipMemcpyAsync(dst, src, bytes,
                      h->opt.mem == DBA_MEM_DEVICE ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice,
                      h->stream));
  return DBA_OK;
}

// Poses n x 7 from the caller into the padded n x 8 state, then normalised.
int poses_in(dba_problem* h, const float* poses) {
  HIPC(hipMemcpy2DAsync(h->pose7, 8 * sizeof(float), poses, 7 * sizeof(float), 7 * sizeof(float),
                        h->n,
                        h->opt.mem == DBA_MEM_DEVICE ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice,
                        h->stream));
  hipLaunchKernelGGL(k_pose_prep, dim3((h->n + 63) / 64), dim3(64), 0, h->stream, h->pose7, h->poseRt,
                     h->n, h->flags);
  HIPC(hipGetLastError());
  return DBA_OK;
}

int check_flags(dba_problem* h) {
  int f = 0;
  HIPC(hipMemcpyAsync(&f, h->flags, sizeof(int), hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  if (f) {
    HIPC(hipMemsetAsync(h->flags, 0, sizeof(int), h->stream));
    if (f & 1) return fail(DBA_ERR_NONFINITE, "a pose is non-finite or has a zero quaternion");
    if (f & 4) return fail(DBA_ERR_NONFINITE, "a weight is negative or non-finite");
    return fail(DBA_ERR_NONFINITE, "a depth or target is non-finite");
  }
  return DBA_OK;
}

int create(const float* poses, const float* inv_depth, int n, int H, int W, const float* K,
           const int32_t* edges, int E, const float* targets, const float* weights, int n_fixed,
           const dba_options* opts, dba_problem* h) {
  if (!poses || !inv_depth || !K || (E > 0 && (!edges || !targets || !weights)))
    return fail(DBA_ERR_ARG, "null input pointer");
  if (n <= 0 || H <= 0 || W <= 0 || E < 0 || n_fixed < 0 || n_fixed > n)
    return fail(DBA_ERR_ARG, "bad sizes");
  if ((int64_t)H * W > (int64_t)1 << 30) return fail(DBA_ERR_ARG, "image too large");
  if (opts) h->opt = *opts;
  if (h->opt.mem != DBA_MEM_HOST && h->opt.mem != DBA_MEM_DEVICE) return fail(DBA_ERR_ARG, "bad mem option");
  h->stream = static_cast<hipStream_t>(h->opt.stream);
  h->n = n;
  h->H = H;
  h->W = W;
  h->E = E;
  h->nf = n_fixed;
  h->P = (int64_t)H * W;
  if (n - n_fixed > kMaxFree)
    return fail(DBA_ERR_LIMIT, "more than " + std::to_string(kMaxFree) + " free frames");
  h->nv = 6 * (n - n_fixed);
  float Kh[4];
  std::vector<int32_t> eh(2 * (size_t)E);
  if (h->opt.mem == DBA_MEM_DEVICE) {
    HIPC(hipMemcpy(Kh, K, sizeof(Kh), hipMemcpyDeviceToHost));
    if (E) HIPC(hipMemcpy(eh.data(), edges, sizeof(int32_t) * 2 * E, hipMemcpyDeviceToHost));
  } else {
    std::memcpy(Kh, K, sizeof(Kh));
    if (E) std::memcpy(eh.data(), edges, sizeof(int32_t) * 2 * E);
  }
  for (int k = 0; k < 4; ++k)
    if (!std::isfinite(Kh[k]) || (k < 2 && Kh[k] == 0.0f)) return fail(DBA_ERR_NONFINITE, "bad intrinsics");
  std::memcpy(h->K, Kh, sizeof(Kh));
  h->h_ei.resize(E);
  h->h_ej.resize(E);
  for (int e = 0; e < E; ++e) {
    const int i = eh[2 * e], j = eh[2 * e + 1];
    if (i < 0 || i >= n || j < 0 || j >= n) return fail(DBA_ERR_ARG, "edge index out of range");
    h->h_ei[e] = i;
    h->h_ej[e] = j;
  }
  std::vector<Group> groups;
  std::vector<Task> tasks;
  std::vector<Unit> units;
  std::vector<int> task_group, blk_ab, blk_ptr, rhs_ptr;
  std::vector<Contrib> blk_ent, rhs_ent;
  CHECK_RC(build_plan(h, groups, tasks, units, task_group, blk_ab, blk_ptr, blk_ent, rhs_ptr,
                      rhs_ent));
  h->n_upper = (int)blk_ab.size() / 2;
  h->n_groups = (int)groups.size();
  h->n_tasks = (int)tasks.size();
  h->n_units = (int)units.size();
  const int fac = h->max_deg ? std::max(n_fields(h->max_deg) * kSub, kWaves * kRec * kRedPitch) : 0;
  h->lin_lds = (size_t)fac * sizeof(float) + cost_lds();
  h->solve_lds = ((size_t)(h->nv + 1) * (h->nv + 1) + 6 * (size_t)std::max(h->nv - 5, 0) +
                  3 * (size_t)h->nv + 4) * sizeof(float);
  {
    // The dynamic-LDS limit is a per-process attribute of each kernel: it is
    // only ever raised, to the largest size any handle has needed, so that a
    // smaller handle created later cannot lower it below an earlier one's.
    static std::mutex mu;
    static size_t lin_max = 65536, solve_max = 65536;
    std::lock_guard<std::mutex> lock(mu);
    if (h->lin_lds > lin_max) {
      HIPC(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_lin<true, true>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)h->lin_lds));
      HIPC(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_lin<false, true>),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)h->lin_lds));
      lin_max = h->lin_lds;
    }
    if (h->solve_lds > solve_max) {
      HIPC(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_solve),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)h->solve_lds));
      // k_cov needs nv (nv + 2) floats, within the solver's size
      HIPC(hipFuncSetAttribute(reinterpret_cast<const void*>(&k_cov),
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)h->solve_lds));
      solve_max = h->solve_lds;
    }
  }

  const int64_t P = h->P;
  Arena& A = h->arena;
  A.add(h->pose7, 8 * (int64_t)n);
  A.add(h->poseRt, 16 * (int64_t)n);
  A.add(h->pose7_stage, 8 * (int64_t)n);
  A.add(h->poseRt_stage, 16 * (int64_t)n);
  A.add(h->dxi, 6 * (int64_t)n);
  A.add(h->depth, n * P);
  A.add(h->dd, n * P);
  A.add(h->targets, 2 * E * P);
  A.add(h->weights, E * P);
  A.add(h->fstore, 8 * n * P);
  A.add(h->estore, 6 * E * P);
  A.add(h->partial, (int64_t)h->n_records * kRec);
  A.add(h->cost_part, std::max(1, h->n_units));
  A.add(h->costs, kCostCap);
  A.add(h->S_dbg, (int64_t)h->nv * h->nv);
  A.add(h->rhs_dbg, h->nv);
  A.add(h->status, 4);
  A.add(h->flags, 4);
  A.add(h->groups, h->n_groups);
  A.add(h->tasks, h->n_tasks);
  A.add(h->units, h->n_units);
  A.add(h->task_group, h->n_tasks);
  A.add(h->blk_ab, (int64_t)blk_ab.size());
  A.add(h->blk_ptr, (int64_t)blk_ptr.size());
  A.add(h->blk_ent, (int64_t)blk_ent.size());
  A.add(h->rhs_ptr, (int64_t)rhs_ptr.size());
  A.add(h->rhs_ent, (int64_t)rhs_ent.size());
  A.add(h->edge_i, E);
  A.add(h->edge_j, E);
  CHECK_RC(A.commit(h->stream));
  if (hipHostMalloc(reinterpret_cast<void**>(&h->h_pin), sizeof(float) * (kCostCap + 4)) != hipSuccess) {
    h->h_pin = nullptr;
    return fail(DBA_ERR_ALLOC, "pinned host buffer");
  }
  CHECK_RC(upload(h, h->groups, groups));
  CHECK_RC(upload(h, h->tasks, tasks));
  CHECK_RC(upload(h, h->units, units));
  CHECK_RC(upload(h, h->task_group, task_group));
  CHECK_RC(upload(h, h->blk_ab, blk_ab));
  CHECK_RC(upload(h, h->blk_ptr, blk_ptr));
  CHECK_RC(upload(h, h->blk_ent, blk_ent));
  CHECK_RC(upload(h, h->rhs_ptr, rhs_ptr));
  CHECK_RC(upload(h, h->rhs_ent, rhs_ent));
  CHECK_RC(upload(h, h->edge_i, h->h_ei));
  CHECK_RC(upload(h, h->edge_j, h->h_ej));
  CHECK_RC(copy_in(h, h->depth, inv_depth, sizeof(float) * n * P));
  CHECK_RC(copy_in(h, h->targets, targets, sizeof(float) * 2 * E * P));
  CHECK_RC(copy_in(h, h->weights, weights, sizeof(float) * E * P));
  CHECK_RC(poses_in(h, poses));
  hipLaunchKernelGGL(k_validate, dim3(256), dim3(256), 0, h->stream, h->depth, n * P, h->targets,
                     2 * E * P, h->weights, E * P, h->flags);
  HIPC(hipGetLastError());
  return check_flags(h);
}

}  // namespace

extern "C" {

int dba_options_default(dba_options* o) {
  if (!o) return fail(DBA_ERR_ARG, "null options");
  o->mem = DBA_MEM_HOST;
  o->stream = nullptr;
  return DBA_OK;
}

void dba_destroy(dba_problem* h) {
  if (!h) return;
  if (h->arena.base) {
    (void)hipStreamSynchronize(h->stream);
    (void)hipFree(h->arena.base);
  }
  if (h->h_pin) (void)hipHostFree(h->h_pin);
  for (float* p : {h->dbg_r, h->dbg_ji, h->dbg_jj, h->dbg_jd, h->cov_buf})
    if (p) (void)hipFree(p);
  for (hipEvent_t e : h->prof_pool) (void)hipEventDestroy(e);
  delete h;
}

int dba_create(const float* poses, const float* inv_depth, int n_frames, int height, int width,
               const float* intrinsics, const int32_t* edges, int n_edges, const float* targets,
               const float* weights, int n_fixed, const dba_options* opts, dba_problem** out) {
  if (!out) return fail(DBA_ERR_ARG, "null output handle");
  *out = nullptr;
  dba_problem* h = new (std::nothrow) dba_problem();
  if (!h) return fail(DBA_ERR_ALLOC, "host allocation");
  dba_options_default(&h->opt);
  const int rc = create(poses, inv_depth, n_frames, height, width, intrinsics, edges, n_edges,
                        targets, weights, n_fixed, opts, h);
  if (rc != DBA_OK) {
    const std::string keep = g_err;
    dba_destroy(h);
    g_err = keep;
    return rc;
  }
  *out = h;
  return DBA_OK;
}

int dba_gn_step(dba_problem* h, dba_step_info* info) {
  if (!h) return fail(DBA_ERR_ARG, "null handle");
  CHECK_RC((launch_lin<false, true>(h, 1)));
  CHECK_RC(launch_assemble(h, 0));
  CHECK_RC(launch_solve(h));
  CHECK_RC((launch_lin<true, false>(h, 1)));
  CHECK_RC(launch_cost_final(h, 1));
  float c[2];
  CHECK_RC(fetch(h, 2, c));
  if (info) {
    info->cost_before = c[0];
    info->cost_after = c[1];
  }
  return DBA_OK;
}

int dba_solve(dba_problem* h, int n_iters, float* costs) {
  if (!h || n_iters < 0) return fail(DBA_ERR_ARG, "bad arguments");
  if (n_iters == 0) {
    CHECK_RC((launch_lin<false, false>(h, 1)));
    CHECK_RC(launch_cost_final(h, 0));
    return fetch(h, 1, costs);
  }
  // chunks of kCostCap - 1 steps between host reads of the costs
  int done = 0;
  while (done < n_iters) {
    const int m = std::min(n_iters - done, kCostCap - 1);
    CHECK_RC((launch_lin<false, true>(h, 1)));
    CHECK_RC(launch_assemble(h, 0));
    CHECK_RC(launch_solve(h));
    for (int k = 1; k < m; ++k) {
      CHECK_RC((launch_lin<true, true>(h, 1)));
      CHECK_RC(launch_assemble(h, k));
      CHECK_RC(launch_solve(h));
    }
    CHECK_RC((launch_lin<true, false>(h, 1)));
    CHECK_RC(launch_cost_final(h, m));
    CHECK_RC(fetch(h, m + 1, costs ? costs + done : nullptr));
    done += m;
  }
  return DBA_OK;
}

int dba_cost(dba_problem* h, float* cost) {
  if (!h || !cost) return fail(DBA_ERR_ARG, "null argument");
  CHECK_RC((launch_lin<false, false>(h, 1)));
  CHECK_RC(launch_cost_final(h, 0));
  return fetch(h, 1, cost);
}

int dba_covariance(dba_problem* h, float* cov) {
  if (!h || !cov) return fail(DBA_ERR_ARG, "null argument");
  const int64_t nv = h->nv;
  if (nv == 0) return DBA_OK;
  if (!h->cov_buf && hipMalloc(&h->cov_buf, sizeof(float) * nv * nv) != hipSuccess) {
    h->cov_buf = nullptr;
    return fail(DBA_ERR_ALLOC, "covariance buffer");
  }
  CHECK_RC((launch_lin<false, true>(h, 1)));
  CHECK_RC(launch_assemble(h, -1));
  hipLaunchKernelGGL(k_cov, dim3(1), dim3(kSolveThreads), h->solve_lds, h->stream, h->S_dbg,
                     h->status, h->cov_buf, h->nv);
  HIPC(hipGetLastError());
  CHECK_RC(fetch(h, 0, nullptr));
  HIPC(hipMemcpyAsync(cov, h->cov_buf, sizeof(float) * nv * nv, hipMemcpyDeviceToHost, h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  return DBA_OK;
}

int dba_get_state(dba_problem* h, float* poses, float* inv_depth) {
  if (!h) return fail(DBA_ERR_ARG, "null handle");
  if (poses)
    HIPC(hipMemcpy2DAsync(poses, 7 * sizeof(float), h->pose7, 8 * sizeof(float), 7 * sizeof(float),
                          h->n, hipMemcpyDeviceToHost, h->stream));
  if (inv_depth)
    HIPC(hipMemcpyAsync(inv_depth, h->depth, sizeof(float) * h->n * h->P, hipMemcpyDeviceToHost,
                        h->stream));
  HIPC(hipStreamSynchronize(h->stream));
  return DBA_OK;
}

// The new state is staged and checked first (depths in the depth-step buffer,
// which holds nothing between steps; poses in their own staging rows) and
// copied over the current state only when it is valid, so a rejected call
// leaves the handle as it was.
int dba_set_state(dba_problem* h, const float* poses, const float* inv_depth) {
  if (!h) return fail(DBA_ERR_ARG, "null handle");
  const size_t dbytes = sizeof(float) * h->n * h->P;
  if (inv_depth) {
    CHECK_RC(copy_in(h, h->dd, inv_depth, dbytes));
    hipLaunchKernelGGL(k_validate, dim3(64), dim3(256), 0, h->stream, h->dd, h->n * h->P,
                       h->targets, (int64_t)0, h->weights, (int64_t)0, h->flags);
    HIPC(hipGetLastError());
  }
  if (poses) {
    HIPC(hipMemcpy2DAsync(h->pose7_stage, 8 * sizeof(float), poses, 7 * sizeof(float),
                          7 * sizeof(float), h->n,
                          h->opt.mem == DBA_MEM_DEVICE ? hipMemcpyDeviceToDevice : hipMemcpyHostToDevice,
                          h->stream));
    hipLaunchKernelGGL(k_pose_prep, dim3((h->n + 63) / 64), dim3(64), 0, h->stream, h->pose7_stage,
                       h->poseRt_stage, h->n, h->flags);
    HIPC(hipGetLastError());
  }
  CHECK_RC(check_flags(h));
  if (inv_depth && dbytes)
    HIPC(hipMemcpyAsync(h->depth, h->dd, dbytes, hipMemcpyDeviceToDevice, h->stream));
  if (poses) {
    HIPC(hipMemcpyAsync(h->pose7, h->pose7_stage, sizeof(float) * 8 * h->n, hipMemcpyDeviceToDevice,
                        h->stream));
    HIPC(hipMemcpyAsync(h->poseRt, h->poseRt_stage, sizeof(float) * 16 * h->n,
                        hipMemcpyDeviceToDevice, h->stream));
  }
  HIPC(hipStreamSynchronize(h->stream));
  return DBA_OK;
}

int dba_get_sizes(const dba_problem* h, int* n_frames, int* n_pixels, int* n_edges, int* n_fixed) {
  if (!h) return fail(DBA_ERR_ARG, "null handle");
  if (n_frames) *n_frames = h->n;
  if (n_pixels) *n_pixels = (int)h->P;
  if (n_edges) *n_edges = h->E;
  if (n_fixed) *n_fixed = h->nf;
  return DBA_OK;
}

int dba_debug_run(dba_problem* h, int stage) {
  if (!h) return fail(DBA_ERR_ARG, "null handle");
  if (stage == DBA_STAGE_ASSEMBLE) {
    CHECK_RC((launch_lin<false, true>(h, 0)));
    CHECK_RC(launch_assemble(h, -1));
    HIPC(hipStreamSynchronize(h->stream));
    if (h->prof_on) CHECK_RC(prof_collect(h));
    return DBA_OK;
  }
  if (stage == DBA_STAGE_JACOBIANS) {
    const int64_t m = (int64_t)h->E * h->P;
    if (m == 0) return DBA_OK;
    if (!h->dbg_r) {
      if (hipMalloc(&h->dbg_r, sizeof(float) * 2 * m) != hipSuccess ||
          hipMalloc(&h->dbg_ji, sizeof(float) * 12 * m) != hipSuccess ||
          hipMalloc(&h->dbg_jj, sizeof(float) * 12 * m) != hipSuccess ||
          hipMalloc(&h->dbg_jd, sizeof(float) * 2 * m) != hipSuccess)
        return fail(DBA_ERR_ALLOC, "inspection buffers");
    }
    hipLaunchKernelGGL(k_debug_jac, dim3((unsigned)((m + 255) / 256)), dim3(256), 0, h->stream,
                       h->poseRt, h->edge_i, h->edge_j, h->depth, h->targets, h->E, (int)h->P, h->W,
                       h->K[0], h->K[1], h->K[2], h->K[3], 1.0f / h->K[0], 1.0f / h->K[1], h->dbg_r,
                       h->dbg_ji, h->dbg_jj, h->dbg_jd);
    HIPC(hipGetLastError());
    HIPC(hipStreamSynchronize(h->stream));
    return DBA_OK;
  }
  return fail(DBA_ERR_ARG, "unknown stage");
}

int64_t dba_debug_size(const dba_problem* h, int which) {
  if (!h) return DBA_ERR_ARG;
  const int64_t n = h->n, P = h->P, E = h->E, nv = h->nv;
  switch (which) {
    case DBA_DBG_S: return 4 * nv * nv;
    case DBA_DBG_RHS: return 4 * nv;
    case DBA_DBG_DXI: return 4 * 6 * n;
    case DBA_DBG_DD: case DBA_DBG_C: case DBA_DBG_GD: return 4 * n * P;
    case DBA_DBG_R: case DBA_DBG_JD: return 4 * 2 * E * P;
    case DBA_DBG_JI: case DBA_DBG_JJ: return 4 * 12 * E * P;
    default: return DBA_ERR_ARG;
  }
}

int dba_debug_get(dba_problem* h, int which, void* host_out, int64_t bytes) {
  if (!h || !host_out) return fail(DBA_ERR_ARG, "null argument");
  const int64_t need = dba_debug_size(h, which);
  if (need < 0 || bytes != need) return fail(DBA_ERR_ARG, "bad debug id or size");
  if (need == 0) return DBA_OK;
  const float* src = nullptr;
  switch (which) {
    case DBA_DBG_S: src = h->S_dbg; break;
    case DBA_DBG_RHS: src = h->rhs_dbg; break;
    case DBA_DBG_DXI: src = h->dxi; break;
    case DBA_DBG_DD: src = h->dd; break;
    case DBA_DBG_R: src = h->dbg_r; break;
    case DBA_DBG_JI: src = h->dbg_ji; break;
    case DBA_DBG_JJ: src = h->dbg_jj; break;
    case DBA_DBG_JD: src = h->dbg_jd; break;
    default: break;
  }
  if (which == DBA_DBG_C || which == DBA_DBG_GD) {
    const int field = which == DBA_DBG_C ? 0 : 1;
    HIPC(hipMemcpy2DAsync(host_out, h->P * sizeof(float), h->fstore + field * h->P,
                          8 * h->P * sizeof(float), h->P * sizeof(float), h->n,
                          hipMemcpyDeviceToHost, h->stream));
  } else {
    if (!src) return fail(DBA_ERR_ARG, "run DBA_STAGE_JACOBIANS first");
    HIPC(hipMemcpyAsync(host_out, src, bytes, hipMemcpyDeviceToHost, h->stream));
  }
  HIPC(hipStreamSynchronize(h->stream));
  return DBA_OK;
}

int dba_profile_enable(dba_problem* h, int kernel_mask, int every) {
  if (!h) return fail(DBA_ERR_ARG, "null handle");
  if (every < 1) return fail(DBA_ERR_ARG, "every must be >= 1");
  h->prof_on = kernel_mask;
  h->prof_every = every;
  for (int k = 0; k < DBA_K_NUM; ++k) h->prof_seen[k] = 0;
  h->prof_recs.clear();
  h->prof_used = 0;
  return DBA_OK;
}

int dba_profile_reset(dba_problem* h) {
  if (!h) return fail(DBA_ERR_ARG, "null handle");
  for (int k = 0; k < DBA_K_NUM; ++k) {
    h->prof_count[k] = 0;
    h->prof_ms[k] = 0.0;
  }
  return DBA_OK;
}

int dba_profile_get(dba_problem* h, int kernel, int64_t* launches, double* total_ms) {
  if (!h || kernel < 0 || kernel >= DBA_K_NUM) return fail(DBA_ERR_ARG, "bad kernel id");
  if (launches) *launches = h->prof_count[kernel];
  if (total_ms) *total_ms = h->prof_ms[kernel];
  return DBA_OK;
}

const char* dba_kernel_name(int kernel) {
  static const char* names[DBA_K_NUM] = {"lin", "assemble", "solve", "cost"};
  return kernel >= 0 && kernel < DBA_K_NUM ? names[kernel] : "unknown";
}

const char* dba_status_string(int code) {
  thread_local std::string msg;
  const char* base = "unknown status";
  switch (code) {
    case DBA_OK: base = "ok"; break;
    case DBA_ERR_ARG: base = "invalid argument"; break;
    case DBA_ERR_NONFINITE: base = "non-finite or invalid value"; break;
    case DBA_ERR_NOT_SPD: base = "reduced system not positive definite"; break;
    case DBA_ERR_DEVICE: base = "HIP runtime error"; break;
    case DBA_ERR_ALLOC: base = "allocation failed"; break;
    case DBA_ERR_LIMIT: base = "size above a compiled limit"; break;
    default: break;
  }
  msg = base;
  if (code != DBA_OK && !g_err.empty()) msg += ": " + g_err;
  return msg.c_str();
}

}  // extern "C"
