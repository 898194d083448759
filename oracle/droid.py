"""ctypes wrapper of the dense frame-graph BA oracle (``droid_oracle.c``) —
TEST INFRASTRUCTURE ONLY, like the rest of ``oracle``.

Arrays come back in fp64 with these shapes (E edges, P = H W pixels, n frames,
nv = 6 (n - n_fixed) free pose coordinates):
r (E, P, 2), Ji / Jj (E, P, 2, 6), Jd (E, P, 2), B (6n, 6n), gc (6n,),
C / gd / dd / depth (n, P), S (nv, nv), rhs (nv,), dxi (n, 6),
poses (n, 7) as [tx, ty, tz, qx, qy, qz, qw] with qw >= 0.
"""

import ctypes as C

import numpy as np

from . import lib

NAMES = dict(r=0, Ji=1, Jj=2, Jd=3, B=4, gc=5, C=6, gd=7, S=8, rhs=9, dxi=10, dd=11, poses=12,
             depth=13)


def _dp(a):
    return a.ctypes.data_as(C.POINTER(C.c_double))


def _fp(a):
    return a.ctypes.data_as(C.POINTER(C.c_float))


class DroidProblem:
    def __init__(self, poses, inv_depth, intrinsics, edges, targets, weights, height, width,
                 n_fixed):
        L = lib()
        f32 = np.float32
        self._keep = [np.ascontiguousarray(poses, dtype=f32),
                      np.ascontiguousarray(inv_depth, dtype=f32),
                      np.ascontiguousarray(intrinsics, dtype=f32),
                      np.ascontiguousarray(edges, dtype=np.int32),
                      np.ascontiguousarray(targets, dtype=f32),
                      np.ascontiguousarray(weights, dtype=f32)]
        po, d, K, e, t, w = self._keep
        self.n, self.H, self.W, self.E = len(po), height, width, len(e)
        self.P = height * width
        self.n_fixed = n_fixed
        self.h = C.c_void_p()
        rc = L.dorc_create(_fp(po), _fp(d), self.n, height, width, _fp(K),
                           e.ctypes.data_as(C.POINTER(C.c_int32)), self.E, _fp(t), _fp(w),
                           n_fixed, C.byref(self.h))
        if rc != 0:
            raise RuntimeError(f"dorc_create failed: {rc}")

    @classmethod
    def from_scene(cls, sc):
        return cls(sc["poses"], sc["inv_depth"], sc["intrinsics"], sc["edges"], sc["targets"],
                   sc["weights"], sc["height"], sc["width"], sc["n_fixed"])

    def __del__(self):
        if getattr(self, "h", None) and self.h.value:
            lib().dorc_destroy(self.h)
            self.h = C.c_void_p()

    def get(self, name):
        which = NAMES[name]
        out = np.empty(lib().dorc_size(self.h, which))
        if lib().dorc_get(self.h, which, out.ctypes.data_as(C.c_void_p)) != 0:
            raise RuntimeError(f"dorc_get({name}) failed")
        E, P, n = self.E, self.P, self.n
        shapes = dict(r=(E, P, 2), Ji=(E, P, 2, 6), Jj=(E, P, 2, 6), Jd=(E, P, 2),
                      B=(6 * n, 6 * n), C=(n, P), gd=(n, P), dd=(n, P), depth=(n, P),
                      S=(6 * (n - self.n_fixed),) * 2, dxi=(n, 6), poses=(n, 7))
        return out.reshape(shapes[name]) if name in shapes else out

    def pose_matrix(self, i):
        T = np.empty(12)
        if lib().dorc_pose_matrix(self.h, i, _dp(T)) != 0:
            raise IndexError(i)
        return T

    def cost(self):
        c = C.c_double()
        rc = lib().dorc_cost(self.h, C.byref(c))
        if rc != 0:
            raise RuntimeError(f"dorc_cost failed: {rc}")
        return c.value

    def covariance(self):
        """Pose marginal covariance S^-1 of the free poses at the current state
        (nv x nv, nv = 6 free poses), from the Cholesky factor of S."""
        nv = 6 * (self.n - self.n_fixed)
        out = np.empty(nv * nv)
        rc = lib().dorc_covariance(self.h, out.ctypes.data_as(C.POINTER(C.c_double)))
        if rc != 0:
            raise RuntimeError(f"dorc_covariance failed: {rc}")
        return out.reshape(nv, nv)

    def gn_step(self):
        c0, c1 = C.c_double(), C.c_double()
        rc = lib().dorc_gn_step(self.h, C.byref(c0), C.byref(c1))
        if rc != 0:
            raise RuntimeError(f"dorc_gn_step failed: {rc}")
        return c0.value, c1.value


def residual_one(Ti, Tj, K, xy, d, target):
    """Residual and Jacobians of one pixel; Ti, Tj as R (row-major, 9) then t (3)."""
    args = [np.ascontiguousarray(a, dtype=np.float64) for a in (Ti, Tj, K, xy)]
    tg = np.ascontiguousarray(target, dtype=np.float64)
    r, Ji, Jj, Jd = np.empty(2), np.empty(12), np.empty(12), np.empty(2)
    clamped = lib().dorc_residual_one(*[_dp(a) for a in args], float(d), _dp(tg), _dp(r),
                                      _dp(Ji), _dp(Jj), _dp(Jd))
    return dict(r=r, Ji=Ji.reshape(2, 6), Jj=Jj.reshape(2, 6), Jd=Jd, clamped=bool(clamped))


def se3_exp(xi):
    xi = np.ascontiguousarray(xi, dtype=np.float64)
    R, t = np.empty(9), np.empty(3)
    lib().dorc_se3_exp(_dp(xi), _dp(R), _dp(t))
    return R.reshape(3, 3), t
