"""ctypes wrapper of the pose-graph oracle (``pgo_oracle.c``) — TEST
INFRASTRUCTURE ONLY, like the rest of ``oracle``.

Arrays come back in fp64 with these shapes (n poses, m edges): poses (n, 6)
as [w, t], r (m, 6) as [r_R, r_t], Ji / Jj (m, 6, 6), Hd (n, 6, 6),
Ho (m, 6, 6), g (n, 6), dx (n, 6).
"""

import ctypes as C

import numpy as np

from . import lib

NAMES = dict(poses=0, r=1, Ji=2, Jj=3, Hd=4, Ho=5, g=6, dx=7)
SHAPES = dict(poses=(-1, 6), r=(-1, 6), Ji=(-1, 6, 6), Jj=(-1, 6, 6), Hd=(-1, 6, 6),
              Ho=(-1, 6, 6), g=(-1, 6), dx=(-1, 6))


class Opts(C.Structure):
    _fields_ = [("lambda0", C.c_double), ("lambda_up", C.c_double), ("lambda_down", C.c_double),
                ("lambda_min", C.c_double), ("lambda_max", C.c_double),
                ("diag_floor", C.c_double), ("pcg_max_iters", C.c_int),
                ("pcg_rel_tol", C.c_double), ("solver", C.c_int)]


class StepInfo(C.Structure):
    _fields_ = [("cost_before", C.c_double), ("cost_after", C.c_double), ("lambda_", C.c_double),
                ("pcg_rel_res", C.c_double), ("accepted", C.c_int), ("pcg_iters", C.c_int)]

    def as_dict(self):
        return dict(cost_before=self.cost_before, cost_after=self.cost_after, lam=self.lambda_,
                    accepted=self.accepted, pcg_iters=self.pcg_iters,
                    pcg_rel_res=self.pcg_rel_res)


def _dp(a):
    return a.ctypes.data_as(C.POINTER(C.c_double))


_sig = False


def _signatures():
    global _sig
    if _sig:
        return lib()
    L = lib()
    d, vp, dp = C.c_double, C.c_void_p, C.POINTER(C.c_double)
    L.porc_opts_default.argtypes = [C.POINTER(Opts)]
    L.porc_create.argtypes = [dp, C.c_int64, C.POINTER(C.c_int32), dp, dp, C.c_int64, C.c_int,
                              C.POINTER(Opts), C.POINTER(vp)]
    L.porc_destroy.argtypes = [vp]
    L.porc_array_size.argtypes = [vp, C.c_int]
    L.porc_array_size.restype = C.c_int64
    L.porc_get.argtypes = [vp, C.c_int, dp]
    L.porc_linearize.argtypes = [vp]
    L.porc_solve_step.argtypes = [vp, C.POINTER(C.c_int), dp]
    L.porc_cost_at.argtypes = [vp, dp, dp]
    L.porc_lm_step.argtypes = [vp, C.POINTER(StepInfo)]
    L.porc_solve.argtypes = [vp, C.c_int, C.POINTER(StepInfo)]
    L.porc_get_lambda.argtypes = [vp]
    L.porc_get_lambda.restype = d
    L.porc_set_lambda.argtypes = [vp, d]
    L.porc_get_cost.argtypes = [vp]
    L.porc_get_cost.restype = d
    L.porc_edge.argtypes = [dp, dp, dp, dp, dp, dp]
    L.porc_retract.argtypes = [dp, dp, dp]
    L.porc_so3_log.argtypes = [dp, dp]
    L.porc_so3_exp.argtypes = [dp, dp]
    _sig = True
    return L


def opts(**kw):
    o = Opts()
    _signatures().porc_opts_default(C.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


class PGOProblem:
    def __init__(self, poses, edges, meas, info, n_fixed=1, **kw):
        L = _signatures()
        self._keep = [np.ascontiguousarray(poses, dtype=np.float64),
                      np.ascontiguousarray(edges, dtype=np.int32),
                      np.ascontiguousarray(meas, dtype=np.float64),
                      np.ascontiguousarray(info, dtype=np.float64)]
        p, e, ms, inf = self._keep
        self.n, self.m = len(p), len(e)
        self.h = C.c_void_p()
        o = opts(**kw)
        rc = L.porc_create(_dp(p), self.n, e.ctypes.data_as(C.POINTER(C.c_int32)), _dp(ms),
                           _dp(inf), self.m, int(n_fixed), C.byref(o), C.byref(self.h))
        if rc != 0:
            raise RuntimeError(f"porc_create failed: {rc}")

    @classmethod
    def from_scene(cls, sc, **kw):
        base = dict(pcg_max_iters=sc["pcg_max_iters"], pcg_rel_tol=sc["pcg_rel_tol"])
        base.update(kw)
        return cls(sc["poses"], sc["edges"], sc["meas"], sc["info"], sc["n_fixed"], **base)

    def __del__(self):
        if getattr(self, "h", None) and self.h.value:
            lib().porc_destroy(self.h)
            self.h = C.c_void_p()

    def get(self, name):
        L = _signatures()
        which = NAMES[name]
        out = np.empty(L.porc_array_size(self.h, which))
        if L.porc_get(self.h, which, _dp(out)) != 0:
            raise RuntimeError("porc_get")
        return out.reshape(SHAPES[name])

    def linearize(self):
        _signatures().porc_linearize(self.h)

    def solve_step(self):
        it, rel = C.c_int(), C.c_double()
        rc = _signatures().porc_solve_step(self.h, C.byref(it), C.byref(rel))
        if rc != 0:
            raise RuntimeError(f"porc_solve_step: {rc}")
        return it.value, rel.value

    def cost_at(self, poses):
        p = np.ascontiguousarray(poses, dtype=np.float64)
        c = C.c_double()
        _signatures().porc_cost_at(self.h, _dp(p), C.byref(c))
        return c.value

    @property
    def cost(self):
        return _signatures().porc_get_cost(self.h)

    @property
    def lam(self):
        return _signatures().porc_get_lambda(self.h)

    @lam.setter
    def lam(self, v):
        _signatures().porc_set_lambda(self.h, v)

    def lm_step(self):
        info = StepInfo()
        rc = _signatures().porc_lm_step(self.h, C.byref(info))
        if rc != 0:
            raise RuntimeError(f"porc_lm_step: {rc}")
        return info.as_dict()

    def solve(self, n_iters):
        infos = (StepInfo * max(n_iters, 1))()
        rc = _signatures().porc_solve(self.h, n_iters, infos)
        if rc != 0:
            raise RuntimeError(f"porc_solve: {rc}")
        return [infos[i].as_dict() for i in range(n_iters)]


def edge(pose_i, pose_j, meas):
    """Residual (6) and Jacobians (6x6 each) of one edge."""
    r, Ji, Jj = np.empty(6), np.empty(36), np.empty(36)
    a, b, m = (np.ascontiguousarray(x, dtype=np.float64) for x in (pose_i, pose_j, meas))
    _signatures().porc_edge(_dp(a), _dp(b), _dp(m), _dp(r), _dp(Ji), _dp(Jj))
    return r, Ji.reshape(6, 6), Jj.reshape(6, 6)


def retract(pose, xi):
    out = np.empty(6)
    a, b = np.ascontiguousarray(pose, dtype=np.float64), np.ascontiguousarray(xi, dtype=np.float64)
    _signatures().porc_retract(_dp(a), _dp(b), _dp(out))
    return out


def so3_log(R):
    w = np.empty(3)
    _signatures().porc_so3_log(_dp(np.ascontiguousarray(R, dtype=np.float64)), _dp(w))
    return w


def so3_exp(w):
    R = np.empty(9)
    _signatures().porc_so3_exp(_dp(np.ascontiguousarray(w, dtype=np.float64)), _dp(R))
    return R.reshape(3, 3)
