"""CPU oracle for bundle adjustment — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never loads it and shares
no code with it.  The arithmetic lives in ``ba_oracle.c`` (plain C loops, fp64)
``droid_oracle.c`` (dense frame-graph BA, wrapped by ``oracle.droid``) and
``pgo_oracle.c`` (pose-graph optimisation, wrapped by ``oracle.pgo``);
this module only builds and marshals.

Parity status: every function is pinned by tests in ``tests/test_oracle_*.py``
(finite differences, dense solves, library routines, closed forms and
statistical invariants); none relies on printed values, because the pages print
no worked bundle-adjustment example.
"""

import ctypes as C
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(HERE, "libba_oracle.so")
# The same sources built with -fopenmp: loops that own their outputs run on
# several threads, every sum keeps its observation order, so the results are
# the plain build's bits (tests/test_oracle_threads.py).
LIB_OMP = os.path.join(HERE, "libba_oracle_omp.so")
SOURCES = [os.path.join(HERE, n) for n in ("ba_oracle.c", "droid_oracle.c", "pgo_oracle.c")
           if os.path.exists(os.path.join(HERE, n))]

(ORC_CAMS, ORC_PTS, ORC_PERM_PT, ORC_PERM_CAM, ORC_PT_PTR, ORC_CAM_PTR, ORC_R, ORC_JC, ORC_JP,
 ORC_W, ORC_RHO, ORC_B, ORC_GC, ORC_C, ORC_GP, ORC_BD, ORC_CINV, ORC_V, ORC_RHS, ORC_M, ORC_DC,
 ORC_DP, ORC_CAMS_TRIAL, ORC_PTS_TRIAL) = range(24)

INT_ARRAYS = {ORC_PERM_PT, ORC_PERM_CAM, ORC_PT_PTR, ORC_CAM_PTR}
NAMES = {
    "cams": ORC_CAMS, "points": ORC_PTS, "perm_pt": ORC_PERM_PT, "perm_cam": ORC_PERM_CAM,
    "pt_ptr": ORC_PT_PTR, "cam_ptr": ORC_CAM_PTR, "r": ORC_R, "Jc": ORC_JC, "Jp": ORC_JP,
    "w": ORC_W, "rho": ORC_RHO, "B": ORC_B, "gc": ORC_GC, "C": ORC_C, "gp": ORC_GP,
    "Bd": ORC_BD, "Cinv": ORC_CINV, "v": ORC_V, "rhs": ORC_RHS, "M": ORC_M, "dc": ORC_DC,
    "dp": ORC_DP, "cams_trial": ORC_CAMS_TRIAL, "points_trial": ORC_PTS_TRIAL,
}


class Opts(C.Structure):
    _fields_ = [("loss", C.c_int), ("huber_delta", C.c_double), ("lambda0", C.c_double),
                ("lambda_up", C.c_double), ("lambda_down", C.c_double),
                ("lambda_min", C.c_double), ("lambda_max", C.c_double),
                ("diag_floor", C.c_double), ("pcg_max_iters", C.c_int),
                ("pcg_rel_tol", C.c_double), ("solver", C.c_int), ("strategy", C.c_int),
                ("dl_radius0", C.c_double), ("dl_gn_damping", C.c_double)]


class StepInfo(C.Structure):
    _fields_ = [("cost_before", C.c_double), ("cost_after", C.c_double), ("lambda_", C.c_double),
                ("pcg_rel_res", C.c_double), ("accepted", C.c_int), ("pcg_iters", C.c_int),
                ("radius", C.c_double), ("gain_ratio", C.c_double), ("step_norm", C.c_double),
                ("step_kind", C.c_int)]

    def as_dict(self):
        return dict(cost_before=self.cost_before, cost_after=self.cost_after,
                    lam=self.lambda_, accepted=self.accepted, pcg_iters=self.pcg_iters,
                    pcg_rel_res=self.pcg_rel_res, radius=self.radius,
                    gain_ratio=self.gain_ratio, step_norm=self.step_norm,
                    step_kind=self.step_kind)


def build(force=True):
    """Compile the oracle with gcc (plain -O2, no FMA contraction), once as is
    and once with OpenMP."""
    if not force and os.path.exists(LIB) and os.path.exists(LIB_OMP):
        return LIB
    for out, extra in ((LIB, []), (LIB_OMP, ["-fopenmp"])):
        cmd = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-ffp-contract=off", *extra, "-o",
               out + ".tmp", *SOURCES, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(out + ".tmp", out)
    return LIB


_libs = {}


def lib(parallel=False):
    """The oracle library: the plain build, or with ``parallel`` the OpenMP
    build (threads per OMP_NUM_THREADS)."""
    if parallel not in _libs:
        path = LIB_OMP if parallel else LIB
        if not os.path.exists(path):
            build()
        L = C.CDLL(path)
        d, i64, i32p = C.c_double, C.c_int64, C.POINTER(C.c_int32)
        dp, vp = C.POINTER(C.c_double), C.c_void_p
        L.orc_create.argtypes = [dp, i64, dp, i64, i32p, i32p, dp, i64, C.POINTER(Opts),
                                 C.POINTER(vp)]
        L.orc_destroy.argtypes = [vp]
        L.orc_array_size.argtypes = [vp, C.c_int]
        L.orc_array_size.restype = i64
        L.orc_get.argtypes = [vp, C.c_int, vp]
        L.orc_set.argtypes = [vp, C.c_int, vp]
        for name in ["orc_linearize", "orc_damp", "orc_schur", "orc_dense_schur_solve",
                     "orc_backsub", "orc_retract"]:
            getattr(L, name).argtypes = [vp]
        L.orc_pcg.argtypes = [vp, C.c_int, d, C.POINTER(C.c_int), dp]
        L.orc_cost_at.argtypes = [vp, dp, dp, dp]
        L.orc_lm_step.argtypes = [vp, C.POINTER(StepInfo)]
        L.orc_solve.argtypes = [vp, C.c_int, C.POINTER(StepInfo)]
        L.orc_backward.argtypes = [vp, dp, dp, dp, C.POINTER(C.c_int), dp]
        L.orc_get_lambda.argtypes = [vp]
        L.orc_get_lambda.restype = d
        L.orc_set_lambda.argtypes = [vp, d]
        L.orc_get_cost.argtypes = [vp]
        L.orc_get_cost.restype = d
        L.orc_schur_matvec.argtypes = [vp, dp, dp]
        L.orc_explicit_S.argtypes = [vp, dp]
        L.orc_covariance.argtypes = [vp, dp]
        L.orc_get_radius.argtypes = [vp]
        L.orc_get_radius.restype = d
        L.orc_set_radius.argtypes = [vp, d]
        L.orc_project_one.argtypes = [dp, dp, dp, C.c_int, d, dp, dp, dp, dp, dp]
        L.orc_retract_camera.argtypes = [dp, dp, dp]
        L.orc_so3_exp.argtypes = [dp, dp]
        L.orc_opts_default.argtypes = [C.POINTER(Opts)]
        L.orc_num_threads.restype = C.c_int
        if hasattr(L, "dorc_create"):
            _droid_signatures(L)
        _libs[parallel] = L
    return _libs[parallel]


def num_threads(parallel=False):
    """Threads the oracle's loops run on."""
    return lib(parallel).orc_num_threads()


def _droid_signatures(L):
    f32p, i32p, vp = C.POINTER(C.c_float), C.POINTER(C.c_int32), C.c_void_p
    dp = C.POINTER(C.c_double)
    L.dorc_create.argtypes = [f32p, f32p, C.c_int, C.c_int, C.c_int, f32p, i32p, C.c_int, f32p,
                              f32p, C.c_int, C.POINTER(vp)]
    L.dorc_destroy.argtypes = [vp]
    L.dorc_cost.argtypes = [vp, dp]
    L.dorc_gn_step.argtypes = [vp, dp, dp]
    L.dorc_covariance.argtypes = [vp, dp]
    L.dorc_get.argtypes = [vp, C.c_int, vp]
    L.dorc_size.argtypes = [vp, C.c_int]
    L.dorc_size.restype = C.c_int64
    L.dorc_residual_one.argtypes = [dp, dp, dp, dp, C.c_double, dp, dp, dp, dp, dp]
    L.dorc_pose_matrix.argtypes = [vp, C.c_int, dp]
    L.dorc_se3_exp.argtypes = [dp, dp, dp]


def _p(a, ctype=C.c_double):
    return a.ctypes.data_as(C.POINTER(ctype))


def default_opts(**kw):
    o = Opts()
    lib().orc_opts_default(C.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def opts_for_scene(sc, **kw):
    base = dict(loss=1 if sc["loss"] == "huber" else 0, huber_delta=sc["huber_delta"],
                pcg_max_iters=sc["pcg_max_iters"], pcg_rel_tol=sc["pcg_rel_tol"])
    base.update(kw)
    return default_opts(**base)


class Problem:
    """Thin ctypes handle around ``orc_problem``."""

    def __init__(self, cams, points, obs_cam, obs_pt, obs_uv, opts=None, parallel=False):
        L = self._L = lib(parallel)
        self._keep = [np.ascontiguousarray(cams, dtype=np.float64),
                      np.ascontiguousarray(points, dtype=np.float64),
                      np.ascontiguousarray(obs_cam, dtype=np.int32),
                      np.ascontiguousarray(obs_pt, dtype=np.int32),
                      np.ascontiguousarray(obs_uv, dtype=np.float64)]
        c, p, oc, op, uv = self._keep
        self.nc, self.np, self.nobs = len(c), len(p), len(oc)
        self.h = C.c_void_p()
        o = opts if opts is not None else default_opts()
        rc = L.orc_create(_p(c), self.nc, _p(p), self.np, _p(oc, C.c_int32), _p(op, C.c_int32),
                          _p(uv), self.nobs, C.byref(o), C.byref(self.h))
        if rc != 0:
            raise RuntimeError(f"orc_create failed: {rc}")

    @classmethod
    def from_scene(cls, sc, parallel=False, **kw):
        return cls(sc["cams"], sc["points"], sc["obs_cam"], sc["obs_pt"], sc["obs_uv"],
                   opts_for_scene(sc, **kw), parallel=parallel)

    def __del__(self):
        if getattr(self, "h", None) and self.h.value:
            self._L.orc_destroy(self.h)
            self.h = C.c_void_p()

    def get(self, name):
        which = NAMES[name]
        n = self._L.orc_array_size(self.h, which)
        out = np.empty(n, dtype=np.int32 if which in INT_ARRAYS else np.float64)
        self._L.orc_get(self.h, which, out.ctypes.data_as(C.c_void_p))
        shapes = {"cams": (-1, 9), "points": (-1, 3), "r": (-1, 2), "Jc": (-1, 2, 9),
                  "Jp": (-1, 2, 3), "B": (-1, 9, 9), "gc": (-1, 9), "C": (-1, 3, 3),
                  "gp": (-1, 3), "Bd": (-1, 9, 9), "Cinv": (-1, 3, 3), "v": (-1, 3),
                  "rhs": (-1, 9), "M": (-1, 9, 9), "dc": (-1, 9), "dp": (-1, 3),
                  "cams_trial": (-1, 9), "points_trial": (-1, 3)}
        return out.reshape(shapes[name]) if name in shapes else out

    def set(self, name, arr):
        arr = np.ascontiguousarray(arr, dtype=np.float64)
        self._L.orc_set(self.h, NAMES[name], arr.ctypes.data_as(C.c_void_p))

    def _check(self, rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed: {rc}")

    def linearize(self):
        self._check(self._L.orc_linearize(self.h), "linearize")

    def damp(self):
        self._check(self._L.orc_damp(self.h), "damp")

    def schur(self):
        self._check(self._L.orc_schur(self.h), "schur")

    def pcg(self, max_iters=50, rel_tol=1e-6):
        it, rel = C.c_int(), C.c_double()
        self._check(self._L.orc_pcg(self.h, max_iters, rel_tol, C.byref(it), C.byref(rel)), "pcg")
        return it.value, rel.value

    def dense_schur_solve(self):
        self._check(self._L.orc_dense_schur_solve(self.h), "dense_schur_solve")

    def backward(self, grad_cams, grad_points):
        """df/du (n_obs x 2, original order) by implicit differentiation of one
        damped Gauss-Newton step at the current parameters and lambda; also
        returns the PCG iteration count and relative residual (0 for the dense
        solver)."""
        gc = np.ascontiguousarray(grad_cams, dtype=np.float64).ravel()
        gp = np.ascontiguousarray(grad_points, dtype=np.float64).ravel()
        assert gc.size == 9 * self.nc and gp.size == 3 * self.np
        out = np.empty(2 * self.nobs)
        it, rel = C.c_int(), C.c_double()
        self._check(self._L.orc_backward(self.h, _p(gc), _p(gp), _p(out), C.byref(it), C.byref(rel)),
                    "backward")
        return out.reshape(-1, 2), it.value, rel.value

    def covariance(self):
        """Camera marginal covariance: the 9x9 diagonal blocks of S~^-1 at the
        current parameters and lambda (n_cams x 9 x 9)."""
        out = np.empty(81 * self.nc)
        self._check(self._L.orc_covariance(self.h, _p(out)), "covariance")
        return out.reshape(-1, 9, 9)

    def backsub(self):
        self._check(self._L.orc_backsub(self.h), "backsub")

    def retract(self):
        self._check(self._L.orc_retract(self.h), "retract")

    def cost_at(self, cams, points):
        c = np.ascontiguousarray(cams, dtype=np.float64)
        p = np.ascontiguousarray(points, dtype=np.float64)
        out = C.c_double()
        self._L.orc_cost_at(self.h, _p(c), _p(p), C.byref(out))
        return out.value

    @property
    def cost(self):
        return self._L.orc_get_cost(self.h)

    @property
    def radius(self):
        return self._L.orc_get_radius(self.h)

    @radius.setter
    def radius(self, v):
        self._L.orc_set_radius(self.h, v)

    @property
    def lam(self):
        return self._L.orc_get_lambda(self.h)

    @lam.setter
    def lam(self, v):
        self._L.orc_set_lambda(self.h, v)

    def lm_step(self):
        info = StepInfo()
        self._check(self._L.orc_lm_step(self.h, C.byref(info)), "lm_step")
        return info.as_dict()

    def solve(self, n_iters):
        infos = (StepInfo * max(n_iters, 1))()
        self._check(self._L.orc_solve(self.h, n_iters, infos), "solve")
        return [infos[i].as_dict() for i in range(n_iters)]

    def schur_matvec(self, x):
        x = np.ascontiguousarray(x, dtype=np.float64).ravel()
        out = np.empty(9 * self.nc)
        self._check(self._L.orc_schur_matvec(self.h, _p(x), _p(out)), "matvec")
        return out

    def explicit_S(self):
        n = 9 * self.nc
        S = np.empty((n, n))
        self._check(self._L.orc_explicit_S(self.h, _p(S)), "explicit_S")
        return S


def project_one(cam, X, uv, loss=0, delta=2.0):
    cam = np.ascontiguousarray(cam, dtype=np.float64)
    X = np.ascontiguousarray(X, dtype=np.float64)
    uv = np.ascontiguousarray(uv, dtype=np.float64)
    r, Jc, Jp = np.empty(2), np.empty(18), np.empty(6)
    w, rho = C.c_double(), C.c_double()
    clamped = lib().orc_project_one(_p(cam), _p(X), _p(uv), loss, delta, _p(r), _p(Jc), _p(Jp),
                                    C.byref(w), C.byref(rho))
    return dict(r=r, Jc=Jc.reshape(2, 9), Jp=Jp.reshape(2, 3), w=w.value, rho=rho.value,
                clamped=bool(clamped))


def retract_camera(cam, delta):
    cam = np.ascontiguousarray(cam, dtype=np.float64)
    delta = np.ascontiguousarray(delta, dtype=np.float64)
    out = np.empty(9)
    lib().orc_retract_camera(_p(cam), _p(delta), _p(out))
    return out


def so3_exp(w):
    w = np.ascontiguousarray(w, dtype=np.float64)
    R = np.empty(9)
    lib().orc_so3_exp(_p(w), _p(R))
    return R.reshape(3, 3)

