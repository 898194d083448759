"""ctypes binding of libpgo (include/pgo.h): argument marshalling only.

Every step of the pose-graph LM iteration runs in the HIP kernels of
``libpgo.so``; this module converts numpy arrays or torch tensors to pointers
and return codes to exceptions.  It raises if the library was not built:
there is no fallback.

Shapes (n poses, m edges): poses (n, 6) as [w, t]; edges (m, 2) int32;
meas (m, 6) as [w_e, t_e]; info (m, 2) as [w_R, w_t].
"""

import ctypes as C
import os

import numpy as np

from .ba import _load_torch_runtime, _ptr

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpgo.so")

PGO_OK, PGO_ERR_ARG, PGO_ERR_NONFINITE, PGO_ERR_NOT_SPD, PGO_ERR_DEVICE, PGO_ERR_ALLOC = \
    0, -1, -2, -3, -4, -5
PGO_MEM_HOST, PGO_MEM_DEVICE = 0, 1
PGO_STAGE_LINEARIZE, PGO_STAGE_STEP = 1, 2
DBG = dict(r=0, Ji=1, Jj=2, Hd=3, Ho=4, g=5, dx=6, pcg=7)
DBG_SHAPE = dict(r=(-1, 6), Ji=(-1, 6, 6), Jj=(-1, 6, 6), Hd=(-1, 6, 6), Ho=(-1, 6, 6),
                 g=(-1, 6), dx=(-1, 6), pcg=(2,))
KERNELS = ["prep", "edge", "pose", "pcg_a", "pcg_b", "retract", "cost"]


class pgo_options(C.Structure):
    _fields_ = [("lambda0", C.c_double), ("lambda_up", C.c_double), ("lambda_down", C.c_double),
                ("lambda_min", C.c_double), ("lambda_max", C.c_double),
                ("diag_floor", C.c_double), ("pcg_max_iters", C.c_int),
                ("pcg_rel_tol", C.c_double), ("mem", C.c_int), ("stream", C.c_void_p)]


class pgo_step_info(C.Structure):
    _fields_ = [("cost_before", C.c_double), ("cost_after", C.c_double), ("lambda_", C.c_double),
                ("pcg_rel_res", C.c_double), ("accepted", C.c_int), ("pcg_iters", C.c_int)]

    def as_dict(self):
        return dict(cost_before=self.cost_before, cost_after=self.cost_after, lam=self.lambda_,
                    accepted=self.accepted, pcg_iters=self.pcg_iters,
                    pcg_rel_res=self.pcg_rel_res)


class PGOError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lib = None
vp, i32, i64, dbl = C.c_void_p, C.c_int, C.c_int64, C.c_double

# Every entry point declared in include/pgo.h, with its ctypes signature.
SIGNATURES = {
    "pgo_options_default": (i32, [C.POINTER(pgo_options)]),
    "pgo_create": (i32, [vp, i64, vp, vp, vp, i64, i32, C.POINTER(pgo_options), C.POINTER(vp)]),
    "pgo_lm_step": (i32, [vp, C.POINTER(pgo_step_info)]),
    "pgo_solve": (i32, [vp, i32, vp]),
    "pgo_cost": (i32, [vp, C.POINTER(dbl)]),
    "pgo_get_poses": (i32, [vp, vp]),
    "pgo_set_lambda": (i32, [vp, dbl]),
    "pgo_get_lambda": (i32, [vp, C.POINTER(dbl)]),
    "pgo_debug_run": (i32, [vp, i32]),
    "pgo_debug_size": (i64, [vp, i32]),
    "pgo_debug_get": (i32, [vp, i32, vp, i64]),
    "pgo_profile_enable": (i32, [vp, i32, i32]),
    "pgo_profile_get": (i32, [vp, i32, C.POINTER(i64), C.POINTER(dbl)]),
    "pgo_destroy": (None, [vp]),
    "pgo_status_string": (C.c_char_p, [i32]),
}


def lib():
    """Load libpgo.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m nonlinear_least_squares_amd.build`")
        _load_torch_runtime()
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _check(rc, what):
    if rc != PGO_OK:
        raise PGOError(rc, f"{what}: {lib().pgo_status_string(rc).decode()}")


def options(**kw):
    o = pgo_options()
    _check(lib().pgo_options_default(C.byref(o)), "pgo_options_default")
    for k, v in kw.items():
        setattr(o, k, v)
    return o


class Problem:
    """One pose graph on the GPU (wraps a pgo_problem handle).

    Inputs are numpy arrays (``mem=PGO_MEM_HOST``) or device torch tensors
    (``mem=PGO_MEM_DEVICE``); ``stream`` is a raw hipStream_t value."""

    def __init__(self, poses, edges, meas, info, n_fixed=1, **opts):
        L = lib()
        keep, ptrs = [], []
        for a, dt in ((poses, np.float64), (edges, np.int32), (meas, np.float64),
                      (info, np.float64)):
            p, k = _ptr(a, dt)
            ptrs.append(p)
            keep.append(k)
        self.n, self.m = len(poses), len(edges)
        self.opts = options(**opts)
        self.h = C.c_void_p()
        rc = L.pgo_create(ptrs[0], self.n, ptrs[1], ptrs[2], ptrs[3], self.m, int(n_fixed),
                          C.byref(self.opts), C.byref(self.h))
        del keep
        _check(rc, "pgo_create")

    @classmethod
    def from_scene(cls, sc, **kw):
        base = dict(pcg_max_iters=sc["pcg_max_iters"], pcg_rel_tol=sc["pcg_rel_tol"])
        base.update(kw)
        return cls(sc["poses"], sc["edges"], sc["meas"], sc["info"], sc["n_fixed"], **base)

    def close(self):
        if getattr(self, "h", None) is not None and self.h.value:
            lib().pgo_destroy(self.h)
            self.h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lm_step(self):
        info = pgo_step_info()
        _check(lib().pgo_lm_step(self.h, C.byref(info)), "pgo_lm_step")
        return info.as_dict()

    def solve(self, n_iters):
        infos = (pgo_step_info * max(n_iters, 1))()
        _check(lib().pgo_solve(self.h, n_iters, infos), "pgo_solve")
        return [infos[i].as_dict() for i in range(n_iters)]

    def cost(self):
        c = C.c_double()
        _check(lib().pgo_cost(self.h, C.byref(c)), "pgo_cost")
        return c.value

    def get_poses(self):
        out = np.empty((self.n, 6))
        _check(lib().pgo_get_poses(self.h, C.c_void_p(out.ctypes.data)), "pgo_get_poses")
        return out

    @property
    def lam(self):
        v = C.c_double()
        _check(lib().pgo_get_lambda(self.h, C.byref(v)), "pgo_get_lambda")
        return v.value

    @lam.setter
    def lam(self, v):
        _check(lib().pgo_set_lambda(self.h, float(v)), "pgo_set_lambda")

    def debug_run(self, upto):
        _check(lib().pgo_debug_run(self.h, upto), "pgo_debug_run")

    def debug_get(self, name):
        which = DBG[name]
        n = lib().pgo_debug_size(self.h, which)
        if n < 0:
            raise PGOError(int(n), "pgo_debug_size")
        out = np.empty(n)
        _check(lib().pgo_debug_get(self.h, which, C.c_void_p(out.ctypes.data), n),
               "pgo_debug_get")
        return out.reshape(DBG_SHAPE[name])

    def profile(self, kernels=None, every=1):
        """Time the named kernels (all when None; an empty list turns timing off),
        every ``every``-th launch of each."""
        names = KERNELS if kernels is None else kernels
        mask = 0
        for n in names:
            mask |= 1 << KERNELS.index(n)
        _check(lib().pgo_profile_enable(self.h, mask, int(every)), "pgo_profile_enable")

    def profile_get(self):
        out = {}
        for k, name in enumerate(KERNELS):
            n, ms = C.c_int64(), C.c_double()
            _check(lib().pgo_profile_get(self.h, k, C.byref(n), C.byref(ms)), "pgo_profile_get")
            out[name] = (n.value, ms.value)
        return out
