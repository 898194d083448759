"""ctypes binding of libdba (include/dba.h): argument marshalling only.

Every step of the dense frame-graph Gauss-Newton iteration runs in the HIP
kernels of ``libdba.so``; this module converts numpy arrays or torch tensors
to pointers and return codes to exceptions.  It raises if the library was not
built: there is no fallback.
"""

import ctypes as C
import os

import numpy as np

from .ba import _load_torch_runtime

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdba.so")

DBA_OK, DBA_ERR_ARG, DBA_ERR_NONFINITE, DBA_ERR_NOT_SPD = 0, -1, -2, -3
DBA_ERR_DEVICE, DBA_ERR_ALLOC, DBA_ERR_LIMIT = -4, -5, -6
DBA_MEM_HOST, DBA_MEM_DEVICE = 0, 1
DBA_STAGE_ASSEMBLE, DBA_STAGE_JACOBIANS = 1, 2
DBG = dict(S=0, rhs=1, dxi=2, dd=3, C=4, gd=5, r=6, Ji=7, Jj=8, Jd=9)
KERNELS = ["lin", "assemble", "solve", "cost"]


class dba_options(C.Structure):
    _fields_ = [("mem", C.c_int), ("stream", C.c_void_p)]


class dba_step_info(C.Structure):
    _fields_ = [("cost_before", C.c_float), ("cost_after", C.c_float)]


class DBAError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lib = None
vp, i32, i64 = C.c_void_p, C.c_int, C.c_int64

# Every entry point declared in include/dba.h, with its ctypes signature.
SIGNATURES = {
    "dba_options_default": (i32, [C.POINTER(dba_options)]),
    "dba_create": (i32, [vp, vp, i32, i32, i32, vp, vp, i32, vp, vp, i32,
                         C.POINTER(dba_options), C.POINTER(vp)]),
    "dba_gn_step": (i32, [vp, C.POINTER(dba_step_info)]),
    "dba_solve": (i32, [vp, i32, vp]),
    "dba_cost": (i32, [vp, C.POINTER(C.c_float)]),
    "dba_get_state": (i32, [vp, vp, vp]),
    "dba_set_state": (i32, [vp, vp, vp]),
    "dba_get_sizes": (i32, [vp, C.POINTER(i32), C.POINTER(i32), C.POINTER(i32), C.POINTER(i32)]),
    "dba_covariance": (i32, [vp, vp]),
    "dba_debug_run": (i32, [vp, i32]),
    "dba_debug_size": (i64, [vp, i32]),
    "dba_debug_get": (i32, [vp, i32, vp, i64]),
    "dba_profile_enable": (i32, [vp, i32, i32]),
    "dba_profile_reset": (i32, [vp]),
    "dba_profile_get": (i32, [vp, i32, C.POINTER(i64), C.POINTER(C.c_double)]),
    "dba_kernel_name": (C.c_char_p, [i32]),
    "dba_destroy": (None, [vp]),
    "dba_status_string": (C.c_char_p, [i32]),
}


def lib():
    """Load libdba.so (raises if it has not been built)."""
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
    if rc != DBA_OK:
        raise DBAError(rc, f"{what}: {lib().dba_status_string(rc).decode()}")


def _ptr(a, dtype):
    if hasattr(a, "data_ptr"):          # torch tensor (host or device)
        import torch
        want = {np.float32: torch.float32, np.int32: torch.int32}[dtype]
        if a.dtype != want or not a.is_contiguous():
            a = a.to(want).contiguous()
        return C.c_void_p(a.data_ptr()), a
    arr = np.ascontiguousarray(a, dtype=dtype)
    return C.c_void_p(arr.ctypes.data), arr


class Problem:
    """One dense frame-graph BA problem on the GPU (wraps a dba_problem)."""

    def __init__(self, poses, inv_depth, intrinsics, edges, targets, weights, height, width,
                 n_fixed, mem=DBA_MEM_HOST, stream=None):
        L = lib()
        keep, ptrs = [], []
        for a, dt in ((poses, np.float32), (inv_depth, np.float32), (intrinsics, np.float32),
                      (edges, np.int32), (targets, np.float32), (weights, np.float32)):
            p, k = _ptr(a, dt)
            ptrs.append(p)
            keep.append(k)
        self.n, self.H, self.W, self.E = len(poses), height, width, len(edges)
        self.P = height * width
        self.n_fixed = n_fixed
        self.mem = mem
        self.opts = dba_options(mem, stream)
        self.h = C.c_void_p()
        rc = L.dba_create(ptrs[0], ptrs[1], self.n, height, width, ptrs[2], ptrs[3], self.E,
                          ptrs[4], ptrs[5], n_fixed, C.byref(self.opts), C.byref(self.h))
        _check(rc, "dba_create")

    @classmethod
    def from_scene(cls, sc, **kw):
        return cls(sc["poses"], sc["inv_depth"], sc["intrinsics"], sc["edges"], sc["targets"],
                   sc["weights"], sc["height"], sc["width"], sc["n_fixed"], **kw)

    def close(self):
        if getattr(self, "h", None) is not None and self.h.value:
            lib().dba_destroy(self.h)
            self.h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def gn_step(self):
        info = dba_step_info()
        _check(lib().dba_gn_step(self.h, C.byref(info)), "dba_gn_step")
        return info.cost_before, info.cost_after

    def solve(self, n_iters):
        costs = np.empty(n_iters + 1, dtype=np.float32)
        _check(lib().dba_solve(self.h, n_iters, C.c_void_p(costs.ctypes.data)), "dba_solve")
        return costs

    def cost(self):
        c = C.c_float()
        _check(lib().dba_cost(self.h, C.byref(c)), "dba_cost")
        return c.value

    def covariance(self):
        """Pose marginal covariance S^-1 (nv x nv float32, nv = 6 free poses)."""
        nv = 6 * (self.n - self.n_fixed)
        out = np.empty((nv, nv), dtype=np.float32)
        _check(lib().dba_covariance(self.h, C.c_void_p(out.ctypes.data)), "dba_covariance")
        return out

    def get_state(self):
        poses = np.empty((self.n, 7), dtype=np.float32)
        depth = np.empty((self.n, self.P), dtype=np.float32)
        _check(lib().dba_get_state(self.h, C.c_void_p(poses.ctypes.data),
                                   C.c_void_p(depth.ctypes.data)), "dba_get_state")
        return poses, depth

    def set_state(self, poses=None, inv_depth=None):
        keep, args = [], []
        for a in (poses, inv_depth):
            if a is None:
                args.append(None)
            else:
                p, k = _ptr(a, np.float32)
                keep.append(k)
                args.append(p)
        _check(lib().dba_set_state(self.h, args[0], args[1]), "dba_set_state")

    def debug_run(self, stage):
        _check(lib().dba_debug_run(self.h, stage), "dba_debug_run")

    def debug_get(self, name):
        which = DBG[name]
        nbytes = lib().dba_debug_size(self.h, which)
        if nbytes < 0:
            raise DBAError(int(nbytes), "dba_debug_size")
        out = np.empty(nbytes // 4, dtype=np.float32)
        _check(lib().dba_debug_get(self.h, which, C.c_void_p(out.ctypes.data), nbytes),
               "dba_debug_get")
        nv = 6 * (self.n - self.n_fixed)
        shapes = dict(S=(nv, nv), dxi=(self.n, 6), dd=(self.n, self.P), C=(self.n, self.P),
                      gd=(self.n, self.P), r=(self.E, self.P, 2), Ji=(self.E, self.P, 2, 6),
                      Jj=(self.E, self.P, 2, 6), Jd=(self.E, self.P, 2))
        return out.reshape(shapes[name]) if name in shapes else out

    def profile(self, kernels=None, every=1):
        """Time the named kernels (all when None; an empty list turns timing off),
        every ``every``-th launch of each."""
        names = KERNELS if kernels is None else kernels
        mask = 0
        for n in names:
            mask |= 1 << KERNELS.index(n)
        _check(lib().dba_profile_enable(self.h, mask, int(every)), "dba_profile_enable")

    def profile_reset(self):
        _check(lib().dba_profile_reset(self.h), "dba_profile_reset")

    def profile_get(self):
        out = {}
        for k, name in enumerate(KERNELS):
            n, ms = C.c_int64(), C.c_double()
            _check(lib().dba_profile_get(self.h, k, C.byref(n), C.byref(ms)), "dba_profile_get")
            out[name] = (n.value, ms.value)
        return out
