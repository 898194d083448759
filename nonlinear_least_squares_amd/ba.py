"""ctypes binding of libba (include/ba.h): argument marshalling only.

Every step of the LM iteration runs in the HIP kernels of ``libba.so``; this
module converts numpy arrays or torch tensors to pointers and return codes to
exceptions.  It raises if the library was not built: there is no fallback.
"""

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libba.so")

BA_OK, BA_ERR_ARG, BA_ERR_NONFINITE, BA_ERR_NOT_SPD, BA_ERR_DEVICE, BA_ERR_ALLOC = 0, -1, -2, -3, -4, -5
BA_MEM_HOST, BA_MEM_DEVICE = 0, 1
BA_LOSS_SQUARED, BA_LOSS_HUBER = 0, 1
BA_STAGE_LINEARIZE, BA_STAGE_SCHUR, BA_STAGE_PCG, BA_STAGE_UPDATE = 1, 2, 3, 4
BA_SOLVER_PCG, BA_SOLVER_DENSE_SCHUR = 0, 1
BA_STRATEGY_LM, BA_STRATEGY_DOGLEG = 0, 1
BA_DENSE_MAX_CAMS = 1536
BA_NOALLOC_MAX_CAMS, BA_NOALLOC_MAX_OBS = 4096, 16384 * 1024

DBG = dict(perm_pt=0, perm_cam=1, pt_ptr=2, cam_ptr=3, r=4, Jc=5, Jp=6, w=7, B=8, gc=9, C=10,
           gp=11, Bd=12, Cinv=13, v=14, rhs=15, M=16, dc=17, dp=18, cams_trial=19,
           points_trial=20, pcg=21, trial_cost=22, S=23)
DBG_INT = {"perm_pt", "perm_cam", "pt_ptr", "cam_ptr"}
DBG_SHAPE = {"r": (-1, 2), "Jc": (-1, 2, 9), "Jp": (-1, 2, 3), "B": (-1, 9, 9), "gc": (-1, 9),
             "C": (-1, 3, 3), "gp": (-1, 3), "Bd": (-1, 9, 9), "Cinv": (-1, 3, 3), "v": (-1, 3),
             "rhs": (-1, 9), "M": (-1, 9, 9), "dc": (-1, 9), "dp": (-1, 3),
             "cams_trial": (-1, 9), "points_trial": (-1, 3)}
KERNELS = ["lin_pt", "lin_cam", "damp_pt", "schur_cam", "precond", "pcg_init", "pcg_pt",
           "pcg_cam", "pcg_q", "pcg_xr", "backsub", "retract", "cost", "ds_runs", "ds_fill",
           "ds_assemble", "ds_panel", "ds_update", "ds_backsolve", "cov_zero", "cov_blocks",
           "dl_obs", "dl_step"]


class ba_options(C.Structure):
    _fields_ = [("loss", C.c_int), ("huber_delta", C.c_double), ("lambda0", C.c_double),
                ("lambda_up", C.c_double), ("lambda_down", C.c_double),
                ("lambda_min", C.c_double), ("lambda_max", C.c_double),
                ("diag_floor", C.c_double), ("pcg_max_iters", C.c_int),
                ("pcg_rel_tol", C.c_double), ("mem", C.c_int), ("stream", C.c_void_p),
                ("solver", C.c_int), ("strategy", C.c_int), ("dl_radius0", C.c_double),
                ("dl_gn_damping", C.c_double)]


class ba_step_info(C.Structure):
    _fields_ = [("cost_before", C.c_double), ("cost_after", C.c_double), ("lambda_", C.c_double),
                ("pcg_rel_res", C.c_double), ("accepted", C.c_int), ("pcg_iters", C.c_int),
                ("radius", C.c_double), ("gain_ratio", C.c_double), ("step_norm", C.c_double),
                ("step_kind", C.c_int)]

    def as_dict(self):
        return dict(cost_before=self.cost_before, cost_after=self.cost_after, lam=self.lambda_,
                    accepted=self.accepted, pcg_iters=self.pcg_iters,
                    pcg_rel_res=self.pcg_rel_res, radius=self.radius,
                    gain_ratio=self.gain_ratio, step_norm=self.step_norm,
                    step_kind=self.step_kind)


class ba_summary(C.Structure):
    _fields_ = [("initial_cost", C.c_double), ("final_cost", C.c_double), ("lambda_", C.c_double),
                ("iterations", C.c_int), ("accepted", C.c_int), ("pcg_iters_total", C.c_int)]


class ba_state(C.Structure):
    _fields_ = [("lambda_", C.c_double), ("cost", C.c_double), ("iteration", C.c_int64),
                ("radius", C.c_double)]


class BAError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{msg} (code {code})")
        self.code = code


_lib = None


def _load_torch_runtime():
    """torch ships its own libamdhip64.so.7 with the same soname as ROCm's; the
    first one loaded serves the whole process.  Importing torch first makes
    libba and torch share torch's runtime, so torch device pointers and
    streams are valid inside libba."""
    try:
        import torch  # noqa: F401
    except ImportError:
        pass

# Every entry point declared in include/ba.h, with its ctypes signature.
SIGNATURES = {
    "ba_options_default": (C.c_int, [C.POINTER(ba_options)]),
    "ba_create": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p, C.c_void_p,
                            C.c_void_p, C.c_int64, C.POINTER(ba_options), C.POINTER(C.c_void_p)]),
    "ba_lm_step": (C.c_int, [C.c_void_p, C.POINTER(ba_step_info)]),
    "ba_solve": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(ba_summary)]),
    "ba_cost": (C.c_int, [C.c_void_p, C.POINTER(C.c_double)]),
    "ba_backward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.POINTER(C.c_int)]),
    "ba_covariance": (C.c_int, [C.c_void_p, C.c_void_p]),
    "ba_get_params": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "ba_set_params": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "ba_get_state": (C.c_int, [C.c_void_p, C.POINTER(ba_state)]),
    "ba_set_state": (C.c_int, [C.c_void_p, C.POINTER(ba_state)]),
    "ba_get_sizes": (C.c_int, [C.c_void_p, C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                               C.POINTER(C.c_int64)]),
    "ba_debug_run": (C.c_int, [C.c_void_p, C.c_int]),
    "ba_debug_size": (C.c_int64, [C.c_void_p, C.c_int]),
    "ba_debug_get": (C.c_int, [C.c_void_p, C.c_int, C.c_void_p, C.c_int64]),
    "ba_profile_enable": (C.c_int, [C.c_void_p, C.c_int, C.c_int]),
    "ba_profile_reset": (C.c_int, [C.c_void_p]),
    "ba_profile_get": (C.c_int, [C.c_void_p, C.c_int, C.POINTER(C.c_int64),
                                 C.POINTER(C.c_double)]),
    "ba_kernel_name": (C.c_char_p, [C.c_int]),
    "ba_cost_noalloc": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_int64, C.c_void_p,
                                  C.c_void_p, C.c_void_p, C.c_int64, C.c_int, C.c_double,
                                  C.c_void_p, C.c_void_p]),
    "ba_destroy": (None, [C.c_void_p]),
    "ba_status_string": (C.c_char_p, [C.c_int]),
}


def lib():
    """Load libba.so (raises if it has not been built)."""
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
    if rc != BA_OK:
        raise BAError(rc, f"{what}: {lib().ba_status_string(rc).decode()}")


def options(**kw):
    o = ba_options()
    _check(lib().ba_options_default(C.byref(o)), "ba_options_default")
    for k, v in kw.items():
        setattr(o, k, v)
    return o


def _ptr(a, dtype):
    """Pointer and keep-alive object for a numpy array or a torch tensor."""
    if hasattr(a, "data_ptr"):          # torch tensor (host or device)
        import torch
        want = {np.float64: torch.float64, np.int32: torch.int32}[dtype]
        if a.dtype != want or not a.is_contiguous():
            a = a.to(want).contiguous()
        return C.c_void_p(a.data_ptr()), a
    arr = np.ascontiguousarray(a, dtype=dtype)
    return C.c_void_p(arr.ctypes.data), arr


def cost_noalloc(cams, points, obs_cam, obs_pt, obs_uv, out, loss=BA_LOSS_SQUARED,
                 huber_delta=2.0, stream=None):
    """ba_cost_noalloc: the cost of the given parameters and observations,
    written to ``out`` (a device tensor of one double), with no handle and no
    device allocation.  Every array is a contiguous device tensor of the
    ba_create layout (float64 parameters and pixels, int32 indices);
    ``stream`` is a raw hipStream_t value (None: the default stream).  The
    call enqueues work and returns without synchronising."""
    ptrs = [C.c_void_p(a.data_ptr()) for a in (cams, points, obs_cam, obs_pt, obs_uv, out)]
    for a, want in ((cams, "float64"), (points, "float64"), (obs_cam, "int32"), (obs_pt, "int32"),
                    (obs_uv, "float64"), (out, "float64")):
        if not a.is_cuda or str(a.dtype) != "torch." + want or not a.is_contiguous():
            raise ValueError(f"cost_noalloc needs contiguous {want} device tensors")
    _check(lib().ba_cost_noalloc(ptrs[0], len(cams), ptrs[1], len(points), ptrs[2], ptrs[3],
                                 ptrs[4], len(obs_cam), int(loss), float(huber_delta), ptrs[5],
                                 C.c_void_p(stream or 0)), "ba_cost_noalloc")
    return out


class Problem:
    """One bundle-adjustment problem on the GPU (wraps a ba_problem handle).

    Inputs are numpy arrays (``mem=BA_MEM_HOST``) or CUDA/HIP torch tensors
    (``mem=BA_MEM_DEVICE``); ``stream`` is a raw hipStream_t value such as
    ``torch.cuda.current_stream().cuda_stream``.
    """

    def __init__(self, cams, points, obs_cam, obs_pt, obs_uv, **opts):
        L = lib()
        self._keep = []
        ptrs = []
        for a, dt in ((cams, np.float64), (points, np.float64), (obs_cam, np.int32),
                      (obs_pt, np.int32), (obs_uv, np.float64)):
            p, k = _ptr(a, dt)
            ptrs.append(p)
            self._keep.append(k)
        self.n_cams, self.n_pts, self.n_obs = len(cams), len(points), len(obs_cam)
        self.opts = options(**opts)
        self.h = C.c_void_p()
        rc = L.ba_create(ptrs[0], self.n_cams, ptrs[1], self.n_pts, ptrs[2], ptrs[3], ptrs[4],
                         self.n_obs, C.byref(self.opts), C.byref(self.h))
        self._keep = None
        _check(rc, "ba_create")

    @classmethod
    def from_scene(cls, sc, **kw):
        base = dict(loss=BA_LOSS_HUBER if sc["loss"] == "huber" else BA_LOSS_SQUARED,
                    huber_delta=sc["huber_delta"], pcg_max_iters=sc["pcg_max_iters"],
                    pcg_rel_tol=sc["pcg_rel_tol"])
        base.update(kw)
        return cls(sc["cams"], sc["points"], sc["obs_cam"], sc["obs_pt"], sc["obs_uv"], **base)

    def close(self):
        if getattr(self, "h", None) is not None and self.h.value:
            lib().ba_destroy(self.h)
            self.h = C.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def lm_step(self):
        info = ba_step_info()
        _check(lib().ba_lm_step(self.h, C.byref(info)), "ba_lm_step")
        return info.as_dict()

    def solve(self, n_iters):
        s = ba_summary()
        _check(lib().ba_solve(self.h, n_iters, C.byref(s)), "ba_solve")
        return dict(initial_cost=s.initial_cost, final_cost=s.final_cost, lam=s.lambda_,
                    iterations=s.iterations, accepted=s.accepted,
                    pcg_iters_total=s.pcg_iters_total)

    def cost(self):
        c = C.c_double()
        _check(lib().ba_cost(self.h, C.byref(c)), "ba_cost")
        return c.value

    def backward(self, grad_cams, grad_points, out=None):
        """df/du (n_obs x 2, original order) by implicit differentiation of one
        damped Gauss-Newton step at the current parameters (ba_backward).
        Inputs are numpy arrays (host handles) or device tensors (device
        handles); for a device handle ``out`` must be a device tensor of
        n_obs x 2 doubles.  Returns (grad_uv, pcg_iters)."""
        pc, kc = _ptr(grad_cams, np.float64)
        pp, kp = _ptr(grad_points, np.float64)
        if out is None:
            out = np.empty((self.n_obs, 2))
        po, ko = _ptr(out, np.float64)
        it = C.c_int()
        _check(lib().ba_backward(self.h, pc, pp, po, C.byref(it)), "ba_backward")
        del kc, kp
        return ko, it.value

    def covariance(self, out=None):
        """Camera marginal covariance: each camera's 9x9 diagonal block of the
        inverse of the damped reduced camera matrix at the current parameters
        and lambda (ba_covariance; needs the dense solver).  ``out``: a device
        tensor of n_cams x 81 doubles for device handles."""
        if out is None:
            out = np.empty((self.n_cams, 9, 9))
        po, ko = _ptr(out, np.float64)
        _check(lib().ba_covariance(self.h, po), "ba_covariance")
        return ko

    def get_params(self):
        cams = np.empty((self.n_cams, 9))
        pts = np.empty((self.n_pts, 3))
        _check(lib().ba_get_params(self.h, C.c_void_p(cams.ctypes.data),
                                   C.c_void_p(pts.ctypes.data)), "ba_get_params")
        return cams, pts

    def set_params(self, cams=None, points=None):
        keep = []
        args = []
        for a in (cams, points):
            if a is None:
                args.append(None)
            else:
                p, k = _ptr(a, np.float64)
                keep.append(k)
                args.append(p)
        _check(lib().ba_set_params(self.h, args[0], args[1]), "ba_set_params")

    def get_state(self):
        st = ba_state()
        _check(lib().ba_get_state(self.h, C.byref(st)), "ba_get_state")
        return dict(lam=st.lambda_, cost=st.cost, iteration=st.iteration, radius=st.radius)

    def set_state(self, lam, iteration=0, radius=0.0):
        st = ba_state(lam, 0.0, iteration, radius)
        _check(lib().ba_set_state(self.h, C.byref(st)), "ba_set_state")

    def debug_run(self, upto):
        _check(lib().ba_debug_run(self.h, upto), "ba_debug_run")

    def debug_get(self, name):
        which = DBG[name]
        nbytes = lib().ba_debug_size(self.h, which)
        if nbytes < 0:
            raise BAError(int(nbytes), "ba_debug_size")
        out = np.empty(nbytes // (4 if name in DBG_INT else 8),
                       dtype=np.int32 if name in DBG_INT else np.float64)
        _check(lib().ba_debug_get(self.h, which, C.c_void_p(out.ctypes.data), nbytes),
               "ba_debug_get")
        if name == "S":
            return out.reshape(9 * self.n_cams, 9 * self.n_cams)
        return out.reshape(DBG_SHAPE[name]) if name in DBG_SHAPE else out

    def profile(self, kernels=None, every=1):
        """Time the named kernels (all when None; an empty list turns timing off),
        every ``every``-th launch of each."""
        names = KERNELS if kernels is None else kernels
        mask = 0
        for n in names:
            mask |= 1 << KERNELS.index(n)
        _check(lib().ba_profile_enable(self.h, mask, int(every)), "ba_profile_enable")

    def profile_reset(self):
        _check(lib().ba_profile_reset(self.h), "ba_profile_reset")

    def profile_get(self):
        out = {}
        for k, name in enumerate(KERNELS):
            n, ms = C.c_int64(), C.c_double()
            _check(lib().ba_profile_get(self.h, k, C.byref(n), C.byref(ms)), "ba_profile_get")
            out[name] = (n.value, ms.value)
        return out
