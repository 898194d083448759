"""The C-ABI libraries load and export every entry point their headers declare.

No compute calls: only host-side functions that never touch a GPU are called
(defaults, status strings, argument checks that fail before any device work).
"""
import ctypes as C
import os
import re

import pytest

from nonlinear_least_squares_amd import ba as bamod
from nonlinear_least_squares_amd import build as buildmod
from nonlinear_least_squares_amd import dba as dbamod
from nonlinear_least_squares_amd import pgo as pgomod

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECL = re.compile(r"^(?:int|void|int64_t|const char\*)\s+\**\s*((?:ba|dba|pgo)_\w+)\s*\(", re.M)


def _declared(header):
    with open(os.path.join(ROOT, "include", header)) as f:
        return sorted(set(DECL.findall(f.read())))


def _ensure(libname):
    path = os.path.join(buildmod.HERE, libname)
    if not os.path.exists(path):
        buildmod.build([libname])
    return path


def test_libba_exports_every_declared_symbol():
    names = _declared("ba.h")
    assert len(names) >= 19
    L = C.CDLL(_ensure("libba.so"))
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    # The Python binding covers the whole ABI, no more and no less.
    assert sorted(bamod.SIGNATURES) == names


def test_host_only_entry_points():
    L = bamod.lib()
    o = bamod.options()
    assert (o.loss, o.huber_delta, o.lambda0, o.pcg_max_iters, o.pcg_rel_tol) == (0, 2.0, 1e-3, 50, 1e-6)
    assert L.ba_options_default(None) == bamod.BA_ERR_ARG
    assert L.ba_status_string(bamod.BA_OK) == b"ok"
    assert b"invalid argument" in L.ba_status_string(bamod.BA_ERR_ARG)
    assert L.ba_kernel_name(0) == b"lin_pt"
    # Argument errors are caught on the host before any device work.
    h = C.c_void_p()
    rc = L.ba_create(None, 1, None, 1, None, None, None, 0, None, C.byref(h))
    assert rc == bamod.BA_ERR_ARG and not h.value
    assert L.ba_lm_step(None, None) == bamod.BA_ERR_ARG
    assert L.ba_debug_size(None, 0) == bamod.BA_ERR_ARG
    # the allocation-free cost rejects null pointers and sizes beyond its
    # scratch array before it looks up the device
    one = (C.c_double * 9)()
    rc = L.ba_cost_noalloc(None, 1, one, 1, None, None, None, 0, 0, 2.0, one, None)
    assert rc == bamod.BA_ERR_ARG
    rc = L.ba_cost_noalloc(one, bamod.BA_NOALLOC_MAX_CAMS + 1, one, 1, None, None, None, 0, 0, 2.0,
                           one, None)
    assert rc == bamod.BA_ERR_ARG and b"BA_NOALLOC_MAX_CAMS" in L.ba_status_string(rc)
    idx = (C.c_int32 * 1)()
    rc = L.ba_cost_noalloc(one, 1, one, 1, idx, idx, one, bamod.BA_NOALLOC_MAX_OBS + 1, 0, 2.0,
                           one, None)
    assert rc == bamod.BA_ERR_ARG
    rc = L.ba_cost_noalloc(one, 1, one, 1, idx, idx, one, 1, 0, -1.0, one, None)
    assert rc == bamod.BA_ERR_ARG
    bad = bamod.options(loss=7)
    cams = (C.c_double * 9)()
    pts = (C.c_double * 3)()
    rc = L.ba_create(cams, 1, pts, 1, None, None, None, 0, C.byref(bad), C.byref(h))
    assert rc == bamod.BA_ERR_ARG and not h.value
    # solver choice: PCG by default; the dense solver is capped by the size of S
    assert o.solver == bamod.BA_SOLVER_PCG
    rc = L.ba_create(cams, 1, pts, 1, None, None, None, 0, C.byref(bamod.options(solver=5)), C.byref(h))
    assert rc == bamod.BA_ERR_ARG and not h.value
    many = (C.c_double * (9 * (bamod.BA_DENSE_MAX_CAMS + 1)))()
    rc = L.ba_create(many, bamod.BA_DENSE_MAX_CAMS + 1, pts, 1, None, None, None, 0,
                     C.byref(bamod.options(solver=bamod.BA_SOLVER_DENSE_SCHUR)), C.byref(h))
    assert rc == bamod.BA_ERR_ARG and not h.value
    assert [L.ba_kernel_name(k) for k in range(len(bamod.KERNELS))] == [n.encode() for n in bamod.KERNELS]


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(bamod, "_lib", None)
    monkeypatch.setattr(bamod, "LIB_PATH", str(tmp_path / "libba.so"))
    with pytest.raises(RuntimeError, match="missing"):
        bamod.lib()


def test_libdba_exports_every_declared_symbol():
    names = _declared("dba.h")
    assert len(names) >= 17
    L = C.CDLL(_ensure("libdba.so"))
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(dbamod.SIGNATURES) == names


def test_libdba_host_only_entry_points():
    _ensure("libdba.so")
    L = dbamod.lib()
    o = dbamod.dba_options()
    assert L.dba_options_default(C.byref(o)) == dbamod.DBA_OK
    assert (o.mem, o.stream) == (dbamod.DBA_MEM_HOST, None)
    assert L.dba_options_default(None) == dbamod.DBA_ERR_ARG
    assert L.dba_status_string(dbamod.DBA_OK) == b"ok"
    assert b"compiled limit" in L.dba_status_string(dbamod.DBA_ERR_LIMIT)
    assert L.dba_kernel_name(0) == b"lin" and L.dba_kernel_name(99) == b"unknown"
    h = C.c_void_p()
    rc = L.dba_create(None, None, 1, 1, 1, None, None, 0, None, None, 0, None, C.byref(h))
    assert rc == dbamod.DBA_ERR_ARG and not h.value
    assert L.dba_gn_step(None, None) == dbamod.DBA_ERR_ARG
    assert L.dba_debug_size(None, 0) == dbamod.DBA_ERR_ARG
    assert L.dba_solve(None, 1, None) == dbamod.DBA_ERR_ARG
    assert L.dba_covariance(None, None) == dbamod.DBA_ERR_ARG
    # sizes are checked before any device work
    buf = (C.c_float * 16)()
    rc = L.dba_create(buf, buf, 2, 2, 2, buf, None, 0, None, None, 3, None, C.byref(h))
    assert rc == dbamod.DBA_ERR_ARG and not h.value


def test_libdba_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(dbamod, "_lib", None)
    monkeypatch.setattr(dbamod, "LIB_PATH", str(tmp_path / "libdba.so"))
    with pytest.raises(RuntimeError, match="missing"):
        dbamod.lib()


def test_libpgo_exports_every_declared_symbol():
    names = _declared("pgo.h")
    assert len(names) >= 15
    L = C.CDLL(_ensure("libpgo.so"))
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing
    assert sorted(pgomod.SIGNATURES) == names


def test_libpgo_host_only_entry_points():
    _ensure("libpgo.so")
    L = pgomod.lib()
    o = pgomod.options()
    assert (o.lambda0, o.lambda_up, o.lambda_down, o.pcg_max_iters, o.pcg_rel_tol, o.mem) == \
        (1e-3, 10.0, 10.0, 200, 1e-8, pgomod.PGO_MEM_HOST)
    assert L.pgo_options_default(None) == pgomod.PGO_ERR_ARG
    assert L.pgo_status_string(pgomod.PGO_OK) == b"ok"
    h = C.c_void_p()
    rc = L.pgo_create(None, 1, None, None, None, 0, 0, None, C.byref(h))
    assert rc == pgomod.PGO_ERR_ARG and not h.value
    assert b"invalid argument" in L.pgo_status_string(rc)
    poses = (C.c_double * 12)()
    # n_fixed beyond n, negative edge count, bad damping schedule: all host checks
    for n_fixed, m, opts in ((3, 0, None), (0, -1, None), (0, 0, pgomod.options(lambda_up=0.5)),
                             (0, 0, pgomod.options(mem=4))):
        rc = L.pgo_create(poses, 2, None, None, None, m, n_fixed,
                          C.byref(opts) if opts is not None else None, C.byref(h))
        assert rc == pgomod.PGO_ERR_ARG and not h.value
    assert L.pgo_lm_step(None, None) == pgomod.PGO_ERR_ARG
    assert L.pgo_solve(None, 1, None) == pgomod.PGO_ERR_ARG
    assert L.pgo_debug_size(None, 0) == pgomod.PGO_ERR_ARG
    assert L.pgo_debug_run(None, 1) == pgomod.PGO_ERR_ARG


def test_libpgo_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(pgomod, "_lib", None)
    monkeypatch.setattr(pgomod, "LIB_PATH", str(tmp_path / "libpgo.so"))
    with pytest.raises(RuntimeError, match="missing"):
        pgomod.lib()
