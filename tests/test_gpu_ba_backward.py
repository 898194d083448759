"""GPU parity of the implicit backward (ba_backward) against the oracle's.

df/du_k = psi'(r_k) J_k H~^-1 G for a random parameter gradient G.  Bars:
with PCG, equal iteration counts and the whole df/du within 1e-8 (norm-wise
relative), as for the forward camera step, or, when both stop at the
iteration cap, within ten times the oracle's own spread under a 1e-13
relative change of the damping; with the dense solver, within
kappa(S) (|dS|/|S| + 8 n eps) + 1e-12, the bound of two backward-stable solves
of reduced systems that differ by the measured dS.  The backward leaves the LM
state as it was, and device-resident arrays give the same bits as host ones.
"""
import numpy as np
import pytest

import oracle
from synthetic import ba_scene, heavy_camera_scene

from test_gpu_ba_parity import CAMERA_TABLES, use_camera_table

pytestmark = pytest.mark.gpu

bamod = pytest.importorskip("nonlinear_least_squares_amd.ba")

EPS = np.finfo(np.float64).eps


def _grads(sc, seed=11):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((len(sc["cams"]), 9)), rng.standard_normal((len(sc["points"]), 3))


def _rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


@pytest.mark.parametrize("config", ["tiny", "small", "medium"])
def test_backward_pcg_parity(config):
    sc = ba_scene(config)
    G_c, G_p = _grads(sc)
    gpu = bamod.Problem.from_scene(sc)
    orc = oracle.Problem.from_scene(sc)
    out, it = gpu.backward(G_c, G_p)
    ref, it_ref, _ = orc.backward(G_c, G_p)
    assert it == it_ref
    bar = 1e-8
    if it_ref >= sc["pcg_max_iters"]:
        # Stopped by the iteration cap, not the tolerance (the walk scene's
        # reduced system): the iterate then depends on rounding.  The bar is
        # the oracle's own spread when the damping moves by 1e-13 relative.
        lam = orc.lam
        orc2 = oracle.Problem.from_scene(sc)
        orc2.lam = lam * (1.0 + 1e-13)
        ref2, _, _ = orc2.backward(G_c, G_p)
        bar = max(bar, 10.0 * _rel(ref2, ref))
    assert _rel(out, ref) <= bar, (_rel(out, ref), bar)


@pytest.mark.parametrize("config", ["tiny", "small", "medium"])
def test_backward_dense_parity(config):
    sc = ba_scene(config)
    G_c, G_p = _grads(sc, seed=12)
    gpu = bamod.Problem.from_scene(sc, solver=bamod.BA_SOLVER_DENSE_SCHUR)
    orc = oracle.Problem.from_scene(sc, solver=1)
    out, it = gpu.backward(G_c, G_p)
    ref, _, _ = orc.backward(G_c, G_p)
    assert it == 0
    # the reduced system of this right-hand side is S of the current state
    gpu.debug_run(bamod.BA_STAGE_SCHUR)
    S = gpu.debug_get("S")
    S_ref = orc.explicit_S()
    n = S.shape[0]
    kappa = np.linalg.cond(S_ref)
    dS = np.linalg.norm(S - S_ref, 2) / np.linalg.norm(S_ref, 2)
    assert _rel(out, ref) <= kappa * (dS + 8 * n * EPS) + 1e-12, (_rel(out, ref), kappa, dS)


def test_backward_huber_tiny_with_outliers():
    sc = ba_scene("tiny", outlier_frac=0.2)
    G_c, G_p = _grads(sc, seed=13)
    kw = dict(loss=bamod.BA_LOSS_HUBER, huber_delta=2.0)
    gpu = bamod.Problem.from_scene(sc, **kw)
    orc = oracle.Problem.from_scene(sc, loss=1, huber_delta=2.0)
    out, it = gpu.backward(G_c, G_p)
    ref, it_ref, _ = orc.backward(G_c, G_p)
    assert it == it_ref
    assert _rel(out, ref) <= 1e-8


def test_backward_leaves_the_lm_state():
    sc = ba_scene("small")
    G_c, G_p = _grads(sc, seed=14)
    a = bamod.Problem.from_scene(sc)
    b = bamod.Problem.from_scene(sc)
    a.solve(3)
    b.solve(3)
    a.backward(G_c, G_p)
    a.solve(3)
    b.solve(3)
    ca, pa = a.get_params()
    cb, pb = b.get_params()
    assert np.array_equal(ca, cb) and np.array_equal(pa, pb)
    assert a.get_state() == b.get_state()


def test_backward_device_arrays_match_host():
    torch = pytest.importorskip("torch")
    sc = ba_scene("tiny")
    G_c, G_p = _grads(sc, seed=15)
    dev = torch.device("cuda:0")
    t = {k: torch.from_numpy(np.ascontiguousarray(sc[k])).to(dev)
         for k in ("cams", "points", "obs_cam", "obs_pt", "obs_uv")}
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    gd = bamod.Problem(t["cams"], t["points"], t["obs_cam"], t["obs_pt"], t["obs_uv"],
                       mem=bamod.BA_MEM_DEVICE, stream=s.cuda_stream)
    gh = bamod.Problem.from_scene(sc)
    out_d = torch.empty((len(sc["obs_cam"]), 2), dtype=torch.float64, device=dev)
    gcd, gpd = torch.from_numpy(G_c).to(dev), torch.from_numpy(G_p).to(dev)
    torch.cuda.synchronize()
    gd.backward(gcd, gpd, out=out_d)
    s.synchronize()
    out_h, _ = gh.backward(G_c, G_p)
    assert np.array_equal(out_d.cpu().numpy(), out_h)


@pytest.mark.parametrize("cameras", CAMERA_TABLES)
def test_backward_heavy_camera(cameras, monkeypatch):
    """The per-observation products of a camera with about 3,200 observations
    in one point band run over several of its chunks (Huber loss, outliers)."""
    use_camera_table(cameras, monkeypatch)
    sc = heavy_camera_scene()
    G_c, G_p = _grads(sc, seed=14)
    gpu = bamod.Problem.from_scene(sc)
    orc = oracle.Problem.from_scene(sc)
    out, it = gpu.backward(G_c, G_p)
    ref, it_ref, _ = orc.backward(G_c, G_p)
    assert it == it_ref
    assert _rel(out, ref) <= 1e-8, _rel(out, ref)
