"""The OpenMP build of the oracle gives the plain build's bits.

Its loops either own their outputs (one observation, camera or point per
iteration) or are owner scans: each thread walks every observation in index
order and adds only those of the cameras (points) it owns, so every sum keeps
the plain loop's order.  The test runs both builds side by side on scenes that
cover squared and Huber loss, repeated (camera, point) pairs, unobserved
points and cameras, a camera far busier than the rest, the PCG and the dense
solver, the dogleg strategy and the implicit backward, and requires every
array to be bitwise equal.
"""
import os

import numpy as np
import pytest

if os.environ.get("OMP_NUM_THREADS", "") in ("", "1"):
    os.environ["OMP_NUM_THREADS"] = "4"    # at least a few threads, read when the build loads

import oracle  # noqa: E402
from synthetic import ba_scene, heavy_camera_scene  # noqa: E402

ARRAYS = ["cams", "points", "r", "Jc", "Jp", "w", "B", "gc", "C", "gp", "Bd", "Cinv", "v", "rhs",
          "M", "dc", "dp", "cams_trial", "points_trial"]


def _edge_scene():
    """Repeated (camera, point) pairs, a long track, an unobserved point and
    an unobserved camera, Huber loss with outliers."""
    sc = ba_scene("tiny", outlier_frac=0.1)
    rng = np.random.default_rng(9)
    oc, op, uv = list(sc["obs_cam"]), list(sc["obs_pt"]), list(sc["obs_uv"])
    k7 = [i for i in range(len(op)) if op[i] == 7][0]
    for _ in range(300):
        oc.append(int(rng.integers(0, 9)))
        op.append(7)
        uv.append(np.array(sc["obs_uv"][k7]) + rng.normal(0, 2.0, 2))
    keep = [i for i in range(len(op)) if op[i] != 11 and oc[i] != 9]
    sc["obs_cam"] = np.array([oc[i] for i in keep], dtype=np.int32)
    sc["obs_pt"] = np.array([op[i] for i in keep], dtype=np.int32)
    sc["obs_uv"] = np.array([uv[i] for i in keep])
    sc["loss"] = "huber"
    return sc


SCENES = {
    "tiny": lambda: ba_scene("tiny"),
    "small": lambda: ba_scene("small"),
    "edge": _edge_scene,
    "heavy": lambda: heavy_camera_scene(n_extra=1500, n_pts=6000),
}


def _pair(sc, **kw):
    return (oracle.Problem.from_scene(sc, **kw),
            oracle.Problem.from_scene(sc, parallel=True, **kw))


def _same(a, b):
    for name in ARRAYS:
        x, y = a.get(name), b.get(name)
        assert np.array_equal(x, y), name
    assert a.cost == b.cost and a.lam == b.lam


def test_threaded_build_runs_on_threads():
    assert oracle.num_threads(False) == 1
    assert oracle.num_threads(True) >= 2


@pytest.mark.parametrize("name", list(SCENES))
def test_lm_steps_bitwise(name):
    sc = SCENES[name]()
    a, b = _pair(sc)
    assert a.cost == b.cost
    assert a.solve(3) == b.solve(3)
    _same(a, b)
    x = np.random.default_rng(5).standard_normal(9 * len(sc["cams"]))
    assert np.array_equal(a.schur_matvec(x), b.schur_matvec(x))


@pytest.mark.parametrize("name", ["tiny", "edge"])
def test_dense_solver_dogleg_and_backward_bitwise(name):
    sc = SCENES[name]()
    a, b = _pair(sc, solver=1)
    assert a.solve(2) == b.solve(2)
    _same(a, b)
    assert np.array_equal(a.covariance(), b.covariance())
    a, b = _pair(sc, strategy=1)
    assert a.solve(4) == b.solve(4)
    _same(a, b)
    rng = np.random.default_rng(3)
    gc, gp = rng.standard_normal((len(sc["cams"]), 9)), rng.standard_normal((len(sc["points"]), 3))
    a, b = _pair(sc)
    a.solve(1)
    b.solve(1)
    ua, ia, _ = a.backward(gc, gp)
    ub, ib, _ = b.backward(gc, gp)
    assert ia == ib and np.array_equal(ua, ub)
