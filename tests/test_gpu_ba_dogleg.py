"""GPU parity of the dogleg strategy (BA_STRATEGY_DOGLEG) against the
oracle's dogleg on the same scenes.

Bars (fp64): per step, until the first step whose cost change is within the
rounding noise of the cost sums (|dC| <= 1e-10 C), the same accept/reject
decision, the same kind of step (Gauss-Newton, cut steepest descent, blend),
the same trust radius, the step norm and the trial cost within 1e-6
relative (a radius set to 3 |h| carries the step norm's tolerance), as long as the Gauss-Newton solve in use reached its
tolerance (a PCG stopped at its iteration cap, as on the medium walk scene,
leaves a step that rounding moves by more than that); the final cost within
1e-6 relative.  With a radius
beyond the Gauss-Newton step the first trial equals, bit for bit, the LM trial
at lambda = dl_gn_damping; a rejected step runs no new solve; runs are
bitwise reproducible.
"""
import numpy as np
import pytest

import oracle
from synthetic import ba_scene
from test_gpu_ba_parity import CAMERA_TABLES, _edge_scene, use_camera_table

pytestmark = pytest.mark.gpu

bamod = pytest.importorskip("nonlinear_least_squares_amd.ba")


def dogleg_traces_agree(g_tr, o_tr, tol):
    converged = True   # of the Gauss-Newton solve the current step uses
    for k, (a, b) in enumerate(zip(g_tr, o_tr)):
        if b["pcg_iters"] > 0:
            converged = b["pcg_rel_res"] <= tol
        if not converged:
            # a PCG stopped at its cap leaves a step that rounding moves by
            # more than the bar; past it the runs may branch
            return k
        assert abs(a["cost_after"] - b["cost_after"]) <= 1e-6 * b["cost_after"], (k, a, b)
        # a radius set to 3 |h| carries the step norm's tolerance
        assert abs(a["radius"] - b["radius"]) <= 1e-6 * b["radius"], (k, a, b)
        if abs(b["cost_after"] - b["cost_before"]) <= 1e-10 * b["cost_before"]:
            return k
        assert a["accepted"] == b["accepted"], (k, a, b)
        assert a["step_kind"] == b["step_kind"], (k, a, b)
        assert abs(a["step_norm"] - b["step_norm"]) <= 1e-6 * b["step_norm"], (k, a, b)
    return len(g_tr)


@pytest.mark.parametrize("config,solver", [("tiny", 0), ("tiny", 1), ("small", 0), ("small", 1),
                                           ("medium", 1), ("medium", 0)])
def test_dogleg_trace_parity(config, solver):
    sc = ba_scene(config)
    n_it = sc["n_iters"] if config != "medium" else 8
    print(f"dogleg {config} solver {solver}: {n_it} iterations", flush=True)
    gpu = bamod.Problem.from_scene(sc, strategy=bamod.BA_STRATEGY_DOGLEG, solver=solver)
    orc = oracle.Problem.from_scene(sc, strategy=1, solver=solver)
    tg = [gpu.lm_step() for _ in range(n_it)]
    to = orc.solve(n_it)
    k = dogleg_traces_agree(tg, to, sc["pcg_rel_tol"])
    print(f"  steps compared {k}; kinds {[t['step_kind'] for t in tg]}", flush=True)
    c_g = gpu.get_state()["cost"]
    assert abs(c_g - orc.cost) <= 1e-6 * orc.cost, (c_g, orc.cost)
    assert sum(t["accepted"] for t in tg) >= 3


def test_large_radius_step_is_the_damped_gauss_newton_step():
    sc = ba_scene("small")
    dl = bamod.Problem.from_scene(sc, strategy=bamod.BA_STRATEGY_DOGLEG, dl_radius0=1e12)
    lm = bamod.Problem.from_scene(sc, lambda0=1e-6)
    a, b = dl.lm_step(), lm.lm_step()
    assert a["step_kind"] == 0
    assert a["cost_after"] == b["cost_after"] and a["pcg_iters"] == b["pcg_iters"]
    assert np.array_equal(dl.get_params()[0], lm.get_params()[0])


def test_rejected_step_reuses_the_gauss_newton_step_and_runs_are_reproducible():
    sc = ba_scene("tiny")
    runs = []
    for _ in range(2):
        g = bamod.Problem.from_scene(sc, strategy=bamod.BA_STRATEGY_DOGLEG)
        tr = [g.lm_step() for _ in range(sc["n_iters"] + 6)]
        runs.append((tr, g.get_params()))
    tr = runs[0][0]
    for a, b in zip(tr, tr[1:]):
        if not a["accepted"]:
            assert b["pcg_iters"] == 0 and b["cost_before"] == a["cost_before"]
    assert any(not t["accepted"] for t in tr)
    assert runs[0][0] == runs[1][0]
    assert np.array_equal(runs[0][1][0], runs[1][1][0]) and np.array_equal(runs[0][1][1], runs[1][1][1])


def test_radius_state_and_options():
    sc = ba_scene("tiny")
    g = bamod.Problem.from_scene(sc, strategy=bamod.BA_STRATEGY_DOGLEG, dl_radius0=0.25)
    assert g.get_state()["radius"] == 0.25
    g.set_state(1e-3, 0, radius=2.0)
    t = g.lm_step()
    assert t["radius"] == 2.0
    g.set_state(1e-3, 0)          # radius 0: left as it is
    assert g.get_state()["radius"] > 0.0
    for bad in (dict(strategy=7), dict(strategy=1, dl_radius0=0.0),
                dict(strategy=1, dl_gn_damping=-1.0)):
        with pytest.raises(bamod.BAError) as e:
            bamod.Problem.from_scene(sc, **bad)
        assert e.value.code == bamod.BA_ERR_ARG


@pytest.mark.parametrize("solver", [0, 1])
def test_dogleg_edge_scene(solver):
    """Repeated runs, a 700-observation point, an unobserved point and an
    unobserved camera (zero gradient: it never moves)."""
    sc = _edge_scene()
    gpu = bamod.Problem.from_scene(sc, strategy=bamod.BA_STRATEGY_DOGLEG, solver=solver,
                                   loss=bamod.BA_LOSS_HUBER)
    orc = oracle.Problem.from_scene(sc, strategy=1, solver=solver)
    tg = [gpu.lm_step() for _ in range(8)]
    to = orc.solve(8)
    dogleg_traces_agree(tg, to, sc["pcg_rel_tol"])
    assert abs(gpu.get_state()["cost"] - orc.cost) <= 1e-6 * orc.cost
    cams, pts = gpu.get_params()
    np.testing.assert_array_equal(pts[11], sc["points"][11])
    np.testing.assert_array_equal(cams[9], sc["cams"][9])


@pytest.mark.parametrize("cameras", CAMERA_TABLES)
def test_dogleg_heavy_camera(cameras, monkeypatch):
    """A camera with about 3,200 observations in one point band: the model
    sums over the observations run over several chunks of that camera."""
    use_camera_table(cameras, monkeypatch)
    from synthetic import heavy_camera_scene
    sc = heavy_camera_scene()
    gpu = bamod.Problem.from_scene(sc, strategy=bamod.BA_STRATEGY_DOGLEG)
    orc = oracle.Problem.from_scene(sc, strategy=1)
    tg = [gpu.lm_step() for _ in range(6)]
    to = orc.solve(6)
    dogleg_traces_agree(tg, to, sc["pcg_rel_tol"])
    assert abs(gpu.get_state()["cost"] - orc.cost) <= 1e-6 * orc.cost
