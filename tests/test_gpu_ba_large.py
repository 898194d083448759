"""Parity at the full large-scene size (1,000 cameras, 400,000 points,
2,203,610 observations), in the launch configuration the benchmark times.

The oracle cannot afford element-by-element comparison of every array at this
size inside a test, so it checks:
  * sampled observations (residual, both Jacobians, robust weight) against the
    oracle's per-observation function,
  * sampled point blocks C_i and camera blocks B_j summed by the oracle's
    per-observation function over that point's or camera's observations,
  * the PCG result through a property that holds at any size: the oracle's
    own implicit Schur operator applied to the GPU step leaves a residual within
    the stopping tolerance of the oracle's right-hand side,
  * one full LM step: cost before, trial cost and the decision.
"""
import numpy as np
import pytest

import oracle
from nonlinear_least_squares_amd import ba as bamod
from synthetic import ba_scene

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def large():
    sc = ba_scene("large")
    return sc


def _close(a, b, tol, floor):
    err = np.linalg.norm(np.asarray(a) - np.asarray(b))
    return err <= tol * max(np.linalg.norm(b), floor)


def test_large_sampled_linearisation(large):
    sc = large
    g = bamod.Problem.from_scene(sc)
    g.debug_run(bamod.BA_STAGE_LINEARIZE)
    r, Jc, Jp, w = (g.debug_get(n) for n in ("r", "Jc", "Jp", "w"))
    loss = 1 if sc["loss"] == "huber" else 0
    rng = np.random.default_rng(44)
    N = len(sc["obs_cam"])
    for k in rng.choice(N, size=2048, replace=False):
        o = oracle.project_one(sc["cams"][sc["obs_cam"][k]], sc["points"][sc["obs_pt"][k]],
                               sc["obs_uv"][k], loss, sc["huber_delta"])
        assert _close(r[k], o["r"], 1e-10, 1e-6)
        assert _close(Jc[k], o["Jc"], 1e-10, 1e-6)
        assert _close(Jp[k], o["Jp"], 1e-10, 1e-6)
        assert abs(w[k] - o["w"]) <= 1e-12
    # point blocks C_i = sum_k w Jp^T Jp over the point's observations
    C = g.debug_get("C").reshape(-1, 3, 3)
    by_pt = np.argsort(sc["obs_pt"], kind="stable")
    ptr = np.searchsorted(sc["obs_pt"][by_pt], np.arange(len(sc["points"]) + 1))
    for i in rng.choice(len(sc["points"]), size=256, replace=False):
        acc = np.zeros((3, 3))
        for k in by_pt[ptr[i]:ptr[i + 1]]:
            o = oracle.project_one(sc["cams"][sc["obs_cam"][k]], sc["points"][i], sc["obs_uv"][k],
                                   loss, sc["huber_delta"])
            acc += o["w"] * o["Jp"].T @ o["Jp"]
        assert _close(C[i], acc, 1e-10, 1e-6)
    # camera blocks B_j over ~2,200 observations each
    B = g.debug_get("B").reshape(-1, 9, 9)
    for j in rng.choice(len(sc["cams"]), size=3, replace=False):
        acc = np.zeros((9, 9))
        for k in np.nonzero(sc["obs_cam"] == j)[0]:
            o = oracle.project_one(sc["cams"][j], sc["points"][sc["obs_pt"][k]], sc["obs_uv"][k],
                                   loss, sc["huber_delta"])
            acc += o["w"] * o["Jc"].T @ o["Jc"]
        assert _close(B[j], acc, 1e-10, 1e-6)


def test_large_pcg_step_solves_the_oracle_system(large):
    sc = large
    g = bamod.Problem.from_scene(sc)
    g.debug_run(bamod.BA_STAGE_PCG)
    dc = g.debug_get("dc").ravel()
    iters, rel = g.debug_get("pcg")
    o = oracle.Problem.from_scene(sc)
    o.linearize()
    o.damp()
    o.schur()
    rhs = o.get("rhs").ravel()
    assert np.linalg.norm(g.debug_get("rhs").ravel() - rhs) <= 1e-9 * np.linalg.norm(rhs)
    res = np.linalg.norm(o.schur_matvec(dc) - rhs) / np.linalg.norm(rhs)
    assert int(iters) < sc["pcg_max_iters"]
    # the GPU stopped at its own relative residual <= 1e-6; the oracle's
    # operator agrees with the GPU's to rounding
    assert rel <= sc["pcg_rel_tol"]
    assert res <= 1.01 * sc["pcg_rel_tol"] + 1e-9, (res, rel)


def test_large_one_lm_step(large):
    sc = large
    g = bamod.Problem.from_scene(sc)
    gi = g.lm_step()
    o = oracle.Problem.from_scene(sc)
    oi = o.lm_step()
    assert abs(gi["cost_before"] - oi["cost_before"]) <= 1e-10 * oi["cost_before"]
    assert abs(gi["cost_after"] - oi["cost_after"]) <= 1e-6 * oi["cost_after"]
    if abs(oi["cost_after"] - oi["cost_before"]) > 1e-10 * oi["cost_before"]:
        assert gi["accepted"] == oi["accepted"]
    assert gi["pcg_iters"] == oi["pcg_iters"]


def test_large_one_dogleg_step(large):
    """One dogleg iteration at full size.  The first radius (1.0) is far below
    the Gauss-Newton step, so the step is the cut steepest descent (or a blend
    when the Cauchy point falls inside): the kind, the radius and the norm
    match the oracle's; the trial cost is held to 1e-6 when the step does not
    depend on a Gauss-Newton solve that stopped at its iteration cap."""
    sc = large
    g = bamod.Problem.from_scene(sc, strategy=bamod.BA_STRATEGY_DOGLEG)
    gi = g.lm_step()
    o = oracle.Problem.from_scene(sc, strategy=1)
    oi = o.lm_step()
    assert abs(gi["cost_before"] - oi["cost_before"]) <= 1e-10 * oi["cost_before"]
    assert gi["step_kind"] == oi["step_kind"] and gi["radius"] == oi["radius"] == 1.0
    assert abs(gi["step_norm"] - oi["step_norm"]) <= 1e-6 * oi["step_norm"]
    if oi["step_kind"] == 1 or oi["pcg_rel_res"] <= sc["pcg_rel_tol"]:
        assert abs(gi["cost_after"] - oi["cost_after"]) <= 1e-6 * oi["cost_after"]
