"""Pins for the oracle's dogleg iteration (``orc_dogleg_step``), checked
against a dense J built in numpy at the same linearisation point:

- with a radius larger than the Gauss-Newton step, the step is h_gn, the
  solution of (J^T W J + mu D) h = -g, and the reported gain ratio is the cost
  decrease over the quadratic model's, L(0) - L(h) = -g^T h - 1/2 h^T H h;
- with a tiny radius, the step is -radius g / |g| (points move additively, so
  their part is read off the trial points);
- in between, |h| equals the radius and h lies on the segment from the
  Cauchy point -alpha g, alpha = |g|^2 / |J g|_W^2, to h_gn;
- along a trace the radius follows its update rule, accepted costs decrease
  strictly, and the final cost equals Levenberg-Marquardt's.
"""
import numpy as np
import pytest

import oracle
from synthetic import ba_scene

MU = 1e-6


def dense_model(P, sc):
    nc, npt = len(sc["cams"]), len(sc["points"])
    Jc, Jp, w = P.get("Jc"), P.get("Jp"), P.get("w")
    n = 9 * nc + 3 * npt
    J = np.zeros((2 * len(w), n))
    for k, (j, i) in enumerate(zip(sc["obs_cam"], sc["obs_pt"])):
        J[2 * k:2 * k + 2, 9 * j:9 * j + 9] = Jc[k]
        J[2 * k:2 * k + 2, 9 * nc + 3 * i:9 * nc + 3 * i + 3] = Jp[k]
    W = np.repeat(w, 2)
    H = J.T @ (W[:, None] * J)
    g = np.concatenate([P.get("gc").ravel(), P.get("gp").ravel()])
    return H, g, nc


def fresh(sc, **kw):
    P = oracle.Problem.from_scene(sc, strategy=1, solver=1, dl_gn_damping=MU, **kw)
    P.linearize()
    return P


def test_large_radius_takes_the_gauss_newton_step_and_the_model_ratio():
    sc = ba_scene("tiny")
    P = fresh(sc)
    H, g, nc = dense_model(P, sc)
    D = np.maximum(np.diag(H), 1e-6)
    h_gn = np.linalg.solve(H + MU * np.diag(D), -g)
    P.radius = 10 * np.linalg.norm(h_gn)
    t = P.lm_step()
    assert t["step_kind"] == 0
    np.testing.assert_allclose(t["step_norm"], np.linalg.norm(h_gn), rtol=1e-7)
    model = -g @ h_gn - 0.5 * h_gn @ H @ h_gn
    np.testing.assert_allclose(t["gain_ratio"], (t["cost_before"] - t["cost_after"]) / model,
                               rtol=1e-7)
    dp = P.get("points_trial").ravel() - sc["points"].ravel() if not t["accepted"] else \
        P.get("points").ravel() - sc["points"].ravel()
    np.testing.assert_allclose(dp, h_gn[9 * nc:], rtol=1e-6, atol=1e-9 * np.abs(h_gn).max())


def test_tiny_radius_takes_the_cut_steepest_descent_step():
    sc = ba_scene("tiny")
    P = fresh(sc)
    H, g, nc = dense_model(P, sc)
    R = 1e-6
    P.radius = R
    t = P.lm_step()
    assert t["step_kind"] == 1
    np.testing.assert_allclose(t["step_norm"], R, rtol=1e-12)
    pts = P.get("points") if t["accepted"] else P.get("points_trial")
    # read off x + h - x: rounding of x (|x| ~ 10) limits the absolute agreement
    np.testing.assert_allclose(pts.ravel() - sc["points"].ravel(), -R * g[9 * nc:] / np.linalg.norm(g),
                               rtol=1e-6, atol=4 * np.finfo(float).eps * np.abs(sc["points"]).max())


def test_blend_lies_on_the_dogleg_at_the_radius():
    sc = ba_scene("tiny")
    P = fresh(sc)
    H, g, nc = dense_model(P, sc)
    D = np.maximum(np.diag(H), 1e-6)
    h_gn = np.linalg.solve(H + MU * np.diag(D), -g)
    alpha = (g @ g) / (g @ H @ g)
    a = -alpha * g
    R = 0.5 * (np.linalg.norm(a) + np.linalg.norm(h_gn))
    assert np.linalg.norm(a) < R < np.linalg.norm(h_gn)
    P.radius = R
    t = P.lm_step()
    assert t["step_kind"] == 2
    np.testing.assert_allclose(t["step_norm"], R, rtol=1e-9)
    pts = P.get("points") if t["accepted"] else P.get("points_trial")
    hp = pts.ravel() - sc["points"].ravel()
    # hp = a_p + beta (h_gn,p - a_p) for one beta in (0, 1)
    d = h_gn[9 * nc:] - a[9 * nc:]
    beta = (hp - a[9 * nc:]) @ d / (d @ d)
    assert 0.0 < beta < 1.0
    np.testing.assert_allclose(hp, a[9 * nc:] + beta * d, rtol=1e-6, atol=1e-9 * np.abs(hp).max())
    # and the whole step, norm R, is that point of the segment
    h = a + beta * (h_gn - a)
    np.testing.assert_allclose(np.linalg.norm(h), R, rtol=1e-6)


@pytest.mark.parametrize("config", ["tiny", "small"])
def test_trace_rules_and_final_cost(config):
    sc = ba_scene(config)
    P = oracle.Problem.from_scene(sc, strategy=1, solver=1)
    tr = P.solve(sc["n_iters"])
    for a, b in zip(tr, tr[1:]):
        R = a["radius"]
        if a["gain_ratio"] > 0.75:
            want = max(R, 3 * a["step_norm"])
        elif a["gain_ratio"] < 0.25:
            want = 0.5 * R
        else:
            want = R
        assert b["radius"] == want, (a, b)
        if not a["accepted"]:
            assert b["pcg_iters"] == 0 and b["cost_before"] == a["cost_before"]
    acc = [t["cost_after"] for t in tr if t["accepted"]]
    assert all(y < x for x, y in zip(acc, acc[1:]))
    L = oracle.Problem.from_scene(sc, solver=1)
    L.solve(sc["n_iters"])
    assert abs(P.cost - L.cost) <= 1e-9 * L.cost


def test_noise_free_scene_converges():
    sc = ba_scene("tiny", noise_px=0.0)
    P = oracle.Problem.from_scene(sc, strategy=1, solver=1)
    c0 = P.cost
    P.solve(25)
    assert P.cost < 1e-12 * c0
