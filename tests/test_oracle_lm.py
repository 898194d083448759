"""Pins for the oracle's LM loop: decision invariants, the damping schedule,
convergence to zero cost on noise-free scenes and the chi-square level of the
final cost on noisy ones (a statistical pin: the pages print no BA values)."""
import numpy as np
import pytest

import oracle
from synthetic import ba_scene


def test_accepted_costs_decrease_and_rejections_keep_parameters():
    sc = ba_scene("tiny")
    P = oracle.Problem.from_scene(sc, lambda0=1e-8)   # small lambda provokes rejections
    lam = P.lam
    seen_reject = False
    for _ in range(15):
        cams0, pts0, cost0 = P.get("cams").copy(), P.get("points").copy(), P.cost
        info = P.lm_step()
        assert info["cost_before"] == cost0 and info["lam"] == lam
        if info["accepted"]:
            assert info["cost_after"] < cost0
            assert P.cost == info["cost_after"]
            assert P.lam == max(lam / 10, 1e-16)
        else:
            seen_reject = True
            np.testing.assert_array_equal(P.get("cams"), cams0)
            np.testing.assert_array_equal(P.get("points"), pts0)
            assert P.cost == cost0
            assert P.lam == min(lam * 10, 1e16)
        lam = P.lam
    assert seen_reject


def test_huge_lambda_gives_tiny_monotone_steps():
    sc = ba_scene("tiny")
    P = oracle.Problem.from_scene(sc, lambda0=1e12)
    infos = P.solve(3)
    for inf in infos:
        assert inf["cost_after"] <= inf["cost_before"] * (1 + 1e-12)
    assert abs(infos[0]["cost_after"] - infos[0]["cost_before"]) < 1e-3 * infos[0]["cost_before"]


def test_noise_free_tiny_converges_to_zero_cost():
    sc = ba_scene("tiny", noise_px=0.0)
    P = oracle.Problem.from_scene(sc)
    c0 = P.cost
    P.solve(30)
    assert P.cost < 1e-12 * c0, (P.cost, c0)


def _chi2_level(n_obs, nc, npt):
    dof = 2 * n_obs - (9 * nc + 3 * npt - 7)
    return 0.5 * dof, 0.5 * np.sqrt(2 * dof)


@pytest.mark.parametrize("config", ["tiny", "small"])
def test_noisy_final_cost_at_chi_square_level(config):
    sc = ba_scene(config)
    P = oracle.Problem.from_scene(sc)
    c_true = P.cost_at(sc["cams_true"], sc["points_true"])
    P.solve(sc["n_iters"])
    mean, sigma = _chi2_level(P.nobs, P.nc, P.np)
    assert P.cost <= c_true
    assert abs(P.cost - mean) < 4 * sigma, (P.cost, mean, sigma)


def test_dense_and_pcg_solvers_agree_on_final_cost():
    sc = ba_scene("tiny")
    a = oracle.Problem.from_scene(sc, solver=0, pcg_rel_tol=1e-12, pcg_max_iters=500)
    b = oracle.Problem.from_scene(sc, solver=1)
    a.solve(10)
    b.solve(10)
    assert abs(a.cost - b.cost) <= 1e-9 * b.cost


def test_huber_reduces_outlier_influence():
    sc = ba_scene("small", outlier_frac=0.05)
    sq = oracle.Problem.from_scene(sc, loss=0)
    hu = oracle.Problem.from_scene(sc, loss=1, huber_delta=2.0)
    sq.solve(8)
    hu.solve(8)
    def point_err(P):
        return np.median(np.linalg.norm(P.get("points") - sc["points_true"], axis=1))
    assert point_err(hu) < point_err(sq)
