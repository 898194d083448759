"""Pins for the pose-graph oracle (``oracle/pgo_oracle.c``).

- SO(3): exp/log round trip, Log against scipy, the inverse right Jacobian by
  differences of Log(Exp(w) Exp(d)).
- Edge Jacobians by central differences through the retraction.
- The residual of the true poses against noise-free measurements is zero.
- H and g against the dense J^T Omega J and J^T Omega r built in numpy.
- The step solves the damped system (dense numpy solve); PCG and the dense
  Cholesky agree at a tight tolerance.
- LM: noise-free graphs converge to zero cost; accepted costs decrease; the
  final cost of a noisy graph sits near its chi-square expectation.
"""
import numpy as np
import pytest
from scipy.spatial.transform import Rotation

from oracle import pgo
from synthetic import pgo_scene


def test_so3_exp_log_round_trip_and_scipy():
    rng = np.random.default_rng(1)
    for _ in range(50):
        w = rng.normal(size=3)
        w *= rng.uniform(0.0, 3.0) / np.linalg.norm(w)
        R = pgo.so3_exp(w)
        np.testing.assert_allclose(R, Rotation.from_rotvec(w).as_matrix(), atol=1e-14)
        np.testing.assert_allclose(pgo.so3_log(R), w, atol=1e-12)
    np.testing.assert_allclose(pgo.so3_log(np.eye(3)), 0.0, atol=1e-15)


def test_edge_jacobians_by_central_differences():
    sc = pgo_scene("tiny")
    rng = np.random.default_rng(2)
    h = 1e-6
    for e in rng.choice(len(sc["edges"]), size=10, replace=False):
        i, j = sc["edges"][e]
        pi, pj, m = sc["poses"][i], sc["poses"][j], sc["meas"][e]
        r, Ji, Jj = pgo.edge(pi, pj, m)
        for k in range(6):
            d = np.zeros(6)
            d[k] = h
            rp, _, _ = pgo.edge(pgo.retract(pi, d), pj, m)
            rm, _, _ = pgo.edge(pgo.retract(pi, -d), pj, m)
            np.testing.assert_allclose((rp - rm) / (2 * h), Ji[:, k], rtol=1e-6, atol=1e-8)
            rp, _, _ = pgo.edge(pi, pgo.retract(pj, d), m)
            rm, _, _ = pgo.edge(pi, pgo.retract(pj, -d), m)
            np.testing.assert_allclose((rp - rm) / (2 * h), Jj[:, k], rtol=1e-6, atol=1e-8)


def test_true_poses_have_zero_residual_without_noise():
    sc = pgo_scene("small", noise=0.0)
    P = pgo.PGOProblem(sc["poses_true"], sc["edges"], sc["meas"], sc["info"], 1)
    assert P.cost < 1e-20


def _dense(P, sc):
    n, m = len(sc["poses"]), len(sc["edges"])
    J = np.zeros((6 * m, 6 * n))
    Ji, Jj = P.get("Ji"), P.get("Jj")
    for e, (i, j) in enumerate(sc["edges"]):
        J[6 * e:6 * e + 6, 6 * i:6 * i + 6] = Ji[e]
        J[6 * e:6 * e + 6, 6 * j:6 * j + 6] = Jj[e]
    om = np.repeat(sc["info"], 3, axis=1).ravel()
    return J, om, P.get("r").ravel()


def test_normal_equations_against_dense_products():
    sc = pgo_scene("tiny")
    P = pgo.PGOProblem.from_scene(sc)
    P.linearize()
    J, om, r = _dense(P, sc)
    H = J.T @ (om[:, None] * J)
    g = J.T @ (om * r)
    n = len(sc["poses"])
    Hd = P.get("Hd")
    for i in range(n):
        np.testing.assert_allclose(Hd[i], H[6 * i:6 * i + 6, 6 * i:6 * i + 6], rtol=1e-12,
                                   atol=1e-9 * np.abs(H).max())
    Ho = P.get("Ho")
    for e, (i, j) in enumerate(sc["edges"]):
        np.testing.assert_allclose(Ho[e], H[6 * i:6 * i + 6, 6 * j:6 * j + 6], rtol=1e-12,
                                   atol=1e-9 * np.abs(H).max())
    np.testing.assert_allclose(P.get("g").ravel(), g, rtol=1e-12, atol=1e-10 * np.abs(g).max())


@pytest.mark.parametrize("solver", [0, 1])
def test_step_solves_the_damped_system(solver):
    sc = pgo_scene("tiny")
    P = pgo.PGOProblem.from_scene(sc, solver=solver, pcg_rel_tol=1e-13, pcg_max_iters=1000)
    P.lam = 1e-2
    P.linearize()
    P.solve_step()
    J, om, r = _dense(P, sc)
    H = J.T @ (om[:, None] * J)
    g = J.T @ (om * r)
    Ht = H + 1e-2 * np.diag(np.maximum(np.diag(H), 1e-6))
    free = np.arange(6, H.shape[0])       # pose 0 is held
    ref = np.linalg.solve(Ht[np.ix_(free, free)], -g[free])
    dx = P.get("dx").ravel()
    assert np.all(dx[:6] == 0.0)
    np.testing.assert_allclose(dx[free], ref, rtol=1e-8, atol=1e-10 * np.abs(ref).max())


def test_noise_free_graph_converges():
    sc = pgo_scene("small", noise=0.0)
    P = pgo.PGOProblem.from_scene(sc, solver=1)
    c0 = P.cost
    P.solve(15)
    assert P.cost < 1e-16 * c0


def test_lm_decreases_and_reaches_chi_square():
    sc = pgo_scene("small")
    P = pgo.PGOProblem.from_scene(sc)
    tr = P.solve(sc["n_iters"])
    acc = [t["cost_after"] for t in tr if t["accepted"]]
    assert all(b < a for a, b in zip(acc, acc[1:]))
    n, m = len(sc["poses"]), len(sc["edges"])
    dof = 6 * m - 6 * (n - 1)
    # 1/2 chi-square with dof degrees of freedom: mean dof/2, sd sqrt(dof/2)
    assert abs(P.cost - dof / 2) < 5 * np.sqrt(dof / 2), (P.cost, dof / 2)
