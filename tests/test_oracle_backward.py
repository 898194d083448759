"""Pins for the oracle's implicit backward (the Theseus note's implicit mode:
differentiate one Newton step h(theta; u) = theta - H~^-1 grad S at the
solution, the damped Gauss-Newton matrix H~ held fixed; u = observed pixels).

- Squared loss: H~ does not depend on u, so the LM step is affine in u and a
  central difference of <G, step(u)> with any step size is the exact
  vector-Jacobian product (up to rounding).
- Huber: d grad S / d u_k = -J_k^T psi'(r_k), so <lambda, grad S(u)> with
  lambda = H~^-1 G differenced in u_k must give -df/du_k; central differences
  away from the threshold.
- Dense closed form: psi'(r_k) J_k H~^-1 G with the full Jacobian and H~ solved
  by numpy, against the oracle's Schur path.
"""
import numpy as np
import pytest

import oracle
from synthetic import ba_scene


def _step(sc, uv, lam, **kw):
    s = dict(sc, obs_uv=uv)
    P = oracle.Problem.from_scene(s, solver=1, **kw)
    P.lam = lam
    P.linearize()
    P.damp()
    P.schur()
    P.dense_schur_solve()
    P.backsub()
    return P.get("dc").ravel(), P.get("dp").ravel()


def _grads(sc, seed=3):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((len(sc["cams"]), 9)), rng.standard_normal((len(sc["points"]), 3))


def test_backward_is_the_derivative_of_the_lm_step_squared_loss():
    sc = ba_scene("tiny")
    lam = 1e-2
    G_c, G_p = _grads(sc)
    P = oracle.Problem.from_scene(sc, solver=1)
    P.lam = lam
    out, _, _ = P.backward(G_c, G_p)
    rng = np.random.default_rng(5)
    uv = sc["obs_uv"]
    for k in rng.choice(len(uv), size=24, replace=False):
        for a in range(2):
            fd = []
            for sgn in (1.0, -1.0):
                u = uv.copy()
                u[k, a] += sgn * 1.0
                dc, dp = _step(sc, u, lam)
                fd.append(G_c.ravel() @ dc + G_p.ravel() @ dp)
            d = (fd[0] - fd[1]) / 2.0
            assert abs(d - out[k, a]) <= 1e-8 * max(1.0, abs(out[k, a])), (k, a, d, out[k, a])


def test_backward_huber_matches_gradient_differences():
    sc = ba_scene("tiny", outlier_frac=0.2)
    delta, lam = 2.0, 1e-2
    G_c, G_p = _grads(sc, seed=4)
    P = oracle.Problem.from_scene(sc, solver=1, loss=1, huber_delta=delta)
    P.lam = lam
    out, _, _ = P.backward(G_c, G_p)
    lc, lp = P.get("dc").ravel(), P.get("dp").ravel()   # lambda = H~^-1 G
    P.linearize()
    e = np.linalg.norm(P.get("r"), axis=1)
    far = np.nonzero(np.abs(e - delta) > 1e-2)[0]
    outside = far[e[far] > delta]
    inside = far[e[far] <= delta]
    assert len(outside) >= 5 and len(inside) >= 5
    pick = np.concatenate([outside[:10], inside[:6]])
    h = 1e-5
    for k in pick:
        for a in range(2):
            vals = []
            for sgn in (1.0, -1.0):
                u = sc["obs_uv"].copy()
                u[k, a] += sgn * h
                Q = oracle.Problem.from_scene(dict(sc, obs_uv=u), loss=1, huber_delta=delta)
                Q.linearize()
                vals.append(lc @ Q.get("gc").ravel() + lp @ Q.get("gp").ravel())
            d = (vals[0] - vals[1]) / (2 * h)
            assert abs(d + out[k, a]) <= 1e-6 * max(1.0, abs(out[k, a])), (k, a, e[k], d, out[k, a])


@pytest.mark.parametrize("loss", [0, 1])
def test_backward_matches_dense_closed_form(loss):
    sc = ba_scene("tiny", outlier_frac=0.2)
    delta, lam = 2.0, 1e-2
    G_c, G_p = _grads(sc, seed=6)
    P = oracle.Problem.from_scene(sc, solver=1, loss=loss, huber_delta=delta)
    P.lam = lam
    out, _, _ = P.backward(G_c, G_p)
    P.linearize()
    nc, npt, N = P.nc, P.np, P.nobs
    Jc, Jp, r, w = P.get("Jc"), P.get("Jp"), P.get("r"), P.get("w")
    J = np.zeros((2 * N, 9 * nc + 3 * npt))
    for k in range(N):
        j, i = sc["obs_cam"][k], sc["obs_pt"][k]
        J[2 * k:2 * k + 2, 9 * j:9 * j + 9] = Jc[k]
        J[2 * k:2 * k + 2, 9 * nc + 3 * i:9 * nc + 3 * i + 3] = Jp[k]
    H = J.T @ (np.repeat(w, 2)[:, None] * J)
    Ht = H + lam * np.diag(np.maximum(np.diag(H), 1e-6))
    lam_vec = np.linalg.solve(Ht, np.concatenate([G_c.ravel(), G_p.ravel()]))
    y = (J @ lam_vec).reshape(N, 2)
    ref = y.copy()
    if loss == 1:
        e = np.linalg.norm(r, axis=1)
        big = e > delta
        rh = r[big] / e[big, None]
        ref[big] = (delta / e[big, None]) * (y[big] - rh * np.sum(rh * y[big], axis=1, keepdims=True))
    np.testing.assert_allclose(out, ref, rtol=1e-9, atol=1e-12 * np.abs(ref).max())
