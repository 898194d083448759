"""Pins for assembly, damping, Schur elimination, PCG and back-substitution.

The references are dense: the full Jacobian is built in numpy from the
per-observation blocks, J^T W J and J^T W r are formed by matrix products, the
damped full system H~ delta = -g is solved by scipy's Cholesky (the library
routine the dense reference step on the NeRF-SLAM page calls), and Schur
elimination is exact algebra, so its result must agree with the full solve.
"""
import numpy as np
import pytest
from scipy.linalg import cho_factor, cho_solve

import oracle
from synthetic import ba_scene


def _dense(P, sc):
    """Dense J (2N x (9 nc + 3 np)), W and r from the oracle's blocks."""
    nc, npt, N = P.nc, P.np, P.nobs
    Jc, Jp, r, w = P.get("Jc"), P.get("Jp"), P.get("r"), P.get("w")
    J = np.zeros((2 * N, 9 * nc + 3 * npt))
    for k in range(N):
        j, i = sc["obs_cam"][k], sc["obs_pt"][k]
        J[2 * k:2 * k + 2, 9 * j:9 * j + 9] = Jc[k]
        J[2 * k:2 * k + 2, 9 * nc + 3 * i:9 * nc + 3 * i + 3] = Jp[k]
    W = np.repeat(w, 2)
    return J, W, r.ravel()


def _scene_with_duplicates(outliers=0.1):
    sc = ba_scene("tiny", outlier_frac=outliers)
    # Repeat a few observations with fresh pixels: repeated (camera, point) pairs.
    rng = np.random.default_rng(2)
    extra = rng.choice(len(sc["obs_cam"]), size=25, replace=False)
    for key in ("obs_cam", "obs_pt"):
        sc[key] = np.concatenate([sc[key], sc[key][extra]]).astype(np.int32)
    sc["obs_uv"] = np.concatenate([sc["obs_uv"], sc["obs_uv"][extra] + rng.normal(0, 3, (25, 2))])
    return sc


@pytest.fixture(params=["plain", "huber_dup"])
def tiny(request):
    if request.param == "plain":
        sc = ba_scene("tiny")
        P = oracle.Problem.from_scene(sc)
    else:
        sc = _scene_with_duplicates()
        P = oracle.Problem.from_scene(sc, loss=1, huber_delta=2.0)
    P.lam = 1e-2
    P.linearize()
    P.damp()
    P.schur()
    return sc, P


def test_assembly_matches_dense_products(tiny):
    sc, P = tiny
    J, W, r = _dense(P, sc)
    H = J.T @ (W[:, None] * J)
    g = J.T @ (W * r)
    nc = P.nc
    B, C, gc, gp = P.get("B"), P.get("C"), P.get("gc"), P.get("gp")
    for j in range(nc):
        blk = H[9 * j:9 * j + 9, 9 * j:9 * j + 9]
        np.testing.assert_allclose(B[j], blk, rtol=0, atol=1e-12 * np.abs(blk).max())
    for i in range(P.np):
        o = 9 * nc + 3 * i
        blk = H[o:o + 3, o:o + 3]
        np.testing.assert_allclose(C[i], blk, rtol=0, atol=1e-12 * max(np.abs(blk).max(), 1e-30))
    np.testing.assert_allclose(gc.ravel(), g[:9 * nc], rtol=0, atol=1e-12 * np.abs(g).max())
    np.testing.assert_allclose(gp.ravel(), g[9 * nc:], rtol=0, atol=1e-12 * np.abs(g).max())


def _damped_dense(P, sc):
    J, W, r = _dense(P, sc)
    H = J.T @ (W[:, None] * J)
    g = J.T @ (W * r)
    d = np.maximum(np.diag(H), 1e-6)
    return H + P.lam * np.diag(d), g


def test_damping_and_point_inverse(tiny):
    sc, P = tiny
    Hd, _ = _damped_dense(P, sc)
    nc = P.nc
    Bd, Cinv = P.get("Bd"), P.get("Cinv")
    for j in range(nc):
        np.testing.assert_allclose(Bd[j], Hd[9 * j:9 * j + 9, 9 * j:9 * j + 9], rtol=1e-13,
                                   atol=1e-13 * np.abs(Bd[j]).max())
    for i in range(P.np):
        o = 9 * nc + 3 * i
        inv = np.linalg.inv(Hd[o:o + 3, o:o + 3])
        np.testing.assert_allclose(Cinv[i], inv, rtol=1e-9, atol=1e-12 * np.abs(inv).max())
    np.testing.assert_allclose(P.get("v"), np.einsum("nij,nj->ni", Cinv, P.get("gp")), rtol=1e-13)


def test_explicit_schur_and_preconditioner_match_dense(tiny):
    sc, P = tiny
    Hd, g = _damped_dense(P, sc)
    n = 9 * P.nc
    Bt, E, Ct = Hd[:n, :n], Hd[:n, n:], Hd[n:, n:]
    S_ref = Bt - E @ np.linalg.solve(Ct, E.T)
    S = P.explicit_S()
    np.testing.assert_allclose(S, S_ref, rtol=0, atol=1e-9 * np.abs(S_ref).max())
    M = P.get("M")
    for j in range(P.nc):
        np.testing.assert_allclose(M[j], S_ref[9 * j:9 * j + 9, 9 * j:9 * j + 9], rtol=0,
                                   atol=1e-9 * np.abs(S_ref).max())
    rhs_ref = -g[:n] + E @ np.linalg.solve(Ct, g[n:])
    np.testing.assert_allclose(P.get("rhs").ravel(), rhs_ref, rtol=0, atol=1e-9 * np.abs(rhs_ref).max())
    x = np.random.default_rng(1).normal(size=n)
    np.testing.assert_allclose(P.schur_matvec(x), S_ref @ x, rtol=0,
                               atol=1e-9 * np.abs(S_ref @ x).max())


def test_schur_plus_backsub_equals_full_dense_solve(tiny):
    """Eliminating the points and back-substituting is exact algebra: the result
    equals the solution of the damped full system by scipy's Cholesky."""
    sc, P = tiny
    Hd, g = _damped_dense(P, sc)
    delta_ref = cho_solve(cho_factor(Hd, lower=True), -g)
    P.dense_schur_solve()
    P.backsub()
    delta = np.concatenate([P.get("dc").ravel(), P.get("dp").ravel()])
    err = np.linalg.norm(delta - delta_ref) / np.linalg.norm(delta_ref)
    assert err < 1e-10, err


@pytest.mark.parametrize("config", ["tiny", "small"])
def test_pcg_converges_to_dense_schur_solution(config):
    sc = ba_scene(config)
    P = oracle.Problem.from_scene(sc)
    P.linearize()
    P.damp()
    P.schur()
    P.dense_schur_solve()
    dc_ref = P.get("dc").copy()
    it, rel = P.pcg(max_iters=9 * P.nc, rel_tol=1e-14)
    assert rel <= 1e-14 or it == 9 * P.nc
    dc = P.get("dc")
    err = np.linalg.norm(dc - dc_ref) / np.linalg.norm(dc_ref)
    assert err < 1e-9, (err, it)


def test_pcg_residual_recurrence_matches_explicit_residual():
    sc = ba_scene("small")
    P = oracle.Problem.from_scene(sc)
    P.linearize()
    P.damp()
    P.schur()
    it, rel = P.pcg(max_iters=50, rel_tol=1e-6)
    assert 0 < it <= 50
    rhs = P.get("rhs").ravel()
    res = rhs - P.schur_matvec(P.get("dc").ravel())
    rel_explicit = np.linalg.norm(res) / np.linalg.norm(rhs)
    assert abs(rel_explicit - rel) <= 1e-8 + 1e-3 * rel, (rel_explicit, rel)
    if it < 50:
        assert rel <= 1e-6


def test_pcg_zero_rhs_gives_zero_step():
    sc = ba_scene("tiny", noise_px=0.0)
    P = oracle.Problem(sc["cams_true"], sc["points_true"], sc["obs_cam"], sc["obs_pt"],
                       sc["obs_uv"])
    P.linearize()
    P.damp()
    P.schur()
    it, _ = P.pcg()
    assert np.abs(P.get("dc")).max() < 1e-6
