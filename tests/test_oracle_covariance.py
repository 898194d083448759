"""Pins for the oracle's camera marginal covariance (``orc_covariance``):
the 9x9 diagonal blocks of S~^-1, S~ the damped reduced camera matrix, from
its Cholesky factor as in the NeRF-SLAM notes' dense step (sec. 3.2).

- By the Schur complement, S~^-1 is the camera block of the inverse of the
  whole damped system; that inverse is formed here from a dense J built in
  numpy, with its own damping, and inverted by numpy.
- For large lambda the coupling through the points fades: each block tends to
  the inverse of the camera's own damped block, B~_j^-1, with a relative
  difference of order 1/lambda^2 (checked against that rate).
- Blocks are symmetric positive definite, and the call leaves the LM state as
  it was.
"""
import numpy as np

import oracle
from synthetic import ba_scene


def _full_damped_H(P, sc, lam, floor=1e-6):
    nc, npt = len(sc["cams"]), len(sc["points"])
    Jc, Jp, w = P.get("Jc"), P.get("Jp"), P.get("w")
    n = 9 * nc + 3 * npt
    J = np.zeros((2 * len(w), n))
    for k, (j, i) in enumerate(zip(sc["obs_cam"], sc["obs_pt"])):
        J[2 * k:2 * k + 2, 9 * j:9 * j + 9] = Jc[k]
        J[2 * k:2 * k + 2, 9 * nc + 3 * i:9 * nc + 3 * i + 3] = Jp[k]
    W = np.repeat(w, 2)
    H = J.T @ (W[:, None] * J)
    d = np.diag(H).copy()
    return H + lam * np.diag(np.maximum(d, floor))


def test_covariance_is_the_camera_block_of_the_full_inverse():
    sc = ba_scene("tiny")
    P = oracle.Problem.from_scene(sc)
    P.solve(3)
    lam = 1e-2
    P.lam = lam
    cov = P.covariance()
    Hinv = np.linalg.inv(_full_damped_H(P, sc, lam))
    nc = len(sc["cams"])
    for j in range(nc):
        ref = Hinv[9 * j:9 * j + 9, 9 * j:9 * j + 9]
        np.testing.assert_allclose(cov[j], ref, rtol=1e-8, atol=1e-8 * np.abs(ref).max())


def test_large_lambda_limit_is_the_camera_block_inverse():
    sc = ba_scene("tiny")
    P = oracle.Problem.from_scene(sc)
    P.linearize()
    errs = []
    for lam in (1e3, 1e4):
        P.lam = lam
        cov = P.covariance()
        B = P.get("B")
        Bd = B + lam * np.maximum(np.diagonal(B, axis1=1, axis2=2), 1e-6)[:, None, :] * np.eye(9)
        ref = np.linalg.inv(Bd)
        errs.append(max(np.linalg.norm(c - r) / np.linalg.norm(r) for c, r in zip(cov, ref)))
    # the coupling enters at second order in 1/lambda: ten times lambda, a
    # hundredth of the difference (with slack for rounding)
    assert errs[0] < 1e-4 and errs[1] < 3e-2 * errs[0], errs


def test_blocks_are_spd_and_state_is_unchanged():
    sc = ba_scene("small")
    P = oracle.Problem.from_scene(sc)
    P.solve(2)
    cams, pts, lam, cost = P.get("cams"), P.get("points"), P.lam, P.cost
    cov = P.covariance()
    asym = [np.linalg.norm(c - c.T) / np.linalg.norm(c) for c in cov]
    assert max(asym) < 1e-12, max(asym)
    assert np.all(np.linalg.eigvalsh(0.5 * (cov + np.transpose(cov, (0, 2, 1)))) > 0)
    assert np.array_equal(P.get("cams"), cams) and np.array_equal(P.get("points"), pts)
    assert P.lam == lam and P.cost == cost
    # the next LM step is the one a fresh run takes
    Q = oracle.Problem.from_scene(sc)
    Q.solve(2)
    a, b = P.lm_step(), Q.lm_step()
    assert a == b
