"""The GPU PCG applies S to the preconditioned residual z and carries p and
q = S p by recurrence, with p.q from Chronopoulos and Gear's identity
p^T S p = z^T S z - beta^2 p_prev^T S p_prev.  Algebraically that is standard
PCG (the O7 reading of the Schur-complement solve on the BA pages); these
tests check, on the oracle's own reduced camera systems, that in fp64 it
stops at the same iteration as standard PCG and lands within the spread that
rounding noise alone gives standard PCG.  CPU only."""
import numpy as np
import pytest

import oracle
from synthetic import ba_scene


def _pcg(S, rhs, Minv, tol, maxit, form, rng=None):
    x = np.zeros_like(rhs)
    r = rhs.copy()
    z = Minv(r)
    rz, rhs_n = r @ z, np.linalg.norm(rhs)
    p = q = pq_prev = rz_prev = None
    hist = []
    for it in range(maxit):
        res = np.linalg.norm(r)
        hist.append(res / rhs_n)
        if it >= 1 and res <= tol * rhs_n:
            return it, x, np.array(hist)
        if form == "standard":
            p = z.copy() if it == 0 else z + (rz / rz_prev) * p
            q = S(p)
            if rng is not None:
                q = q * (1.0 + 1e-15 * rng.standard_normal(q.shape))
            pq = p @ q
        else:
            Sz = S(z)
            zSz = z @ Sz
            if it == 0:
                p, q, pq = z.copy(), Sz, zSz
            else:
                beta = rz / rz_prev
                pq = zSz - beta * beta * pq_prev
                p, q = z + beta * p, Sz + beta * q
        alpha = rz / pq
        x, r = x + alpha * p, r - alpha * q
        z = Minv(r)
        rz_prev, rz, pq_prev = rz, r @ z, pq
    return maxit, x, np.array(hist)


def _system(sc, lam_scale):
    P = oracle.Problem.from_scene(sc)
    P.linearize()
    P.lam = P.lam * lam_scale
    P.damp()
    P.schur()
    Mi = np.linalg.inv(P.get("M"))
    return P, P.get("rhs").ravel(), lambda v: np.einsum("jab,jb->ja", Mi, v.reshape(-1, 9)).ravel()


@pytest.mark.parametrize("config,lam_scale", [("tiny", 1.0), ("tiny", 1e-3), ("small", 1.0), ("small", 1e-3),
                                              ("medium", 1e-3)])
def test_recurrence_form_tracks_standard_pcg(config, lam_scale):
    sc = ba_scene(config)
    P, rhs, Minv = _system(sc, lam_scale)
    tol, maxit = sc["pcg_rel_tol"], sc["pcg_max_iters"]
    it0, x0, h0 = _pcg(P.schur_matvec, rhs, Minv, tol, maxit, "standard")
    it1, x1, h1 = _pcg(P.schur_matvec, rhs, Minv, tol, maxit, "recurrence")
    itn, xn, hn = _pcg(P.schur_matvec, rhs, Minv, tol, maxit, "standard", np.random.default_rng(7))
    assert it1 == it0 == itn
    n = len(h0)
    d_form = np.max(np.abs(h1[:n] - h0) / h0)
    d_noise = np.max(np.abs(hn[:n] - h0) / h0)
    dx_form = np.linalg.norm(x1 - x0) / np.linalg.norm(x0)
    dx_noise = np.linalg.norm(xn - x0) / np.linalg.norm(x0)
    # the variant stays within a few times the spread that 1e-15 noise in S p
    # gives standard PCG, or within plain fp64 rounding where that spread is tiny
    assert d_form <= max(10 * d_noise, 1e-9), (d_form, d_noise)
    assert dx_form <= max(10 * dx_noise, 1e-11), (dx_form, dx_noise)
    # and it solves the system as well as standard PCG does: on ill-conditioned
    # systems the true residual of both drifts above the recursive one
    def true_res(x):
        return np.linalg.norm(rhs - P.schur_matvec(x)) / np.linalg.norm(rhs)
    assert true_res(x1) <= max(1.01 * tol, 3 * max(true_res(x0), true_res(xn)))
