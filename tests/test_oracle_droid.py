"""Pins of the dense frame-graph BA oracle (fp64) against what the pages and
the mathematics fix, independently of the oracle's own formulas:

* the image model re-derived with scipy rotations and 4x4 matrix inverses
  (NeRF-SLAM reproduction notes, sec. 2.2),
* central finite differences of that independent model for every Jacobian,
* the SE(3) exponential against scipy's matrix exponential,
* H = J^T W J and b = -J^T W r against a dense numpy J (sec. 3.1),
* the Schur step against a dense solve of the full normal equations (sec. 3.2),
* the retraction against T <- expm(xi^) T,
* noise-free convergence to the true poses and depths.
"""
import numpy as np
import pytest
from scipy.linalg import expm
from scipy.spatial.transform import Rotation

from oracle import droid
from synthetic.droid import droid_scene


def hat6(xi):
    M = np.zeros((4, 4))
    p = xi[3:]
    M[:3, :3] = [[0, -p[2], p[1]], [p[2], 0, -p[0]], [-p[1], p[0], 0]]
    M[:3, 3] = xi[:3]
    return M


def mat_of(T12):
    T = np.eye(4)
    T[:3, :3] = np.asarray(T12[:9]).reshape(3, 3)
    T[:3, 3] = T12[9:]
    return T


def flat(T):
    return np.concatenate([T[:3, :3].ravel(), T[:3, 3]])


def pose7_to_mat(p):
    T = np.eye(4)
    T[:3, :3] = Rotation.from_quat(np.asarray(p[3:], dtype=np.float64)).as_matrix()
    T[:3, 3] = p[:3]
    return T


def model(Ti, Tj, K, xy, d, target):
    """Independent image model: back-project with 1/d, move by Tj Ti^-1, project."""
    fx, fy, cx, cy = K
    Xi = np.array([(xy[0] - cx) / fx, (xy[1] - cy) / fy, 1.0]) / max(d, 1e-6)
    Xj = (Tj @ np.linalg.inv(Ti) @ np.append(Xi, 1.0))[:3]
    z = max(Xj[2], 1e-6)
    return np.array([fx * Xj[0] / z + cx, fy * Xj[1] / z + cy]) - target


def random_pose(rng, rot=0.3, trans=0.5):
    T = np.eye(4)
    T[:3, :3] = Rotation.from_rotvec(rng.normal(0, rot, 3)).as_matrix()
    T[:3, 3] = rng.normal(0, trans, 3)
    return T


K = np.array([50.0, 52.0, 31.5, 23.5])


def test_residual_matches_independent_model():
    rng = np.random.default_rng(11)
    for _ in range(50):
        Ti, Tj = random_pose(rng, trans=0.1), random_pose(rng, trans=0.1)
        xy = rng.uniform([0, 0], [63, 47])
        d = rng.uniform(0.2, 1.0)
        tg = rng.uniform(0, 60, 2)
        out = droid.residual_one(flat(Ti), flat(Tj), K, xy, d, tg)
        ref = model(Ti, Tj, K, xy, d, tg)
        np.testing.assert_allclose(out["r"], ref, rtol=1e-12, atol=1e-10)
        assert not out["clamped"]


def test_hand_example():
    # identity poses: the pixel re-projects onto itself; a pure x-translation
    # of 0.1 with inverse depth 0.5 (depth 2) shifts it by fx * 0.1 / 2 = 2.5.
    I = flat(np.eye(4))
    out = droid.residual_one(I, I, K, [10.0, 20.0], 0.5, [10.0, 20.0])
    np.testing.assert_allclose(out["r"], [0.0, 0.0], atol=1e-13)
    Tj = np.eye(4)
    Tj[0, 3] = 0.1
    out = droid.residual_one(I, flat(Tj), K, [10.0, 20.0], 0.5, [10.0, 20.0])
    np.testing.assert_allclose(out["r"], [2.5, 0.0], atol=1e-12)
    # d/dd of the x shift fx * tx * d is fx * tx = 5
    np.testing.assert_allclose(out["Jd"], [5.0, 0.0], atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_jacobians_central_differences(seed):
    rng = np.random.default_rng(seed)
    h = 1e-6
    for _ in range(10):
        Ti, Tj = random_pose(rng, trans=0.1), random_pose(rng, trans=0.1)
        xy = rng.uniform([0, 0], [63, 47])
        d = rng.uniform(0.2, 1.0)
        tg = rng.uniform(0, 60, 2)
        out = droid.residual_one(flat(Ti), flat(Tj), K, xy, d, tg)
        Ji = np.empty((2, 6))
        Jj = np.empty((2, 6))
        for k in range(6):
            e = np.zeros(6)
            e[k] = h
            Ji[:, k] = (model(expm(hat6(e)) @ Ti, Tj, K, xy, d, tg)
                        - model(expm(hat6(-e)) @ Ti, Tj, K, xy, d, tg)) / (2 * h)
            Jj[:, k] = (model(Ti, expm(hat6(e)) @ Tj, K, xy, d, tg)
                        - model(Ti, expm(hat6(-e)) @ Tj, K, xy, d, tg)) / (2 * h)
        Jd = (model(Ti, Tj, K, xy, d + h, tg) - model(Ti, Tj, K, xy, d - h, tg)) / (2 * h)
        scale = max(np.abs(Ji).max(), np.abs(Jj).max(), 1.0)
        np.testing.assert_allclose(out["Ji"], Ji, atol=1e-6 * scale)
        np.testing.assert_allclose(out["Jj"], Jj, atol=1e-6 * scale)
        np.testing.assert_allclose(out["Jd"], Jd, atol=1e-6 * max(np.abs(Jd).max(), 1.0))


def test_clamps_zero_their_derivatives():
    I = flat(np.eye(4))
    # inverse depth below the floor: the point sits at depth 1e6 whatever d is
    out = droid.residual_one(I, I, K, [40.0, 30.0], 1e-9, [0.0, 0.0])
    assert out["clamped"]
    np.testing.assert_array_equal(out["Jd"], [0.0, 0.0])
    # point behind camera j: z clamped at 1e-6, no depth column in the projection
    Tj = np.eye(4)
    Tj[2, 3] = -5.0
    out = droid.residual_one(I, flat(Tj), K, [31.5, 23.5], 0.5, [0.0, 0.0])
    assert out["clamped"]
    np.testing.assert_array_equal(out["Jj"][:, 2], [0.0, 0.0])


@pytest.mark.parametrize("scale", [0.0, 1e-9, 1e-5, 3e-3, 0.02, 0.7, 3.0])
def test_se3_exp_matches_matrix_exponential(scale):
    rng = np.random.default_rng(int(scale * 1e9) % 1000)
    for _ in range(5):
        xi = np.concatenate([rng.normal(0, 1, 3), scale * rng.normal(0, 1, 3)])
        R, t = droid.se3_exp(xi)
        ref = expm(hat6(xi))
        np.testing.assert_allclose(R, ref[:3, :3], atol=1e-14)
        np.testing.assert_allclose(t, ref[:3, 3], atol=1e-13)


def small_problem(noise=0.5, seed=7):
    sc = droid_scene(seed=seed, n_frames=4, height=6, width=8, hops=2, cx=3.5, cy=2.5,
                     noise_px=noise)
    return sc, droid.DroidProblem.from_scene(sc)


def dense_system(P, sc):
    """Dense J (residual rows x [poses, depths]) and W from the oracle's blocks."""
    n, Pp, E = P.n, P.P, P.E
    Ji, Jj, Jd, r = P.get("Ji"), P.get("Jj"), P.get("Jd"), P.get("r")
    m = 2 * E * Pp
    J = np.zeros((m, 6 * n + n * Pp))
    for e, (i, j) in enumerate(sc["edges"]):
        for p in range(Pp):
            rows = slice(2 * (e * Pp + p), 2 * (e * Pp + p) + 2)
            J[rows, 6 * i:6 * i + 6] += Ji[e, p]
            J[rows, 6 * j:6 * j + 6] += Jj[e, p]
            J[rows, 6 * n + i * Pp + p] = Jd[e, p]
    w = np.repeat(sc["weights"].astype(np.float64).ravel(), 2)
    return J, w, r.ravel()


def test_assembly_against_dense_normal_equations():
    sc, P = small_problem()
    P.gn_step()  # linearises at the initial parameters, then moves them
    J, w, r = dense_system(P, sc)
    H = J.T @ (w[:, None] * J)
    g = J.T @ (w * r)
    n6 = 6 * P.n
    np.testing.assert_allclose(P.get("B"), H[:n6, :n6], rtol=1e-12, atol=1e-12 * abs(H).max())
    np.testing.assert_allclose(P.get("gc"), g[:n6], rtol=1e-12, atol=1e-12 * abs(g).max())
    np.testing.assert_allclose(P.get("C").ravel(), np.diag(H)[n6:], rtol=1e-12)
    np.testing.assert_allclose(P.get("gd").ravel(), g[n6:], rtol=1e-12,
                               atol=1e-12 * abs(g).max())
    # the depth block is diagonal: each depth only enters residuals of its own frame
    Hdd = H[n6:, n6:]
    assert np.count_nonzero(Hdd - np.diag(np.diag(Hdd))) == 0


def test_schur_step_equals_dense_solve():
    sc, P = small_problem()
    P.gn_step()
    J, w, r = dense_system(P, sc)
    nf, n6 = P.n_fixed, 6 * P.n
    free = np.r_[6 * nf:n6, n6:J.shape[1]]
    Jf = J[:, free]
    H = Jf.T @ (w[:, None] * Jf)
    b = -Jf.T @ (w * r)
    x = np.linalg.solve(H, b)
    nv = n6 - 6 * nf
    dxi = P.get("dxi")
    np.testing.assert_array_equal(dxi[:nf], 0.0)
    np.testing.assert_allclose(dxi[nf:].ravel(), x[:nv], rtol=1e-9, atol=1e-11 * abs(x).max())
    np.testing.assert_allclose(P.get("dd").ravel(), x[nv:], rtol=1e-9,
                               atol=1e-11 * abs(x).max())
    # the reduced matrix is the Schur complement of the depth block
    Hcc, Hcd, Hdd = H[:nv, :nv], H[:nv, nv:], np.diag(H[nv:, nv:])
    S = Hcc - (Hcd / Hdd) @ Hcd.T
    np.testing.assert_allclose(P.get("S"), S, rtol=1e-10, atol=1e-12 * abs(S).max())
    np.testing.assert_allclose(P.get("rhs"), b[:nv] - (Hcd / Hdd) @ b[nv:], rtol=1e-10,
                               atol=1e-12 * abs(b).max())


def test_retraction_is_left_exponential():
    sc, P = small_problem()
    T0 = [mat_of(P.pose_matrix(i)) for i in range(P.n)]
    d0 = P.get("depth")
    P.gn_step()
    dxi, dd = P.get("dxi"), P.get("dd")
    for i in range(P.n):
        np.testing.assert_allclose(mat_of(P.pose_matrix(i)), expm(hat6(dxi[i])) @ T0[i],
                                   atol=1e-13)
    np.testing.assert_allclose(P.get("depth"), d0 + dd, rtol=1e-15)


def test_pose_readback_matches_input():
    sc, P = small_problem()
    out = P.get("poses")
    for i in range(P.n):
        np.testing.assert_allclose(pose7_to_mat(out[i]), pose7_to_mat(sc["poses"][i]),
                                   atol=1e-7)
        assert out[i, 6] >= 0


def test_cost_matches_independent_model():
    sc, P = small_problem()
    Kc = sc["intrinsics"].astype(np.float64)
    T = [pose7_to_mat(p.astype(np.float64)) for p in sc["poses"]]
    s = 0.0
    for e, (i, j) in enumerate(sc["edges"]):
        for p in range(P.P):
            xy = (p % P.W, p // P.W)
            r = model(T[i], T[j], Kc, xy, float(sc["inv_depth"][i, p]),
                      sc["targets"][e, p].astype(np.float64))
            s += 0.5 * float(sc["weights"][e, p]) * (r @ r)
    # float32 quaternions are renormalised the same way on both sides
    assert abs(P.cost() - s) <= 1e-9 * s


def test_noise_free_converges_to_truth():
    sc = droid_scene(noise_px=0.0)
    P = droid.DroidProblem.from_scene(sc)
    c0 = P.cost()
    for _ in range(sc["n_iters"]):
        P.gn_step()
    # targets are float32: the floor is their rounding, far below 1e-10 C0
    assert P.cost() < 1e-10 * c0
    est = P.get("poses")
    for i in range(P.n):
        Te, Tt = pose7_to_mat(est[i]), pose7_to_mat(sc["poses_true"][i].astype(np.float64))
        assert np.abs(Te - Tt).max() < 1e-5
    np.testing.assert_allclose(P.get("depth"), sc["inv_depth_true"], rtol=1e-4)


def test_noisy_converges_below_truth_and_fixed_poses_stay():
    sc = droid_scene(n_frames=6, height=12, width=16, hops=3, cx=7.5, cy=5.5)
    P = droid.DroidProblem.from_scene(sc)
    p0 = P.get("poses")
    costs = [P.gn_step() for _ in range(sc["n_iters"])]
    for c0, c1 in costs:
        assert c1 <= c0 * (1 + 1e-12)
    tr = dict(sc, poses=sc["poses_true"], inv_depth=sc["inv_depth_true"])
    assert P.cost() < droid.DroidProblem.from_scene(tr).cost()
    np.testing.assert_array_equal(P.get("poses")[:2], p0[:2])


def test_invalid_inputs_rejected():
    sc = droid_scene(n_frames=4, height=6, width=8, hops=2, cx=3.5, cy=2.5)
    bad = sc["edges"].copy()
    bad[0, 1] = 4
    with pytest.raises(RuntimeError):
        droid.DroidProblem(sc["poses"], sc["inv_depth"], sc["intrinsics"], bad, sc["targets"],
                           sc["weights"], 6, 8, 2)
    with pytest.raises(RuntimeError):
        droid.DroidProblem(sc["poses"], sc["inv_depth"], sc["intrinsics"], sc["edges"],
                           sc["targets"], sc["weights"], 6, 8, 5)


def test_covariance_is_pose_block_of_inverse_normal_matrix():
    """The pose covariance is the free-pose block of the inverse of the full
    normal matrix (block inversion: that block is the inverse of the Schur
    complement of the depths); it is symmetric positive definite."""
    sc, P = small_problem()
    cov = P.covariance()
    J, w, r = dense_system(P, sc)
    nf, n6 = P.n_fixed, 6 * P.n
    free = np.r_[6 * nf:n6, n6:J.shape[1]]
    Jf = J[:, free]
    H = Jf.T @ (w[:, None] * Jf)
    nv = n6 - 6 * nf
    ref = np.linalg.inv(H)[:nv, :nv]
    np.testing.assert_allclose(cov, ref, rtol=1e-8, atol=1e-10 * abs(ref).max())
    np.testing.assert_allclose(cov, cov.T, rtol=0, atol=1e-12 * abs(cov).max())
    assert np.linalg.eigvalsh(cov).min() > 0
    # covariance times the reduced matrix is the identity
    np.testing.assert_allclose(cov @ P.get("S"), np.eye(nv), atol=1e-8)
