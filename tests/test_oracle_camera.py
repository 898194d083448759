"""Pins for the oracle's per-observation model: SO(3) maps, projection,
Jacobians, robust kernel and camera retraction.

Each pin checks the oracle against something other than itself: scipy's
Rotation (a library routine), hand-computed numbers, the generator's
independent image model, central finite differences and closed forms.
"""
import numpy as np
import pytest
from scipy.spatial.transform import Rotation

import oracle
from synthetic import ba_scene
from synthetic.ba import image_model


def _rand_rotvecs(rng, n, max_angle=np.pi):
    axis = rng.normal(size=(n, 3))
    axis /= np.linalg.norm(axis, axis=1, keepdims=True)
    ang = rng.uniform(0.0, max_angle, size=n)
    return axis * ang[:, None]


def test_so3_exp_matches_scipy():
    rng = np.random.default_rng(0)
    ws = np.concatenate([_rand_rotvecs(rng, 200), _rand_rotvecs(rng, 50, 1e-6),
                         np.array([[0, 0, 0], [1e-9, -2e-9, 3e-9], [np.pi - 1e-9, 0, 0]])])
    for w in ws:
        R = oracle.so3_exp(w)
        np.testing.assert_allclose(R, Rotation.from_rotvec(w).as_matrix(), atol=2e-15, rtol=0)
        np.testing.assert_allclose(R.T @ R, np.eye(3), atol=2e-15)
        assert abs(np.linalg.det(R) - 1.0) < 2e-15


def test_so3_exp_small_angle_branch_is_continuous():
    w = np.array([0.3, -0.4, 0.5])
    w = w / np.linalg.norm(w)
    a = oracle.so3_exp(w * 1e-8 * (1 - 1e-9))
    b = oracle.so3_exp(w * 1e-8 * (1 + 1e-9))
    np.testing.assert_allclose(a, b, atol=1e-15)


def test_projection_hand_example():
    # Identity rotation, t = 0, f = 500, k1 = 0.1, k2 = 0.2, X = (1, 2, 10):
    # p = (0.1, 0.2), n = 0.05, s = 1 + 0.005 + 0.0005 = 1.0055,
    # u = 500 * 1.0055 * (0.1, 0.2) = (50.275, 100.55).
    cam = np.array([0, 0, 0, 0, 0, 0, 500.0, 0.1, 0.2])
    out = oracle.project_one(cam, [1.0, 2.0, 10.0], [0.0, 0.0])
    np.testing.assert_allclose(out["r"], [50.275, 100.55], rtol=1e-14)
    # Residual is predicted minus observed.
    out = oracle.project_one(cam, [1.0, 2.0, 10.0], [50.0, 100.0])
    np.testing.assert_allclose(out["r"], [0.275, 0.55], rtol=1e-12)
    # Translation moves the point in the camera frame: t = (0, 0, 10) doubles the depth.
    cam2 = cam.copy()
    cam2[3:6] = [0, 0, 10.0]
    out = oracle.project_one(cam2, [2.0, 4.0, 10.0], [0.0, 0.0])
    np.testing.assert_allclose(out["r"], [50.275, 100.55], rtol=1e-14)


def test_projection_matches_independent_image_model():
    sc = ba_scene("small", noise_px=0.0)
    cams, pts = sc["cams_true"], sc["points_true"]
    rots = Rotation.from_rotvec(cams[:, :3])
    idx = np.arange(0, len(sc["obs_cam"]), 37)
    oc, op = sc["obs_cam"][idx], sc["obs_pt"][idx]
    uv, _ = image_model(rots[oc], cams[oc, 3:6], cams[oc, 6], cams[oc, 7], cams[oc, 8], pts[op])
    for n, (j, i) in enumerate(zip(oc, op)):
        out = oracle.project_one(cams[j], pts[i], uv[n])
        assert np.all(np.abs(out["r"]) < 1e-9)


def _perturb(cam, X, col, h):
    cam = cam.copy()
    X = X.copy()
    if col < 3:
        e = np.zeros(3)
        e[col] = h
        cam[:3] = (Rotation.from_rotvec(e) * Rotation.from_rotvec(cam[:3])).as_rotvec()
    elif col < 9:
        cam[col] += h
    else:
        X[col - 9] += h
    return cam, X


def _fd_jacobian(cam, X, uv):
    J = np.empty((2, 12))
    for col in range(12):
        ref = np.abs(cam[col]) if 3 <= col < 9 else (np.abs(X[col - 9]) if col >= 9 else 1.0)
        h = 1e-6 * max(1.0, ref)
        cp, Xp = _perturb(cam, X, col, h)
        cm, Xm = _perturb(cam, X, col, -h)
        rp = oracle.project_one(cp, Xp, uv)["r"]
        rm = oracle.project_one(cm, Xm, uv)["r"]
        J[:, col] = (rp - rm) / (2 * h)
    return J


def _check_fd(cam, X, uv, tol=1e-6):
    out = oracle.project_one(cam, X, uv)
    J = np.concatenate([out["Jc"], out["Jp"]], axis=1)
    Jfd = _fd_jacobian(cam, X, uv)
    scale = np.abs(J).max()
    err = np.abs(J - Jfd).max() / scale
    assert err < tol, (err, J, Jfd)


def test_jacobians_match_central_differences_on_tiny():
    sc = ba_scene("tiny")
    for k in range(len(sc["obs_cam"])):
        j, i = sc["obs_cam"][k], sc["obs_pt"][k]
        _check_fd(sc["cams"][j], sc["points"][i], sc["obs_uv"][k])


def test_jacobians_with_strong_distortion_and_large_rotations():
    rng = np.random.default_rng(3)
    for _ in range(200):
        w = _rand_rotvecs(rng, 1)[0]
        R = Rotation.from_rotvec(w).as_matrix()
        Pc = np.array([rng.uniform(-3, 3), rng.uniform(-3, 3), rng.uniform(2, 8)])
        t = rng.normal(size=3)
        X = R.T @ (Pc - t)
        cam = np.concatenate([w, t, [rng.uniform(300, 800), rng.normal(0, 0.2), rng.normal(0, 0.2)]])
        _check_fd(cam, X, rng.normal(0, 50, size=2))


def test_depth_clamp_branch():
    # A point behind the camera: depth clamped at 1e-6, so du/dP_z is zero.
    cam = np.array([0, 0, 0, 0, 0, 0, 500.0, 0.0, 0.0])
    out = oracle.project_one(cam, [1e-7, 2e-7, -1.0], [0.0, 0.0])
    assert out["clamped"]
    np.testing.assert_allclose(out["r"], [500 * 0.1, 500 * 0.2], rtol=1e-12)
    assert out["Jp"][0, 2] == 0.0 and out["Jp"][1, 2] == 0.0
    assert out["Jc"][0, 5] == 0.0 and out["Jc"][1, 5] == 0.0


def test_huber_weight_and_cost():
    cam = np.array([0, 0, 0, 0, 0, 0, 500.0, 0.0, 0.0])
    X = np.array([0.0, 0.0, 10.0])
    # Residual (3, 4): norm 5 > delta 2 -> rho = 2 (5 - 1) = 8, w = 2 / 5.
    out = oracle.project_one(cam, X, [-3.0, -4.0], loss=1, delta=2.0)
    np.testing.assert_allclose(out["r"], [3.0, 4.0], rtol=1e-15)
    assert out["rho"] == pytest.approx(8.0, rel=1e-15)
    assert out["w"] == pytest.approx(0.4, rel=1e-15)
    # Inside the quadratic zone: norm 1 -> rho = 0.5, w = 1.
    out = oracle.project_one(cam, X, [-0.6, -0.8], loss=1, delta=2.0)
    assert out["rho"] == pytest.approx(0.5, rel=1e-14) and out["w"] == 1.0
    # Continuity at e = delta.
    a = oracle.project_one(cam, X, [-2.0 * 0.6, -2.0 * 0.8], loss=1, delta=2.0)
    b = oracle.project_one(cam, X, [-2.0 * 0.6 * (1 + 1e-12), -2.0 * 0.8 * (1 + 1e-12)], loss=1,
                           delta=2.0)
    assert abs(a["rho"] - b["rho"]) < 1e-10 and abs(a["w"] - b["w"]) < 1e-10
    # delta -> infinity reduces Huber to squared loss exactly.
    for uv in ([-30.0, 7.0], [1.0, 2.0]):
        h = oracle.project_one(cam, X, uv, loss=1, delta=1e300)
        s = oracle.project_one(cam, X, uv, loss=0)
        assert h["rho"] == s["rho"] and h["w"] == s["w"] == 1.0


def test_gradient_matches_finite_difference_of_cost():
    """g = sum w J^T r is the exact gradient of sum rho (Huber included)."""
    sc = ba_scene("tiny", outlier_frac=0.1)
    P = oracle.Problem.from_scene(sc, loss=1, huber_delta=2.0)
    P.linearize()
    gc, gp = P.get("gc"), P.get("gp")
    cams, pts = sc["cams"], sc["points"]
    rng = np.random.default_rng(5)
    for _ in range(12):
        j = rng.integers(len(cams))
        col = rng.integers(9)
        h = 1e-6 * (max(1.0, abs(cams[j, col])) if col >= 3 else 1.0)
        cp, cm = cams.copy(), cams.copy()
        cp[j], _ = _perturb(cams[j], np.zeros(3), col, h)
        cm[j], _ = _perturb(cams[j], np.zeros(3), col, -h)
        fd = (P.cost_at(cp, pts) - P.cost_at(cm, pts)) / (2 * h)
        assert abs(fd - gc[j, col]) <= 1e-6 * max(1.0, abs(gc[j, col])), (j, col, fd, gc[j, col])
    for _ in range(12):
        i = rng.integers(len(pts))
        col = rng.integers(3)
        h = 1e-6 * max(1.0, abs(pts[i, col]))
        pp, pm = pts.copy(), pts.copy()
        pp[i, col] += h
        pm[i, col] -= h
        fd = (P.cost_at(cams, pp) - P.cost_at(cams, pm)) / (2 * h)
        assert abs(fd - gp[i, col]) <= 1e-6 * max(1.0, abs(gp[i, col]))


def test_retraction_matches_rotation_composition():
    rng = np.random.default_rng(7)
    ws = np.concatenate([_rand_rotvecs(rng, 100), _rand_rotvecs(rng, 20, 1e-9),
                         _rand_rotvecs(rng, 20) * 0 + np.array([np.pi - 1e-7, 0, 0])])
    for w in ws:
        d = rng.normal(0, 0.3, size=9)
        cam = np.concatenate([w, rng.normal(size=3), [500.0, 0.01, -0.01]])
        out = oracle.retract_camera(cam, d)
        Rexp = (Rotation.from_rotvec(d[:3]) * Rotation.from_rotvec(w)).as_matrix()
        np.testing.assert_allclose(Rotation.from_rotvec(out[:3]).as_matrix(), Rexp, atol=5e-15)
        assert np.linalg.norm(out[:3]) <= np.pi + 1e-12
        np.testing.assert_array_equal(out[3:], cam[3:] + d[3:])
    # A zero step is the identity on the parameters (up to the Exp/Log round trip).
    cam = np.concatenate([_rand_rotvecs(rng, 1)[0], rng.normal(size=6)])
    out = oracle.retract_camera(cam, np.zeros(9))
    np.testing.assert_allclose(out[:3], cam[:3], atol=1e-14)
