"""Seeded synthetic dense (DROID-style) bundle-adjustment scenes, float32.

A ring of keyframes, each with a per-pixel inverse-depth map on a 48 x 64 grid,
and a frame graph whose edges ``(i, j)`` carry one 2-D target per pixel of frame
``i``: the position where that pixel should land in frame ``j``, plus a
confidence weight.  Poses are world-to-camera and stored as 7 floats
``[tx, ty, tz, qx, qy, qz, qw]``.

Settings: 16 keyframes with centres on a circle of radius 0.3 in the x-y plane,
small random yaw and pitch, looking along +z; pinhole intrinsics f = 50,
c = (31.5, 23.5); true inverse depth ~ U(0.2, 1.0); edges (i, i+k mod 16) for
k = 1..4 (64 edges); targets = true projection + N(0, 0.5^2) px; weights
~ U(0.1, 1); poses 2..15 perturbed by the exponential of a N(0, 0.01^2) twist,
inverse depths multiplied by exp(N(0, 0.1^2)).  The forward model used to
place the targets is written on scipy's ``Rotation`` and ``expm`` only.
"""

import numpy as np
from scipy.linalg import expm
from scipy.spatial.transform import Rotation

DROID = dict(n_frames=16, height=48, width=64, seed=5, fx=50.0, fy=50.0, cx=31.5, cy=23.5,
             ring=0.3, n_iters=8, n_fixed=2, hops=4)


def _twist_matrix(xi):
    rho, phi = xi[:3], xi[3:]
    M = np.zeros((4, 4))
    M[:3, :3] = np.array([[0, -phi[2], phi[1]], [phi[2], 0, -phi[0]], [-phi[1], phi[0], 0]])
    M[:3, 3] = rho
    return M


def _to_pose7(T):
    q = Rotation.from_matrix(T[:3, :3]).as_quat()       # x, y, z, w
    if q[3] < 0:
        q = -q
    return np.concatenate([T[:3, 3], q])


def _synth_pixels(Ti, Tj, ys, xs, inv_depth, K):
    """Synthesis-only: where pixel (x, y) of frame i with inverse depth lands in frame j."""
    fx, fy, cx, cy = K
    ray = np.stack([(xs - cx) / fx, (ys - cy) / fy, np.ones_like(xs)], axis=1)
    Xi = ray / inv_depth[:, None]
    Tij = Tj @ np.linalg.inv(Ti)
    Xj = Xi @ Tij[:3, :3].T + Tij[:3, 3]
    return np.stack([fx * Xj[:, 0] / Xj[:, 2] + cx, fy * Xj[:, 1] / Xj[:, 2] + cy], axis=1), Xj[:, 2]


def droid_scene(seed=None, noise_px=0.5, pose_sigma=0.01, depth_sigma=0.1, **over):
    cfg = dict(DROID)
    cfg.update(over)
    if seed is None:
        seed = cfg["seed"]
    rng = np.random.Generator(np.random.PCG64(seed))
    n, H, W = cfg["n_frames"], cfg["height"], cfg["width"]
    K = (cfg["fx"], cfg["fy"], cfg["cx"], cfg["cy"])

    T_true = np.empty((n, 4, 4))
    for i in range(n):
        a = 2.0 * np.pi * i / n
        c = cfg["ring"] * np.array([np.cos(a), np.sin(a), 0.0])
        yaw, pitch = rng.normal(0.0, 0.02, size=2)
        R = Rotation.from_euler("yx", [yaw, pitch]).as_matrix()
        T = np.eye(4)
        T[:3, :3] = R
        T[:3, 3] = -R @ c
        T_true[i] = T
    d_true = rng.uniform(0.2, 1.0, size=(n, H, W))

    edges = np.array([(i, (i + k) % n) for i in range(n) for k in range(1, cfg["hops"] + 1)],
                     dtype=np.int32)
    ys, xs = np.meshgrid(np.arange(H, dtype=float), np.arange(W, dtype=float), indexing="ij")
    ys, xs = ys.ravel(), xs.ravel()
    targets = np.empty((len(edges), H * W, 2))
    for e, (i, j) in enumerate(edges):
        uv, z = _synth_pixels(T_true[i], T_true[j], ys, xs, d_true[i].ravel(), K)
        assert z.min() > 0.1
        targets[e] = uv
    targets += rng.normal(0.0, noise_px, size=targets.shape)
    weights = rng.uniform(0.1, 1.0, size=(len(edges), H * W))

    T_init = T_true.copy()
    for i in range(cfg["n_fixed"], n):
        T_init[i] = expm(_twist_matrix(rng.normal(0.0, pose_sigma, size=6))) @ T_true[i]
    d_init = d_true * np.exp(rng.normal(0.0, depth_sigma, size=d_true.shape))

    f32 = np.float32
    return dict(
        poses=np.stack([_to_pose7(T) for T in T_init]).astype(f32),
        poses_true=np.stack([_to_pose7(T) for T in T_true]).astype(f32),
        inv_depth=d_init.reshape(n, H * W).astype(f32),
        inv_depth_true=d_true.reshape(n, H * W).astype(f32),
        intrinsics=np.array(K, dtype=f32), edges=edges,
        targets=targets.reshape(len(edges), H * W, 2).astype(f32),
        weights=weights.astype(f32), height=H, width=W,
        n_fixed=cfg["n_fixed"], n_iters=cfg["n_iters"], seed=seed,
    )
