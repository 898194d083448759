"""Seeded synthetic pose graphs (SE(3) poses, relative-pose measurements).

A pose is stored as 6 doubles ``[w0, w1, w2, t0, t1, t2]``: ``w`` the
axis-angle vector of the body-to-world rotation ``R`` and ``t`` the body origin
in the world, so a body point ``x`` sits at ``R x + t``.  An edge ``(i, j)``
measures the pose of ``j`` in the frame of ``i``, ``T_i^-1 T_j``: rotation
``R_i^T R_j`` and translation ``R_i^T (t_j - t_i)``, each drawn around the
truth with Gaussian noise, and carries the information weights of its
rotation and translation parts.

The layout imitates the sphere benchmarks named on the eager-mode BA summary
(sphere-a; and parking-garage: odometry chains plus loop closures): poses on
a sphere, ``n_rings`` latitude rings of ``per_ring`` poses each, visited ring
by ring; odometry edges join consecutive poses and loop-closure edges join
each pose to the pose below it on the previous ring.  Each pose faces along
its ring (x axis along the direction of travel, z outwards).

Configurations:

* ``tiny``   : 4 rings x 8 poses (32 poses, 55 edges).
* ``small``  : 10 x 20 (200 poses, 379 edges).
* ``sphere`` : 50 x 50 (2,500 poses, 4,949 edges), the size of the sphere
  benchmarks.
* ``medium`` : 100 x 100 (10,000 poses, 19,899 edges).
* ``large``  : 512 x 1024 (524,288 poses, 1,047,551 edges): as many poses as
  the batched pose-graph benchmark of the Theseus note holds in total (256
  graphs of 2,048 poses), here as one connected graph.

Every draw comes from ``numpy.random.Generator(PCG64(seed))``; the forward
model (composition of the true poses) is written on scipy's ``Rotation`` and
shares no code with either solver.
"""

import numpy as np
from scipy.spatial.transform import Rotation

PGO_CONFIGS = {
    "tiny": dict(n_rings=4, per_ring=8, seed=31, n_iters=10),
    "small": dict(n_rings=10, per_ring=20, seed=32, n_iters=15),
    "sphere": dict(n_rings=50, per_ring=50, seed=33, n_iters=20),
    "medium": dict(n_rings=100, per_ring=100, seed=35, n_iters=20),
    "large": dict(n_rings=512, per_ring=1024, seed=34, n_iters=20),
}

SPHERE_RADIUS = 10.0
SIGMA_T = 0.05       # measurement noise, translation (units)
SIGMA_R = 0.01       # measurement noise, rotation (rad)
INIT_T = 0.2         # initial error, translation (units)
INIT_R = 0.05        # initial error, rotation (rad)


def _true_poses(n_rings, per_ring):
    a, b = np.meshgrid(np.arange(n_rings), np.arange(per_ring), indexing="ij")
    lat = (np.pi * (a + 1) / (n_rings + 1) - np.pi / 2).ravel()
    lon = (2 * np.pi * b / per_ring).ravel()
    out = np.stack([np.cos(lat) * np.cos(lon), np.cos(lat) * np.sin(lon), np.sin(lat)], axis=1)
    east = np.stack([-np.sin(lon), np.cos(lon), np.zeros_like(lon)], axis=1)
    north = np.cross(out, east)
    R = np.stack([east, north, out], axis=2)   # columns: body axes in world
    return R, SPHERE_RADIUS * out


def _edges(n_rings, per_ring):
    n = n_rings * per_ring
    e = [(k, k + 1) for k in range(n - 1)]
    e += [(k - per_ring, k) for k in range(per_ring, n)]
    return np.array(e, dtype=np.int32)


def pgo_scene(config="tiny", seed=None, noise=1.0, init=1.0, **over):
    """Draw one pose graph.  Returns a dict with ``poses`` (initial values,
    n x 6), ``poses_true``, ``edges`` (m x 2 int32), ``meas`` (m x 6 measured
    relative poses, axis-angle and translation), ``info`` (m x 2: weights of
    the rotation and translation residuals), ``n_fixed`` (pose 0 is held) and
    the solver settings."""
    cfg = dict(PGO_CONFIGS[config])
    cfg.update(over)
    if seed is None:
        seed = cfg["seed"]
    rng = np.random.Generator(np.random.PCG64(seed))
    Rt, tt = _true_poses(cfg["n_rings"], cfg["per_ring"])
    n = len(Rt)
    E = _edges(cfg["n_rings"], cfg["per_ring"])
    m = len(E)
    rot = Rotation.from_matrix(Rt)
    i, j = E[:, 0], E[:, 1]
    rel_R = rot[i].inv() * rot[j]
    rel_t = rot[i].inv().apply(tt[j] - tt[i])
    nr = rng.normal(0.0, SIGMA_R * noise, size=(m, 3))
    nt = rng.normal(0.0, SIGMA_T * noise, size=(m, 3))
    meas_R = rel_R * Rotation.from_rotvec(nr)
    meas = np.concatenate([meas_R.as_rotvec(), rel_t + nt], axis=1)
    info = np.tile([1.0 / SIGMA_R ** 2, 1.0 / SIGMA_T ** 2], (m, 1))
    er = rng.normal(0.0, INIT_R * init, size=(n, 3))
    et = rng.normal(0.0, INIT_T * init, size=(n, 3))
    er[0] = 0.0
    et[0] = 0.0
    R0 = rot * Rotation.from_rotvec(er)
    poses = np.concatenate([R0.as_rotvec(), tt + et], axis=1)
    poses_true = np.concatenate([rot.as_rotvec(), tt], axis=1)
    return dict(poses=np.ascontiguousarray(poses), poses_true=np.ascontiguousarray(poses_true),
                edges=np.ascontiguousarray(E), meas=np.ascontiguousarray(meas),
                info=np.ascontiguousarray(info), n_fixed=1, n_iters=cfg["n_iters"],
                pcg_max_iters=200, pcg_rel_tol=1e-8, config=config, seed=seed)


def pgo_summary(sc):
    return f"pose graph {sc['config']}: {len(sc['poses'])} poses, {len(sc['edges'])} edges"
