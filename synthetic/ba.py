"""Seeded synthetic bundle-adjustment scenes (9-parameter cameras, 3-D points).

Camera parameters are stored as 9 doubles per camera:
``[w0, w1, w2, t0, t1, t2, f, k1, k2]`` with ``w`` the axis-angle vector of the
world-to-camera rotation ``R`` (a point ``X`` maps to ``P = R X + t``), ``f`` the
focal length in pixels and ``k1, k2`` the radial distortion coefficients applied
to the normalised image coordinates.  The principal point is 0.

The forward image model used to synthesise observations is: ``p = P_xy / P_z``,
``n = |p|^2``, ``u = f (1 + k1 n + k2 n^2) p``.  It is written on scipy's
``Rotation`` so that it shares no code with either solver.

Configurations (sizes from the workload list of the task):

* ``tiny``   : 10 ring cameras, 200 points, 4 distinct cameras per point (800
  observations), 1 px noise, squared loss, 10 LM iterations.
* ``small``  : 50 ring cameras, 8,000 points, track length 2 + Binomial(6, 1/3)
  (about 32,000 observations), 1 px noise, 20 LM iterations.
* ``medium`` : 250 cameras on a random-walk trajectory, 60,000 points spawned in
  the view of an anchor camera, visibility by a view frustum, 3-12 views per
  point (about 300,000 observations), 1 px noise, 2 % outliers, Huber 2 px;
  the initial rotation error turns each camera about its own centre.
* ``large``  : 1,000 ring cameras, 400,000 points, power-law track lengths on
  {2..50} with exponent 2.02 (about 2.2 M observations), 1 px noise, 5 %
  outliers, Huber 2 px, 30 LM iterations.
* ``wide``   : as ``large`` with 1,500 ring cameras and 90,000 points (about
  500,000 observations), 20 LM iterations.

``heavy_camera_scene`` adds to a ring scene one camera that sees thousands of
points of one contiguous index range (a camera far busier than the rest).

Every draw comes from ``numpy.random.Generator(PCG64(seed))``.
"""

import numpy as np
from scipy.spatial.transform import Rotation

CONFIGS = {
    "tiny": dict(n_cams=10, n_pts=200, seed=1, layout="ring", tracks="fixed4",
                 outlier_frac=0.0, loss="squared", huber_delta=2.0, n_iters=10,
                 pcg_max_iters=50, pcg_rel_tol=1e-6),
    "small": dict(n_cams=50, n_pts=8000, seed=2, layout="ring", tracks="binom",
                  outlier_frac=0.0, loss="squared", huber_delta=2.0, n_iters=20,
                  pcg_max_iters=50, pcg_rel_tol=1e-6),
    "medium": dict(n_cams=250, n_pts=60000, seed=3, layout="walk", tracks="frustum",
                   outlier_frac=0.02, loss="huber", huber_delta=2.0, n_iters=20,
                   pcg_max_iters=50, pcg_rel_tol=1e-6),
    "large": dict(n_cams=1000, n_pts=400000, seed=4, layout="ring", tracks="powerlaw",
                  outlier_frac=0.05, loss="huber", huber_delta=2.0, n_iters=30,
                  pcg_max_iters=50, pcg_rel_tol=1e-6),
    # more cameras than whole per-camera rows of the point passes fit in one
    # compute unit's LDS (the library then reads the camera data from memory)
    "wide": dict(n_cams=1500, n_pts=90000, seed=6, layout="ring", tracks="powerlaw",
                 outlier_frac=0.05, loss="huber", huber_delta=2.0, n_iters=20,
                 pcg_max_iters=50, pcg_rel_tol=1e-6),
}

RING_RADIUS = 20.0      # ring cameras sit 20 units from the centre of the point box
BOX_HALF = 5.0          # points fill a 10 x 10 x 10 box around the origin
IMG_HALF = (320.0, 240.0)   # 640 x 480 image for the frustum test
WALK_STEP = 4.3         # forward step of the random-walk trajectory
WALK_NEAR, WALK_FAR = 0.5, 30.0


def _look_at(center, target, up=(0.0, 1.0, 0.0)):
    """World-to-camera rotation whose optical (+z) axis points at ``target``."""
    z = np.asarray(target, float) - np.asarray(center, float)
    z /= np.linalg.norm(z)
    x = np.cross(z, np.asarray(up, float))
    x /= np.linalg.norm(x)
    y = np.cross(z, x)
    return np.stack([x, y, z])          # rows are the camera axes in world frame


def image_model(rot, t, f, k1, k2, X):
    """Synthesis-only forward model: pixel coordinates and camera-frame depth.

    ``rot`` is a scipy Rotation holding one rotation per row of ``X``.
    """
    P = rot.apply(X) + t
    p = P[:, :2] / P[:, 2:3]
    n = np.sum(p * p, axis=1, keepdims=True)
    s = 1.0 + k1[:, None] * n + k2[:, None] * n * n
    return f[:, None] * s * p, P[:, 2]


def _ring_cameras(rng, n_cams):
    ang = 2.0 * np.pi * np.arange(n_cams) / n_cams
    centers = np.stack([RING_RADIUS * np.cos(ang), np.zeros(n_cams),
                        RING_RADIUS * np.sin(ang)], axis=1)
    R = np.stack([_look_at(c, (0.0, 0.0, 0.0)) for c in centers])
    return R, centers


def _walk_cameras(rng, n_cams):
    R = np.empty((n_cams, 3, 3))
    centers = np.empty((n_cams, 3))
    c = np.zeros(3)
    yaw = 0.0
    for j in range(n_cams):
        heading = np.array([np.sin(yaw), 0.0, np.cos(yaw)])
        base = _look_at(c, c + heading)
        pitch, roll = rng.normal(0.0, 0.01, size=2)
        tilt = Rotation.from_euler("xz", [pitch, roll]).as_matrix()
        R[j] = tilt @ base
        centers[j] = c
        c = c + heading * WALK_STEP + rng.normal(0.0, 0.05, size=3)
        yaw += rng.normal(0.0, 0.03)
    return R, centers


def _distinct_cameras(rng, n_cams, lengths):
    """For each point, ``lengths[i]`` distinct cameras drawn uniformly."""
    n_pts = len(lengths)
    maxlen = int(lengths.max())
    width = max(2 * maxlen, 16)
    out = np.empty((n_pts, maxlen), dtype=np.int64)
    todo = np.arange(n_pts)
    while len(todo):
        cand = rng.integers(0, n_cams, size=(len(todo), width))
        order = np.argsort(cand, axis=1, kind="stable")
        srt = np.take_along_axis(cand, order, axis=1)
        dup_sorted = np.zeros_like(srt, dtype=bool)
        dup_sorted[:, 1:] = srt[:, 1:] == srt[:, :-1]
        dup = np.zeros_like(dup_sorted)
        np.put_along_axis(dup, order, dup_sorted, axis=1)
        keep = ~dup
        rank = np.cumsum(keep, axis=1)
        ok = rank[:, -1] >= lengths[todo]
        for row in np.nonzero(ok)[0]:
            i = todo[row]
            cams = cand[row][keep[row]][: lengths[i]]
            out[i, : lengths[i]] = cams
        todo = todo[~ok]
    return out


def _track_lengths(rng, kind, n_pts, n_cams):
    if kind == "fixed4":
        return np.full(n_pts, 4, dtype=np.int64)
    if kind == "binom":
        return 2 + rng.binomial(6, 1.0 / 3.0, size=n_pts)
    if kind == "powerlaw":
        L = np.arange(2, 51)
        p = L.astype(float) ** -2.02
        p /= p.sum()
        return rng.choice(L, size=n_pts, p=p)
    raise ValueError(kind)


def _frustum_tracks(rng, R, t, f, k1, k2, n_pts):
    """Spawn points in anchor views and keep the cameras whose frustum holds them."""
    n_cams = len(R)
    rots = Rotation.from_matrix(R)
    X = np.empty((n_pts, 3))
    tracks = []
    todo = np.arange(n_pts)
    while len(todo):
        m = len(todo)
        anchor = rng.integers(0, n_cams, size=m)
        pix = rng.uniform(-1.0, 1.0, size=(m, 2)) * np.array(IMG_HALF)
        depth = rng.uniform(3.0, 25.0, size=m)
        pc = np.concatenate([pix / f[anchor, None] * depth[:, None], depth[:, None]], axis=1)
        Xw = rots[anchor].inv().apply(pc - t[anchor])
        vis = np.zeros((m, n_cams), dtype=bool)
        for j in range(n_cams):
            jj = np.full(m, j)
            u, z = image_model(rots[jj], t[jj], f[jj], k1[jj], k2[jj], Xw)
            vis[:, j] = ((z > WALK_NEAR) & (z < WALK_FAR)
                         & (np.abs(u[:, 0]) <= IMG_HALF[0]) & (np.abs(u[:, 1]) <= IMG_HALF[1]))
        vis[np.arange(m), anchor] = True
        cnt = vis.sum(axis=1)
        ok = cnt >= 3
        for row in np.nonzero(ok)[0]:
            i = todo[row]
            cams = np.nonzero(vis[row])[0]
            if len(cams) > 12:
                others = cams[cams != anchor[row]]
                pick = rng.choice(others, size=11, replace=False)
                cams = np.concatenate([[anchor[row]], pick])
            X[i] = Xw[row]
            tracks.append((i, cams))
        todo = todo[~ok]
    tracks.sort(key=lambda e: e[0])
    return X, [c for _, c in tracks]


def ba_scene(config="tiny", seed=None, noise_px=1.0, outlier_frac=None,
             rot_sigma=0.01, trans_sigma=0.01, point_sigma=0.1, shuffle=True, **over):
    """Draw one scene.  Returns a dict of numpy arrays plus solver settings.

    ``cams``/``points`` are the perturbed initial values, ``cams_true`` and
    ``points_true`` the ground truth, ``obs_cam``/``obs_pt`` int32 indices and
    ``obs_uv`` the (N, 2) observed pixels.
    """
    cfg = dict(CONFIGS[config])
    cfg.update(over)
    if seed is None:
        seed = cfg["seed"]
    if outlier_frac is None:
        outlier_frac = cfg["outlier_frac"]
    rng = np.random.Generator(np.random.PCG64(seed))
    n_cams, n_pts = cfg["n_cams"], cfg["n_pts"]

    if cfg["layout"] == "ring":
        R, centers = _ring_cameras(rng, n_cams)
    else:
        R, centers = _walk_cameras(rng, n_cams)
    t_true = -np.einsum("nij,nj->ni", R, centers)
    f = rng.uniform(400.0, 600.0, size=n_cams)
    k1 = rng.normal(0.0, 1e-3, size=n_cams)
    k2 = rng.normal(0.0, 1e-3, size=n_cams)

    if cfg["tracks"] == "frustum":
        X_true, tracks = _frustum_tracks(rng, R, t_true, f, k1, k2, n_pts)
        lengths = np.array([len(c) for c in tracks])
        obs_cam = np.concatenate(tracks)
    else:
        X_true = rng.uniform(-BOX_HALF, BOX_HALF, size=(n_pts, 3))
        lengths = _track_lengths(rng, cfg["tracks"], n_pts, n_cams)
        cams = _distinct_cameras(rng, n_cams, lengths)
        mask = np.arange(cams.shape[1])[None, :] < lengths[:, None]
        obs_cam = cams[mask]
    obs_pt = np.repeat(np.arange(n_pts), lengths)
    n_obs = len(obs_cam)

    rots = Rotation.from_matrix(R)
    uv_true, depth = image_model(rots[obs_cam], t_true[obs_cam], f[obs_cam],
                                 k1[obs_cam], k2[obs_cam], X_true[obs_pt])
    assert depth.min() > 0.5
    noise = rng.normal(0.0, 1.0, size=(n_obs, 2)) * noise_px
    if outlier_frac > 0:
        is_out = rng.random(n_obs) < outlier_frac
        outl = rng.uniform(-50.0, 50.0, size=(n_obs, 2))
        noise = np.where(is_out[:, None], outl, noise)
    else:
        is_out = np.zeros(n_obs, dtype=bool)
    obs_uv = uv_true + noise

    w_true = rots.as_rotvec()
    eps = rng.normal(0.0, rot_sigma, size=(n_cams, 3))
    w_init = (Rotation.from_rotvec(eps) * rots).as_rotvec()
    t_init = t_true + rng.normal(0.0, trans_sigma, size=(n_cams, 3))
    if cfg["layout"] == "walk":
        # The walk runs hundreds of units from the origin; turning R about the
        # origin with t held would move each camera centre by eps |centre|
        # (about 10 units) and put near points behind it.  Turn the camera
        # about its own centre instead (t carried along), so the depth clamp
        # never fires at the initial values.
        t_init = Rotation.from_rotvec(eps).apply(t_true) + (t_init - t_true)
    X_init = X_true + rng.normal(0.0, point_sigma, size=(n_pts, 3))

    cams_true = np.concatenate([w_true, t_true, f[:, None], k1[:, None], k2[:, None]], axis=1)
    cams_init = np.concatenate([w_init, t_init, f[:, None], k1[:, None], k2[:, None]], axis=1)

    if shuffle:
        order = rng.permutation(n_obs)
        obs_cam, obs_pt, obs_uv, is_out = obs_cam[order], obs_pt[order], obs_uv[order], is_out[order]

    return dict(
        cams=np.ascontiguousarray(cams_init), points=np.ascontiguousarray(X_init),
        cams_true=np.ascontiguousarray(cams_true), points_true=np.ascontiguousarray(X_true),
        obs_cam=np.ascontiguousarray(obs_cam, dtype=np.int32),
        obs_pt=np.ascontiguousarray(obs_pt, dtype=np.int32),
        obs_uv=np.ascontiguousarray(obs_uv), is_outlier=is_out,
        loss=cfg["loss"], huber_delta=cfg["huber_delta"], n_iters=cfg["n_iters"],
        pcg_max_iters=cfg["pcg_max_iters"], pcg_rel_tol=cfg["pcg_rel_tol"],
        config=config, seed=seed,
    )


def scene_summary(sc):
    n_c, n_p, n_o = len(sc["cams"]), len(sc["points"]), len(sc["obs_cam"])
    return f"{sc['config']}: {n_c} cameras, {n_p} points, {n_o} observations"


def heavy_camera_scene(n_extra=3000, camera=0, config="small", n_pts=12000, seed=None,
                       loss="huber", outlier_frac=0.02):
    """A ring scene in which camera ``camera`` additionally observes points
    0 .. n_extra - 1 (one observation each, synthesised like the others: the
    true projection plus 1 px noise, ``outlier_frac`` of them replaced by
    uniform +-50 px outliers).  With ``n_pts`` = 12,000 those points fill the
    lowest quarter of the point indices, so the camera holds about 3,200
    observations of points in that quarter."""
    sc = ba_scene(config, seed=seed, n_pts=n_pts, outlier_frac=outlier_frac)
    rng = np.random.Generator(np.random.PCG64(1000 + sc["seed"]))
    ct, Xt = sc["cams_true"], sc["points_true"]
    pts = np.arange(n_extra)
    cam = np.full(n_extra, camera)
    rots = Rotation.from_rotvec(ct[cam, 0:3])
    uv, depth = image_model(rots, ct[cam, 3:6], ct[cam, 6], ct[cam, 7], ct[cam, 8], Xt[pts])
    assert depth.min() > 0.5
    noise = rng.normal(0.0, 1.0, size=(n_extra, 2))
    out = rng.random(n_extra) < outlier_frac
    noise = np.where(out[:, None], rng.uniform(-50.0, 50.0, size=(n_extra, 2)), noise)
    order = rng.permutation(len(sc["obs_cam"]) + n_extra)
    sc["obs_cam"] = np.ascontiguousarray(np.concatenate([sc["obs_cam"], cam])[order], dtype=np.int32)
    sc["obs_pt"] = np.ascontiguousarray(np.concatenate([sc["obs_pt"], pts])[order], dtype=np.int32)
    sc["obs_uv"] = np.ascontiguousarray(np.concatenate([sc["obs_uv"], uv + noise])[order])
    sc["is_outlier"] = np.concatenate([sc["is_outlier"], out])[order]
    sc["loss"] = loss
    sc["config"] = f"{config} with a heavy camera"
    return sc
