"""GPU parity: libba (HIP, gfx950) against the CPU oracle on the same seeded inputs.

Bars (fp64): sparsity structure bit-exact; residuals, Jacobians, weights and
every Hessian / Schur block within 1e-10 per block (Frobenius norm, relative
to the block, floored at 1e-6 of the array's RMS block norm so near-zero
blocks are judged against the array's scale); the PCG camera step within 1e-8
at equal PCG iteration counts; the final cost after the fixed LM iteration
count within 1e-6 relative.  Accept/reject decisions and trial costs must
agree on every step until the first one whose cost change is within the
rounding noise of the cost sum (|dC| <= 1e-10 C), where either decision is
correct.  Blocks built from inverted point blocks (C~^-1, v, S_jj, rhs) are
held to the larger of 1e-10 and the first-order error bound of a Cholesky
inverse, 32 kappa eps per point block, carried to the cameras; residuals to
the larger of 1e-10 and the first-order effect of rounding the camera-frame
point P = R X + t (large world coordinates with near points cancel there).
"""
import numpy as np
import pytest

import oracle
from synthetic import ba_scene, heavy_camera_scene

pytestmark = pytest.mark.gpu

bamod = pytest.importorskip("nonlinear_least_squares_amd.ba")

BLOCK_TOL = 1e-10


def blocks_close(name, got, ref, tol=BLOCK_TOL):
    """Per-block Frobenius check; tol is a scalar or one relative tolerance per block."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    n = ref.shape[0]
    g = got.reshape(n, -1)
    r = ref.reshape(n, -1)
    assert np.all(np.isfinite(g)), name
    err = np.linalg.norm(g - r, axis=1)
    norm = np.linalg.norm(r, axis=1)
    rms = np.sqrt(np.mean(norm ** 2)) if n else 0.0
    scale = np.maximum(norm, 1e-6 * rms)
    bound = np.asarray(tol) * scale
    bad = np.nonzero(err > bound)[0]
    worst = float(np.max(err / np.maximum(scale, 1e-300))) if n else 0.0
    assert len(bad) == 0, f"{name}: {len(bad)}/{n} blocks off, worst relative error {worst:.3e}"
    return worst


EPS = np.finfo(np.float64).eps


def inverse_bounds(orc, sc):
    """First-order bounds for quantities built from the inverted point blocks.

    Inverting C~_i by Cholesky has a forward error of order kappa(C~_i) eps in
    any correct implementation, so two correct implementations may differ by
    that much.  Per point: 32 kappa_i eps relative for C~^-1 and v; per camera
    the absolute error of E C~^-1 E^T (and of E v) is bounded by summing each
    observation's ||E_k||^2 ||C~_i^-1|| 32 kappa_i eps (and ||E_k|| ||v_i||
    32 kappa_i eps).  Returns relative tolerances per point and per camera,
    never below the 1e-10 bar."""
    Cinv = orc.get("Cinv")
    kappa = np.linalg.cond(Cinv)
    tol_pt = np.maximum(BLOCK_TOL, 32 * kappa * EPS)
    Jc, Jp, w = orc.get("Jc"), orc.get("Jp"), orc.get("w")
    E = w[:, None, None] * np.einsum("kra,krb->kab", Jc, Jp)
    En = np.linalg.norm(E.reshape(len(E), -1), axis=1)
    pt, cam = sc["obs_pt"], sc["obs_cam"]
    cinv_n = np.linalg.norm(Cinv.reshape(len(Cinv), -1), axis=1)
    v_n = np.linalg.norm(orc.get("v"), axis=1)
    nc = len(sc["cams"])
    abs_M = np.bincount(cam, weights=En ** 2 * cinv_n[pt] * 32 * kappa[pt] * EPS, minlength=nc)
    abs_r = np.bincount(cam, weights=En * v_n[pt] * 32 * kappa[pt] * EPS, minlength=nc)
    M_n = np.linalg.norm(orc.get("M").reshape(nc, -1), axis=1)
    r_n = np.linalg.norm(orc.get("rhs"), axis=1)
    tol_M = np.maximum(BLOCK_TOL, abs_M / np.maximum(M_n, 1e-300) + BLOCK_TOL)
    tol_r = np.maximum(BLOCK_TOL, abs_r / np.maximum(r_n, 1e-300) + BLOCK_TOL)
    return dict(Cinv=tol_pt, v=tol_pt, M=tol_M, rhs=tol_r)


def traces_agree(g_tr, o_tr, cost_tol=1e-6):
    """Accept/reject decisions and trial costs agree on every step up to the
    first one whose oracle cost change is within the rounding noise of the
    cost sums; after such a step the two runs may legitimately branch."""
    for a, b in zip(g_tr, o_tr):
        if abs(a["cost_after"] - b["cost_after"]) > cost_tol * b["cost_after"]:
            return False
        margin = abs(b["cost_after"] - b["cost_before"])
        if margin <= 1e-10 * b["cost_before"]:
            return True
        if a["accepted"] != b["accepted"]:
            return False
    return True


# Camera layouts of the point passes, chosen at creation by size; the
# environment switches select the other two on scenes that would not get them.
CAMERA_TABLES = ["lds", "vectors", "memory"]


def use_camera_table(kind, monkeypatch):
    """For handles created next: whole camera rows in LDS (the default up to
    1,076 cameras), only the PCG's camera vectors in LDS with the geometry read
    from memory (chosen by size up to 2,240 cameras), or the camera table and
    vectors read from memory."""
    if kind == "vectors":
        monkeypatch.setenv("BA_SPLIT_LDS_CAMERAS", "1")
    elif kind == "memory":
        monkeypatch.setenv("BA_NO_LDS_CAMERAS", "1")


def make_pair(sc, **kw):
    gpu = bamod.Problem.from_scene(sc, **kw)
    orc = oracle.Problem.from_scene(sc, **kw)
    return gpu, orc


@pytest.fixture(scope="module", params=["tiny", "small", "medium"])
def scene(request):
    return ba_scene(request.param)


def test_structure_bit_exact(scene):
    gpu, orc = make_pair(scene)
    for name in ("perm_pt", "perm_cam", "pt_ptr", "cam_ptr"):
        np.testing.assert_array_equal(gpu.debug_get(name), orc.get(name), err_msg=name)


def residual_bounds(orc, sc):
    """Per observation: the larger of 1e-10 and the first-order effect on the
    residual of rounding P = R X + t, |Jp| 8 eps (|X| + |t|) relative to |r|.
    Where world coordinates are large and the point is near (the walk scene:
    |X| ~ 1e3 at depths ~0.5), P cancels and two correct projections differ by
    about that much."""
    Jp, r = orc.get("Jp"), orc.get("r")
    X = sc["points"][sc["obs_pt"]]
    t = sc["cams"][sc["obs_cam"], 3:6]
    bound = (np.linalg.norm(Jp.reshape(len(Jp), -1), axis=1) * 8 * EPS
             * (np.linalg.norm(X, axis=1) + np.linalg.norm(t, axis=1)))
    return np.maximum(BLOCK_TOL, bound / np.maximum(np.linalg.norm(r, axis=1), 1e-300) + BLOCK_TOL)


def test_linearisation_parity(scene):
    gpu, orc = make_pair(scene)
    gpu.debug_run(bamod.BA_STAGE_LINEARIZE)
    orc.linearize()
    for name in ("r", "Jc", "Jp", "w", "B", "gc", "C", "gp"):
        got, ref = gpu.debug_get(name), orc.get(name)
        if name == "w":
            got, ref = got[:, None], ref[:, None]
        blocks_close(name, got, ref, residual_bounds(orc, scene) if name == "r" else BLOCK_TOL)


@pytest.mark.parametrize("lam", [1e-2, 1e-6])
def test_schur_parity(scene, lam):
    gpu, orc = make_pair(scene)
    gpu.set_state(lam)
    orc.lam = lam
    gpu.debug_run(bamod.BA_STAGE_SCHUR)
    orc.linearize()
    orc.damp()
    orc.schur()
    blocks_close("Bd", gpu.debug_get("Bd"), orc.get("Bd"))
    tols = inverse_bounds(orc, scene)
    for name in ("Cinv", "v", "rhs", "M"):
        blocks_close(name, gpu.debug_get(name), orc.get(name), tols[name])


@pytest.mark.parametrize("config", ["tiny", "small"])
@pytest.mark.parametrize("cameras", CAMERA_TABLES)
def test_pcg_and_update_parity(config, cameras, monkeypatch):
    # the camera table of these scenes fits in LDS; the environment switches,
    # read when the handle is created, select the other layouts
    use_camera_table(cameras, monkeypatch)
    sc = ba_scene(config)
    gpu, orc = make_pair(sc)
    gpu.debug_run(bamod.BA_STAGE_UPDATE)
    orc.linearize()
    orc.damp()
    orc.schur()
    it, rel = orc.pcg(sc["pcg_max_iters"], sc["pcg_rel_tol"])
    orc.backsub()
    orc.retract()
    g_it, g_rel = gpu.debug_get("pcg")
    assert int(g_it) == it, (g_it, it)
    assert abs(g_rel - rel) <= 1e-6 * max(rel, 1e-300) + 1e-12
    dc, dc_ref = gpu.debug_get("dc"), orc.get("dc")
    assert np.linalg.norm(dc - dc_ref) <= 1e-8 * np.linalg.norm(dc_ref)
    dp, dp_ref = gpu.debug_get("dp"), orc.get("dp")
    assert np.linalg.norm(dp - dp_ref) <= 1e-8 * np.linalg.norm(dp_ref)
    blocks_close("cams_trial", gpu.debug_get("cams_trial"), orc.get("cams_trial"), 1e-8)
    blocks_close("points_trial", gpu.debug_get("points_trial"), orc.get("points_trial"), 1e-8)
    trial = float(gpu.debug_get("trial_cost")[0])
    ref = orc.cost_at(orc.get("cams_trial"), orc.get("points_trial"))
    assert abs(trial - ref) <= 1e-8 * ref


@pytest.mark.parametrize("config", ["tiny", "small"])
def test_lm_final_cost_parity(config):
    sc = ba_scene(config)
    gpu, orc = make_pair(sc)
    assert abs(gpu.cost() - orc.cost) <= 1e-12 * orc.cost
    n = sc["n_iters"]
    g_tr = [gpu.lm_step() for _ in range(n)]
    o_tr = orc.solve(n)
    assert traces_agree(g_tr, o_tr)
    final, ref = gpu.get_state()["cost"], orc.cost
    assert abs(final - ref) <= 1e-6 * ref, (final, ref)
    cams, pts = gpu.get_params()
    assert abs(gpu.cost() - final) <= 1e-12 * final


def test_medium_three_lm_steps():
    sc = ba_scene("medium")
    gpu, orc = make_pair(sc)
    g_tr = [gpu.lm_step() for _ in range(3)]
    o_tr = orc.solve(3)
    assert traces_agree(g_tr, o_tr)
    for a, b in zip(g_tr, o_tr):
        assert a["pcg_iters"] == b["pcg_iters"]


def test_noise_free_tiny_converges_on_gpu():
    sc = ba_scene("tiny", noise_px=0.0)
    gpu = bamod.Problem.from_scene(sc)
    c0 = gpu.cost()
    gpu.solve(30)
    assert gpu.cost() < 1e-12 * c0


def test_bitwise_determinism():
    sc = ba_scene("small")
    a = bamod.Problem.from_scene(sc)
    b = bamod.Problem.from_scene(sc)
    a.solve(4)
    b.solve(4)
    ca, pa = a.get_params()
    cb, pb = b.get_params()
    assert np.array_equal(ca, cb) and np.array_equal(pa, pb)
    assert a.get_state() == b.get_state()


def _edge_scene():
    """Repeated (camera, point) pairs, a point longer than a tile (carry across
    sub-tiles and wavefronts), an unobserved point and an unobserved camera."""
    sc = ba_scene("tiny", outlier_frac=0.1)
    rng = np.random.default_rng(9)
    oc, op, uv = list(sc["obs_cam"]), list(sc["obs_pt"]), list(sc["obs_uv"])
    # Point 7 observed 700 times (cameras repeat): spans several 256-wide sub-tiles.
    for _ in range(700):
        k = [i for i in range(len(op)) if op[i] == 7][0]
        oc.append(int(rng.integers(0, 9)))
        op.append(7)
        uv.append(np.array(sc["obs_uv"][k]) + rng.normal(0, 2.0, 2))
    # Remove every observation of point 11 and of camera 9.
    keep = [i for i in range(len(op)) if op[i] != 11 and oc[i] != 9]
    sc["obs_cam"] = np.array([oc[i] for i in keep], dtype=np.int32)
    sc["obs_pt"] = np.array([op[i] for i in keep], dtype=np.int32)
    sc["obs_uv"] = np.array([uv[i] for i in keep])
    sc["loss"] = "huber"
    return sc


def test_camera_layouts_bitwise(monkeypatch):
    """The three camera layouts differ only in where the point passes find the
    camera data (R in the camera table is formed from the same quaternion by
    the same function as the LDS rows' R, and every sum keeps its order), so
    five LM steps leave the same parameters, cost and damping to the bit."""
    sc = ba_scene("small")
    runs = []
    for kind in CAMERA_TABLES:
        with monkeypatch.context() as m:
            use_camera_table(kind, m)
            g = bamod.Problem.from_scene(sc)
        tr = [g.lm_step() for _ in range(5)]
        runs.append((tr, g.get_params(), g.get_state()))
    for tr, (cams, pts), st in runs[1:]:
        assert tr == runs[0][0]
        assert np.array_equal(cams, runs[0][1][0]) and np.array_equal(pts, runs[0][1][1])
        assert st == runs[0][2]


@pytest.mark.parametrize("cameras", CAMERA_TABLES)
@pytest.mark.parametrize("queued", [False, True])
def test_scene_without_observations(queued, cameras, monkeypatch):
    """Cameras and points with no observations at all: the cost is 0, the
    reduced system is the damping alone with a zero right-hand side, so the PCG
    stops before its first iteration; no step lowers the cost strictly, so
    every step is rejected and the parameters stay, as in the oracle's run.
    Step by step and queued (ba_solve), in all three camera layouts (every
    point-pass wavefront has an empty range)."""
    use_camera_table(cameras, monkeypatch)
    sc = dict(ba_scene("tiny"))
    sc["obs_cam"] = np.zeros(0, np.int32)
    sc["obs_pt"] = np.zeros(0, np.int32)
    sc["obs_uv"] = np.zeros((0, 2))
    gpu, orc = make_pair(sc)
    o_tr = orc.solve(3)
    if queued:
        s = gpu.solve(3)
        assert s["accepted"] == 0 and s["pcg_iters_total"] == 0 and s["final_cost"] == 0.0
    else:
        g_tr = [gpu.lm_step() for _ in range(3)]
        for a, b in zip(g_tr, o_tr):
            assert a["accepted"] == b["accepted"] == 0
            assert a["pcg_iters"] == b["pcg_iters"] == 0
            assert a["cost_before"] == a["cost_after"] == 0.0
    cams, pts = gpu.get_params()
    assert np.array_equal(cams, sc["cams"]) and np.array_equal(pts, sc["points"])
    st = gpu.get_state()
    assert st["cost"] == 0.0 and abs(st["lam"] - 10 * o_tr[-1]["lam"]) <= 1e-15 * st["lam"]


def test_edge_cases_parity():
    sc = _edge_scene()
    gpu, orc = make_pair(sc)
    for name in ("perm_pt", "perm_cam", "pt_ptr", "cam_ptr"):
        np.testing.assert_array_equal(gpu.debug_get(name), orc.get(name), err_msg=name)
    gpu.debug_run(bamod.BA_STAGE_SCHUR)
    orc.linearize()
    orc.damp()
    orc.schur()
    for name in ("B", "gc", "C", "gp", "Bd"):
        blocks_close(name, gpu.debug_get(name), orc.get(name))
    tols = inverse_bounds(orc, sc)
    for name in ("Cinv", "v", "rhs", "M"):
        blocks_close(name, gpu.debug_get(name), orc.get(name), tols[name])
    gpu2, orc2 = make_pair(sc)
    g_tr = [gpu2.lm_step() for _ in range(6)]
    o_tr = orc2.solve(6)
    assert traces_agree(g_tr, o_tr)
    assert abs(gpu2.get_state()["cost"] - orc2.cost) <= 1e-6 * orc2.cost
    cams, pts = gpu2.get_params()
    np.testing.assert_array_equal(pts[11], sc["points"][11])   # unobserved: never moves


def test_device_validation_errors():
    sc = ba_scene("tiny")
    bad = sc["obs_cam"].copy()
    bad[17] = 10
    with pytest.raises(bamod.BAError) as e:
        bamod.Problem(sc["cams"], sc["points"], bad, sc["obs_pt"], sc["obs_uv"])
    assert e.value.code == bamod.BA_ERR_ARG
    uv = sc["obs_uv"].copy()
    uv[3, 1] = np.inf
    with pytest.raises(bamod.BAError) as e:
        bamod.Problem(sc["cams"], sc["points"], sc["obs_cam"], sc["obs_pt"], uv)
    assert e.value.code == bamod.BA_ERR_NONFINITE


def test_checkpoint_resume_bitwise():
    sc = ba_scene("small")
    full = bamod.Problem.from_scene(sc)
    full.solve(8)
    first = bamod.Problem.from_scene(sc)
    first.solve(4)
    cams, pts = first.get_params()
    st = first.get_state()
    second = bamod.Problem.from_scene(sc)
    second.set_params(cams, pts)
    second.set_state(st["lam"], st["iteration"])
    assert second.get_state()["cost"] == st["cost"]
    second.solve(4)
    c1, p1 = full.get_params()
    c2, p2 = second.get_params()
    assert np.array_equal(c1, c2) and np.array_equal(p1, p2)


def test_device_resident_inputs_on_torch_stream():
    torch = pytest.importorskip("torch")
    sc = ba_scene("tiny")
    dev = torch.device("cuda:0")
    s = torch.cuda.Stream()
    t = {k: torch.from_numpy(np.ascontiguousarray(sc[k])).to(dev)
         for k in ("cams", "points", "obs_cam", "obs_pt", "obs_uv")}
    torch.cuda.synchronize()
    gpu = bamod.Problem(t["cams"], t["points"], t["obs_cam"], t["obs_pt"], t["obs_uv"],
                        mem=bamod.BA_MEM_DEVICE, stream=s.cuda_stream)
    host = bamod.Problem.from_scene(sc)
    gpu.solve(5)
    host.solve(5)
    assert gpu.get_state() == host.get_state()


def _max_band_segment(sc, bands=4):
    """Longest run of one camera's observations whose points share one of the
    library's point-index bands (its camera passes cut such a run into chunks
    of at most 1,024 observations)."""
    key = sc["obs_cam"].astype(np.int64) * bands + (sc["obs_pt"].astype(np.int64) * bands) // len(sc["points"])
    return int(np.bincount(key).max())


@pytest.mark.parametrize("cameras", CAMERA_TABLES)
def test_heavy_camera_multi_chunk_parity(cameras, monkeypatch):
    """One camera with about 3,200 observations in one point band: its
    camera-order segment is split into several chunks, whose partials the
    per-camera kernels (B and g_c, rhs and S_jj, the PCG's camera side) add in
    chunk order.  All three camera layouts, selected by the environment
    switches read at creation."""
    use_camera_table(cameras, monkeypatch)
    sc = heavy_camera_scene()
    assert _max_band_segment(sc) > 2048
    gpu, orc = make_pair(sc)
    gpu.debug_run(bamod.BA_STAGE_SCHUR)
    orc.linearize()
    orc.damp()
    orc.schur()
    for name in ("B", "gc", "C", "gp", "Bd"):
        blocks_close(name, gpu.debug_get(name), orc.get(name))
    tols = inverse_bounds(orc, sc)
    for name in ("Cinv", "v", "rhs", "M"):
        blocks_close(name, gpu.debug_get(name), orc.get(name), tols[name])
    gpu.debug_run(bamod.BA_STAGE_UPDATE)
    it, rel = orc.pcg(sc["pcg_max_iters"], sc["pcg_rel_tol"])
    orc.backsub()
    g_it, _ = gpu.debug_get("pcg")
    assert int(g_it) == it
    dc, dc_ref = gpu.debug_get("dc"), orc.get("dc")
    assert np.linalg.norm(dc - dc_ref) <= 1e-8 * np.linalg.norm(dc_ref)
    dp, dp_ref = gpu.debug_get("dp"), orc.get("dp")
    assert np.linalg.norm(dp - dp_ref) <= 1e-8 * np.linalg.norm(dp_ref)
    gpu2, orc2 = make_pair(sc)
    g_tr = [gpu2.lm_step() for _ in range(6)]
    o_tr = orc2.solve(6)
    assert traces_agree(g_tr, o_tr)
    assert abs(gpu2.get_state()["cost"] - orc2.cost) <= 1e-6 * orc2.cost


def test_rejected_set_params_leaves_the_handle():
    """ba_set_params with a non-finite camera fails and changes nothing: the
    parameters, the cost and the next LM step are those of an untouched
    handle, bit for bit."""
    sc = ba_scene("small")
    a = bamod.Problem.from_scene(sc)
    b = bamod.Problem.from_scene(sc)
    a.solve(2)
    b.solve(2)
    cams, pts = a.get_params()
    bad = cams.copy()
    bad[3, 4] = np.nan
    with pytest.raises(bamod.BAError) as e:
        a.set_params(bad, pts)
    assert e.value.code == bamod.BA_ERR_NONFINITE
    bad_pts = pts.copy()
    bad_pts[7, 1] = np.inf
    with pytest.raises(bamod.BAError) as e:
        a.set_params(None, bad_pts)
    assert e.value.code == bamod.BA_ERR_NONFINITE
    ca, pa = a.get_params()
    assert np.array_equal(ca, cams) and np.array_equal(pa, pts)
    assert a.get_state() == b.get_state()
    assert a.lm_step() == b.lm_step()
    ca, pa = a.get_params()
    cb, pb = b.get_params()
    assert np.array_equal(ca, cb) and np.array_equal(pa, pb)
