"""Parity of the fp32 gfx950 dense frame-graph BA path (libdba) with the fp64
CPU oracle, on the same seeded inputs.

Tolerances (fp32 path against an fp64 oracle):
  * per-residual J_i, J_j, J_d and the depth blocks C, g_d: per-block
    relative 1e-4 (a few hundred fp32 roundings on O(1) quantities); r:
    1e-4 relative plus 16 fp32 ulps of the pixel-sized operands of its
    operations;
  * B and g_c: per 6x6 block, 1e-4 of the block's norm plus 1e-6 of the
    largest block (fp32 sums over ~3,000 pixels per edge);
  * the reduced matrix S = B - E C^-1 E^T: per block, 2e-4 of
    |B| + |E C^-1 E^T| (the two terms cancel; each carries fp32 sum error);
  * the pose step per component: its difference from the oracle's, less the
    part that the measured difference of the two reduced systems explains
    exactly, within the fp32 Cholesky solve's componentwise backward error
    carried through |S^-1| (pose_step_check), the two parts checked to be
    well below the step; and its backward error in the oracle's system,
    |S dxi - rhs| <= 2e-3 |rhs|;
  * the depth step per pixel: its difference, less the exact effect of the
    pose-step difference through the pixel's coupling rows, within 1e-4
    relative fp32 arithmetic on the terms of the pixel's back-substitution
    (depth_step_check);
  * costs after each of the 8 Gauss-Newton steps: 1e-3 relative.
"""
import numpy as np
import pytest
from scipy.spatial.transform import Rotation

from oracle import droid as odroid
from synthetic.droid import droid_scene

pytestmark = pytest.mark.gpu
EPS32 = float(np.finfo(np.float32).eps)

SMALL = dict(n_frames=4, height=6, width=8, hops=2, cx=3.5, cy=2.5)
MID = dict(n_frames=6, height=20, width=28, hops=3, cx=13.5, cy=9.5)


def gpu():
    from nonlinear_least_squares_amd import dba
    return dba


def blocks_close(a, b, tol, floor_frac=1e-6, axes=None):
    """Per-block Frobenius comparison over the trailing block axes."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    ax = axes if axes is not None else tuple(range(1, a.ndim))
    err = np.sqrt(((a - b) ** 2).sum(axis=ax))
    ref = np.sqrt((b ** 2).sum(axis=ax))
    bound = tol * np.maximum(ref, floor_frac * ref.max())
    bad = np.nonzero(err > bound)[0]
    assert bad.size == 0, (f"{bad.size} blocks out of tolerance, worst "
                           f"{(err / np.maximum(ref, 1e-300)).max():.3e} at {bad[:5]}")


def pose_mat(p):
    T = np.eye(4)
    T[:3, :3] = Rotation.from_quat(np.asarray(p[3:], dtype=np.float64)).as_matrix()
    T[:3, 3] = p[:3]
    return T


def pose_step_check(S_ref, rhs_ref, S_g, rhs_g, x_g):
    """Per component: (error of the device's pose step, what the measured
    difference of the two systems explains, bound on the rest).

    The device solves its own fp32 system S_g x = rhs_g by Cholesky, so
    (S_g + dS) x_g = rhs_g with |dS| <= gamma_{3n+1} |L| |L^T| (the
    componentwise backward error of a Cholesky solve, u = 2^-24), and the
    oracle's x_ref solves S_ref x = rhs_ref in fp64.  Subtracting gives the
    identity x_g - x_ref = S_ref^-1 ((rhs_g - rhs_ref) - (S_g - S_ref) x_g)
    - S_ref^-1 dS x_g: the first term is computed from the measured
    differences, the second is at most |S_ref^-1| gamma |L| |L^T| |x_g|
    (twice that allowed, |L| being taken from S_g in fp64)."""
    n = S_ref.shape[0]
    u = 2.0 ** -24
    gam = (3 * n + 1) * u / (1 - (3 * n + 1) * u)
    Sinv = np.linalg.inv(S_ref)
    L = np.linalg.cholesky(0.5 * (S_g + S_g.T))
    ax = np.abs(x_g)
    explained = Sinv @ ((rhs_g - rhs_ref) - (S_g - S_ref) @ x_g)
    rest = 2.0 * np.abs(Sinv) @ (gam * (np.abs(L) @ (np.abs(L.T) @ ax)))
    return explained, rest


def depth_step_check(O, sc, d_xi, xi_g):
    """Per pixel: (the part of |dd_g - dd_ref| the pose-step difference d_xi
    explains, bound on the rest).  A pixel's step is
    dd = -(g_d + sum_e w Jd^T (Ji xi_i + Jj xi_j)) / C over the edges e that
    leave its frame, C = sum_e w Jd^T Jd; a pose-step difference d_xi moves it
    by -sum_e w Jd^T (Ji d_xi_i + Jj d_xi_j) / C exactly.  The rest is the
    fp32 arithmetic on the pixel's terms (its Jacobians, C and g_d, each held
    to 1e-4 relative of the oracle's): 1e-4 of
    (|g_d| + sum_e |Jd|^T w (|Ji| |xi_i| + |Jj| |xi_j|)) / C and of |dd|."""
    Ji, Jj, Jd = O.get("Ji"), O.get("Jj"), O.get("Jd")
    w = sc["weights"].astype(np.float64)
    n, P = len(sc["poses"]), O.P
    ax = np.abs(xi_g)
    moved, mag = np.zeros((n, P)), np.zeros((n, P))
    for e, (i, j) in enumerate(sc["edges"]):
        wJd = Jd[e] * w[e][:, None]
        moved[i] -= (wJd * (Ji[e] @ d_xi[i] + Jj[e] @ d_xi[j])).sum(-1)
        mag[i] += (np.abs(wJd) * (np.abs(Ji[e]) @ ax[i] + np.abs(Jj[e]) @ ax[j])).sum(-1)
    C = O.get("C")
    Cs = np.where(C > 0, C, 1.0)
    rest = 1e-4 * ((np.abs(O.get("gd")) + mag) / Cs + np.abs(O.get("dd")))
    return np.where(C > 0, moved / Cs, 0.0), np.where(C > 0, rest, 0.0)


def free_blocks(M, nf):
    n6 = M.shape[0]
    return M[6 * nf:, 6 * nf:] if n6 > 0 else M


def to_blocks(M):
    nb = M.shape[0] // 6
    return M.reshape(nb, 6, nb, 6).transpose(0, 2, 1, 3).reshape(nb * nb, 6, 6)


@pytest.fixture(scope="module")
def scenes():
    return {"small": droid_scene(**SMALL), "mid": droid_scene(**MID), "full": droid_scene()}


@pytest.mark.parametrize("name", ["small", "mid", "full"])
def test_residuals_and_jacobians(scenes, name):
    sc = scenes[name]
    G = gpu().Problem.from_scene(sc)
    G.debug_run(gpu().DBA_STAGE_JACOBIANS)
    O = odroid.DroidProblem.from_scene(sc)
    O.gn_step()  # linearises at the initial state first
    E, P = O.E, O.P
    # r = f X/Z + c - target: besides 1e-4 relative, each of its ~8 fp32
    # operations rounds at the size of its operands, which are of order
    # f |X/Z| <= f + |u - c|, c, the target and u itself
    r, r_ref = G.debug_get("r").astype(np.float64), O.get("r")
    tg = sc["targets"].astype(np.float64)
    f, c = sc["intrinsics"][:2].astype(np.float64), sc["intrinsics"][2:].astype(np.float64)
    u = r_ref + tg
    bound = 1e-4 * np.abs(r_ref) + 16 * EPS32 * (f + np.abs(u - c) + np.abs(c) + np.abs(tg) +
                                                 np.abs(u))
    assert (np.abs(r - r_ref) <= bound).all(), np.max(np.abs(r - r_ref) / bound)
    for nm in ("Ji", "Jj"):
        blocks_close(G.debug_get(nm).reshape(E * P, 12), O.get(nm).reshape(E * P, 12), 1e-4)
    blocks_close(G.debug_get("Jd").reshape(E * P, 2), O.get("Jd").reshape(E * P, 2), 1e-4)


@pytest.mark.parametrize("name", ["small", "mid", "full"])
def test_assembly_without_elimination(scenes, name):
    sc = scenes[name]
    G = gpu().Problem.from_scene(sc)
    G.debug_run(gpu().DBA_STAGE_ASSEMBLE)
    O = odroid.DroidProblem.from_scene(sc)
    O.gn_step()
    nf = sc["n_fixed"]
    B = free_blocks(O.get("B"), nf)
    blocks_close(to_blocks(G.debug_get("S")), to_blocks(B), 1e-4)
    gc = O.get("gc")[6 * nf:]
    blocks_close(G.debug_get("rhs").reshape(-1, 6), -gc.reshape(-1, 6), 1e-4)


@pytest.mark.parametrize("name", ["small", "mid", "full"])
def test_one_step(scenes, name):
    sc = scenes[name]
    nf = sc["n_fixed"]
    G = gpu().Problem.from_scene(sc)
    O = odroid.DroidProblem.from_scene(sc)
    c0, c1 = G.gn_step()
    o0, o1 = O.gn_step()
    assert abs(c0 - o0) <= 1e-4 * o0
    assert abs(c1 - o1) <= 1e-3 * o1
    # depth blocks
    blocks_close(G.debug_get("C")[..., None], O.get("C")[..., None], 1e-4, axes=(2,))
    gd_ref = O.get("gd")
    assert np.abs(G.debug_get("gd") - gd_ref).max() <= 1e-4 * np.abs(gd_ref).max() + 1e-30
    # reduced system: S against |B| + |E C^-1 E^T| of the oracle
    S_ref = O.get("S")
    B = free_blocks(O.get("B"), nf)
    scale = np.sqrt((to_blocks(B) ** 2).sum(axis=(1, 2))) + \
        np.sqrt((to_blocks(B - S_ref) ** 2).sum(axis=(1, 2)))
    err = np.sqrt(((to_blocks(G.debug_get("S")) - to_blocks(S_ref)) ** 2).sum(axis=(1, 2)))
    assert (err <= 2e-4 * scale + 1e-12).all(), (err / np.maximum(scale, 1e-30)).max()
    rhs_ref = O.get("rhs")
    rhs = G.debug_get("rhs").astype(np.float64)
    assert np.linalg.norm(rhs - rhs_ref) <= 2e-4 * np.linalg.norm(rhs_ref) + \
        1e-4 * np.abs(O.get("gc")).max()
    # pose step: per component within the bound of the two solves, and the
    # backward error in the oracle's system
    dxi = G.debug_get("dxi").astype(np.float64)
    dxi_ref = O.get("dxi")
    np.testing.assert_array_equal(dxi[:nf], 0.0)
    x = dxi[nf:].ravel()
    assert np.linalg.norm(S_ref @ x - rhs_ref) <= 2e-3 * np.linalg.norm(rhs_ref)
    S_g = G.debug_get("S").astype(np.float64)
    expl, rest = pose_step_check(S_ref, rhs_ref, S_g, rhs, x)
    x_ref = dxi_ref[nf:].ravel()
    pres = np.abs(x - x_ref - expl)
    assert (pres <= rest).all(), (pres / rest).max()
    # neither part is vacuous: both stay well below the step itself
    assert np.linalg.norm(expl) <= 0.05 * np.linalg.norm(x_ref)
    assert np.linalg.norm(rest) <= 0.25 * np.linalg.norm(x_ref)
    # depth step, per pixel
    dd, dd_ref = G.debug_get("dd").astype(np.float64), O.get("dd")
    dmov, drest = depth_step_check(O, sc, dxi - dxi_ref, dxi)
    dres = np.abs(dd - dd_ref - dmov)
    assert (dres <= drest).all(), (dres / np.maximum(drest, 1e-300)).max()
    print(f"{name}: pose step residual / bound <= {(pres / rest).max():.3f}, depth step "
          f"residual / bound <= {(dres / np.maximum(drest, 1e-300)).max():.3f}", flush=True)
    # new state
    gp, gdp = G.get_state()
    op = O.get("poses")
    for i in range(len(op)):
        assert np.abs(pose_mat(gp[i]) - pose_mat(op[i])).max() <= 1e-4
    np.testing.assert_allclose(gdp, O.get("depth"), rtol=1e-3, atol=1e-5)


def test_eight_steps_match_oracle_costs(scenes):
    sc = scenes["full"]
    G = gpu().Problem.from_scene(sc)
    costs = G.solve(sc["n_iters"])
    O = odroid.DroidProblem.from_scene(sc)
    ref = [O.cost()] + [O.gn_step()[1] for _ in range(sc["n_iters"])]
    np.testing.assert_allclose(costs, ref, rtol=1e-3)
    gp, gdp = G.get_state()
    op = O.get("poses")
    for i in range(len(op)):
        assert np.abs(pose_mat(gp[i]) - pose_mat(op[i])).max() <= 1e-3
    assert np.abs(gdp - O.get("depth")).max() <= 1e-3 * np.abs(O.get("depth")).max()


def test_solve_equals_repeated_steps_bitwise(scenes):
    sc = scenes["mid"]
    A = gpu().Problem.from_scene(sc)
    B = gpu().Problem.from_scene(sc)
    ca = A.solve(4)
    cb = [B.gn_step() for _ in range(4)]
    assert list(ca[:4]) == [c[0] for c in cb]
    assert ca[4] == cb[3][1]
    for k in range(3):
        assert cb[k][1] == cb[k + 1][0]      # cost after == next cost before, bit for bit
    pa, da = A.get_state()
    pb, db = B.get_state()
    assert np.array_equal(pa, pb) and np.array_equal(da, db)
    assert A.cost() == ca[4]


def test_bitwise_deterministic(scenes):
    sc = scenes["full"]
    out = []
    for _ in range(2):
        G = gpu().Problem.from_scene(sc)
        c = G.solve(3)
        p, d = G.get_state()
        out.append((c, p, d, G.debug_get("S")))
    for a, b in zip(out[0], out[1]):
        assert np.array_equal(a, b)


def test_noise_free_converges_to_truth():
    sc = droid_scene(noise_px=0.0)
    G = gpu().Problem.from_scene(sc)
    costs = G.solve(sc["n_iters"])
    assert costs[-1] < 1e-7 * costs[0]
    p, d = G.get_state()
    for i in range(len(p)):
        assert np.abs(pose_mat(p[i]) - pose_mat(sc["poses_true"][i])).max() < 2e-4
    np.testing.assert_allclose(d, sc["inv_depth_true"], rtol=2e-3)


def test_unbalanced_graph_matches_oracle():
    """Frames with no out-edge, a repeated edge, a self-edge, an edge into a
    fixed frame and a pixel whose weights are all zero."""
    sc = droid_scene(**MID)
    edges = np.array([[0, 1], [1, 2], [1, 2], [2, 3], [3, 3], [3, 0], [4, 5], [2, 5], [4, 1]],
                     dtype=np.int32)
    rng = np.random.default_rng(3)
    P = sc["height"] * sc["width"]
    targets = np.empty((len(edges), P, 2), np.float32)
    for e, (i, j) in enumerate(edges):       # reuse the generated targets for the same pair
        k = np.nonzero((sc["edges"][:, 0] == i) & (sc["edges"][:, 1] == j))[0]
        targets[e] = sc["targets"][k[0]] if len(k) else \
            rng.uniform(0, 20, size=(P, 2)).astype(np.float32)
    weights = rng.uniform(0.1, 1.0, size=(len(edges), P)).astype(np.float32)
    weights[:, 5] = 0.0
    args = (sc["poses"], sc["inv_depth"], sc["intrinsics"], edges, targets, weights,
            sc["height"], sc["width"], 2)
    G = gpu().Problem(*args)
    O = odroid.DroidProblem(*args)
    for _ in range(2):
        c0, c1 = G.gn_step()
        o0, o1 = O.gn_step()
        assert abs(c0 - o0) <= 1e-4 * o0 and abs(c1 - o1) <= 1e-3 * o1
    dd = G.debug_get("dd")
    assert (dd[:, 5] == 0).all() and (dd[5] == 0).all()   # no coupling: no depth step
    gp, gdp = G.get_state()
    np.testing.assert_allclose(gdp, O.get("depth"), rtol=1e-3, atol=1e-4)


def test_all_fixed_moves_depths_only():
    sc = droid_scene(**SMALL)
    sc = dict(sc, n_fixed=sc["poses"].shape[0])
    G = gpu().Problem.from_scene(sc)
    O = odroid.DroidProblem.from_scene(sc)
    p0, _ = G.get_state()
    c = G.gn_step()
    o = O.gn_step()
    assert abs(c[1] - o[1]) <= 1e-3 * o[1]
    p1, d1 = G.get_state()
    assert np.array_equal(p0, p1)
    np.testing.assert_allclose(d1, O.get("depth"), rtol=1e-3, atol=1e-5)


def test_errors():
    dba = gpu()
    sc = droid_scene(**SMALL)
    base = dict(poses=sc["poses"], inv_depth=sc["inv_depth"], intrinsics=sc["intrinsics"],
                edges=sc["edges"], targets=sc["targets"], weights=sc["weights"],
                height=sc["height"], width=sc["width"], n_fixed=2)

    def make(**over):
        kw = dict(base)
        kw.update(over)
        return dba.Problem(**kw)

    with pytest.raises(dba.DBAError) as ex:
        make(edges=np.array([[0, 9]] * len(sc["edges"]), np.int32))
    assert ex.value.code == dba.DBA_ERR_ARG
    w = sc["weights"].copy()
    w[1, 3] = -1.0
    with pytest.raises(dba.DBAError) as ex:
        make(weights=w)
    assert ex.value.code == dba.DBA_ERR_NONFINITE
    d = sc["inv_depth"].copy()
    d[0, 0] = np.nan
    with pytest.raises(dba.DBAError) as ex:
        make(inv_depth=d)
    assert ex.value.code == dba.DBA_ERR_NONFINITE
    p = sc["poses"].copy()
    p[1, 3:] = 0.0
    with pytest.raises(dba.DBAError) as ex:
        make(poses=p)
    assert ex.value.code == dba.DBA_ERR_NONFINITE
    # out-degree above the limit
    n = 12
    big = droid_scene(n_frames=n, height=4, width=4, hops=9, cx=1.5, cy=1.5)
    with pytest.raises(dba.DBAError) as ex:
        dba.Problem.from_scene(big)
    assert ex.value.code == dba.DBA_ERR_LIMIT
    # no edges: nothing constrains the poses
    G = make(edges=np.zeros((0, 2), np.int32), targets=np.zeros((0, 48, 2), np.float32),
             weights=np.zeros((0, 48), np.float32))
    assert G.cost() == 0.0
    with pytest.raises(dba.DBAError) as ex:
        G.gn_step()
    assert ex.value.code == dba.DBA_ERR_NOT_SPD
    # the failed step left the state alone and the handle usable
    p0, d0 = G.get_state()
    assert np.array_equal(d0, sc["inv_depth"])


def test_failed_step_leaves_state_and_recovers(scenes):
    """A reduced system that cannot be factored (a free frame no edge
    touches) fails the step without changing the state."""
    sc = droid_scene(**SMALL)
    keep = (sc["edges"][:, 0] != 3) & (sc["edges"][:, 1] != 3)
    G = gpu().Problem(sc["poses"], sc["inv_depth"], sc["intrinsics"], sc["edges"][keep],
                      sc["targets"][keep], sc["weights"][keep], sc["height"], sc["width"], 2)
    p0, d0 = G.get_state()
    with pytest.raises(gpu().DBAError) as ex:
        G.solve(3)
    assert ex.value.code == gpu().DBA_ERR_NOT_SPD
    p1, d1 = G.get_state()
    assert np.array_equal(p0, p1) and np.array_equal(d0, d1)


def test_device_inputs_on_a_stream(scenes):
    import torch
    dba = gpu()
    sc = scenes["mid"]
    dev = torch.device("cuda", 0)
    s = torch.cuda.Stream()
    t = {k: torch.from_numpy(np.ascontiguousarray(sc[k])).to(dev)
         for k in ("poses", "inv_depth", "intrinsics", "edges", "targets", "weights")}
    torch.cuda.synchronize()
    G = dba.Problem(t["poses"], t["inv_depth"], t["intrinsics"], t["edges"], t["targets"],
                    t["weights"], sc["height"], sc["width"], sc["n_fixed"],
                    mem=dba.DBA_MEM_DEVICE, stream=s.cuda_stream)
    H = dba.Problem.from_scene(sc)
    assert np.array_equal(G.solve(3), H.solve(3))
    G.set_state(t["poses"], t["inv_depth"])
    pg, dg = G.get_state()
    ph, dh = dba.Problem.from_scene(sc).get_state()
    assert np.array_equal(pg, ph) and np.array_equal(dg, dh)


def test_state_roundtrip(scenes):
    dba = gpu()
    sc = scenes["small"]
    G = dba.Problem.from_scene(sc)
    p, d = G.get_state()
    q = p[:, 3:]
    np.testing.assert_allclose(np.linalg.norm(q, axis=1), 1.0, atol=1e-6)
    assert (q[:, 3] >= 0).all()
    G.gn_step()
    G.set_state(p, d)
    p2, d2 = G.get_state()
    # translations and depths come back bit for bit; the quaternion is
    # normalised again on the way in, which may move its last bits
    assert np.array_equal(p[:, :3], p2[:, :3]) and np.array_equal(d, d2)
    np.testing.assert_allclose(p2[:, 3:], p[:, 3:], rtol=0, atol=4 * EPS32)


@pytest.mark.parametrize("name", ["small", "mid", "full"])
def test_pose_covariance(scenes, name):
    """S^-1 (fp32, one workgroup) against the oracle's fp64 S^-1 at the same
    state.  First-order perturbation bound for an inverse: the relative
    Frobenius error is at most kappa(S) d / (1 - kappa(S) d), d the relative
    difference of the two reduced matrices plus the factorisation's own
    n eps32; the test allows 4x that.  The state and the cost do not change."""
    sc = scenes[name]
    G = gpu().Problem.from_scene(sc)
    O = odroid.DroidProblem.from_scene(sc)
    p0, d0 = G.get_state()
    c0 = G.cost()
    X = G.covariance().astype(np.float64)
    ref = O.covariance()
    S_ref = O.get("S")
    S_gpu = G.debug_get("S").astype(np.float64)   # this linearisation
    nv = S_ref.shape[0]
    kappa = np.linalg.cond(S_ref)
    d = np.linalg.norm(S_gpu - S_ref) / np.linalg.norm(S_ref) + nv * EPS32
    assert kappa * d < 0.25, (kappa, d)
    rel = np.linalg.norm(X - ref) / np.linalg.norm(ref)
    assert rel <= 4 * kappa * d / (1 - kappa * d), (rel, kappa, d)
    assert np.linalg.norm(X - X.T) <= 4 * kappa * d * np.linalg.norm(ref)
    assert np.linalg.eigvalsh(0.5 * (X + X.T)).min() > 0
    p1, d1 = G.get_state()
    assert np.array_equal(p0, p1) and np.array_equal(d0, d1)
    assert G.cost() == c0


def test_pose_covariance_all_fixed_is_empty():
    sc = droid_scene(**SMALL)
    sc = dict(sc, n_fixed=sc["poses"].shape[0])
    G = gpu().Problem.from_scene(sc)
    assert G.covariance().shape == (0, 0)


def test_rejected_set_state_leaves_the_state(scenes):
    """dba_set_state with a non-finite depth or a zero quaternion fails and
    changes nothing: the state and the next step match an untouched handle."""
    dba = gpu()
    sc = scenes["small"]
    G = dba.Problem.from_scene(sc)
    H = dba.Problem.from_scene(sc)
    G.gn_step()
    H.gn_step()
    p0, d0 = G.get_state()
    bad_d = d0.copy()
    bad_d.flat[3] = np.nan
    with pytest.raises(dba.DBAError) as ex:
        G.set_state(p0, bad_d)
    assert ex.value.code == dba.DBA_ERR_NONFINITE
    bad_p = p0.copy()
    bad_p[1, 3:] = 0.0
    with pytest.raises(dba.DBAError) as ex:
        G.set_state(bad_p, None)
    assert ex.value.code == dba.DBA_ERR_NONFINITE
    p1, d1 = G.get_state()
    assert np.array_equal(p0, p1) and np.array_equal(d0, d1)
    assert G.gn_step() == H.gn_step()


def test_handles_of_different_sizes():
    """Above 64 KiB the solver's dynamic-LDS limit is a per-process kernel
    attribute: a handle with 24 free frames (the largest reduced system, 144
    unknowns), then one with 21, then steps of both, each against the oracle
    (the second handle must not lower the limit below the first's need)."""
    kw = dict(height=8, width=10, hops=2, cx=4.5, cy=3.5)
    big, mid = droid_scene(n_frames=26, **kw), droid_scene(n_frames=23, **kw)
    Gb = gpu().Problem.from_scene(big)
    Gm = gpu().Problem.from_scene(mid)
    for sc, G in ((mid, Gm), (big, Gb)):
        O = odroid.DroidProblem.from_scene(sc)
        c0, c1 = G.gn_step()
        o0, o1 = O.gn_step()
        assert abs(c0 - o0) <= 1e-4 * o0 and abs(c1 - o1) <= 1e-3 * o1, (c0, c1, o0, o1)
