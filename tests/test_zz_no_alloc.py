"""ba_cost_noalloc (the cost with no handle and no device allocation) against
the existing entry point ba_cost of a handle built from the same inputs.

Both evaluate every observation's rho with the same camera table bits and the
same per-observation arithmetic; only the order of the final sum differs
(point order in the handle, the caller's order here), so the two totals of N
non-negative terms agree within N eps of the cost (the error bound of a
floating-point sum of non-negative terms in any order).

Two calls in a row share the GPU's scratch array: a larger scene first, then a
smaller one, so stale partials of the first call would show in the second.
"""
import numpy as np
import pytest

from synthetic import ba_scene

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
bamod = pytest.importorskip("nonlinear_least_squares_amd.ba")

EPS = np.finfo(np.float64).eps


def _device(sc, dev):
    return [torch.from_numpy(np.ascontiguousarray(sc[k])).to(dev)
            for k in ("cams", "points", "obs_cam", "obs_pt", "obs_uv")]


def _loss(sc):
    return bamod.BA_LOSS_HUBER if sc["loss"] == "huber" else bamod.BA_LOSS_SQUARED


def test_cost_noalloc_matches_ba_cost_on_two_calls():
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream().cuda_stream
    scenes = [ba_scene("medium"), ba_scene("tiny")]   # the second call is smaller
    assert len(scenes[1]["obs_cam"]) < len(scenes[0]["obs_cam"])
    outs = []
    for sc in scenes:
        print(f"noalloc cost: {sc['config']} ({len(sc['obs_cam'])} observations)", flush=True)
        t = _device(sc, dev)
        out = torch.full((1,), -1.0, dtype=torch.float64, device=dev)
        bamod.cost_noalloc(*t, out, loss=_loss(sc), huber_delta=sc["huber_delta"], stream=stream)
        torch.cuda.synchronize()
        got = float(out.item())
        ref = bamod.Problem.from_scene(sc).cost()
        n = len(sc["obs_cam"])
        assert np.isfinite(got)
        assert abs(got - ref) <= n * EPS * ref, (sc["config"], got, ref)
        outs.append(got)
    # the same call again gives the same bits (fixed reduction order)
    sc = scenes[1]
    t = _device(sc, dev)
    out = torch.empty((1,), dtype=torch.float64, device=dev)
    bamod.cost_noalloc(*t, out, loss=_loss(sc), huber_delta=sc["huber_delta"], stream=stream)
    torch.cuda.synchronize()
    assert float(out.item()) == outs[1]


def test_cost_noalloc_flags_out_of_range_index_and_rejects_sizes():
    dev = torch.device("cuda:0")
    sc = ba_scene("tiny")
    cams, pts, oc, op, uv = _device(sc, dev)
    bad = oc.clone()
    bad[5] = len(sc["cams"])          # one past the last camera: never read
    out = torch.zeros((1,), dtype=torch.float64, device=dev)
    bamod.cost_noalloc(cams, pts, bad, op, uv, out)
    torch.cuda.synchronize()
    assert np.isnan(float(out.item()))
    # sizes beyond the scratch array's limits are rejected before device work
    L = bamod.lib()
    import ctypes as C
    p = [C.c_void_p(a.data_ptr()) for a in (cams, pts, oc, op, uv, out)]
    rc = L.ba_cost_noalloc(p[0], bamod.BA_NOALLOC_MAX_CAMS + 1, p[1], len(sc["points"]), p[2],
                           p[3], p[4], len(sc["obs_cam"]), 0, 2.0, p[5], None)
    assert rc == bamod.BA_ERR_ARG
    assert b"BA_NOALLOC_MAX_CAMS" in L.ba_status_string(rc)
    rc = L.ba_cost_noalloc(p[0], len(sc["cams"]), p[1], len(sc["points"]), p[2], p[3], p[4],
                           bamod.BA_NOALLOC_MAX_OBS + 1, 0, 2.0, p[5], None)
    assert rc == bamod.BA_ERR_ARG


def test_cost_noalloc_under_graph_capture():
    """The call enqueues only kernel launches, so it can be captured; each
    replay (with eager work and synchronisations between replays) gives the
    eager result's bits."""
    dev = torch.device("cuda:0")
    sc = ba_scene("small")
    t = _device(sc, dev)
    eager = torch.empty((1,), dtype=torch.float64, device=dev)
    bamod.cost_noalloc(*t, eager, loss=_loss(sc), huber_delta=sc["huber_delta"],
                       stream=torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    out = torch.zeros((1,), dtype=torch.float64, device=dev)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bamod.cost_noalloc(*t, out, loss=_loss(sc), huber_delta=sc["huber_delta"],
                           stream=s.cuda_stream)
    for _ in range(3):
        out.fill_(-1.0)
        g.replay()
        torch.cuda.synchronize()
        assert float(out.item()) == float(eager.item())
        # eager work on the same scratch between replays
        other = torch.empty((1,), dtype=torch.float64, device=dev)
        tt = _device(ba_scene("tiny"), dev)
        bamod.cost_noalloc(*tt, other, stream=torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
