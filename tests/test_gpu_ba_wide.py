"""Parity on the wide scene (1,500 ring cameras, 90,000 points, about 495,000
observations, Huber loss): more cameras than whole camera rows fit in one
compute unit's LDS, so the library chooses by size, with no switch, the
vectors layout: the PCG and back-substitution point passes keep only the
cameras' 9-vectors in LDS and read each observation's camera geometry from
memory.  The PCG and LM tests also run the memory layout (everything read from
memory, chosen by size past 2,240 cameras) under its environment switch.

Bars as for the other scenes: every block of the linearisation within 1e-10,
the blocks built from inverted point blocks within their first-order bound,
the PCG camera step within 1e-8 at the oracle's iteration count, the point
step within 1e-8, and a three-step LM trace with the final cost within 1e-6.
"""
import numpy as np
import pytest

import oracle
from synthetic import ba_scene

from test_gpu_ba_parity import (blocks_close, inverse_bounds, residual_bounds, traces_agree,
                                use_camera_table)

pytestmark = pytest.mark.gpu

bamod = pytest.importorskip("nonlinear_least_squares_amd.ba")


@pytest.fixture(scope="module")
def wide():
    return ba_scene("wide")


def test_wide_linearisation_and_schur(wide):
    sc = wide
    g = bamod.Problem.from_scene(sc)
    o = oracle.Problem.from_scene(sc)
    g.debug_run(bamod.BA_STAGE_SCHUR)
    o.linearize()
    o.damp()
    o.schur()
    for name in ("r", "Jc", "Jp", "w", "B", "gc", "C", "gp", "Bd"):
        got, ref = g.debug_get(name), o.get(name)
        if name == "w":
            got, ref = got[:, None], ref[:, None]
        blocks_close(name, got, ref, residual_bounds(o, sc) if name == "r" else 1e-10)
    tols = inverse_bounds(o, sc)
    for name in ("Cinv", "v", "rhs", "M"):
        blocks_close(name, g.debug_get(name), o.get(name), tols[name])


@pytest.mark.parametrize("cameras", ["vectors", "memory"])
def test_wide_pcg_and_backsubstitution(wide, cameras, monkeypatch):
    use_camera_table(cameras, monkeypatch)
    sc = wide
    g = bamod.Problem.from_scene(sc)
    o = oracle.Problem.from_scene(sc)
    g.debug_run(bamod.BA_STAGE_UPDATE)
    o.linearize()
    o.damp()
    o.schur()
    it, rel = o.pcg(sc["pcg_max_iters"], sc["pcg_rel_tol"])
    o.backsub()
    o.retract()
    g_it, g_rel = g.debug_get("pcg")
    assert int(g_it) == it, (g_it, it)
    dc, dc_ref = g.debug_get("dc"), o.get("dc")
    assert np.linalg.norm(dc - dc_ref) <= 1e-8 * np.linalg.norm(dc_ref)
    dp, dp_ref = g.debug_get("dp"), o.get("dp")
    assert np.linalg.norm(dp - dp_ref) <= 1e-8 * np.linalg.norm(dp_ref)
    trial = float(g.debug_get("trial_cost")[0])
    ref = o.cost_at(o.get("cams_trial"), o.get("points_trial"))
    assert abs(trial - ref) <= 1e-8 * ref


@pytest.mark.parametrize("cameras", ["vectors", "memory"])
def test_wide_three_lm_steps(wide, cameras, monkeypatch):
    use_camera_table(cameras, monkeypatch)
    sc = wide
    g = bamod.Problem.from_scene(sc)
    o = oracle.Problem.from_scene(sc)
    g_tr = [g.lm_step() for _ in range(3)]
    o_tr = o.solve(3)
    assert traces_agree(g_tr, o_tr)
    for a, b in zip(g_tr, o_tr):
        assert a["pcg_iters"] == b["pcg_iters"]
    assert abs(g.get_state()["cost"] - o.cost) <= 1e-6 * o.cost



@pytest.mark.parametrize("n_cams", [1076, 1077])
def test_layout_boundary_scenes(n_cams):
    """The largest scene whose whole camera rows fit in LDS (1,076 cameras:
    the table fills the compute unit's LDS less room for the kernels' own LDS
    variables) and the smallest that takes the vectors layout, each created
    after a tiny handle and stepped in turn with it (the LDS limit is a
    per-process kernel attribute and must hold for every handle): the PCG
    step, the point step and three LM steps against the oracle."""
    sc = ba_scene("wide", n_cams=n_cams, n_pts=6000, seed=40 + n_cams % 2, n_iters=3)
    small = bamod.Problem.from_scene(ba_scene("tiny"))
    g = bamod.Problem.from_scene(sc)
    small.lm_step()
    o = oracle.Problem.from_scene(sc)
    g.debug_run(bamod.BA_STAGE_UPDATE)
    o.linearize()
    o.damp()
    o.schur()
    it, rel = o.pcg(sc["pcg_max_iters"], sc["pcg_rel_tol"])
    o.backsub()
    g_it, g_rel = g.debug_get("pcg")
    assert int(g_it) == it, (g_it, it)
    dc, dc_ref = g.debug_get("dc"), o.get("dc")
    assert np.linalg.norm(dc - dc_ref) <= 1e-8 * np.linalg.norm(dc_ref)
    dp, dp_ref = g.debug_get("dp"), o.get("dp")
    assert np.linalg.norm(dp - dp_ref) <= 1e-8 * np.linalg.norm(dp_ref)
    g = bamod.Problem.from_scene(sc)
    small.lm_step()
    o = oracle.Problem.from_scene(sc)
    g_tr = [g.lm_step() for _ in range(3)]
    o_tr = o.solve(3)
    assert traces_agree(g_tr, o_tr)
    assert abs(g.get_state()["cost"] - o.cost) <= 1e-6 * o.cost
