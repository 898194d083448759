"""ba_solve queues its LM steps without reading each one back: the accept or
reject decision, the damping update and the copy of an accepted trial into the
current parameters run on the device.  These tests hold it to the step-by-step
path (ba_lm_step, whose decision is taken on the host): same decisions, same
arithmetic, so the parameters, cost, damping and iteration count must agree
bit for bit, and the summary must add up the per-step records.

Each case stops before the LM reaches the rounding level of its cost sum: on
the small scene the relative cost change is 3e-13 at the fifth step and at
most 4e-15 after it, where the decision rests on the last bit of the cost and
either one is correct (the stored-trace tests draw the same line).  The other
scenes stay above 1e-3 over the steps compared.
"""
import numpy as np
import pytest

from synthetic import ba_scene

from test_gpu_ba_parity import _edge_scene

pytestmark = pytest.mark.gpu

bamod = pytest.importorskip("nonlinear_least_squares_amd.ba")


def _same_state(a, b):
    ca, pa = a.get_params()
    cb, pb = b.get_params()
    assert np.array_equal(ca, cb) and np.array_equal(pa, pb)
    assert a.get_state() == b.get_state()


def _scene(name):
    if name == "edge":
        return _edge_scene(), {}
    if name == "medium-dense":
        return ba_scene("medium"), dict(solver=bamod.BA_SOLVER_DENSE_SCHUR)
    return ba_scene(name), {}


@pytest.mark.parametrize("name,n", [("small", 5), ("edge", 8), ("medium", 6),
                                    ("medium-dense", 5), ("wide", 4), ("large", 20)])
def test_queued_solve_matches_steps(name, n):
    sc, kw = _scene(name)
    print(f"queued solve against steps: {name}, {n} LM iterations", flush=True)
    a = bamod.Problem.from_scene(sc, **kw)
    b = bamod.Problem.from_scene(sc, **kw)
    tr = [a.lm_step() for _ in range(n)]
    s = b.solve(n)
    _same_state(a, b)
    assert s["iterations"] == n
    assert s["accepted"] == sum(t["accepted"] for t in tr)
    assert s["pcg_iters_total"] == sum(t["pcg_iters"] for t in tr)
    assert s["initial_cost"] == tr[0]["cost_before"]
    assert s["final_cost"] == a.get_state()["cost"]


def test_queued_solve_mixed_with_steps():
    """Queued runs, single steps between them (the linearisation state and the
    record buffer carried across calls), and a longer run that grows the
    record buffer."""
    sc = ba_scene("small")
    a = bamod.Problem.from_scene(sc)
    b = bamod.Problem.from_scene(sc)
    for _ in range(5):
        a.lm_step()
    b.solve(1)
    b.lm_step()
    b.solve(3)
    _same_state(a, b)


def test_queued_solve_timed_counts():
    """With every launch timed, the queued run counts one point-pass launch per
    PCG iteration that ran and one linearisation per step that followed an
    accepted one (plus the first), and leaves the results unchanged."""
    sc = ba_scene("small")
    a = bamod.Problem.from_scene(sc)
    b = bamod.Problem.from_scene(sc)
    tr = [a.lm_step() for _ in range(5)]
    b.profile()
    b.solve(5)
    _same_state(a, b)
    prof = b.profile_get()
    assert prof["pcg_pt"][0] == sum(t["pcg_iters"] for t in tr)
    assert prof["lin_pt"][0] == 1 + sum(t["accepted"] for t in tr[:-1])
    assert prof["backsub"][0] == 5


def test_queued_solve_not_spd_leaves_state():
    """With no floor on the damping term an unobserved camera's damped block is
    zero: both paths report BA_ERR_NOT_SPD at the first step, and the queued
    steps after it change nothing."""
    sc = _edge_scene()
    a = bamod.Problem.from_scene(sc, diag_floor=0.0)
    b = bamod.Problem.from_scene(sc, diag_floor=0.0)
    c0, p0 = b.get_params()
    st0 = b.get_state()
    with pytest.raises(bamod.BAError) as e:
        a.lm_step()
    assert e.value.code == bamod.BA_ERR_NOT_SPD
    with pytest.raises(bamod.BAError) as e:
        b.solve(3)
    assert e.value.code == bamod.BA_ERR_NOT_SPD
    _same_state(a, b)
    c1, p1 = b.get_params()
    assert np.array_equal(c0, c1) and np.array_equal(p0, p1)
    assert b.get_state() == st0
