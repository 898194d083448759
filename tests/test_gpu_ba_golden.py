"""LM runs on the GPU replayed against the oracle's stored traces.

tests/golden/ba_lm_traces.json holds the oracle's per-iteration LM traces on
the medium walk scene (20 iterations), the large scene (30; the benchmark
times the first 20 from a fresh handle) and the wide scene (20), written by
tests/golden/make_ba_traces.py, which calls only the oracle and the scene
generators.

The medium scene is also replayed with the dense reduced-camera solver
("medium-dense"), the solver the eager-mode BA summary names for problems of
that size: its reduced system is too ill-conditioned for block-Jacobi PCG to
reach the 1e-6 tolerance within 50 iterations on most steps.

Bars: the accept/reject decisions and the trial costs within 1e-6 relative on
every iteration up to the first whose cost change is within the rounding noise
of the cost sums (|dC| <= 1e-10 C), after which either decision is correct;
the cost after the fixed iteration count within 1e-6 relative.  A PCG stopped
at its iteration cap leaves an iterate that rounding moves (tests/
test_pcg_formulation.py measures the spread): where the oracle accepts such a
step, the runs may branch after it, so the trace is compared up to and
including that step and the final cost is not required to match.
"""
import json
import os

import numpy as np
import pytest

from synthetic import ba_scene

from test_gpu_ba_parity import traces_agree

pytestmark = pytest.mark.gpu

bamod = pytest.importorskip("nonlinear_least_squares_amd.ba")

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "ba_lm_traces.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _compared_prefix(steps, cap):
    """Iterations to compare: all, or up to and including the first accepted
    step whose PCG stopped at the cap without reaching the tolerance."""
    for k, b in enumerate(steps):
        if b["accepted"] and b["pcg_iters"] >= cap:
            return k + 1, False
    return len(steps), True


@pytest.mark.parametrize("config,n", [("medium", 20), ("medium-dense", 20), ("large", 20),
                                      ("large", 30), ("wide", 20)])
def test_lm_trace_against_golden(golden, config, n):
    ref = golden[config]
    scene, _, solver = config.partition("-")
    sc = ba_scene(scene)
    assert len(sc["obs_cam"]) == ref["n_obs"] and len(sc["points"]) == ref["n_pts"]
    steps = ref["steps"][:n]
    kw = dict(solver=bamod.BA_SOLVER_DENSE_SCHUR) if solver == "dense" else {}
    print(f"golden trace: {config}, {n} LM iterations", flush=True)
    g = bamod.Problem.from_scene(sc, **kw)
    tr = [g.lm_step() for _ in range(n)]
    m, whole = _compared_prefix(steps, sc["pcg_max_iters"]) if not kw else (n, True)
    for k, (a, b) in enumerate(zip(tr, steps)):
        print(f"  {k:2d} gpu {a['accepted']} {a['pcg_iters']:2d} {a['cost_after']:.12e}   "
              f"oracle {b['accepted']} {b['pcg_iters']:2d} {b['cost_after']:.12e}", flush=True)
    for a, b in zip(tr[:m], steps[:m]):
        assert abs(a["cost_before"] - b["cost_before"]) <= 1e-6 * b["cost_before"]
    assert traces_agree(tr[:m], steps[:m])
    if not whole:
        print(f"  compared the first {m} iterations (iteration {m} accepted a capped PCG step)")
        return
    final, want = g.get_state()["cost"], steps[-1]["cost"]
    assert abs(final - want) <= 1e-6 * want, (final, want)
    # the same run through ba_solve, as the benchmark calls it
    h = bamod.Problem.from_scene(sc, **kw)
    s = h.solve(n)
    assert abs(s["final_cost"] - want) <= 1e-6 * want
    assert s["accepted"] == sum(t["accepted"] for t in tr)
