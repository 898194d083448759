"""Pose-graph parity at the size of the large benchmark graph (524,288 poses,
1,047,551 edges), in the launch configuration the benchmark times (256 PCG
blocks of sixteen wavefronts): sampled edges (residual and both Jacobian
blocks) against the oracle's per-edge function, and one full LM step (cost
before, trial cost, decision) against the oracle's."""
import numpy as np
import pytest

from oracle import pgo as opgo
from synthetic import pgo_scene

pytestmark = pytest.mark.gpu

pgomod = pytest.importorskip("nonlinear_least_squares_amd.pgo")


@pytest.fixture(scope="module")
def large():
    return pgo_scene("large")


def test_large_sampled_edges(large):
    sc = large
    g = pgomod.Problem.from_scene(sc)
    g.debug_run(pgomod.PGO_STAGE_LINEARIZE)
    r, Ji, Jj = g.debug_get("r"), g.debug_get("Ji"), g.debug_get("Jj")
    rng = np.random.default_rng(45)
    for e in rng.choice(len(sc["edges"]), size=2048, replace=False):
        i, j = sc["edges"][e]
        ro, Jio, Jjo = opgo.edge(sc["poses"][i], sc["poses"][j], sc["meas"][e])
        for got, ref in ((r[e], ro), (Ji[e], Jio), (Jj[e], Jjo)):
            err = np.linalg.norm(got - ref)
            assert err <= 1e-10 * max(np.linalg.norm(ref), 1e-6), (e, err)


def test_large_one_lm_step(large):
    sc = large
    print("pose graph large: one LM step on the GPU and in the oracle", flush=True)
    g = pgomod.Problem.from_scene(sc)
    gi = g.lm_step()
    o = opgo.PGOProblem.from_scene(sc)
    oi = o.lm_step()
    assert abs(gi["cost_before"] - oi["cost_before"]) <= 1e-10 * oi["cost_before"]
    assert abs(gi["cost_after"] - oi["cost_after"]) <= 1e-6 * oi["cost_after"]
    assert gi["accepted"] == oi["accepted"] and gi["pcg_iters"] == oi["pcg_iters"]
