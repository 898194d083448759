"""Pins for the oracle's sparsity structure: observation orderings and CSR
offsets against numpy's lexsort / bincount, brute force on small inputs, and
the input validation error paths."""
import numpy as np
import pytest

import oracle
from synthetic import ba_scene


def _brute_perm(primary, secondary):
    n = len(primary)
    return np.array(sorted(range(n), key=lambda k: (primary[k], secondary[k], k)), dtype=np.int32)


@pytest.mark.parametrize("config", ["tiny", "small"])
def test_orderings_match_lexsort(config):
    sc = ba_scene(config)
    P = oracle.Problem.from_scene(sc)
    k = np.arange(len(sc["obs_cam"]))
    np.testing.assert_array_equal(P.get("perm_pt"), np.lexsort((k, sc["obs_cam"], sc["obs_pt"])))
    np.testing.assert_array_equal(P.get("perm_cam"), np.lexsort((k, sc["obs_pt"], sc["obs_cam"])))
    np.testing.assert_array_equal(
        P.get("pt_ptr"), np.concatenate([[0], np.cumsum(np.bincount(sc["obs_pt"], minlength=P.np))]))
    np.testing.assert_array_equal(
        P.get("cam_ptr"), np.concatenate([[0], np.cumsum(np.bincount(sc["obs_cam"], minlength=P.nc))]))


def test_orderings_brute_force_with_duplicates_and_empty_segments():
    rng = np.random.default_rng(11)
    nc, npt, n = 5, 9, 60
    oc = rng.integers(0, nc - 1, size=n).astype(np.int32)      # camera nc-1 never observed
    op = rng.integers(0, npt - 2, size=n).astype(np.int32)     # last two points never observed
    oc[10:14] = 2
    op[10:14] = 3                                               # repeated (camera, point) pair
    cams = np.tile([0.0, 0, 0, 0, 0, 20.0, 500.0, 0, 0], (nc, 1))
    pts = rng.uniform(-1, 1, size=(npt, 3))
    uv = rng.normal(size=(n, 2))
    P = oracle.Problem(cams, pts, oc, op, uv)
    np.testing.assert_array_equal(P.get("perm_pt"), _brute_perm(op, oc))
    np.testing.assert_array_equal(P.get("perm_cam"), _brute_perm(oc, op))
    ptr = P.get("pt_ptr")
    assert ptr[-1] == ptr[-2] == ptr[-3] == n
    cptr = P.get("cam_ptr")
    assert cptr[-1] == cptr[-2] == n


def test_invalid_inputs_are_rejected():
    cams = np.tile([0.0, 0, 0, 0, 0, 20.0, 500.0, 0, 0], (2, 1))
    pts = np.zeros((3, 3))
    uv = np.zeros((2, 2))
    with pytest.raises(RuntimeError):
        oracle.Problem(cams, pts, [0, 2], [0, 1], uv)            # camera index out of range
    with pytest.raises(RuntimeError):
        oracle.Problem(cams, pts, [0, 1], [0, -1], uv)           # negative point index
    bad = uv.copy()
    bad[1, 0] = np.nan
    with pytest.raises(RuntimeError):
        oracle.Problem(cams, pts, [0, 1], [0, 1], bad)           # non-finite observation
