"""The GPU tests' comparison helpers, checked on the CPU with masks the oracle
made and mistakes planted in copies of them."""
import numpy as np
import pytest

import oracle as O
import synth_inputs as si
from parity_utils import MAX_EXEMPT_DIFFERING, compare_masks


@pytest.fixture(scope="module")
def routed():
    wl = si.Workload(801, "helpers", 1, 2, 64, "f32", (8, 32, 32), (2, 4, 4), (0.9,), 2, 0.0,
                     "u13")
    q, k, _ = si.make_inputs(wl)
    geo = O.geometry(wl.grid, wl.block)
    p = float(np.float32(0.9))
    return O.route(q.numpy(), k.numpy(), geo, p, 2), p


def test_exemption_causes_make_up_the_rule(routed):
    res, p = routed
    close, near = O.row_exemption_causes(res["diag"], p, 2)
    assert np.array_equal(close | near, O.row_exemptions(res["diag"], p, 2))
    assert not O.row_exemption_causes(res["diag"], 1.0, 2)[0].any()


def test_identical_masks_pass_with_counts(routed):
    res, p = routed
    c = compare_masks(res["keep"].copy(), res, p, 2)
    rows = res["keep"].shape[1] * res["keep"].shape[2]
    assert c["mismatched"] == 0 and c["exempt_differing"] == 0
    assert c["exact"] + c["exempt"] == rows
    assert c["exempt_mass_close"] + c["exempt_near_tie"] == c["exempt"]


def test_a_changed_exact_row_fails(routed):
    res, p = routed
    exempt = O.row_exemptions(res["diag"], p, 2)
    h, i = map(int, np.argwhere(~exempt[0])[0])
    bad = res["keep"].copy()
    j = int(np.nonzero(~bad[0, h, i])[0][0]) if (~bad[0, h, i]).any() else (i + 1) % bad.shape[-1]
    bad[0, h, i, j] = ~bad[0, h, i, j]
    with pytest.raises(AssertionError):
        compare_masks(bad, res, p, 2)


def test_too_many_differing_exempt_rows_fail(routed):
    # every exempt row whose set can move by one block without breaking the
    # per-row invariants is changed: more than the allowed fraction differ
    res, p = routed
    keep = res["keep"].copy()
    exempt = O.row_exemptions(res["diag"], p, 2)
    P = res["P"]
    changed = 0
    for h, i in map(tuple, np.argwhere(exempt[0])):
        row = keep[0, h, i]
        cand = [j for j in np.nonzero(~row)[0]]
        if cand:
            row[cand[0]] = True          # one more block: mass and floor still hold
            changed += 1
    rows = keep.shape[1] * keep.shape[2]
    if changed <= MAX_EXEMPT_DIFFERING * rows:
        pytest.skip("too few exempt rows in this fixture to exceed the bound")
    with pytest.raises(AssertionError):
        compare_masks(keep, res, p, 2)
