"""Pins for the oracle's slack fill and work schedule (CPU)."""
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_slack_golden():
    n = 0
    with open(os.path.join(GOLDEN, "slack_tiny.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            nb, P, keep, slack, want = [c.strip() for c in line.split("|")]
            nb = int(nb)
            P = np.array([float(x) for x in P.split(",")]).reshape(1, 1, nb, nb)
            keep = np.array([int(x) for x in keep.split(",")], dtype=bool).reshape(1, 1, nb, nb)
            want = np.array([int(x) for x in want.split(",")], dtype=bool).reshape(1, 1, nb, nb)
            got, _ = O.slack_fill(P, keep, float(slack))
            np.testing.assert_array_equal(got, want, err_msg=line)
            n += 1
    assert n == 4


def _slack_bruteforce(P, keep, slack):
    """Independent per-head fill using Python's sort on (-P, linear index)."""
    out = keep.copy()
    B, H, nb, _ = P.shape
    budget = math.ceil(slack * nb * nb)
    for b in range(B):
        for h in range(H):
            pairs = [(i, j) for i in range(nb) for j in range(nb) if not keep[b, h, i, j]]
            pairs.sort(key=lambda ij: (-P[b, h, ij[0], ij[1]], ij[0] * nb + ij[1]))
            need = budget - int(keep[b, h].sum())
            for i, j in pairs[:max(need, 0)]:
                out[b, h, i, j] = True
    return out


@pytest.mark.parametrize("seed", range(6))
def test_slack_fill_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    grid, block, H, d = (3, 6, 7), (2, 4, 4), 3, 8
    N = grid[0] * grid[1] * grid[2]
    Q = rng.standard_normal((1, N, H, d)) * 3
    K = rng.standard_normal((1, N, H, d)) * 3
    geo = O.geometry(grid, block)
    slack = float(rng.choice([0.3, 0.5, 0.8]))
    res = O.route(Q, K, geo, 0.5, 1, slack=slack)
    ref = _slack_bruteforce(res["P"], res["base_keep"], slack)
    np.testing.assert_array_equal(res["keep"], ref)
    budget = math.ceil(slack * geo.nb ** 2)
    for h in range(H):
        base = int(res["base_keep"][0, h].sum())
        got = int(res["keep"][0, h].sum())
        assert got == max(base, budget)
        added = res["keep"][0, h] & ~res["base_keep"][0, h]
        unkept = ~res["keep"][0, h]
        if added.any() and unkept.any():
            assert res["P"][0, h][added].min() >= res["P"][0, h][unkept].max()


def _check_schedule(order, counts, key):
    rows = counts.size
    assert sorted(order.tolist()) == list(range(rows))
    keys = [key(r) for r in order]
    assert keys == sorted(keys)


def test_schedule_modes():
    rng = np.random.default_rng(0)
    counts = rng.integers(1, 9, 60)
    np.testing.assert_array_equal(O.schedule(counts, "head_major"), np.arange(60))
    o = O.schedule(counts, "nnz_sorted")
    _check_schedule(o, counts, lambda r: (-counts[r], r))
    o = O.schedule(counts, "head_phased", items_per_head=10, heads_per_phase=2)
    _check_schedule(o, counts, lambda r: (r // 20, -counts[r], r))
    # an explicit tiny case
    c = [2, 5, 5, 1, 5, 2]
    assert O.schedule(c, "nnz_sorted").tolist() == [1, 2, 4, 0, 5, 3]
    assert O.schedule(c, "head_phased", items_per_head=3).tolist() == [1, 2, 0, 4, 5, 3]


def test_schedule_xcd_local_hand_case():
    """Five heads of two items each on two queues, worked by hand.  Head costs
    5, 9, 4, 9, 1; placed cost descending with ties by head (1, 3, 0, 2, 4),
    each onto the least loaded queue with ties by queue: 1 -> q0 (9, 0),
    3 -> q1 (9, 9), 0 -> q0 (14, 9), 2 -> q1 (14, 13), 4 -> q1 (14, 14).
    Queue 0 lists heads 1, 0 and queue 1 heads 3, 2, 4, each head's items in
    natural order."""
    c = [3, 2, 4, 5, 2, 2, 9, 0, 1, 0]
    got = O.schedule(c, "xcd_local", items_per_head=2, n_queues=2)
    assert got.tolist() == [2, 3, 0, 1, 6, 7, 4, 5, 8, 9]
    # one queue: heads cost descending (ties by head), items natural
    assert O.schedule(c, "xcd_local", items_per_head=2, n_queues=1).tolist() == \
        [2, 3, 6, 7, 0, 1, 4, 5, 8, 9]
    # every item exactly once, for random costs and eight queues
    rng = np.random.default_rng(3)
    counts = rng.integers(0, 50, 40 * 7)
    o = O.schedule(counts, "xcd_local", items_per_head=7)
    assert sorted(o.tolist()) == list(range(counts.size))
    # items of one head stay together and in natural order
    for h in range(40):
        pos = [int(np.where(o == h * 7 + i)[0][0]) for i in range(7)]
        assert pos == list(range(pos[0], pos[0] + 7))
