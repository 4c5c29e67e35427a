"""Pins for the oracle's dynamic slack fill and its telemetry budget (CPU)."""
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield [c.strip() for c in line.split("|")]


def test_dynamic_fill_golden():
    n = 0
    for P, keep, budget, theta, want in _lines("dynamic_slack_tiny.txt"):
        P = np.array([float(x) for x in P.split(",")]).reshape(1, 2, 2, 2)
        keep = np.array([int(x) for x in keep.split(",")], dtype=bool).reshape(1, 2, 2, 2)
        want = np.array([int(x) for x in want.split(",")], dtype=bool).reshape(1, 2, 2, 2)
        got, info = O.dynamic_slack_fill(P, keep, int(budget), float(theta))
        np.testing.assert_array_equal(got, want)
        assert info["added"] == int(want.sum() - keep.sum())
        n += 1
    assert n == 5


def test_budget_golden():
    n = 0
    for recs, fill, max_pairs, want in _lines("slack_budget_tiny.txt"):
        rows = [[0, 0] + [int(x) for x in r.split(":")] for r in recs.split(";")]
        assert O.slack_budget(rows, float(fill), int(max_pairs)) == int(want)
        n += 1
    assert n == 6


def _fill_bruteforce(P, keep, budget, theta):
    """Independent fill: Python's sorted over (-P, linear index) of every pair."""
    B, H, nb, _ = P.shape
    out = keep.copy()
    pairs = []
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                for j in range(nb):
                    if not keep[b, h, i, j] and P[b, h, i, j] >= theta:
                        pairs.append((-P[b, h, i, j], ((b * H + h) * nb + i) * nb + j, (b, h, i, j)))
    for _, _, idx in sorted(pairs)[:budget]:
        out[idx] = True
    return out


@pytest.mark.parametrize("seed", range(8))
def test_dynamic_fill_matches_bruteforce(seed):
    rng = np.random.default_rng(seed)
    B, H, nb = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(2, 7))
    # quantised probabilities so that ties are common
    P = rng.integers(0, 6, size=(B, H, nb, nb)) / 8.0
    keep = rng.random((B, H, nb, nb)) < 0.4
    budget = int(rng.integers(0, B * H * nb * nb + 2))
    theta = float(rng.choice([0.0, 0.125, 0.3, 0.6]))
    got, info = O.dynamic_slack_fill(P, keep, budget, theta)
    np.testing.assert_array_equal(got, _fill_bruteforce(P, keep, budget, theta))
    assert (got >= keep).all()                                  # only adds
    added = got & ~keep
    assert info["added"] == int(added.sum()) == min(budget, info["candidates"])
    assert (P[added] >= theta).all()
    if info["added"] and info["added"] < info["candidates"]:
        assert P[added].min() >= np.max(P[~got & (P >= theta)])   # nothing better left out


def test_dynamic_fill_monotone_in_budget():
    rng = np.random.default_rng(5)
    P = rng.random((1, 2, 5, 5))
    keep = rng.random(P.shape) < 0.3
    prev = keep
    for budget in range(0, 40, 3):
        got, _ = O.dynamic_slack_fill(P, keep, budget, 0.1)
        assert (got >= prev).all()
        prev = got


def test_budget_properties():
    # equal busy: no idle capacity
    assert O.slack_budget([[0, 0, 5, 77]] * 9, 1.0, 10 ** 9) == 0
    # two workers: closed form floor(fill * (T - b) * tiles / (T + b))
    for T, b, tiles, fill in ((1000, 600, 80, 1.0), (999, 1, 7, 0.3), (5, 4, 1000, 0.9)):
        want = math.floor(fill * (T - b) * tiles / (T + b))
        assert O.slack_budget([[0, 0, tiles, T], [0, 0, 0, b]], fill, 10 ** 9) == want
    assert O.slack_budget([[0, 0, 10, 100], [0, 0, 10, 50]], 0.0, 10 ** 9) == 0
    assert O.slack_budget([[0, 0, 10, 100], [0, 0, 10, 50]], 1.0, 2) == 2
