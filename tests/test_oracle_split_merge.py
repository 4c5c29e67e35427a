"""Pins for the oracle's split-and-merge pieces (CPU): the cut of heavy work
items into parts, and the log-sum-exp merge of partial attentions."""
import math
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _triples(text, width):
    text = text.strip()
    if not text:
        return []
    out = [tuple(int(x) for x in part.split()) for part in text.split(";")]
    assert all(len(t) == width for t in out)
    return out


def test_split_units_golden():
    n = 0
    with open(os.path.join(GOLDEN, "split_units_tiny.txt")) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            counts, split, max_parts, units, cut = [c.strip() for c in line.split("|")]
            counts = [int(x) for x in counts.split(",")]
            got_u, got_c = O.split_units(counts, int(split), int(max_parts))
            assert got_u == _triples(units, 4), line
            assert got_c == _triples(cut, 3), line
            n += 1
    assert n == 8


@pytest.mark.parametrize("seed", range(8))
def test_split_units_invariants(seed):
    rng = np.random.default_rng(seed)
    counts = rng.integers(0, 40, size=int(rng.integers(1, 60)))
    split = int(rng.integers(1, 12))
    max_parts = int(rng.integers(0, 120))
    units, cut = O.split_units(counts, split, max_parts)
    # units tile every item's list, in order, with non-empty near-equal parts
    by_item = {}
    for item, t0, t1, slot in units:
        by_item.setdefault(item, []).append((t0, t1, slot))
    assert [u[0] for u in units] == sorted(u[0] for u in units)
    assert sorted(by_item) == list(range(len(counts)))
    heavy_seen, cut_items = 0, []
    for item, parts in by_item.items():
        nt = int(counts[item])
        assert parts[0][0] == 0 and parts[-1][1] == nt
        assert all(a[1] == b[0] for a, b in zip(parts, parts[1:]))
        if len(parts) > 1:
            lens = [t1 - t0 for t0, t1, _ in parts]
            assert min(lens) >= 1 and max(lens) - min(lens) <= 1
            assert len(parts) == math.ceil(nt / split) and nt > split
            cut_items.append(item)
        else:
            assert parts[0][2] == -1
    # slots: consecutive from 0, within the budget; the cut items are the
    # heaviest of those that want cutting (nt descending, ties by index), and
    # the next of them would not have fitted
    slots = [s for _, _, _, s in units if s >= 0]
    assert slots == list(range(len(slots))) and len(slots) <= max_parts
    wanting = sorted((i for i, nt in enumerate(counts) if nt > split),
                     key=lambda i: (-counts[i], i))
    assert sorted(cut_items) == sorted(wanting[:len(cut_items)])
    if len(cut_items) < len(wanting):
        nxt = wanting[len(cut_items)]
        assert len(slots) + math.ceil(counts[nxt] / split) > max_parts
    assert [c[0] for c in cut] == cut_items
    for item, slot0, parts in cut:
        assert [s for _, _, s in by_item[item]] == list(range(slot0, slot0 + parts))


def _dense(q, k, v):
    s = q @ k.T / math.sqrt(q.shape[1])
    s -= s.max(axis=1, keepdims=True)
    w = np.exp(s)
    return (w / w.sum(axis=1, keepdims=True)) @ v


@pytest.mark.parametrize("seed", range(6))
def test_merge_of_disjoint_parts_is_attention_over_the_union(seed):
    rng = np.random.default_rng(100 + seed)
    n, m, d = 7, int(rng.integers(5, 50)), 16
    scale = float(rng.choice([0.5, 3.0, 12.0]))         # up to very peaked softmax
    q = rng.standard_normal((n, d)) * scale
    k = rng.standard_normal((m, d)) * scale
    v = rng.standard_normal((m, d))
    nparts = int(rng.integers(1, 6))
    label = rng.integers(0, nparts, size=m)               # random disjoint key sets
    parts = [O.partial_attention(q, k[label == p], v[label == p]) for p in range(nparts)]
    got = O.merge_partials(parts)
    np.testing.assert_allclose(got, _dense(q, k, v), rtol=1e-10, atol=1e-12)


def test_partial_attention_lse_and_empty_part():
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((3, 8)) for _ in range(3))
    o, lse = O.partial_attention(q, k, v)
    s = q @ k.T / math.sqrt(8)
    np.testing.assert_allclose(lse, np.log(np.exp(s).sum(axis=1)), rtol=1e-12)
    np.testing.assert_allclose(o, _dense(q, k, v), rtol=1e-12)
    oe, le = O.partial_attention(q, k[:0], v[:0])
    assert (oe == 0).all() and np.isneginf(le).all()
    # an empty part changes nothing
    np.testing.assert_allclose(O.merge_partials([(o, lse), (oe, le)]), o, rtol=1e-12)
    with pytest.raises(ValueError):
        O.merge_partials([(oe, le)])
