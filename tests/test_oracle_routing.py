"""Pins for the oracle's pooled Top-p routing, floor, repair and CSR (CPU)."""
import itertools
import math
import os

import numpy as np
import pytest
import scipy.special

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield [c.strip() for c in line.split("|")]


def test_select_row_golden():
    n = 0
    for P, i, p, k, kept in _golden("select_rows.txt"):
        prow = np.array([float(x) for x in P.split(",")])
        got, _ = O.select_row(prow, int(i), float(p), int(k))
        assert got == [int(x) for x in kept.split(",")], (P, i, p, k)
        n += 1
    assert n >= 10


def test_probabilities_are_a_row_softmax():
    rng = np.random.default_rng(3)
    Qp, Kp = rng.standard_normal((2, 1, 2, 9, 16))
    P = O.block_probabilities(Qp, Kp)
    S = np.einsum("bhid,bhjd->bhij", Qp, Kp) / 4.0
    np.testing.assert_allclose(P, scipy.special.softmax(S, axis=-1), rtol=1e-13, atol=0)
    np.testing.assert_allclose(P.sum(-1), 1.0, atol=1e-14)
    assert (P > 0).all()


@pytest.mark.parametrize("nb,p,m_expected", [(8, 0.9, 8), (308, 0.9, 278), (308, 0.45, 139), (10, 0.25, 3)])
def test_uniform_row_closed_form(nb, p, m_expected):
    # identical pooled keys give P = 1/nb exactly tied; m = ceil(p * nb) and the
    # lowest indices are kept: 277/308 < 0.9 <= 278/308.
    Kp = np.ones((1, 1, nb, 4))
    Qp = np.random.default_rng(0).standard_normal((1, 1, nb, 4))
    P = O.block_probabilities(Qp, Kp)
    np.testing.assert_allclose(P, 1.0 / nb, rtol=1e-14)
    for i in (0, nb // 2, nb - 1):
        kept, dg = O.select_row(P[0, 0, i], i, p, 1)
        assert dg["m"] == m_expected == math.ceil(p * nb - 1e-9)
        assert kept == sorted(set(range(m_expected)) | {i})


def _bruteforce_min_set(prow, p):
    """Smallest cardinality reaching p, and the max-mass set among those."""
    nb = len(prow)
    for size in range(1, nb + 1):
        best = None
        for sub in itertools.combinations(range(nb), size):
            mass = sum(prow[j] for j in sub)
            if mass >= p and (best is None or mass > best[0]):
                best = (mass, set(sub))
        if best is not None:
            return size, best[1]
    return nb, set(range(nb))


@pytest.mark.parametrize("seed", range(12))
def test_topp_is_minimal_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    nb = int(rng.integers(3, 11))
    logits = rng.standard_normal(nb) * rng.uniform(0.5, 3.0)
    prow = scipy.special.softmax(logits)
    for p in (0.3, 0.6, 0.9, 0.97):
        size, best = _bruteforce_min_set(prow, p)
        i = int(rng.integers(nb))
        kept, dg = O.select_row(prow, i, p, 1)
        assert dg["m"] == size
        assert set(kept) == best | {i}


@pytest.mark.parametrize("seed", range(4))
def test_floor_limit_is_stable_topk(seed):
    rng = np.random.default_rng(seed)
    nb = 12
    prow = scipy.special.softmax(rng.integers(0, 4, nb).astype(float))   # many exact ties
    for k in (1, 2, 5, 12, 20):
        for i in (0, 7):
            kept, _ = O.select_row(prow, i, 1e-12, k)
            ref = sorted(range(nb), key=lambda j: (-prow[j], j))[:min(k, nb)]
            assert kept == sorted(set(ref) | {i})


def _tiny_case(seed, grid=(3, 6, 7), block=(2, 4, 4), H=3, d=16):
    rng = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    Q = rng.standard_normal((1, N, H, d)) * 2
    K = rng.standard_normal((1, N, H, d)) * 2
    return O.geometry(grid, block), Q, K


@pytest.mark.parametrize("p,k", [(0.5, 1), (0.9, 2), (0.99, 3), (1.0, 1), (0.3, 20)])
def test_route_invariants(p, k):
    geo, Q, K = _tiny_case(11)
    res = O.route(Q, K, geo, p, k)
    nb = geo.nb
    rp, ci = res["row_ptr"], res["col_idx"]
    P = res["P"].reshape(-1, nb)
    assert rp[0] == 0 and rp[-1] == ci.size
    for r in range(rp.size - 1):
        cols = ci[rp[r]:rp[r + 1]]
        i = r % nb
        assert (np.diff(cols) > 0).all()
        assert i in cols
        assert cols.size >= min(k, nb)
        assert P[r, cols].sum() >= min(p, 1.0) - 1e-12
        if p >= 1.0:
            assert cols.size == nb
    assert res["head_nnz"].sum() == ci.size
    back = O.csr_to_keep(rp, ci, 1, Q.shape[2], nb)
    np.testing.assert_array_equal(back, res["keep"])


def test_route_matches_select_row():
    geo, Q, K = _tiny_case(5, grid=(4, 8, 8), block=(2, 4, 4), H=2, d=8)
    res = O.route(Q, K, geo, 0.8, 2)
    nb = geo.nb
    P = res["P"]
    for h in range(2):
        for i in range(nb):
            kept, dg = O.select_row(P[0, h, i], i, 0.8, 2)
            assert kept == np.nonzero(res["keep"][0, h, i])[0].tolist()
            assert dg["m"] == res["diag"]["m"][0, h, i]


def test_route_nan_input_keeps_csr_well_formed():
    geo, Q, K = _tiny_case(9)
    Q[0, 5, 1, 3] = np.nan
    K[0, 17, 2, 0] = np.inf
    res = O.route(Q, K, geo, 0.9, 2)
    nb = geo.nb
    rp, ci = res["row_ptr"], res["col_idx"]
    for r in range(rp.size - 1):
        cols = ci[rp[r]:rp[r + 1]]
        assert 1 <= cols.size <= nb and (r % nb) in cols
        assert (np.diff(cols) > 0).all() and cols.min() >= 0 and cols.max() < nb


def test_exemption_rule_flags_only_fragile_rows():
    # a row whose mass lands exactly on p is fragile; one far from p is not
    prow = np.array([0.5, 0.25, 0.125, 0.125])
    _, dg = O.select_row(prow, 0, 0.75, 1)
    ex = O.row_exemptions({k: np.array([v]) for k, v in dg.items()}, 0.75, 1)
    assert ex[0]
    _, dg = O.select_row(prow, 0, 0.7, 1)
    ex = O.row_exemptions({k: np.array([v]) for k, v in dg.items()}, 0.7, 1)
    assert not ex[0]
    # floor decides the count: exact even though the mass sits on p
    _, dg = O.select_row(prow, 0, 0.75, 3)
    ex = O.row_exemptions({k: np.array([v]) for k, v in dg.items()}, 0.75, 3)
    assert not ex[0]
    # near tie at the cut
    prow = np.array([0.4, 0.2, 0.2 * (1 - 1e-7), 0.2 * (1 + 1e-7) - 1e-12])
    prow = prow / prow.sum()
    _, dg = O.select_row(prow, 0, 0.5, 1)
    ex = O.row_exemptions({k: np.array([v]) for k, v in dg.items()}, 0.5, 1)
    assert ex[0]
