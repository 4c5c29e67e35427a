"""Pins for the oracle's 3D blocking and pooling (CPU only)."""
import itertools
import os

import numpy as np
import pytest

import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                yield line


def test_block_index_golden():
    for line in _golden_rows("block_index.txt"):
        v = [int(x) for x in line.split()]
        grid, block, (t, h, w), (blk, slot, tok) = v[0:3], v[3:6], v[6:9], v[9:12]
        geo = O.geometry(grid, block)
        assert O.token_block_slot(t, h, w, geo) == (blk, slot)
        assert O.block_members(geo)[blk, slot] == tok


@pytest.mark.parametrize("grid,block,nb,padded", [
    ((4, 8, 8), (2, 4, 4), 8, (4, 8, 8)),
    ((21, 30, 52), (2, 8, 8), 308, (22, 32, 56)),
    ((21, 45, 80), (2, 8, 8), 660, (22, 48, 80)),
    ((81, 30, 52), (2, 8, 8), 1148, (82, 32, 56)),
])
def test_geometry_of_workloads(grid, block, nb, padded):
    geo = O.geometry(grid, block)
    assert geo.nb == nb and geo.padded == padded


@pytest.mark.parametrize("grid,block", [((4, 8, 8), (2, 4, 4)), ((3, 5, 7), (2, 2, 4)),
                                        ((5, 6, 9), (2, 4, 4)), ((1, 3, 3), (1, 2, 2))])
def test_members_are_a_bijection_and_boxed(grid, block):
    geo = O.geometry(grid, block)
    T, H, W = grid
    bt, bh, bw = block
    _, nbh, nbw = geo.nblk
    m = O.block_members(geo)
    real = m[m >= 0]
    assert sorted(real.tolist()) == list(range(T * H * W))
    assert (m < 0).sum() == geo.nb * geo.bt_tokens - T * H * W
    for blk in range(geo.nb):
        tb, rem = divmod(blk, nbh * nbw)
        hb, wb = divmod(rem, nbw)
        prev = None
        for slot in range(geo.bt_tokens):
            n = m[blk, slot]
            st, rem2 = divmod(slot, bh * bw)
            sh, sw = divmod(rem2, bw)
            t, h, w = tb * bt + st, hb * bh + sh, wb * bw + sw
            if n < 0:
                assert t >= T or h >= H or w >= W
                continue
            # decode the token index independently and compare coordinates
            assert (n // (H * W), (n // W) % H, n % W) == (t, h, w)
            if prev is not None:
                assert n > prev          # row-major slots visit tokens in increasing order
            prev = n


def _pool_bruteforce(X, grid, block):
    """Per-block means by plain coordinate arithmetic, no member table."""
    T, H, W = grid
    bt, bh, bw = block
    nbt, nbh, nbw = (-(-T // bt), -(-H // bh), -(-W // bw))
    B, N, Hh, d = X.shape
    sums = np.zeros((B, Hh, nbt * nbh * nbw, d))
    cnt = np.zeros(nbt * nbh * nbw)
    for t, h, w in itertools.product(range(T), range(H), range(W)):
        blk = ((t // bt) * nbh + h // bh) * nbw + w // bw
        sums[:, :, blk, :] += X[:, (t * H + h) * W + w, :, :]
        cnt[blk] += 1
    return sums / cnt[None, None, :, None]


@pytest.mark.parametrize("grid,block", [((4, 8, 8), (2, 4, 4)), ((3, 5, 7), (2, 2, 4))])
def test_pool_matches_bruteforce(grid, block):
    rng = np.random.default_rng(7)
    X = rng.standard_normal((2, grid[0] * grid[1] * grid[2], 3, 5))
    geo = O.geometry(grid, block)
    np.testing.assert_allclose(O.pool(X, geo), _pool_bruteforce(X, grid, block), rtol=0, atol=1e-13)


def test_pool_constant_and_linear():
    geo = O.geometry((3, 5, 7), (2, 2, 4))
    N = 3 * 5 * 7
    c = np.full((1, N, 2, 4), 3.25)
    np.testing.assert_array_equal(O.pool(c, geo), 3.25)
    rng = np.random.default_rng(1)
    X, Y = rng.standard_normal((2, 1, N, 2, 4))
    np.testing.assert_allclose(O.pool(2 * X - 0.5 * Y, geo),
                               2 * O.pool(X, geo) - 0.5 * O.pool(Y, geo), atol=1e-13)


def test_smallest_partial_block_counts():
    # hand-derived: the last 480p block covers 1 frame x 6 rows x 4 columns
    geo = O.geometry((21, 30, 52), (2, 8, 8))
    m = O.block_members(geo)
    valid = (m >= 0).sum(axis=1)
    assert valid[307] == 24 and valid.min() == 24 and valid.max() == 128
