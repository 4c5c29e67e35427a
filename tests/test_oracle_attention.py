"""Pins for the oracle's block-sparse attention (CPU)."""
import numpy as np
import pytest
import torch

import oracle as O


def _inputs(seed, grid, H, d, scale=1.5):
    rng = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    return [rng.standard_normal((1, N, H, d)) * s for s in (scale, scale, 1.0)]


def _sdpa(Q, K, V, mask=None):
    """torch SDPA on the CPU in float64; mask[h] is a [N, N] bool (True = attend)."""
    q = torch.from_numpy(Q).permute(0, 2, 1, 3)
    k = torch.from_numpy(K).permute(0, 2, 1, 3)
    v = torch.from_numpy(V).permute(0, 2, 1, 3)
    m = None if mask is None else torch.from_numpy(mask)[None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m)
    return o.permute(0, 2, 1, 3).numpy()


def _token_mask(geo, row_ptr, col_idx, H):
    """Token-level mask expanded from the block CSR by coordinate arithmetic."""
    T, Hg, W = geo.grid
    bt, bh, bw = geo.block
    _, nbh, nbw = geo.nblk
    N = T * Hg * W
    blk_of = np.empty(N, dtype=np.int64)
    for t in range(T):
        for h in range(Hg):
            for w in range(W):
                blk_of[(t * Hg + h) * W + w] = ((t // bt) * nbh + h // bh) * nbw + w // bw
    mask = np.zeros((H, N, N), dtype=bool)
    for h in range(H):
        for n in range(N):
            r = h * geo.nb + blk_of[n]
            kept = set(col_idx[row_ptr[r]:row_ptr[r + 1]].tolist())
            mask[h, n] = np.isin(blk_of, list(kept))
    return mask


@pytest.mark.parametrize("grid,block", [((4, 8, 8), (2, 4, 4)), ((3, 5, 7), (2, 2, 4))])
def test_dense_when_p_is_one(grid, block):
    Q, K, V = _inputs(1, grid, 2, 16)
    geo = O.geometry(grid, block)
    res = O.route(Q, K, geo, 1.0, 1)
    Os = O.sparse_attention(Q, K, V, geo, res["row_ptr"], res["col_idx"])
    Od = O.dense_attention(Q, K, V)
    np.testing.assert_allclose(Os, Od, atol=1e-12, rtol=0)
    np.testing.assert_allclose(Od, _sdpa(Q, K, V), atol=1e-12, rtol=0)


@pytest.mark.parametrize("p,k", [(0.5, 1), (0.8, 2), (0.95, 3)])
def test_sparse_equals_masked_sdpa(p, k):
    grid, block = (3, 6, 7), (2, 4, 4)
    Q, K, V = _inputs(2, grid, 3, 8, scale=2.5)
    geo = O.geometry(grid, block)
    res = O.route(Q, K, geo, p, k)
    assert res["col_idx"].size < 3 * geo.nb * geo.nb or p >= 0.95   # really sparse at low p
    Os = O.sparse_attention(Q, K, V, geo, res["row_ptr"], res["col_idx"])
    ref = _sdpa(Q, K, V, _token_mask(geo, res["row_ptr"], res["col_idx"], 3))
    np.testing.assert_allclose(Os, ref, atol=1e-12, rtol=0)


def test_constant_values_and_single_key():
    grid, block = (1, 1, 5), (1, 1, 4)        # block 1 holds one real token (n = 4)
    Q, K, V = _inputs(3, grid, 1, 4)
    geo = O.geometry(grid, block)
    row_ptr = np.array([0, 2, 3])
    col_idx = np.array([0, 1, 1])              # row 0 keeps both, row 1 only itself
    Vc = np.full_like(V, -0.75)
    Oc = O.sparse_attention(Q, K, Vc, geo, row_ptr, col_idx)
    np.testing.assert_allclose(Oc, -0.75, atol=1e-15)
    Os = O.sparse_attention(Q, K, V, geo, row_ptr, col_idx)
    np.testing.assert_array_equal(Os[0, 4, 0], V[0, 4, 0])


def test_row_subset_leaves_others_unset():
    grid, block = (4, 8, 8), (2, 4, 4)
    Q, K, V = _inputs(4, grid, 2, 8)
    geo = O.geometry(grid, block)
    res = O.route(Q, K, geo, 0.9, 2)
    full = O.sparse_attention(Q, K, V, geo, res["row_ptr"], res["col_idx"])
    part = O.sparse_attention(Q, K, V, geo, res["row_ptr"], res["col_idx"], rows=[3, 12])
    members = O.block_members(geo)
    for r in (3, 12):
        h, i = divmod(r, geo.nb)
        tok = members[i][members[i] >= 0]
        np.testing.assert_array_equal(part[0, tok, h], full[0, tok, h])
    assert np.isnan(part).sum() == part.size - 2 * 32 * 8
