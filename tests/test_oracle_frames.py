"""Pins for the oracle's frame-level (fine-grained) Top-p inside kept blocks
and its attention (CPU): hand-derived cases, brute force over subsets,
coordinate arithmetic, the p_frame = 1 reduction to block routing, and torch
SDPA with a token mask built from the frame masks."""
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _inputs(seed, grid, H, d, scale=1.5):
    rng = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    return [rng.standard_normal((1, N, H, d)) * s for s in (scale, scale, 1.0)]


def _golden():
    rows = []
    for line in open(os.path.join(ROOT, "tests", "golden", "frames_tiny.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        f = [x.strip() for x in line.split("|")]
        rows.append(([float(x) for x in f[0].split(",")], [int(x) for x in f[1].split(",")],
                     int(f[2]), int(f[3]), float(f[4]), int(f[5]),
                     [int(x) for x in f[6].split(",")]))
    return rows


@pytest.mark.parametrize("case", _golden())
def test_hand_derived_cases(case):
    masses, cands, bt, own_blk, pf, kf, want = case
    nf = (max(cands) // bt + 1) * bt + bt
    scores = np.full(nf, -50.0)
    cand = np.zeros(nf, dtype=bool)
    for mval, f in zip(masses, cands):
        scores[f] = math.log(mval)
        cand[f] = True
    keep, _ = O.select_frames_row(scores, cand, range(own_blk * bt, (own_blk + 1) * bt), pf, kf)
    assert sorted(np.nonzero(keep)[0].tolist()) == want


def test_frame_members_by_coordinates():
    geo = O.geometry((5, 6, 7), (2, 4, 4))
    fm = O.frame_members(geo)
    bt, bh, bw = geo.block
    T, Hg, W = geo.grid
    _, nbh, nbw = geo.nblk
    seen = set()
    for t in range(T):
        for h in range(Hg):
            for w in range(W):
                n = (t * Hg + h) * W + w
                j = ((t // bt) * nbh + h // bh) * nbw + w // bw
                tau = t % bt
                assert n in fm[j, tau]
                seen.add(n)
    assert sorted(seen) == sorted(fm[fm >= 0].tolist())


def test_frame_pool_by_coordinates():
    grid, block = (5, 6, 7), (2, 4, 4)
    geo = O.geometry(grid, block)
    X = _inputs(3, grid, 2, 8)[0]
    Kf, counts = O.frame_pool(X, geo)
    T, Hg, W = grid
    bt, bh, bw = block
    _, nbh, nbw = geo.nblk
    sums = np.zeros((geo.nb, bt, 2, 8))
    cnt = np.zeros((geo.nb, bt), dtype=np.int64)
    for t in range(T):
        for h in range(Hg):
            for w in range(W):
                j = ((t // bt) * nbh + h // bh) * nbw + w // bw
                sums[j, t % bt] += X[0, (t * Hg + h) * W + w]
                cnt[j, t % bt] += 1
    assert np.array_equal(cnt, counts)
    ok = cnt > 0
    ref = np.zeros_like(sums)
    ref[ok] = sums[ok] / cnt[ok][:, None, None]
    np.testing.assert_allclose(Kf[0].transpose(1, 2, 0, 3), ref, atol=1e-12, rtol=0)
    assert (counts[:, 1] == 0).sum() == geo.nblk[1] * geo.nblk[2]   # last t-block: one frame


@pytest.mark.parametrize("seed", range(12))
def test_minimal_set_by_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    nf = 12
    scores = rng.normal(0, 1.5, nf)
    cand = rng.random(nf) < 0.8
    cand[0] = True
    pf = float(rng.uniform(0.2, 0.99))
    kf = int(rng.integers(1, 4))
    keep, dg = O.select_frames_row(scores, cand, [], pf, kf)
    idx = np.nonzero(cand)[0]
    pc = np.exp(scores[idx] - scores[idx].max())
    pc /= pc.sum()
    best = None
    for mask in range(1, 1 << idx.size):
        sel = [b for b in range(idx.size) if (mask >> b) & 1]
        mass = pc[sel].sum()
        if mass >= pf - 1e-12:
            if best is None or len(sel) < best[0] or (len(sel) == best[0] and mass > best[1]):
                best = (len(sel), mass, sel)
    size = max(best[0], min(kf, idx.size))
    if size == best[0]:
        want = set(idx[best[2]].tolist())
    else:   # the floor binds: the `size` largest
        want = set(idx[np.argsort(-pc, kind="stable")[:size]].tolist())
    assert set(np.nonzero(keep)[0].tolist()) == want


@pytest.mark.parametrize("pf,kf", [(0.5, 1), (0.8, 3), (0.95, 2)])
def test_invariants(pf, kf):
    grid, block = (5, 8, 12), (2, 4, 4)
    Q, K, _ = _inputs(4, grid, 2, 16, scale=2.0)
    geo = O.geometry(grid, block)
    res = O.route_frames(Q, K, geo, 0.9, 2, pf)
    fk, keep, counts = res["frame_keep"], res["keep"], res["frame_counts"]
    bt = block[0]
    Kf, _ = O.frame_pool(K, geo)
    for h in range(2):
        for i in range(geo.nb):
            row = fk[0, h, i]
            assert not row[~keep[0, h, i]].any()              # only inside kept blocks
            assert not row[counts == 0].any()                 # only frames with tokens
            assert row[i][counts[i] > 0].all()                # own block whole
            cand = np.repeat(keep[0, h, i], bt) & (counts > 0).reshape(-1)
            assert row.reshape(-1).sum() >= min(kf, cand.sum())
            sc = Kf[0, h].reshape(-1, 16) @ res["Qp"][0, h, i] / 4.0
            pc = np.where(cand, np.exp(sc - sc[cand].max()), 0.0)
            pc /= pc.sum()
            assert pc[row.reshape(-1)].sum() >= pf - 1e-12
    # frame_mask lines up with the CSR
    rp, ci, fm = res["row_ptr"], res["col_idx"], res["frame_mask"]
    for r in range(2 * geo.nb):
        h, i = divmod(r, geo.nb)
        for e in range(rp[r], rp[r + 1]):
            bits = [(int(fm[e]) >> t) & 1 for t in range(bt)]
            assert bits == fk[0, h, i, ci[e]].astype(int).tolist()


def test_p_frame_one_keeps_every_frame_of_every_kept_block():
    grid, block = (5, 8, 12), (2, 4, 4)
    Q, K, V = _inputs(5, grid, 2, 16)
    geo = O.geometry(grid, block)
    res = O.route_frames(Q, K, geo, 0.8, 2, 1.0)
    counts = res["frame_counts"]
    want = [sum(1 << t for t in range(block[0]) if counts[j, t] > 0) for j in res["col_idx"]]
    assert res["frame_mask"].tolist() == want
    Of = O.sparse_attention_frames(Q, K, V, geo, res["row_ptr"], res["col_idx"], res["frame_mask"])
    Ob = O.sparse_attention(Q, K, V, geo, res["row_ptr"], res["col_idx"])
    np.testing.assert_allclose(Of, Ob, atol=1e-12, rtol=0)


def _sdpa(Q, K, V, mask):
    q = torch.from_numpy(Q).permute(0, 2, 1, 3)
    k = torch.from_numpy(K).permute(0, 2, 1, 3)
    v = torch.from_numpy(V).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v,
                                                         attn_mask=torch.from_numpy(mask)[None])
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("pf", [0.6, 0.9])
def test_attention_equals_masked_sdpa(pf):
    grid, block = (5, 6, 7), (2, 4, 4)
    Q, K, V = _inputs(6, grid, 2, 8, scale=2.5)
    geo = O.geometry(grid, block)
    res = O.route_frames(Q, K, geo, 0.85, 2, pf)
    rp, ci, fm = res["row_ptr"], res["col_idx"], res["frame_mask"]
    T, Hg, W = grid
    bt, bh, bw = block
    _, nbh, nbw = geo.nblk
    N = T * Hg * W
    blk = np.empty(N, dtype=np.int64)
    tau = np.empty(N, dtype=np.int64)
    for t in range(T):
        for h in range(Hg):
            for w in range(W):
                n = (t * Hg + h) * W + w
                blk[n] = ((t // bt) * nbh + h // bh) * nbw + w // bw
                tau[n] = t % bt
    mask = np.zeros((2, N, N), dtype=bool)
    for h in range(2):
        for n in range(N):
            r = h * geo.nb + blk[n]
            kept = {(int(ci[e]), t) for e in range(rp[r], rp[r + 1]) for t in range(bt)
                    if (int(fm[e]) >> t) & 1}
            mask[h, n] = [(blk[m], tau[m]) in kept for m in range(N)]
    ref = _sdpa(Q, K, V, mask)
    got = O.sparse_attention_frames(Q, K, V, geo, rp, ci, fm)
    np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)
    # a planted mistake: dropping one kept frame changes the output
    fm2 = fm.copy()
    e = int(np.nonzero(fm2)[0][0])
    fm2[e] &= fm2[e] - 1
    if fm2.sum() < fm.sum():
        got2 = O.sparse_attention_frames(Q, K, V, geo, rp, ci, fm2)
        assert not np.allclose(got2, ref, atol=1e-9)
