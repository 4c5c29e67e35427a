"""Comparison helpers for the GPU parity tests (test code; uses the oracle)."""
from __future__ import annotations

import math

import numpy as np

import oracle as O

# Output tolerances: bf16 workloads max |d| <= 2e-2 and mean |d| <= 2e-3;
# float32 workload max |d| <= 1e-4 (oracle attention fed the GPU's own mask).
TOL_BF16_MAX, TOL_BF16_MEAN, TOL_F32_MAX = 2e-2, 2e-3, 1e-4


# At most this fraction of all rows may be exempt rows where the GPU and the
# oracle keep different sets (float32 deciding a near-threshold row the other
# way); rows outside the exemption rule may differ nowhere.
MAX_EXEMPT_DIFFERING = 0.005


def compare_masks(gpu_keep: np.ndarray, res: dict, p: float, k_floor: int, key: str = "keep"):
    """Row-by-row comparison of a GPU mask with the oracle's.

    Rows outside the float32 exemption rule (oracle.row_exemptions) must match
    exactly.  Exempt rows must keep the own block, at least min(k_floor, nb)
    blocks, mass >= p - 1e-4 (oracle P), a size within 1 of the oracle's and a
    symmetric difference of at most 2 blocks; and at most MAX_EXEMPT_DIFFERING
    of all rows may be exempt rows that differ from the oracle.
    Returns a dict of counts (exempt rows split by reason: mass within 1e-4 of
    p, near tie at the cut); raises AssertionError on any violation.
    """
    ref = res[key]
    B, H, nb, _ = ref.shape
    P = res["P"]
    close, near_tie = O.row_exemption_causes(res["diag"], p, k_floor)
    exempt = close | near_tie
    exact_rows = mism = ex_ok = ex_equal = 0
    bad = []
    for b in range(B):
        for h in range(H):
            eq = (gpu_keep[b, h] == ref[b, h]).all(axis=1)
            for i in range(nb):
                if not exempt[b, h, i]:
                    if eq[i]:
                        exact_rows += 1
                    else:
                        mism += 1
                        if len(bad) < 5:
                            bad.append((b, h, i, np.nonzero(gpu_keep[b, h, i] != ref[b, h, i])[0]))
                    continue
                g = gpu_keep[b, h, i]
                kept = int(g.sum())
                assert g[i], (b, h, i, "own block missing")
                assert kept >= min(k_floor, nb), (b, h, i, kept)
                if p < 1.0:
                    assert P[b, h, i][g].sum() >= p - 1e-4, (b, h, i)
                assert abs(kept - int(ref[b, h, i].sum())) <= 1, (b, h, i)
                assert int((g != ref[b, h, i]).sum()) <= 2, (b, h, i)
                ex_ok += 1
                ex_equal += int(eq[i])
    assert mism == 0, f"{mism} non-exempt rows differ, e.g. {bad}"
    rows = B * H * nb
    differing = ex_ok - ex_equal
    assert differing <= MAX_EXEMPT_DIFFERING * rows, (differing, rows)
    return dict(exact=exact_rows, exempt=ex_ok, exempt_mass_close=int(close.sum()),
                exempt_near_tie=int((near_tie & ~close).sum()), exempt_but_equal=ex_equal,
                exempt_differing=differing, mismatched=mism)


def check_slack(gpu_keep: np.ndarray, gpu_base: np.ndarray, P: np.ndarray, slack: float,
                tie_rel: float = 1e-5):
    """GPU slack fill against the oracle fill applied to the GPU's own base mask.

    Pairs chosen differently may only be pairs whose probability is within a
    relative 1e-5 of the head's selection threshold (float32 versus float64
    probabilities).  Every head must hold exactly max(base, budget) pairs.
    """
    ref, info = O.slack_fill(P, gpu_base, slack)
    B, H, nb, _ = P.shape
    budget = int(math.ceil(float(slack) * nb * nb))
    diffs = 0
    for b in range(B):
        for h in range(H):
            g, r = gpu_keep[b, h], ref[b, h]
            assert int(g.sum()) == max(int(gpu_base[b, h].sum()), budget), (b, h)
            assert (g[gpu_base[b, h]]).all(), (b, h, "base pair dropped")
            d = g != r
            if d.any():
                thr = info[(b, h)]["last"]
                near = np.abs(P[b, h][d] - thr) <= tie_rel * thr
                assert near.all(), (b, h, int(d.sum()), P[b, h][d][~near][:4], thr)
                diffs += int(d.sum())
    return diffs


def sample_rows(row_ptr: np.ndarray, B: int, H: int, nb: int, geo, n_heads=8, n_blocks=16,
                seed=0):
    """Seeded sample of rows: n_heads heads (always the heaviest and lightest)
    x n_blocks query blocks (always the heaviest row of the head and one
    partially padded block)."""
    rng = np.random.default_rng(seed)
    counts = np.diff(row_ptr).reshape(B * H, nb)
    head_nnz = counts.sum(axis=1)
    heads = {int(head_nnz.argmax()), int(head_nnz.argmin())}
    others = [x for x in range(B * H) if x not in heads]
    rng.shuffle(others)
    heads |= set(others[: max(0, n_heads - len(heads))])
    members = O.block_members(geo)
    partial = [i for i in range(nb) if (members[i] < 0).any()]
    rows = []
    for bh in sorted(heads):
        blocks = {int(counts[bh].argmax())}
        if partial:
            blocks.add(int(rng.choice(partial)))
        rest = [i for i in range(nb) if i not in blocks]
        rng.shuffle(rest)
        blocks |= set(rest[: max(0, n_blocks - len(blocks))])
        rows += [bh * nb + i for i in sorted(blocks)]
    return rows


def compare_outputs(o_gpu: np.ndarray, o_ref: np.ndarray, geo, rows, H: int, dtype: str):
    """Compare outputs of the real query tokens of the given rows."""
    members = O.block_members(geo)
    nb = geo.nb
    errs = []
    for r in rows:
        bh, i = divmod(int(r), nb)
        b, h = divmod(bh, H)
        tok = members[i][members[i] >= 0]
        errs.append(np.abs(o_gpu[b, tok, h, :].astype(np.float64) - o_ref[b, tok, h, :]).ravel())
    e = np.concatenate(errs)
    assert np.isfinite(e).all()
    if dtype == "f32":
        assert e.max() <= TOL_F32_MAX, e.max()
    else:
        assert e.max() <= TOL_BF16_MAX, e.max()
        assert e.mean() <= TOL_BF16_MEAN, e.mean()
    return float(e.max()), float(e.mean())


def pair_groups(geo, heads: int):
    """Work items of the bf16 attention kernel, head by head: t-neighbour pairs
    (even t leads) over the first 2*(nbt//2) planes; if nbt is odd, the last
    plane's h-neighbour pairs (even h leads); if nbh is odd too, that plane's
    last row's w-neighbour pairs (even w leads); if nbw is odd as well, the
    last block alone.  Returns [(row_a, row_b or -1)]."""
    nbt, nbh, nbw = geo.nblk

    def blk(t, h, w):
        return (t * nbh + h) * nbw + w

    per_head = []
    for tp in range(nbt // 2):
        for h in range(nbh):
            for w in range(nbw):
                per_head.append((blk(2 * tp, h, w), blk(2 * tp + 1, h, w)))
    if nbt % 2:
        t = nbt - 1
        for hp in range(nbh // 2):
            for w in range(nbw):
                per_head.append((blk(t, 2 * hp, w), blk(t, 2 * hp + 1, w)))
        if nbh % 2:
            h = nbh - 1
            for wp in range(nbw // 2):
                per_head.append((blk(t, h, 2 * wp), blk(t, h, 2 * wp + 1)))
            if nbw % 2:
                per_head.append((blk(t, h, nbw - 1), -1))
    out = []
    for bh in range(heads):
        for a, b in per_head:
            out.append((bh * geo.nb + a, bh * geo.nb + b if b >= 0 else -1))
    return out


def check_dynamic_slack(gpu_keep: np.ndarray, gpu_base: np.ndarray, P: np.ndarray, budget: int,
                        theta: float, tie_rel: float = 1e-5):
    """GPU dynamic slack fill against the oracle fill applied to the GPU's own
    base mask.  Pairs chosen differently may only be pairs whose probability is
    within a relative 1e-5 of the selection threshold or of theta (float32
    versus float64 probabilities).  The GPU keeps every base pair, and adds as
    many pairs as the oracle unless a candidate sits at theta.  Returns the
    number of differing pairs and the oracle's info."""
    ref, info = O.dynamic_slack_fill(P, gpu_base, budget, theta)
    assert (gpu_keep[gpu_base]).all(), "base pair dropped"
    added = int(gpu_keep.sum() - gpu_base.sum())
    at_theta = np.abs(P[~gpu_base] - theta) <= tie_rel * max(theta, 1e-30)
    if not at_theta.any():
        assert added == info["added"], (added, info)
    d = gpu_keep != ref
    if d.any():
        thr = info["last"] if info["added"] else theta
        near = (np.abs(P[d] - thr) <= tie_rel * thr) | (np.abs(P[d] - theta) <= tie_rel * theta)
        assert near.all(), (int(d.sum()), P[d][~near][:4], thr, theta)
    return int(d.sum()), info
