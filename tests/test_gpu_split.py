"""GPU parity of the split-and-merge attention (through the C ABI).

Heavy work items are cut into parts along their union key-block lists, each
part leaves float32 partials, and a merge kernel joins them by log-sum-exp.
Checked here: the work-unit table against oracle.split_units (bit-exact); the
output against the oracle's sparse attention (bf16 max |d| <= 2e-2, mean
|d| <= 2e-3); items left whole bitwise equal to the plain attention; the two
sorted queues bitwise equal to each other; every kept tile done exactly once;
a workspace reused with another cut leaves no trace.
"""
import math

import numpy as np
import pytest
import torch

import adaptive_block_sparse_amd as A
import oracle as O
import synth_inputs as si
from parity_utils import compare_outputs, pair_groups, sample_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda:0"


def _wl(cfg, grid, block, heads, d, p=(0.9,), k_floor=2):
    return si.Workload(cfg, f"split-{cfg}", 1, heads, d, "bf16", grid, block, p, k_floor, 0.0,
                       "u13")


SMALL = {
    "d128-bt128-ragged": _wl(101, (5, 12, 20), (2, 8, 8), 3, 128),
    "d64-bt64-ragged": _wl(102, (3, 20, 12), (1, 8, 8), 2, 64),
    "d128-bt32": _wl(103, (4, 9, 10), (2, 4, 4), 2, 128),
    "d64-bt128-onetile": _wl(104, (2, 8, 8), (2, 8, 8), 2, 64),
    "batch2": si.Workload(107, "split-107-batch2", 2, 3, 128, "bf16", (4, 10, 12), (2, 8, 8),
                          (0.9,), 2, 0.0, "u13"),
    "pair-w-odd": _wl(109, (2, 8, 40), (2, 8, 8), 2, 128),
    "block-4x4x4": _wl(111, (9, 10, 11), (4, 4, 4), 2, 128),
    "block-4x4x8": _wl(114, (7, 10, 13), (4, 4, 8), 3, 128),
    "pair-tiers": _wl(116, (5, 20, 40), (2, 8, 8), 2, 128),
}


def _union_counts(rp, ci, geo, heads):
    counts = []
    for a, b in pair_groups(geo, heads):
        cols = set(ci[rp[a]:rp[a + 1]].tolist())
        if b >= 0:
            cols |= set(ci[rp[b]:rp[b + 1]].tolist())
        counts.append(len(cols))
    return counts


def _wanted(counts, split):
    return sum(math.ceil(n / split) for n in counts if n > split)


class Case:
    """Inputs, mask and plain attention output of one workload."""

    def __init__(self, wl, p=None, inputs=None):
        self.wl = wl
        p = float(np.float32(wl.p[0] if p is None else p))
        print(f"[gpu case] split {wl.name} p={p}", flush=True)
        self.inputs = si.make_inputs(wl) if inputs is None else inputs
        self.q, self.k, self.v = (t.to(DEV) for t in self.inputs)
        self.plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
        self.mask = A.route(self.plan, self.q, self.k, p, wl.k_floor)
        self.o_plain = A.attend(self.plan, self.q, self.k, self.v, self.mask,
                                sched=A.SCHED_HEAD_PHASED)
        torch.cuda.synchronize()
        self.geo = O.geometry(wl.grid, wl.block)
        self.rp, self.ci = self.mask.to_host()
        self.bh = wl.batch * wl.heads
        self.groups = pair_groups(self.geo, self.bh)
        self.counts = _union_counts(self.rp, self.ci, self.geo, self.bh)

    def run_split(self, split, max_parts, sched=A.SCHED_NNZ_SORTED, ws=None):
        print(f"[gpu case]   split={split} max_parts={max_parts} sched={sched}", flush=True)
        if ws is None:
            ws = A.workspace(A.attend_split_ws_bytes(self.plan, max_parts), DEV)
        tel = torch.zeros(A.attend_grid(self.plan, sched) * 4, dtype=torch.int64, device=DEV)
        o = torch.full_like(self.q, float("nan"))
        A.attend_prepare_split(self.plan, self.k, self.v, self.mask, sched, split, max_parts, ws)
        A.attend_run_split(self.plan, self.q, self.mask, o, sched, max_parts, ws, telemetry=tel)
        torch.cuda.synchronize()
        units, cut = O.split_units(self.counts, split, max_parts)
        got = ws[: len(units) * 16].view(torch.int32).cpu().numpy().reshape(-1, 4)
        np.testing.assert_array_equal(got, np.array(units, dtype=np.int32).reshape(-1, 4))
        t = tel.cpu().numpy().reshape(-1, 4)
        assert int(t[:, 2].sum()) == self.ci.size            # every kept tile done once
        return o.float().cpu().numpy(), units, cut

    def whole_rows(self, cut):
        cut_items = {c[0] for c in cut}
        return [r for it, pair in enumerate(self.groups) if it not in cut_items
                for r in pair if r >= 0]

    def check_rows_equal(self, o1, o2, rows):
        members = O.block_members(self.geo)
        for r in rows:
            bh, i = divmod(int(r), self.geo.nb)
            b, h = divmod(bh, self.wl.heads)
            tok = members[i][members[i] >= 0]
            assert np.array_equal(o1[b, tok, h, :], o2[b, tok, h, :]), r


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("split", [1, 3])
def test_split_everything_small(name, split):
    c = Case(SMALL[name])
    max_parts = _wanted(c.counts, split)
    o, units, cut = c.run_split(split, max_parts)
    assert len(cut) == sum(1 for n in c.counts if n > split)
    rows = range(c.bh * c.geo.nb)
    o_ref = O.sparse_attention(*(t.float().numpy() for t in c.inputs), c.geo, c.rp, c.ci)
    print("max/mean err", compare_outputs(o, o_ref, c.geo, rows, c.wl.heads, "bf16"))
    o_plain = c.o_plain.float().cpu().numpy()
    c.check_rows_equal(o, o_plain, c.whole_rows(cut))
    print("split vs plain max |d|", float(np.nanmax(np.abs(o - o_plain))))
    # the other sorted queue gives the same bits
    o2, _, _ = c.run_split(split, max_parts, sched=A.SCHED_HEAD_PHASED)
    assert np.array_equal(o, o2)


def test_split_budget_cuts_the_heaviest():
    c = Case(SMALL["d128-bt128-ragged"])
    split = 2
    full = _wanted(c.counts, split)
    max_parts = full // 3
    o, units, cut = c.run_split(split, max_parts)   # unit table checked against the oracle
    assert 0 < len(cut) < sum(1 for n in c.counts if n > split)
    lightest_cut = min(c.counts[it] for it, _, _ in cut)
    assert all(c.counts[it] <= lightest_cut for it in range(len(c.counts))
               if it not in {x[0] for x in cut})
    o_ref = O.sparse_attention(*(t.float().numpy() for t in c.inputs), c.geo, c.rp, c.ci)
    compare_outputs(o, o_ref, c.geo, range(c.bh * c.geo.nb), c.wl.heads, "bf16")
    c.check_rows_equal(o, c.o_plain.float().cpu().numpy(), c.whole_rows(cut))


def test_nothing_cut_is_bitwise_plain():
    c = Case(SMALL["batch2"])
    o_plain = c.o_plain.float().cpu().numpy()
    for split, max_parts in ((1, 0), (10 ** 6, 64)):
        o, _, cut = c.run_split(split, max_parts)
        assert cut == []
        assert np.array_equal(o, o_plain)


def test_workspace_reused_with_another_cut():
    c = Case(SMALL["d128-bt32"])
    max_parts = _wanted(c.counts, 1)
    ws = A.workspace(A.attend_split_ws_bytes(c.plan, max_parts), DEV)
    c.run_split(1, max_parts, ws=ws)
    o_again, _, _ = c.run_split(4, max_parts // 2, ws=ws)   # fewer, longer parts, same memory
    o_fresh, _, _ = c.run_split(4, max_parts // 2)
    assert np.array_equal(o_again, o_fresh)


def test_dense_mask_split():
    """p = 1 keeps every block: the split result is plain softmax attention."""
    c = Case(SMALL["d64-bt64-ragged"], p=1.0)
    assert c.ci.size == c.bh * c.geo.nb ** 2
    o, _, _ = c.run_split(5, _wanted(c.counts, 5))
    o_ref = O.dense_attention(*(t.float().numpy() for t in c.inputs))
    compare_outputs(o, o_ref, c.geo, range(c.bh * c.geo.nb), c.wl.heads, "bf16")


@pytest.mark.slow
def test_split_full_480p():
    """The 480p layer (40 heads, 32 760 tokens, p = 0.9) with parts of at most
    64 union entries and one slot per item on average, then parts of at most
    96 entries and 256 slots, in the launch configuration the benchmark times:
    unit tables exact, sampled rows against the oracle, whole items bitwise
    equal to the plain path."""
    wl = si.WORKLOADS[1]
    c = Case(wl)
    o, units, cut = c.run_split(64, len(c.groups))
    assert len(cut) > 0
    # a budget of 256 slots: only the heaviest items are cut
    o2, _, cut2 = c.run_split(96, 256)
    assert 0 < len(cut2) < len(cut)
    whole2 = set(c.whole_rows(cut2))
    q, k, v = (t.float().numpy() for t in c.inputs)
    rows = sample_rows(c.rp, wl.batch, wl.heads, c.geo.nb, c.geo, seed=1)
    o_ref = O.sparse_attention(q, k, v, c.geo, c.rp, c.ci, rows=rows)
    print("max/mean err", compare_outputs(o, o_ref, c.geo, rows, wl.heads, "bf16"))
    print("max/mean err, 256 slots", compare_outputs(o2, o_ref, c.geo, rows, wl.heads, "bf16"))
    whole = set(c.whole_rows(cut))
    plain = c.o_plain.float().cpu().numpy()
    c.check_rows_equal(o, plain, [r for r in rows if r in whole])
    c.check_rows_equal(o2, plain, [r for r in rows if r in whole2])


BLOCKS = [(2, 4, 4), (1, 4, 8), (2, 2, 8), (1, 8, 8), (2, 4, 8), (4, 4, 4),
          (2, 8, 8), (4, 4, 8), (1, 8, 16), (8, 4, 4)]


def _draw(i):
    """A seeded small bf16 layer with a random cut: block shape, grid (ragged
    tails, grids below one block along an axis), heads, d, p, k_floor, the
    longest part and the slot budget (between none and every wanted part)."""
    rng = np.random.default_rng([2027, i])
    block = BLOCKS[int(rng.integers(len(BLOCKS)))]
    while True:
        grid = tuple(int(rng.integers(1, 3 * b + 1)) for b in block)
        if grid[0] * grid[1] * grid[2] <= 4000:
            break
    heads = int(rng.integers(1, 4))
    d = int(rng.choice([64, 128]))
    p = float(np.float32(rng.choice([0.3, 0.6, 0.9, 1.0])))
    k_floor = int(rng.integers(1, 6))
    split = int(rng.choice([1, 2, 3, 5, 8]))
    frac = float(rng.choice([0.0, 0.3, 1.0]))
    return _wl(400 + i, grid, block, heads, d, (p,), k_floor), split, frac


RANDOM = [_draw(i) for i in range(24)]


@pytest.mark.parametrize("wl,split,frac", RANDOM,
                         ids=[f"{w.name}-{w.grid}-{w.block}-h{w.heads}-d{w.head_dim}-p{w.p[0]:.2f}"
                              f"-S{s}-f{f}" for w, s, f in RANDOM])
def test_split_random_shapes(wl, split, frac):
    """Seeded random layers and cuts: the unit table exact (in run_split),
    every row against the oracle, items left whole bitwise equal to the plain
    path, both sorted queues bitwise equal."""
    c = Case(wl)
    max_parts = int(frac * _wanted(c.counts, split))
    o, units, cut = c.run_split(split, max_parts)
    rows = range(c.bh * c.geo.nb)
    o_ref = O.sparse_attention(*(t.float().numpy() for t in c.inputs), c.geo, c.rp, c.ci)
    print("max/mean err", compare_outputs(o, o_ref, c.geo, rows, c.wl.heads, "bf16"))
    c.check_rows_equal(o, c.o_plain.float().cpu().numpy(), c.whole_rows(cut))
    o2, _, _ = c.run_split(split, max_parts, sched=A.SCHED_HEAD_PHASED)
    assert np.array_equal(o, o2)
