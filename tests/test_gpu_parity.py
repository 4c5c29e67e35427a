"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Masks: bit-exact on every row outside the float32 exemption rule; exempt rows
checked for the invariants.  Outputs: the oracle attention is fed the GPU's own
mask; bf16 max |d| <= 2e-2 and mean |d| <= 2e-3, float32 max |d| <= 1e-4.
Small shapes are compared on every row; the full workloads on a seeded sample
of 8 heads x 16 query blocks (always the heaviest/lightest heads, the heaviest
row and a partially padded block), in the launch configuration the benchmark
times.
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

import adaptive_block_sparse_amd as A
import oracle as O
import synth_inputs as si
from parity_utils import check_slack, compare_masks, compare_outputs, pair_groups, sample_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda:0"


def _wl(cfg, grid, block, heads, d, dtype, p=(0.9,), k_floor=2, tau="u13"):
    return si.Workload(cfg, f"test-{cfg}", 1, heads, d, dtype, grid, block, p, k_floor, 0.0, tau)


SMALL = {
    "bf16-d128-bt128-ragged": _wl(101, (5, 12, 20), (2, 8, 8), 3, 128, "bf16"),
    "bf16-d64-bt64-ragged": _wl(102, (3, 20, 12), (1, 8, 8), 2, 64, "bf16"),
    "bf16-d128-bt32": _wl(103, (4, 9, 10), (2, 4, 4), 2, 128, "bf16"),
    "bf16-d64-bt128-onetile": _wl(104, (2, 8, 8), (2, 8, 8), 2, 64, "bf16"),
    "f32-d128-bt32": _wl(105, (3, 10, 9), (2, 4, 4), 2, 128, "f32"),
    "f32-tiny-cfg0": si.WORKLOADS[0],
    "bf16-batch2": si.Workload(107, "test-107-batch2", 2, 3, 128, "bf16", (4, 10, 12), (2, 8, 8),
                               (0.9,), 2, 0.0, "u13"),
    "bf16-pair-h": _wl(108, (2, 16, 24), (2, 8, 8), 2, 128, "bf16"),       # nbt = 1: pairs along h
    "bf16-pair-w-odd": _wl(109, (2, 8, 40), (2, 8, 8), 2, 128, "bf16"),    # nbt = nbh = 1, nbw = 5
    "bf16-d64-bt128": _wl(110, (5, 12, 20), (2, 8, 8), 2, 64, "bf16"),
    "bf16-block-4x4x4": _wl(111, (9, 10, 11), (4, 4, 4), 2, 128, "bf16"),
    # 128-token blocks of other shapes, cut on every axis: real counts 128, 96,
    # 80, 64, 60, 48, 40, 30 (and 128, 80, 40, 25), so whole padding chunks,
    # padding-only second subtiles, short-block copies and packed slots of
    # several extents all occur
    "bf16-block-4x4x8": _wl(114, (7, 10, 13), (4, 4, 8), 3, 128, "bf16"),
    "bf16-block-1x8x16": _wl(115, (3, 13, 21), (1, 8, 16), 2, 128, "bf16"),
    # 3 x 3 x 5 blocks: t-pairs, then h-pairs in the last plane, w-pairs in its
    # last row and one block alone, so every tier of the work-item rule runs
    "bf16-pair-tiers": _wl(116, (5, 20, 40), (2, 8, 8), 2, 128, "bf16"),
    "f32-d64-bt128": _wl(112, (3, 9, 10), (2, 8, 8), 2, 64, "f32"),
}


def _run(wl, p, k_floor, slack=0.0, sched=None, inputs=None, telemetry=False):
    """Route and attend; sched None = the library's default for the shape (the
    schedule the benchmark times)."""
    q, k, v = inputs if inputs is not None else si.make_inputs(wl)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    sched = A.default_sched(plan) if sched is None else sched
    print(f"[gpu case] {wl.name} p={p} k_floor={k_floor} slack={slack} sched={sched}", flush=True)
    mask = A.route(plan, qd, kd, p, k_floor, slack)
    tel = None
    if telemetry:
        tel = torch.zeros(A.attend_grid(plan, sched) * 4, dtype=torch.int64, device=DEV)
    o = A.attend(plan, qd, kd, vd, mask, sched=sched, telemetry=tel)
    torch.cuda.synchronize()
    return dict(q=q, k=k, v=v, plan=plan, mask=mask, o=o.float().cpu().numpy(),
                tel=None if tel is None else tel.cpu().numpy().reshape(-1, 4))


def _np(t):
    return t.float().numpy()


@pytest.mark.parametrize("name", list(SMALL))
def test_small_full_parity(name):
    wl = SMALL[name]
    p = float(np.float32(wl.p[0]))
    r = _run(wl, p, wl.k_floor, telemetry=True)
    geo = O.geometry(wl.grid, wl.block)
    res = O.route(_np(r["q"]), _np(r["k"]), geo, p, wl.k_floor)
    rp, ci = r["mask"].to_host()
    keep = O.csr_to_keep(rp, ci, wl.batch, wl.heads, geo.nb)
    counts = compare_masks(keep, res, p, wl.k_floor)
    print("mask rows", counts)
    assert (np.diff(rp) > 0).all()
    assert r["mask"].head_nnz.cpu().numpy().sum() == ci.size
    o_ref = O.sparse_attention(_np(r["q"]), _np(r["k"]), _np(r["v"]), geo, rp, ci)
    rows = range(wl.batch * wl.heads * geo.nb)
    print("max/mean err", compare_outputs(r["o"], o_ref, geo, rows, wl.heads, wl.dtype))
    assert r["tel"][:, 2].sum() == ci.size          # every kept tile done exactly once
    # every schedule gives the same bits
    for sched in (A.SCHED_NNZ_SORTED, A.SCHED_HEAD_MAJOR, A.SCHED_HEAD_PHASED,
                  A.SCHED_XCD_LOCAL):
        o2 = _run(wl, p, wl.k_floor, sched=sched, inputs=(r["q"], r["k"], r["v"]))["o"]
        assert np.array_equal(o2, r["o"])


@pytest.mark.parametrize("name", ["bf16-d128-bt128-ragged", "f32-tiny-cfg0", "bf16-block-4x4x8"])
def test_dense_when_p_is_one(name):
    wl = SMALL[name]
    r = _run(wl, 1.0, 1)
    rp, ci = r["mask"].to_host()
    geo = O.geometry(wl.grid, wl.block)
    assert ci.size == wl.heads * geo.nb * geo.nb
    o_ref = O.dense_attention(_np(r["q"]), _np(r["k"]), _np(r["v"]))
    compare_outputs(r["o"], o_ref, geo, range(wl.heads * geo.nb), wl.heads, wl.dtype)


def test_floor_above_nb_and_single_block():
    wl = SMALL["bf16-d128-bt128-ragged"]
    r = _run(wl, 0.5, 1000)
    rp, ci = r["mask"].to_host()
    geo = O.geometry(wl.grid, wl.block)
    assert ci.size == wl.heads * geo.nb * geo.nb
    one = _wl(106, (2, 8, 8), (2, 8, 8), 2, 128, "bf16")
    r = _run(one, 0.3, 1)
    rp, ci = r["mask"].to_host()
    assert rp.tolist() == [0, 1, 2] and ci.tolist() == [0, 0]
    o_ref = O.dense_attention(_np(r["q"]), _np(r["k"]), _np(r["v"]))
    compare_outputs(r["o"], o_ref, O.geometry(one.grid, one.block), [0, 1], 2, "bf16")


@pytest.mark.parametrize("p,slack", [(0.3, 0.5), (0.5, 0.7), (0.2, 0.97)])
def test_slack_fill_active(p, slack):
    """Heads below the budget: the fill must add exactly the oracle's pairs
    (up to float32 near-ties at the threshold)."""
    wl = SMALL["bf16-d128-bt128-ragged"]
    p = float(np.float32(p))
    inputs = si.make_inputs(wl)
    geo = O.geometry(wl.grid, wl.block)
    base = _run(wl, p, 1, inputs=inputs)
    r = _run(wl, p, 1, slack=slack, inputs=inputs)
    brp, bci = base["mask"].to_host()
    rp, ci = r["mask"].to_host()
    base_keep = O.csr_to_keep(brp, bci, 1, wl.heads, geo.nb)
    keep = O.csr_to_keep(rp, ci, 1, wl.heads, geo.nb)
    res = O.route(_np(inputs[0]), _np(inputs[1]), geo, p, 1)
    compare_masks(base_keep, res, p, 1)
    budget = int(np.ceil(np.float64(np.float32(slack)) * geo.nb ** 2))
    assert (base_keep.reshape(wl.heads, -1).sum(1) < budget).any()      # the fill is active
    print("slack pairs off the oracle", check_slack(keep, base_keep, res["P"], np.float32(slack)))
    o_ref = O.sparse_attention(_np(inputs[0]), _np(inputs[1]), _np(inputs[2]), geo, rp, ci)
    compare_outputs(r["o"], o_ref, geo, range(wl.heads * geo.nb), wl.heads, wl.dtype)


@pytest.mark.slow
def test_slack_fill_active_long_horizon():
    """The long-horizon shape at p = 0.3 so that heads fall below the 15 %
    budget; full mask check, sampled outputs."""
    wl = si.WORKLOADS[4]
    p = float(np.float32(0.3))
    inputs = si.make_inputs(wl)
    geo = O.geometry(wl.grid, wl.block)
    base = _run(wl, p, wl.k_floor, inputs=inputs)
    r = _run(wl, p, wl.k_floor, slack=wl.slack, inputs=inputs, telemetry=True)
    brp, bci = base["mask"].to_host()
    rp, ci = r["mask"].to_host()
    base_keep = O.csr_to_keep(brp, bci, 1, wl.heads, geo.nb)
    keep = O.csr_to_keep(rp, ci, 1, wl.heads, geo.nb)
    q, k, v = (_np(t) for t in inputs)
    res = O.route(q, k, geo, p, wl.k_floor)
    print("base mask rows", compare_masks(base_keep, res, p, wl.k_floor))
    dens = base_keep.reshape(wl.heads, -1).mean(1)
    print("base density per head", np.round(dens, 3))
    print("slack pairs off the oracle", check_slack(keep, base_keep, res["P"], np.float32(wl.slack)))
    assert r["tel"][:, 2].sum() == ci.size
    rows = sample_rows(rp, 1, wl.heads, geo.nb, geo, seed=44)
    o_ref = O.sparse_attention(q, k, v, geo, rp, ci, rows=rows)
    print("max/mean err", compare_outputs(r["o"], o_ref, geo, rows, wl.heads, wl.dtype))


def test_schedules_are_bitwise_identical():
    wl = SMALL["bf16-d128-bt128-ragged"]
    inputs = si.make_inputs(wl)
    outs = [_run(wl, 0.8, 2, sched=s, inputs=inputs)["o"] for s in (0, 1, 2, 3)]
    for other in outs[1:]:
        assert np.array_equal(outs[0], other)


def test_pooled_means_and_schedule_array():
    wl = SMALL["bf16-d128-bt128-ragged"]
    q, k, v = si.make_inputs(wl)
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    ws = A.workspace(plan.route_ws_bytes, DEV)
    mask = A.route(plan, q.to(DEV), k.to(DEV), 0.8, 2, ws=ws)
    torch.cuda.synchronize()
    geo = O.geometry(wl.grid, wl.block)
    n = wl.batch * wl.heads * geo.nb * wl.head_dim
    pooled = ws[: 2 * n * 4].view(torch.float32).cpu().numpy()
    np.testing.assert_allclose(pooled[:n].reshape(1, wl.heads, geo.nb, -1), O.pool(_np(q), geo),
                               rtol=1e-5, atol=1e-5)
    np.testing.assert_allclose(pooled[n:].reshape(1, wl.heads, geo.nb, -1), O.pool(_np(k), geo),
                               rtol=1e-5, atol=1e-5)
    rp, _ = mask.to_host()
    counts = np.diff(rp)
    groups = pair_groups(geo, wl.batch * wl.heads)
    assert sorted([r for gr in groups for r in gr if r >= 0]) == list(range(counts.size))
    costs = [counts[a] + (counts[b] if b >= 0 else 0) for a, b in groups]
    aws = A.workspace(plan.attend_ws_bytes, DEV)
    gph = len(groups) // wl.heads
    for mode, sched in (("nnz_sorted", 0), ("head_major", 1), ("head_phased", 2)):
        A.attend_prepare(plan, k.to(DEV), v.to(DEV), mask, sched, aws)
        torch.cuda.synchronize()
        got = aws[: len(groups) * 4].view(torch.int32).cpu().numpy()
        want = O.schedule(costs, mode, items_per_head=gph, heads_per_phase=plan.heads_per_phase)
        np.testing.assert_array_equal(got, want)
    # XCD-local queues (one per XCD, eight on MI355X), against the oracle's
    A.attend_prepare(plan, k.to(DEV), v.to(DEV), mask, A.SCHED_XCD_LOCAL, aws)
    torch.cuda.synchronize()
    got = aws[: len(groups) * 4].view(torch.int32).cpu().numpy()
    want = O.schedule(costs, "xcd_local", items_per_head=gph, n_queues=8)
    np.testing.assert_array_equal(got, want)


def test_wide_logit_range_moves_the_reference():
    """Scores that climb by more than 2^8 (in exp2 units) from one key block to
    the next, with every block kept: walking the blocks in ascending order, a
    query's running reference must move at every block, so the kernel's
    rescale path (taken only on jumps above 2^8) runs again and again.
    Outputs still match the oracle."""
    wl = SMALL["bf16-d128-bt128-ragged"]
    geo = O.geometry(wl.grid, wl.block)
    blk = np.full(wl.tokens, -1)
    for j, mem in enumerate(O.block_members(geo)):
        blk[mem[mem >= 0]] = j
    rng = np.random.default_rng(2024)
    q = np.zeros((1, wl.tokens, wl.heads, wl.head_dim), np.float32)
    q[..., 0] = 8.0
    k = (0.25 * rng.standard_normal(q.shape)).astype(np.float32)
    k[..., 0] = 10.0 * blk[None, :, None]            # score 80 j: 10.2 exp2 units per block
    v = rng.standard_normal(q.shape).astype(np.float32)
    step = 8.0 * 10.0 * 1.4426950408889634 / np.sqrt(wl.head_dim)
    assert step > 8.0
    qt, kt, vt = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    r = _run(wl, 1.0, wl.k_floor, inputs=(qt, kt, vt), sched=A.SCHED_XCD_LOCAL)
    rp, ci = r["mask"].to_host()
    assert (np.diff(rp) == geo.nb).all()            # every block kept
    o_ref = O.sparse_attention(_np(r["q"]), _np(r["k"]), _np(r["v"]), geo, rp, ci)
    rows = range(wl.batch * wl.heads * geo.nb)
    print("max/mean err", compare_outputs(r["o"], o_ref, geo, rows, wl.heads, wl.dtype))


def _exp2_bound(q, k, d):
    """Per head: log2(e)/sqrt(d) x the largest query norm x the largest key
    norm (bf16 values, float64): the Cauchy-Schwarz bound on |scores| in the
    exp2 domain that decides between the kernel's two softmax walks."""
    qn = np.sqrt((q.astype(np.float64) ** 2).sum(-1)).max(axis=(0, 1))
    kn = np.sqrt((k.astype(np.float64) ** 2).sum(-1)).max(axis=(0, 1))
    return 1.4426950408889634 / np.sqrt(d) * qn * kn


def test_both_softmax_walks_in_one_launch():
    """Head 0: random inputs (bound about 20: every item walked against the
    reference 0).  Head 1: queries and keys along one direction, the keys half
    aligned and half opposed, scaled so that the bound sits just below 32: the
    probabilities span about 2^-29 .. 2^29 against the reference 0.  Head 2:
    the same scaled past 32, walked with the running maximum.  Every output
    against the oracle, and every schedule gives the same bits."""
    wl = SMALL["bf16-d128-bt128-ragged"]
    assert wl.heads == 3
    d = wl.head_dim
    rng = np.random.default_rng(31)
    shape = (1, wl.tokens, wl.heads, d)
    q = rng.standard_normal(shape).astype(np.float32)
    k = rng.standard_normal(shape).astype(np.float32)
    v = rng.standard_normal(shape).astype(np.float32)
    u = rng.standard_normal(d)
    u /= np.linalg.norm(u)
    sign = np.where(np.arange(wl.tokens) % 2 == 0, 1.0, -1.0)
    for h, target in ((1, 29.0), (2, 36.0)):
        scale = np.sqrt(target * np.sqrt(d) / 1.4426950408889634)   # |q| = |k| = scale
        q[0, :, h] = scale * u + 0.01 * rng.standard_normal((wl.tokens, d))
        k[0, :, h] = sign[:, None] * scale * u + 0.01 * rng.standard_normal((wl.tokens, d))
    qt, kt, vt = (torch.from_numpy(x).to(torch.bfloat16) for x in (q, k, v))
    bound = _exp2_bound(_np(qt), _np(kt), d)
    print("exp2-domain bounds per head", bound)
    assert bound[0] < 30 and 28 < bound[1] < 31.5 and bound[2] > 33
    p = float(np.float32(wl.p[0]))
    r = _run(wl, p, wl.k_floor, inputs=(qt, kt, vt))
    geo = O.geometry(wl.grid, wl.block)
    rp, ci = r["mask"].to_host()
    o_ref = O.sparse_attention(_np(r["q"]), _np(r["k"]), _np(r["v"]), geo, rp, ci)
    rows = range(wl.batch * wl.heads * geo.nb)
    print("max/mean err", compare_outputs(r["o"], o_ref, geo, rows, wl.heads, wl.dtype))
    for sched in (A.SCHED_NNZ_SORTED, A.SCHED_HEAD_MAJOR, A.SCHED_XCD_LOCAL):
        o2 = _run(wl, p, wl.k_floor, sched=sched, inputs=(r["q"], r["k"], r["v"]))["o"]
        assert np.array_equal(o2, r["o"])


def test_nan_input_keeps_mask_well_formed():
    wl = SMALL["bf16-d128-bt128-ragged"]
    q, k, v = si.make_inputs(wl)
    q[0, 5, 1, 3] = float("nan")
    r = _run(wl, 0.9, 2, inputs=(q, k, v))
    rp, ci = r["mask"].to_host()
    geo = O.geometry(wl.grid, wl.block)
    for row in range(rp.size - 1):
        cols = ci[rp[row]:rp[row + 1]]
        assert 1 <= cols.size <= geo.nb and (row % geo.nb) in cols
        assert (np.diff(cols) > 0).all()


def test_maximum_blocks_per_head():
    """nb = 4096, the largest the library accepts (16 x 16 x 16 blocks of
    2 x 4 x 4 tokens): full mask check, sampled outputs."""
    wl = _wl(113, (32, 64, 64), (2, 4, 4), 1, 64, "bf16", k_floor=3)
    inputs = si.make_inputs(wl)
    p = float(np.float32(0.9))
    r = _run(wl, p, 3, inputs=inputs)
    geo = O.geometry(wl.grid, wl.block)
    assert geo.nb == 4096
    q, k, v = (_np(t) for t in inputs)
    res = O.route(q, k, geo, p, 3)
    rp, ci = r["mask"].to_host()
    keep = O.csr_to_keep(rp, ci, 1, 1, geo.nb)
    print("mask rows", compare_masks(keep, res, p, 3))
    rows = sample_rows(rp, 1, 1, geo.nb, geo, n_heads=1, n_blocks=24, seed=113)
    o_ref = O.sparse_attention(q, k, v, geo, rp, ci, rows=rows)
    print("max/mean err", compare_outputs(r["o"], o_ref, geo, rows, 1, "bf16"))


# ---------------------------------------------------------------------------
# Full workloads, sampled attention rows, launch configuration of the benchmark
# ---------------------------------------------------------------------------
FULL = [(1, 0.9), (3, 0.95), (2, 0.9), (2, 0.95), (4, 0.9)]


@pytest.mark.slow
@pytest.mark.parametrize("cfg,p", FULL)
def test_full_workload_parity(cfg, p):
    wl = si.WORKLOADS[cfg]
    p = float(np.float32(p))
    inputs = si.make_inputs(wl)
    r = _run(wl, p, wl.k_floor, slack=wl.slack, inputs=inputs, telemetry=True)
    q, k, v = (_np(t) for t in inputs)
    geo = O.geometry(wl.grid, wl.block)
    res = O.route(q, k, geo, p, wl.k_floor)
    rp, ci = r["mask"].to_host()
    keep = O.csr_to_keep(rp, ci, wl.batch, wl.heads, geo.nb)
    if wl.slack > 0:
        base = _run(wl, p, wl.k_floor, slack=0.0, inputs=inputs)
        brp, bci = base["mask"].to_host()
        base_keep = O.csr_to_keep(brp, bci, wl.batch, wl.heads, geo.nb)
        print("base mask rows", compare_masks(base_keep, res, p, wl.k_floor))
        print("slack pairs off the oracle", check_slack(keep, base_keep, res["P"], wl.slack))
    else:
        print("mask rows", compare_masks(keep, res, p, wl.k_floor))
    dens = np.diff(rp).reshape(wl.heads, geo.nb).sum(1) / geo.nb ** 2
    print(f"kept density per head: min {dens.min():.3f} median {np.median(dens):.3f} "
          f"max {dens.max():.3f}")
    assert r["tel"][:, 2].sum() == ci.size
    rows = sample_rows(rp, wl.batch, wl.heads, geo.nb, geo, seed=cfg)
    o_ref = O.sparse_attention(q, k, v, geo, rp, ci, rows=rows)
    print("max/mean err", compare_outputs(r["o"], o_ref, geo, rows, wl.heads, wl.dtype))
    if cfg == 1:
        # the same outputs under the other schedules, bitwise
        for s in (A.SCHED_NNZ_SORTED, A.SCHED_HEAD_MAJOR, A.SCHED_HEAD_PHASED,
                  A.SCHED_XCD_LOCAL):
            o2 = _run(wl, p, wl.k_floor, sched=s, inputs=inputs)["o"]
            assert np.array_equal(o2, r["o"])
        # and the benchmark's pipeline: the K/V re-layout on a second stream
        # beside routing and the schedule kernels, joined by an event before
        # the attention run
        qd, kd, vd = (t.to(DEV) for t in inputs)
        plan = r["plan"]
        sched = A.default_sched(plan)
        main, side = torch.cuda.current_stream(), torch.cuda.Stream()
        ws = A.workspace(plan.attend_ws_bytes, DEV)
        o3 = torch.empty_like(qd)
        fork, join = torch.cuda.Event(), torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        A.attend_relayout(plan, kd, vd, ws, stream=side)
        join.record(side)
        m3 = A.route(plan, qd, kd, p, wl.k_floor)
        A.attend_schedule(plan, m3, sched, ws)
        main.wait_event(join)
        A.attend_run(plan, qd, kd, m3, o3, sched, ws)
        torch.cuda.synchronize()
        assert np.array_equal(o3.float().cpu().numpy(), r["o"])


def test_relayout_after_routing_beside_the_schedule():
    """abs_attend_relayout on a second stream after abs_route, while
    abs_attend_schedule runs on the first; the run after an event join gives
    the same bits as abs_attend on one stream (the benchmark's pipeline)."""
    wl = SMALL["bf16-d128-bt128-ragged"]
    inputs = si.make_inputs(wl)
    want = _run(wl, 0.9, 2, sched=A.SCHED_HEAD_PHASED, inputs=inputs)["o"]
    q, k, v = (t.to(DEV) for t in inputs)
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ws = A.workspace(plan.attend_ws_bytes, DEV)
    o = torch.empty_like(q)
    fork, join = torch.cuda.Event(), torch.cuda.Event()
    for _ in range(2):                       # the second pass reuses the workspace
        mask = A.route(plan, q, k, 0.9, 2)
        fork.record(main)
        side.wait_event(fork)
        A.attend_relayout(plan, k, v, ws, stream=side)
        join.record(side)
        A.attend_schedule(plan, mask, A.SCHED_HEAD_PHASED, ws)
        main.wait_event(join)
        A.attend_run(plan, q, k, mask, o, A.SCHED_HEAD_PHASED, ws)
        torch.cuda.synchronize()
        assert np.array_equal(o.float().cpu().numpy(), want)


def test_relayout_beside_routing_on_a_second_stream():
    """abs_attend_relayout on a second stream, overlapping abs_route, then
    abs_attend_schedule and the run after an event join: the same bits as
    abs_attend on one stream."""
    wl = SMALL["bf16-d128-bt128-ragged"]
    inputs = si.make_inputs(wl)
    want = _run(wl, 0.9, 2, sched=A.SCHED_XCD_LOCAL, inputs=inputs)["o"]
    q, k, v = (t.to(DEV) for t in inputs)
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    ws = A.workspace(plan.attend_ws_bytes, DEV)
    o = torch.empty_like(q)
    fork, join = torch.cuda.Event(), torch.cuda.Event()
    for _ in range(2):                       # the second pass reuses the workspace
        fork.record(main)
        side.wait_event(fork)
        A.attend_relayout(plan, k, v, ws, stream=side)
        join.record(side)
        mask = A.route(plan, q, k, 0.9, 2)
        main.wait_event(join)
        A.attend_schedule(plan, mask, A.SCHED_XCD_LOCAL, ws)
        A.attend_run(plan, q, k, mask, o, A.SCHED_XCD_LOCAL, ws)
        torch.cuda.synchronize()
        assert np.array_equal(o.float().cpu().numpy(), want)


def test_mfma_probe_runs():
    """The measurement aid: a short probe launch gives finite sums, a positive
    rate and a clock64 rate inside the chip's range."""
    import bench
    r = bench.mfma_probe(DEV, iters=200, workgroups=256, launches=2)
    print("probe", r)
    assert r["tflops"] > 0
    assert 0.5 < r["clock64_ghz"] < 3.0
    for qpw in (32, 64):
        r = bench.attn_loop_probe(DEV, qpw, iters=100, workgroups=256, launches=2)
        print("loop probe", r)
        assert r["tflops"] > 0
        assert 0.5 < r["clock64_ghz"] < 3.0
