"""GPU parity of fine-grained routing (Top-p over frames inside the kept
blocks) and of the frame-restricted attention, through the C ABI, against the
CPU oracle.  Block masks as in the other parity tests; frame masks bit-exact on
every row whose block set matches the oracle's and whose frame cut is outside
the float32 exemption rule; outputs within the bf16 tolerances, the oracle fed
the GPU's own masks."""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_amd as A
import oracle as O
import synth_inputs as si
from parity_utils import compare_masks, compare_outputs, sample_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda:0"


def _wl(cfg, grid, block, heads, d, k_floor=2):
    return si.Workload(cfg, f"frames-{cfg}", 1, heads, d, "bf16", grid, block, (0.9,), k_floor,
                       0.0, "u13")


SMALL = {
    # 2x8x8 blocks, the last t-plane of blocks cut to one frame, h and w cut too
    "2x8x8-ragged": _wl(401, (5, 12, 20), (2, 8, 8), 3, 128),
    "2x8x8-d64": _wl(402, (6, 16, 24), (2, 8, 8), 2, 64),
    # four frames a block, cut on every axis (frames of 16 or fewer tokens)
    "4x4x8-ragged": _wl(403, (7, 10, 13), (4, 4, 8), 2, 128),
    # one frame a block: the frame level re-runs Top-p over the kept blocks
    "1x8x16": _wl(404, (3, 13, 21), (1, 8, 16), 2, 128),
}


def _frame_keep(rp, ci, fm, B, H, nb, bt):
    keep = np.zeros((B * H * nb, nb, bt), dtype=bool)
    for r in range(B * H * nb):
        for e in range(rp[r], rp[r + 1]):
            for t in range(bt):
                keep[r, ci[e], t] = (int(fm[e]) >> t) & 1
    return keep.reshape(B, H, nb, nb, bt)


def compare_frames(gpu_fk, gpu_keep, res, p_frame, k_floor, bt):
    """Frame masks row by row where the block sets agree: exact outside the
    exemption rule (oracle frame diagnostics), invariants inside it."""
    B, H, nb, _ = res["keep"].shape
    close, near = O.row_exemption_causes(res["frame_diag"], p_frame, k_floor)
    exempt = close | near
    same_blocks = (gpu_keep == res["keep"]).all(axis=-1)
    counts = res["frame_counts"]
    n_exact = n_exempt = n_skipped = 0
    for b in range(B):
        for h in range(H):
            for i in range(nb):
                g = gpu_fk[b, h, i]
                # always: frames only inside kept blocks and with real tokens,
                # the own block whole
                assert not g[~gpu_keep[b, h, i]].any(), (b, h, i)
                assert not g[counts == 0].any(), (b, h, i)
                assert g[i][counts[i] > 0].all(), (b, h, i, "own frames")
                if not same_blocks[b, h, i]:
                    n_skipped += 1
                    continue
                if not exempt[b, h, i]:
                    assert np.array_equal(g, res["frame_keep"][b, h, i]), (b, h, i)
                    n_exact += 1
                else:
                    cand = int((res["keep"][b, h, i][:, None] & (counts > 0)).sum())
                    assert g.sum() >= min(k_floor, cand), (b, h, i)
                    assert abs(int(g.sum()) - int(res["frame_keep"][b, h, i].sum())) <= 1
                    assert int((g != res["frame_keep"][b, h, i]).sum()) <= 2
                    n_exempt += 1
    assert n_exact > 0
    return dict(exact=n_exact, exempt=n_exempt, block_row_differs=n_skipped)


def _run(wl, p, k_floor, p_frame, sched=None, inputs=None):
    q, k, v = inputs if inputs is not None else si.make_inputs(wl)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    print(f"[gpu case] frames {wl.name} grid={wl.grid} block={wl.block} p={p} p_frame={p_frame} "
          f"sched={sched}", flush=True)
    mask, fm = A.route_frames(plan, qd, kd, p, k_floor, p_frame)
    o = A.attend_frames(plan, qd, kd, vd, mask, fm, sched=sched)
    torch.cuda.synchronize()
    rp, ci = mask.to_host()
    return dict(q=q, k=k, v=v, rp=rp, ci=ci, fm=fm[: ci.size].cpu().numpy(),
                o=o.float().cpu().numpy(), plan=plan, mask=mask, fm_t=fm)


def _np(t):
    return t.float().numpy()


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("p_frame", [0.7, 0.9])
def test_small_frames_parity(name, p_frame):
    wl = SMALL[name]
    p, pf = float(np.float32(0.9)), float(np.float32(p_frame))
    r = _run(wl, p, wl.k_floor, pf)
    geo = O.geometry(wl.grid, wl.block)
    bt = wl.block[0]
    res = O.route_frames(_np(r["q"]), _np(r["k"]), geo, p, wl.k_floor, pf)
    keep = O.csr_to_keep(r["rp"], r["ci"], 1, wl.heads, geo.nb)
    print("block rows", compare_masks(keep, res, p, wl.k_floor))
    fk = _frame_keep(r["rp"], r["ci"], r["fm"], 1, wl.heads, geo.nb, bt)
    print("frame rows", compare_frames(fk, keep, res, pf, wl.k_floor, bt))
    o_ref = O.sparse_attention_frames(_np(r["q"]), _np(r["k"]), _np(r["v"]), geo, r["rp"],
                                      r["ci"], r["fm"])
    rows = range(wl.heads * geo.nb)
    print("max/mean err", compare_outputs(r["o"], o_ref, geo, rows, wl.heads, "bf16"))
    # the same bits under every schedule
    for sched in (A.SCHED_NNZ_SORTED, A.SCHED_HEAD_MAJOR, A.SCHED_HEAD_PHASED,
                  A.SCHED_XCD_LOCAL):
        o2 = _run(wl, p, wl.k_floor, pf, sched=sched, inputs=(r["q"], r["k"], r["v"]))["o"]
        assert np.array_equal(o2, r["o"])


@pytest.mark.parametrize("name", ["2x8x8-ragged", "4x4x8-ragged"])
def test_p_frame_one_is_the_block_path(name):
    """p_frame = 1 keeps every real frame of every kept block: the same CSR as
    abs_route and, through the frame kernel, the same bits as abs_attend."""
    wl = SMALL[name]
    inputs = si.make_inputs(wl)
    p = float(np.float32(0.9))
    r = _run(wl, p, wl.k_floor, 1.0, inputs=inputs)
    geo = O.geometry(wl.grid, wl.block)
    qd, kd, vd = (t.to(DEV) for t in inputs)
    plan = r["plan"]
    m2 = A.route(plan, qd, kd, p, wl.k_floor)
    o2 = A.attend(plan, qd, kd, vd, m2)
    torch.cuda.synchronize()
    rp2, ci2 = m2.to_host()
    assert np.array_equal(rp2, r["rp"]) and np.array_equal(ci2, r["ci"])
    res = O.route_frames(_np(inputs[0]), _np(inputs[1]), geo, p, wl.k_floor, 1.0)
    counts = res["frame_counts"]
    want = [sum(1 << t for t in range(wl.block[0]) if counts[j, t] > 0) for j in r["ci"]]
    assert r["fm"].tolist() == want
    assert np.array_equal(o2.float().cpu().numpy(), r["o"])


@pytest.mark.slow
def test_frames_480p_sampled():
    wl = si.WORKLOADS[1]
    p, pf = float(np.float32(0.9)), float(np.float32(0.9))
    inputs = si.make_inputs(wl)
    r = _run(wl, p, wl.k_floor, pf, inputs=inputs)
    geo = O.geometry(wl.grid, wl.block)
    q, k, v = (_np(t) for t in inputs)
    res = O.route_frames(q, k, geo, p, wl.k_floor, pf)
    keep = O.csr_to_keep(r["rp"], r["ci"], 1, wl.heads, geo.nb)
    print("block rows", compare_masks(keep, res, p, wl.k_floor))
    fk = _frame_keep(r["rp"], r["ci"], r["fm"], 1, wl.heads, geo.nb, wl.block[0])
    print("frame rows", compare_frames(fk, keep, res, pf, wl.k_floor, wl.block[0]))
    kept_frames = int(sum(bin(int(x)).count("1") for x in r["fm"]))
    print("kept frames", kept_frames, "of", 2 * r["ci"].size)
    rows = sample_rows(r["rp"], 1, wl.heads, geo.nb, geo, seed=41)
    o_ref = O.sparse_attention_frames(q, k, v, geo, r["rp"], r["ci"], r["fm"], rows=rows)
    print("max/mean err", compare_outputs(r["o"], o_ref, geo, rows, wl.heads, "bf16"))
