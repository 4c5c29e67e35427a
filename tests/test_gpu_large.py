"""Shape ceilings on the GPU.

* The largest block count per head the plan accepts, nb = 8192 (128-token
  blocks cut by the grid on every axis): the widest routing rows (a row of
  8192 blocks in one wave's registers) and block numbers past 4096 in the
  attention kernel's block table.
* A layer whose Q, K, V and O tensors hold more than 2^31 elements each (64
  heads x 266 240 tokens x d = 128): every element offset of the pooling, the
  K/V re-layout and the attention loads and stores must be 64-bit, and the
  attention kernel's tile copies, addressed as a 64-bit scalar base plus a
  32-bit lane offset, reach tiles whose address has bit 31 of its low half
  set (the base's low half must be zero-extended, not sign-extended).  Heads 0
  and 63 carry the seeded synthetic inputs and are checked against the oracle
  (pooled means, the whole mask outside the exemption rule, sampled outputs
  that include the highest token offsets); the other heads are seeded random
  normal values that fill the layout.
"""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_amd as A
import oracle as O
import synth_inputs as si
from parity_utils import compare_masks, compare_outputs, sample_rows

pytestmark = [pytest.mark.gpu, pytest.mark.slow]
DEV = "cuda:0"
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)


def _np(t):
    return t.float().numpy()


def test_largest_block_count_per_head():
    wl = si.Workload(114, "test-114-nb8192", 1, 1, 128, "bf16", (31, 125, 250), (2, 8, 8),
                     (0.9,), 3, 0.0, "u13")
    geo = O.geometry(wl.grid, wl.block)
    assert geo.nb == 8192
    q, k, v = si.make_inputs(wl)
    p = float(np.float32(0.9))
    plan = A.plan_init(1, 1, 128, wl.grid, wl.block, "bf16")
    print(f"[gpu case] {wl.name} nb={geo.nb} tokens={wl.tokens}", flush=True)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    mask = A.route(plan, qd, kd, p, wl.k_floor)
    o = A.attend(plan, qd, kd, vd, mask)
    torch.cuda.synchronize()
    rp, ci = mask.to_host()
    qn, kn, vn = _np(q), _np(k), _np(v)
    res = O.route(qn, kn, geo, p, wl.k_floor)
    keep = O.csr_to_keep(rp, ci, 1, 1, geo.nb)
    print("mask rows", compare_masks(keep, res, p, wl.k_floor))
    rows = sorted(set(sample_rows(rp, 1, 1, geo.nb, geo, n_heads=1, n_blocks=16, seed=114)
                      + [geo.nb - 1, geo.nb - 2]))
    o_ref = O.sparse_attention(qn, kn, vn, geo, rp, ci, rows=rows)
    print("max/mean err", compare_outputs(_np(o.cpu()), o_ref, geo, rows, 1, "bf16"))


def test_tensors_beyond_2_31_elements():
    B, H, d = 1, 64, 128
    wl = si.Workload(115, "test-115-2e31", B, H, d, "bf16", (16, 128, 130), (2, 8, 8), (0.9,), 4,
                     0.0, "u13")
    N = wl.tokens
    assert N * H * d > 2 ** 31
    geo = O.geometry(wl.grid, wl.block)
    checked = (0, H - 1)
    q2, k2, v2 = si.make_inputs(wl, heads=list(checked))
    gen = torch.Generator(device=DEV)
    full = []
    for stream, src in enumerate((q2, k2, v2)):
        gen.manual_seed(115 * 16 + stream)
        t = torch.randn((B, N, H, d), generator=gen, device=DEV, dtype=torch.bfloat16)
        for slot, h in enumerate(checked):
            t[:, :, h, :] = src[:, :, slot, :].to(DEV)
        full.append(t)
    qd, kd, vd = full
    p = float(np.float32(0.9))
    plan = A.plan_init(B, H, d, wl.grid, wl.block, "bf16")
    print(f"[gpu case] {wl.name} elements={N * H * d} nb={geo.nb}", flush=True)
    rws = A.workspace(plan.route_ws_bytes, DEV)
    mask = A.route(plan, qd, kd, p, wl.k_floor, ws=rws)
    o = A.attend(plan, qd, kd, vd, mask)
    torch.cuda.synchronize()
    n = B * H * geo.nb * d
    pooled = rws[: 2 * n * 4].view(torch.float32).view(2, B, H, geo.nb, d)
    rp, ci = mask.to_host()
    nb = geo.nb
    for slot, h in enumerate(checked):
        qn = _np(q2[:, :, slot:slot + 1, :])
        kn = _np(k2[:, :, slot:slot + 1, :])
        vn = _np(v2[:, :, slot:slot + 1, :])
        # pooled means of this head (the pooling kernel's loads)
        np.testing.assert_allclose(pooled[0, :, h:h + 1].cpu().numpy(), O.pool(qn, geo),
                                   rtol=1e-5, atol=1e-5)
        np.testing.assert_allclose(pooled[1, :, h:h + 1].cpu().numpy(), O.pool(kn, geo),
                                   rtol=1e-5, atol=1e-5)
        # this head's rows of the mask
        r0, r1 = h * nb, (h + 1) * nb
        rph = rp[r0:r1 + 1] - rp[r0]
        cih = ci[rp[r0]:rp[r1]]
        res = O.route(qn, kn, geo, p, wl.k_floor)
        keep = O.csr_to_keep(rph, cih, 1, 1, nb)
        print(f"head {h} mask rows", compare_masks(keep, res, p, wl.k_floor))
        # outputs of sampled query blocks, the last ones (highest offsets) included
        rows = sorted(set(sample_rows(rph, 1, 1, nb, geo, n_heads=1, n_blocks=4, seed=115 + h)
                          + [nb - 1]))
        o_ref = O.sparse_attention(qn, kn, vn, geo, rph, cih, rows=rows)
        oh = _np(o[:, :, h:h + 1, :].cpu())
        print(f"head {h} max/mean err", compare_outputs(oh, o_ref, geo, rows, 1, "bf16"))
