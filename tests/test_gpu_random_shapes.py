"""Parity on a seeded draw of small shapes.

Forty-eight layers whose grid, block shape (32, 64 or 128 tokens), head count,
head dimension, dtype, p and k_floor are drawn from a seeded generator,
ragged tails included (grid sides that are not multiples of the block side,
grids smaller than one block along an axis).  Each is routed and attended on
the GPU and checked against the oracle: the whole mask outside the exemption
rule, the outputs of every row (or of a seeded sample when the layer is
larger), every kept tile done once, and every schedule giving the same bits.
"""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_amd as A
import oracle as O
import synth_inputs as si
from parity_utils import compare_masks, compare_outputs, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

BLOCKS = [(2, 4, 4), (1, 4, 8), (2, 2, 8), (1, 8, 8), (2, 4, 8), (4, 4, 4),
          (2, 8, 8), (4, 4, 8), (1, 8, 16), (8, 4, 4)]


def _draw(i):
    rng = np.random.default_rng([2026, i])
    block = BLOCKS[int(rng.integers(len(BLOCKS)))]
    while True:
        grid = tuple(int(rng.integers(1, 3 * b + 1)) for b in block)
        if grid[0] * grid[1] * grid[2] <= 4000:
            break
    heads = int(rng.integers(1, 4))
    d = int(rng.choice([64, 128]))
    dtype = "f32" if rng.random() < 0.2 else "bf16"
    p = float(np.float32(rng.choice([0.3, 0.6, 0.8, 0.9, 0.95, 1.0])))
    k_floor = int(rng.integers(1, 6))
    return si.Workload(300 + i, f"random-{i}", 1, heads, d, dtype, grid, block, (p,), k_floor,
                       0.0, "u13")


CASES = [_draw(i) for i in range(48)]


@pytest.mark.parametrize("wl", CASES, ids=[f"{w.name}-{w.grid}-{w.block}-h{w.heads}-d{w.head_dim}-"
                                           f"{w.dtype}-p{w.p[0]:.2f}-k{w.k_floor}" for w in CASES])
def test_random_shape_parity(wl):
    p, k_floor = wl.p[0], wl.k_floor
    q, k, v = si.make_inputs(wl)
    geo = O.geometry(wl.grid, wl.block)
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    print(f"[gpu case] {wl.name} grid={wl.grid} block={wl.block} nb={geo.nb} p={p} "
          f"k_floor={k_floor}", flush=True)
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    mask = A.route(plan, qd, kd, p, k_floor)
    sched = A.default_sched(plan)
    tel = torch.zeros(A.attend_grid(plan, sched) * 4, dtype=torch.int64, device=DEV)
    o = A.attend(plan, qd, kd, vd, mask, sched=sched, telemetry=tel)
    torch.cuda.synchronize()
    rp, ci = mask.to_host()
    qn, kn, vn = (t.float().numpy() for t in (q, k, v))
    res = O.route(qn, kn, geo, p, k_floor)
    keep = O.csr_to_keep(rp, ci, wl.batch, wl.heads, geo.nb)
    print("mask rows", compare_masks(keep, res, p, k_floor))
    rows = list(range(wl.batch * wl.heads * geo.nb))
    if len(rows) > 96:
        rows = sample_rows(rp, wl.batch, wl.heads, geo.nb, geo, n_heads=wl.heads, n_blocks=32,
                           seed=wl.cfg)
    o_ref = O.sparse_attention(qn, kn, vn, geo, rp, ci, rows=rows)
    on = o.float().cpu().numpy()
    print("max/mean err", compare_outputs(on, o_ref, geo, rows, wl.heads, wl.dtype))
    assert tel.cpu().numpy().reshape(-1, 4)[:, 2].sum() == ci.size
    for s in (A.SCHED_NNZ_SORTED, A.SCHED_HEAD_MAJOR, A.SCHED_HEAD_PHASED, A.SCHED_XCD_LOCAL):
        o2 = A.attend(plan, qd, kd, vd, mask, sched=s)
        assert torch.equal(o2, o)
