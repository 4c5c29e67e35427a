"""The no-allocation routing entry point (abs_route_noalloc, static per-GPU
scratch) against abs_route with a caller workspace: identical masks, on two
calls in a row, the second with a smaller input."""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_amd as A
import synth_inputs as si

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda:0"


def _wl(cfg, grid, block, heads, d, dtype, p, k_floor, slack):
    return si.Workload(cfg, f"noalloc-{cfg}", 1, heads, d, dtype, grid, block, (p,), k_floor,
                       slack, "u13")


def _masks(wl, p, slack):
    q, k, _ = si.make_inputs(wl)
    qd, kd = q.to(DEV), k.to(DEV)
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    assert plan.route_ws_bytes <= A.ROUTE_NOALLOC_SCRATCH_BYTES
    print(f"[gpu case] noalloc {wl.name} grid={wl.grid} heads={wl.heads} p={p} slack={slack}",
          flush=True)
    ref = A.route(plan, qd, kd, p, wl.k_floor, slack)
    got = A.Mask(plan, DEV)
    # stale contents in the caller's mask buffers must not matter
    got.row_ptr.fill_(-7)
    got.col_idx.fill_(-7)
    got.head_nnz.fill_(-7)
    A.route_noalloc(plan, qd, kd, p, wl.k_floor, slack, mask=got)
    torch.cuda.synchronize()
    rp, ci = ref.to_host()
    rp2, ci2 = got.to_host()
    return (rp, ci, ref.head_nnz.cpu().numpy()), (rp2, ci2, got.head_nnz.cpu().numpy())


@pytest.mark.parametrize("slack", [0.0, 0.5])
def test_noalloc_matches_route_twice_second_smaller(slack):
    p = float(np.float32(0.3 if slack else 0.9))
    big = _wl(301, (21, 30, 52), (2, 8, 8), 4, 128, "bf16", p, 4, slack)   # 480p grid, 4 heads
    small = _wl(302, (5, 12, 20), (2, 8, 8), 2, 64, "bf16", p, 2, slack)
    for wl in (big, small):
        ref, got = _masks(wl, p, slack)
        for a, b in zip(ref, got):
            assert np.array_equal(a, b)
        assert ref[1].size == int(ref[0][-1]) > 0
