"""GPU parity of the dynamic slack fill and its telemetry budget (C ABI).

The budget kernel is integer work on the telemetry records: bit-exact against
oracle.slack_budget on the same records.  The fill is compared with
oracle.dynamic_slack_fill applied to the GPU's own base mask (pairs may differ
only at float32 near-ties with the selection threshold or theta).  Attention
on the filled mask is compared with the oracle as everywhere else.
"""
import numpy as np
import pytest
import torch

import adaptive_block_sparse_amd as A
import oracle as O
import synth_inputs as si
from parity_utils import check_dynamic_slack, compare_masks, compare_outputs, sample_rows

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

DEV = "cuda:0"


def _wl(cfg, grid, block, heads, d):
    return si.Workload(cfg, f"dslack-{cfg}", 1, heads, d, "bf16", grid, block, (0.9,), 2, 0.0,
                       "u13")


SMALL = {
    "d128-bt128-ragged": _wl(101, (5, 12, 20), (2, 8, 8), 3, 128),
    "d64-bt64-ragged": _wl(102, (3, 20, 12), (1, 8, 8), 2, 64),
    "d128-bt32": _wl(103, (4, 9, 10), (2, 4, 4), 2, 128),
}


def _np(t):
    return t.float().numpy()


class Case:
    def __init__(self, wl, p=0.9, k_floor=None, inputs=None):
        self.wl = wl
        self.p = float(np.float32(p))
        self.kf = wl.k_floor if k_floor is None else k_floor
        print(f"[gpu case] dynamic slack {wl.name} p={self.p}", flush=True)
        self.inputs = si.make_inputs(wl) if inputs is None else inputs
        self.q, self.k, self.v = (t.to(DEV) for t in self.inputs)
        self.plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
        self.geo = O.geometry(wl.grid, wl.block)
        self.base = A.route(self.plan, self.q, self.k, self.p, self.kf)
        torch.cuda.synchronize()
        brp, bci = self.base.to_host()
        self.base_keep = O.csr_to_keep(brp, bci, wl.batch, wl.heads, self.geo.nb)
        self.res = O.route(_np(self.inputs[0]), _np(self.inputs[1]), self.geo, self.p, self.kf)

    def fill(self, budget, theta):
        print(f"[gpu case]   budget={budget} theta={theta}", flush=True)
        b = torch.tensor([budget], dtype=torch.int64, device=DEV)
        m = A.route_dynamic(self.plan, self.q, self.k, self.p, self.kf, theta, b)
        torch.cuda.synchronize()
        rp, ci = m.to_host()
        keep = O.csr_to_keep(rp, ci, self.wl.batch, self.wl.heads, self.geo.nb)
        assert m.head_nnz.cpu().numpy().sum() == ci.size
        return m, keep, rp, ci


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("budget,theta", [(0, 0.0), (37, 0.0), (500, 0.002), (10 ** 9, 0.004)])
def test_dynamic_fill_small(name, budget, theta):
    c = Case(SMALL[name])
    compare_masks(c.base_keep, c.res, c.p, c.kf)
    theta = float(np.float32(theta))
    m, keep, rp, ci = c.fill(budget, theta)
    diffs, info = check_dynamic_slack(keep, c.base_keep, c.res["P"], budget, theta)
    print("added", info["added"], "of", info["candidates"], "candidates; pairs off the oracle", diffs)
    if budget == 0:
        assert np.array_equal(keep, c.base_keep)
    o = A.attend(c.plan, c.q, c.k, c.v, m)
    torch.cuda.synchronize()
    o_ref = O.sparse_attention(*(_np(t) for t in c.inputs), c.geo, rp, ci)
    rows = range(c.wl.batch * c.wl.heads * c.geo.nb)
    compare_outputs(o.float().cpu().numpy(), o_ref, c.geo, rows, c.wl.heads, "bf16")


def _telemetry_run(c, mask, sched):
    n = A.attend_grid(c.plan, sched)
    tel = torch.zeros(n * 4, dtype=torch.int64, device=DEV)
    A.attend(c.plan, c.q, c.k, c.v, mask, sched=sched, telemetry=tel)
    torch.cuda.synchronize()
    return tel


@pytest.mark.parametrize("sched", [A.SCHED_XCD_LOCAL, A.SCHED_HEAD_PHASED])
def test_budget_kernel_matches_oracle(sched):
    c = Case(SMALL["d128-bt128-ragged"])
    tel = _telemetry_run(c, c.base, sched)
    records = tel.cpu().numpy().reshape(-1, 4)
    assert int(records[:, 2].sum()) == int(c.base_keep.sum())
    out = torch.zeros(1, dtype=torch.int64, device=DEV)
    for fill, cap in ((1.0, 10 ** 12), (0.37, 10 ** 12), (0.0, 10 ** 12), (1.0, 5)):
        fill = float(np.float32(fill))
        A.slack_budget(c.plan, sched, tel, fill, cap, out)
        torch.cuda.synchronize()
        want = O.slack_budget(records, fill, cap)
        print("fill", fill, "cap", cap, "budget", int(out.item()), "oracle", want)
        assert int(out.item()) == want


@pytest.mark.slow
def test_dynamic_slack_480p_loop():
    """The 480p layer: base launch -> telemetry -> budget kernel -> routing with
    the fill -> attention, all on the device in stream order.  Budget bit-exact,
    fill against the oracle on the GPU's base mask, sampled attention rows."""
    wl = si.WORKLOADS[1]
    c = Case(wl, k_floor=wl.k_floor)
    sched = A.SCHED_XCD_LOCAL
    tel = _telemetry_run(c, c.base, sched)
    budget = torch.zeros(1, dtype=torch.int64, device=DEV)
    theta = float(np.float32(1e-3))
    A.slack_budget(c.plan, sched, tel, 1.0, 10 ** 9, budget)
    m = A.route_dynamic(c.plan, c.q, c.k, c.p, c.kf, theta, budget)
    o = A.attend(c.plan, c.q, c.k, c.v, m, sched=sched)
    torch.cuda.synchronize()
    want = O.slack_budget(tel.cpu().numpy().reshape(-1, 4), 1.0, 10 ** 9)
    assert int(budget.item()) == want and want > 0
    rp, ci = m.to_host()
    keep = O.csr_to_keep(rp, ci, 1, wl.heads, c.geo.nb)
    diffs, info = check_dynamic_slack(keep, c.base_keep, c.res["P"], want, theta)
    print("budget", want, "added", info["added"], "pairs off the oracle", diffs)
    q, k, v = (_np(t) for t in c.inputs)
    rows = sample_rows(rp, 1, wl.heads, c.geo.nb, c.geo, seed=7)
    o_ref = O.sparse_attention(q, k, v, c.geo, rp, ci, rows=rows)
    print("max/mean err", compare_outputs(o.float().cpu().numpy(), o_ref, c.geo, rows, wl.heads,
                                          "bf16"))
