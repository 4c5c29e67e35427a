"""Host-side logic of bench.py (CPU): the per-CU aggregation of telemetry
records, the multi-GPU refusal, and the profile lookup."""
import json
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _hw(se, sa, cu):
    return (se << 13) | (sa << 12) | (cu << 8)


def test_cu_key_fields():
    assert bench.cu_key(_hw(5, 1, 9), 3) == (3, 5, 1, 9)
    assert bench.cu_key(_hw(0, 0, 0) | 0xff, 0x13) == (3, 0, 0, 0)   # low bits and high XCC bits ignored


def test_imbalance_sums_workgroups_per_cu():
    # two workgroups on one CU add up; max/mean over the three CUs
    recs = np.array([
        [_hw(0, 0, 1), 0, 10, 100],
        [_hw(0, 0, 1), 0, 20, 50],     # same CU as the first
        [_hw(0, 0, 2), 0, 15, 120],
        [_hw(1, 0, 1), 1, 15, 180],
    ])
    r = bench.imbalance(recs)
    assert r["cus"] == 3
    tiles = np.array([30, 15, 15], float)
    busy = np.array([150, 120, 180], float)
    assert abs(r["tiles_max_over_mean"] - tiles.max() / tiles.mean()) < 1e-12
    assert abs(r["busy_max_over_mean"] - busy.max() / busy.mean()) < 1e-12


def test_balanced_records_give_one():
    recs = np.array([[_hw(0, 0, c), x, 7, 70] for x in range(8) for c in range(4)])
    r = bench.imbalance(recs)
    assert r["cus"] == 32 and r["tiles_max_over_mean"] == 1.0 and r["busy_max_over_mean"] == 1.0


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2 and "one GPU" in p.stderr


def test_traffic_profile_lookup():
    # the committed profile gives a byte count for the workload and queue it was
    # taken on (while the kernel source is unchanged), and nothing for another
    # queue or workload
    path = os.path.join(ROOT, "profiles", "attn_bf16_wan22_480p_hbm_traffic.md")
    sched = next(l.split(":", 1)[1].strip() for l in open(path) if l.startswith("sched:"))
    t = bench.measured_traffic(1, sched)
    assert t is None or t > 1e9
    assert bench.measured_traffic(1, "head_major") is None
    assert bench.measured_traffic(2, sched) is None


def test_code_digest_ignores_comments_only(tmp_path):
    # the profile match survives comment edits and fails on any code edit
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) {  /* note */\n  return x + 1;   // one\n}\n")
    b = tmp_path / "b.hip"
    b.write_text("/* other\n   header */\nint f(int x) {\n\n  return x + 1;\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("// header\nint f(int x) {  /* note */\n  return x + 2;   // one\n}\n")
    assert bench.code_digest(str(a)) == bench.code_digest(str(b))
    assert bench.code_digest(str(a)) != bench.code_digest(str(c))


def test_cpu_description_names_the_machine():
    d = bench.cpu_description()
    assert d["affinity_cores"] == len(os.sched_getaffinity(0)) and d["blas_threads"] >= 1
    assert d["cpu_model"] is None or isinstance(d["cpu_model"], str)


def test_mask_parity_counts_on_the_oracles_own_mask():
    import oracle as O
    import synth_inputs as si
    wl = si.Workload(802, "counts", 1, 2, 64, "f32", (8, 32, 32), (2, 4, 4), (0.9,), 2, 0.0,
                     "u13")
    q, k, _ = si.make_inputs(wl)
    geo = O.geometry(wl.grid, wl.block)
    p = float(np.float32(0.9))
    res = O.route(q.numpy(), k.numpy(), geo, p, 2)
    rp, ci, _ = O.keep_to_csr(res["keep"])
    c = bench.mask_parity_counts(res, p, 2, rp, ci)
    assert c["rows"] == 2 * geo.nb
    assert c["exact_checked_differing"] == 0 and c["exempt_differing"] == 0
    assert c["exact_checked_equal"] + c["exempt_equal"] == c["rows"]
    assert c["exempt_mass_close"] + c["exempt_near_tie"] == c["exempt_equal"]
    # one planted change in an exact-checked row is counted there
    exempt = O.row_exemptions(res["diag"], p, 2)
    h, i = map(int, np.argwhere(~exempt[0])[0])
    keep = res["keep"].copy()
    j = (i + 1) % geo.nb
    keep[0, h, i, j] = ~keep[0, h, i, j]
    rp2, ci2, _ = O.keep_to_csr(keep)
    assert bench.mask_parity_counts(res, p, 2, rp2, ci2)["exact_checked_differing"] == 1


def test_executed_flop_lookup_is_bound_to_workload_and_queue():
    assert bench.measured_executed_flop(2, "head_phased") is None
    assert bench.measured_executed_flop(1, "head_major") is None
