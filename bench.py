#!/usr/bin/env python3
"""Benchmark: one adaptive block-sparse attention layer per step on one MI355X.

A step is the whole hot path on one synthetic input batch: route (3D-block
pooling, pooled scores, Top-p + k_floor + own-block repair, CSR; slack fill
when the workload has one) followed by attend (K/V re-layout, work schedule,
persistent block-sparse attention).  Inputs are resident in HBM before the
timed region.  Prints one JSON line.

  python bench.py [--steps K] [--warmup W] [--workload 1] [--sched head_phased]
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector
PEAK_HBM_GBS = 8000.0


def cu_key(hw_id: int, xcc: int):
    """(XCC, shader engine, shader array, CU) from the HW_ID / XCC_ID registers."""
    return (xcc & 0xF, (hw_id >> 13) & 0x7, (hw_id >> 12) & 0x1, (hw_id >> 8) & 0xF)


def imbalance(tel: np.ndarray):
    per_cu_tiles, per_cu_busy = {}, {}
    for hw, xcc, tiles, busy in tel.tolist():
        k = cu_key(int(hw), int(xcc))
        per_cu_tiles[k] = per_cu_tiles.get(k, 0) + tiles
        per_cu_busy[k] = per_cu_busy.get(k, 0) + busy
    t = np.array(list(per_cu_tiles.values()), dtype=np.float64)
    b = np.array(list(per_cu_busy.values()), dtype=np.float64)
    return dict(cus=len(t), tiles_max_over_mean=float(t.max() / t.mean()),
                busy_max_over_mean=float(b.max() / b.mean()))


def code_digest(*paths: str) -> str:
    """sha256 of C++/HIP sources with their comments and blank space removed:
    it changes when the code changes, not when only a comment does."""
    import hashlib
    import re
    parts = []
    for path in paths:
        text = open(path).read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        parts.append("\n".join(" ".join(line.split()) for line in text.splitlines()
                               if line.strip()))
    return hashlib.sha256("\n\f\n".join(parts).encode()).hexdigest()


# the sources compiled into the attention kernel
ATTEND_SOURCES = [os.path.join(ROOT, "adaptive_block_sparse_amd", "csrc", f)
                  for f in ("attend.hip", "internal.h", "device_common.h")]


def measured_traffic(workload_cfg: int, sched: str):
    """HBM bytes per launch of the attention kernel from the committed rocprofv3
    FETCH_SIZE/WRITE_SIZE summary, if it was taken on this workload and launch
    and the kernel code has not changed since (else None)."""
    path = os.path.join(ROOT, "profiles", "attn_bf16_wan22_480p_hbm_traffic.md")
    if workload_cfg != 1 or not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith((" ", "|", "#")):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    if (fields.get("attend_code_sha256") != code_digest(*ATTEND_SOURCES)
            or fields.get("sched") != sched
            or "traffic_bytes_per_launch" not in fields):
        return None
    return int(fields["traffic_bytes_per_launch"])


def _profile_fields(name: str):
    path = os.path.join(ROOT, "profiles", name)
    fields = {}
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith((" ", "|", "#", "*")):
                key, _, val = line.partition(":")
                fields[key.strip()] = val.strip()
    return fields


def measured_executed_flop(workload_cfg: int, sched: str):
    """bf16 MFMA flop executed per launch of the attention kernel, from the
    committed rocprofv3 SQ_INSTS_VALU_MFMA_MOPS_BF16 summary, if it was taken
    on this workload and launch and the kernel code has not changed since
    (else None)."""
    if workload_cfg != 1:
        return None
    f = _profile_fields("attn_bf16_wan22_480p_mfma_lds_counters.md")
    if (f.get("attend_code_sha256") != code_digest(*ATTEND_SOURCES) or f.get("sched") != sched
            or "executed_flop_per_launch" not in f):
        return None
    return float(f["executed_flop_per_launch"])


def cpu_description():
    """CPU model, the cores this process may run on, and the BLAS threads."""
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    affinity = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max(int(i.get("num_threads", 1)) for i in threadpool_info()) or 1
    except Exception:
        blas = affinity
    return {"cpu_model": model, "affinity_cores": affinity, "blas_threads": blas}


def mask_parity_counts(res: dict, p: float, k_floor: int, rp, ci):
    """The GPU mask against the oracle's, row by row (counts only; the GPU
    tests assert): rows the float32 exemption rule leaves exact-checked and
    whether they match, and exempt rows by reason and whether they match."""
    import oracle as O
    B, H, nb, _ = res["base_keep"].shape
    keep = O.csr_to_keep(rp, ci, B, H, nb)
    ref = res["keep"]
    same = (keep == ref).all(axis=-1)
    close, near = O.row_exemption_causes(res["diag"], p, k_floor)
    exempt = close | near
    return {"rows": int(same.size),
            "exact_checked_equal": int((same & ~exempt).sum()),
            "exact_checked_differing": int((~same & ~exempt).sum()),
            "exempt_mass_close": int(close.sum()),
            "exempt_near_tie": int((near & ~close).sum()),
            "exempt_equal": int((same & exempt).sum()),
            "exempt_differing": int((~same & exempt).sum())}


def block_valid_counts(grid, block) -> np.ndarray:
    """Real tokens in each 3D block (row-major block order)."""
    per_axis = []
    for g, b in zip(grid, block):
        n = -(-g // b)
        per_axis.append(np.array([min(b, g - i * b) for i in range(n)], dtype=np.float64))
    return np.einsum("i,j,k->ijk", *per_axis).ravel()


def _probe_lib():
    import ctypes
    path = os.path.join(ROOT, "adaptive_block_sparse_amd", "libabs_probe.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -m adaptive_block_sparse_amd.build)")
    lib = ctypes.CDLL(path)
    V = ctypes.c_void_p
    lib.abs_probe_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, V, V, V]
    lib.abs_probe_attn_loop.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, V, V, V]
    lib.abs_probe_wall_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int32)]
    return lib


def _time_probe(dev, launch, threads: int, workgroups: int, launches: int):
    """Median time of `launches` timed launches (after two untimed ones) and
    the median clock64 rate against the wall clock inside the loops."""
    import ctypes
    import torch
    lib = _probe_lib()
    out = torch.empty(workgroups * threads, dtype=torch.float32, device=dev)
    clocks = torch.zeros(workgroups * 2, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream()
    khz = ctypes.c_int32(0)
    if lib.abs_probe_wall_clock_khz(ctypes.byref(khz)) != 0 or khz.value <= 0:
        raise RuntimeError("wall clock rate query failed")
    times, clk = [], []
    for i in range(2 + launches):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        rc = launch(lib, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(clocks.data_ptr()),
                    ctypes.c_void_p(stream.cuda_stream))
        e1.record(stream)
        if rc != 0:
            raise RuntimeError(f"probe launch returned {rc}")
        torch.cuda.synchronize()
        if i >= 2:
            times.append(e0.elapsed_time(e1) * 1e-3)
            c = clocks.cpu().numpy().reshape(-1, 2).astype(np.float64)
            clk.append(float(np.median(c[:, 0] / (c[:, 1] / (khz.value * 1e3)))) / 1e9)
    assert bool(torch.isfinite(out).all())
    return float(np.median(times)), float(np.median(clk))


def mfma_probe(dev, iters: int = 40000, workgroups: int = 512, launches: int = 5):
    """Sustained bf16 MFMA rate of this GPU on its own (libabs_probe.so, a
    measurement aid): every wave issues v_mfma_f32_32x32x16_bf16 back to back
    on varied operands, four independent accumulators.  512 workgroups of four
    waves are two waves on every SIMD, all resident at once (the attention
    kernel's occupancy); one wave per SIMD (256) sustains less.  Median of
    `launches` timed launches after two untimed ones.  clock64_ghz is the rate
    of the device's clock64 counter against its wall clock during the loops."""
    t, clk = _time_probe(dev, lambda lib, o, c, s: lib.abs_probe_mfma_bf16(iters, workgroups, o, c, s),
                         256, workgroups, launches)
    flop = workgroups * 4 * iters * 4 * 32 * 32 * 16 * 2
    return {"tflops": round(flop / t / 1e12, 1), "clock64_ghz": round(clk, 3),
            "ms_per_launch": round(t * 1e3, 3), "iters": iters, "workgroups": workgroups,
            "waves_per_simd": workgroups // 256, "launches": launches}


def attn_loop_probe(dev, queries_per_wave: int = 32, iters: int = 12000, workgroups: int = 256,
                    launches: int = 5):
    """Rate of the attention kernel's per-subtile arithmetic on its own
    (libabs_probe.so): scores, FAST-walk softmax and PV products of one 32-key
    subtile a round, operands from LDS, with no copies, barrier, padding or
    work items.  32 queries per wave: two waves per SIMD, as in the kernel; 64:
    one wave per SIMD holding two query groups."""
    threads = 512 if queries_per_wave == 32 else 256
    t, clk = _time_probe(dev, lambda lib, o, c, s: lib.abs_probe_attn_loop(
        queries_per_wave, iters, workgroups, o, c, s), threads, workgroups, launches)
    flop = workgroups * iters * (threads // 64) * (queries_per_wave // 32) * 16 * 32768
    return {"tflops": round(flop / t / 1e12, 1), "clock64_ghz": round(clk, 3),
            "ms_per_launch": round(t * 1e3, 3), "queries_per_wave": queries_per_wave,
            "iters": iters, "workgroups": workgroups, "launches": launches}


def cpu_baseline(wl, p, inputs, rp, ci, budget_s=20.0):
    """The oracle, as it stands, on the host cores: full routing of every row,
    attention on a seeded row sample extrapolated by kept tiles."""
    import oracle as O
    cpu = cpu_description()
    q, k, v = (t.float().numpy() for t in inputs)
    geo = O.geometry(wl.grid, wl.block)
    t0 = time.perf_counter()
    res = O.route(q, k, geo, p, wl.k_floor, wl.slack)
    t_route = time.perf_counter() - t0
    counts = np.diff(rp)
    rng = np.random.default_rng(7)
    order = rng.permutation(counts.size)
    done_rows, done_tiles, t_att = 0, 0, 0.0
    for r in order:
        t1 = time.perf_counter()
        O.sparse_attention(q, k, v, geo, rp, ci, rows=[int(r)])
        t_att += time.perf_counter() - t1
        done_rows += 1
        done_tiles += int(counts[r])
        if t_route + t_att > budget_s and done_rows >= 8:
            break
    total_tiles = int(counts.sum())
    t_layer = t_route + t_att * total_tiles / done_tiles
    return dict(t_layer_s=t_layer, t_route_s=t_route, rows=done_rows, tiles=done_tiles,
                total_tiles=total_tiles, cores=cpu["blas_threads"], cpu=cpu, route=res)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=1)
    ap.add_argument("--p", type=float, default=None)
    ap.add_argument("--frames", type=float, default=None, metavar="P_FRAME",
                    help="fine-grained routing: after the block-level Top-p, Top-p over the "
                         "frames of each row's kept blocks (abs_route_frames, abs_attend_frames)")
    ap.add_argument("--slack", type=float, default=None,
                    help="per-head slack budget as a fraction of nb^2 (default: the workload's; "
                         "0 turns the fixed fill off)")
    ap.add_argument("--heads", type=int, default=None,
                    help="run only the first H heads of the workload (one rank's share when "
                         "the layer is sharded by head across GPUs)")
    ap.add_argument("--sched", default=None,
                    choices=["nnz_sorted", "head_major", "head_phased", "xcd_local"],
                    help="work order (default: the library's choice for the shape; "
                         "head_phased with --split)")
    ap.add_argument("--split", type=int, default=None,
                    help="split-and-merge attention: cut work items whose union list is longer "
                         "than SPLIT entries into parts, merge the parts by log-sum-exp")
    ap.add_argument("--max-parts", type=int, default=None,
                    help="partial-result slots for --split (default: two per persistent "
                         "workgroup)")
    ap.add_argument("--dynamic-slack", type=float, default=None, metavar="FILL",
                    help="dynamic slack fill: a base launch's telemetry gives the idle capacity; "
                         "FILL of it (0..1) is filled with the highest-P unkept pairs")
    ap.add_argument("--slack-theta", type=float, default=1e-3,
                    help="score threshold of the dynamic fill (P >= theta)")
    ap.add_argument("--slack-cap", type=int, default=None,
                    help="cap on pairs the dynamic fill adds (default: 5%% of the base mask)")
    ap.add_argument("--pipeline", default="beside_route",
                    choices=["beside_route", "beside_route_only", "after_route", "serial"],
                    help="where the mask-independent K/V re-layout runs: on a second stream "
                         "beside routing and the mask-dependent schedule kernels (default); "
                         "beside routing only (the schedule kernels wait for it); on a second "
                         "stream after routing, beside the schedule kernels; or after routing "
                         "on one stream")
    ap.add_argument("--no-overlap", action="store_true",
                    help="the same as --pipeline serial")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--timed-only", action="store_true",
                    help="run only the warmup and timed steps (no schedule sweep, cold step or "
                         "dense comparator): every attention launch is then one of the timed "
                         "configuration, as profiler summaries need")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (for HBM counter scaling)")
    ap.add_argument("--mfma-peak", action="store_true",
                    help="run only the probes: the bf16 MFMA rate this GPU sustains on its own "
                         "at one, two and three waves per SIMD and its clock meanwhile, and the "
                         "attention kernel's per-subtile arithmetic alone at 32 and 64 queries "
                         "per wave")
    ap.add_argument("--probe-launches", type=int, default=5,
                    help="timed launches of each probe (about 10 ms each)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(a layer would shard by head, each GPU attending its own heads).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = "cuda:0"

    if args.copy_calibration:
        x = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "launches": 3}))
        return
    if args.mfma_peak:
        n = args.probe_launches
        print(json.dumps({"mfma_probe_bf16": [mfma_probe(dev, workgroups=w, launches=n)
                                              for w in (256, 512, 768)],
                          "attn_loop_probe": [attn_loop_probe(dev, qpw, launches=n)
                                              for qpw in (32, 64)]}))
        return

    import adaptive_block_sparse_amd as A
    import synth_inputs as si

    wl = si.WORKLOADS[args.workload]
    if args.heads is not None:
        if not 1 <= args.heads <= wl.heads:
            print(f"--heads must be in 1..{wl.heads}", file=sys.stderr)
            sys.exit(2)
        wl = dataclasses.replace(wl, heads=args.heads, name=f"{wl.name}-first{args.heads}heads")
    if args.slack is not None:
        if not 0.0 <= args.slack < 1.0:
            print("--slack must be in [0, 1)", file=sys.stderr)
            sys.exit(2)
        wl = dataclasses.replace(wl, slack=args.slack)
    p = float(np.float32(args.p if args.p is not None else wl.p[0]))
    split = args.split is not None
    frames = args.frames is not None
    if frames and (split or args.dynamic_slack is not None or wl.dtype != "bf16"):
        print("--frames runs the plain bf16 path (no --split, no --dynamic-slack)", file=sys.stderr)
        sys.exit(2)
    if frames:
        wl = dataclasses.replace(wl, slack=0.0)
        args.no_cpu_baseline = True
    if split and args.sched not in (None, "nnz_sorted", "head_phased"):
        print("--split runs on the sorted queues: --sched nnz_sorted or head_phased",
              file=sys.stderr)
        sys.exit(2)
    print(f"[bench] generating {wl.name}", file=sys.stderr, flush=True)
    inputs = si.make_inputs(wl)
    q, k, v = (t.to(dev) for t in inputs)
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    if args.sched is None:
        args.sched = "head_phased" if split else {v_: k_ for k_, v_ in A.SCHEDULES.items()}[
            A.default_sched(plan)]
    sched = A.SCHEDULES[args.sched]
    mask = A.Mask(plan, dev)
    rws = A.workspace(plan.route_ws_bytes, dev)
    max_parts = 0
    if split:
        # default: two slots per persistent workgroup (the heaviest items are cut first)
        max_parts = (args.max_parts if args.max_parts is not None
                     else 2 * A.attend_grid(plan, sched))
        aws = A.workspace(A.attend_split_ws_bytes(plan, max_parts), dev)
    else:
        aws = A.workspace(plan.attend_ws_bytes, dev)
    o = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def prepare(msk, s_, ws_=None):
        ws_ = aws if ws_ is None else ws_
        if split:
            A.attend_prepare_split(plan, k, v, msk, s_, args.split, max_parts, ws_)
        else:
            A.attend_prepare(plan, k, v, msk, s_, ws_)

    def run(msk, out, s_, telemetry=None, ws_=None):
        ws_ = aws if ws_ is None else ws_
        if split:
            A.attend_run_split(plan, q, msk, out, s_, max_parts, ws_, telemetry=telemetry)
        else:
            A.attend_run(plan, q, k, msk, out, s_, ws_, telemetry=telemetry)

    # dynamic slack: one base launch's telemetry sets the budget (on the device)
    dyn = None
    o2_dyn = torch.empty_like(q) if args.dynamic_slack is not None else None
    if args.dynamic_slack is not None:
        if args.sched == "head_major":
            print("--dynamic-slack needs a persistent queue", file=sys.stderr)
            sys.exit(2)
        bmask = A.route(plan, q, k, p, wl.k_floor, wl.slack, ws=rws)   # the base mask
        base_tiles = bmask.nnz()
        cap = args.slack_cap if args.slack_cap is not None else base_tiles // 20
        tel0 = torch.zeros(A.attend_grid(plan, sched) * 4, dtype=torch.int64, device=dev)
        budget_t = torch.zeros(1, dtype=torch.int64, device=dev)
        bws = A.workspace(aws.numel(), dev)
        prepare(bmask, sched, bws)
        for _ in range(3):
            run(bmask, o, sched, ws_=bws)
        run(bmask, o, sched, telemetry=tel0, ws_=bws)
        A.slack_budget(plan, sched, tel0, args.dynamic_slack, cap, budget_t)
        torch.cuda.synchronize()
        dyn = {"fill": args.dynamic_slack, "theta": args.slack_theta, "cap": cap,
               "budget": int(budget_t.item()), "base_tiles": base_tiles,
               "base_busy_max_over_mean": round(imbalance(
                   tel0.cpu().numpy().reshape(-1, 4))["busy_max_over_mean"], 4)}

    # The K/V re-layout does not depend on the mask, so it can run on a second
    # stream (default priority).  Beside routing and the schedule kernels (the
    # default), routing and the re-layout share HBM bandwidth: the routing
    # kernels take longer, but the two finish sooner than one after the other
    # (480p, same box: 0.42-0.43 ms from the step's start to the attention
    # launch, against 0.44-0.46 with the schedule kernels waiting for the
    # re-layout and 0.47 with the re-layout beside the schedule kernels only or
    # everything on one stream).
    pipeline = "serial" if (split or args.no_overlap) else args.pipeline
    side = torch.cuda.Stream(device=dev)
    fork, join = torch.cuda.Event(), torch.cuda.Event()

    fm_t = (torch.empty(int(plan.col_capacity), dtype=torch.int32, device=dev) if frames
            else None)
    p_frame = float(np.float32(args.frames)) if frames else None

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        if frames:
            # routing with the frame level, then the prologue and attention in one call
            A.route_frames(plan, q, k, p, wl.k_floor, p_frame, mask=mask, frame_mask=fm_t, ws=rws)
            if ev is not None:
                ev[1].record(stream)
                ev[2].record(stream)
            A.attend_frames(plan, q, k, v, mask, fm_t, sched=sched, o=o, ws=aws)
            if ev is not None:
                ev[3].record(stream)
            return
        if pipeline in ("beside_route", "beside_route_only"):
            fork.record(stream)            # after the previous step's attention
            side.wait_event(fork)
            A.attend_relayout(plan, k, v, aws, stream=side)
            join.record(side)
        if dyn is not None:
            A.route_dynamic(plan, q, k, p, wl.k_floor, args.slack_theta, budget_t, mask=mask,
                            ws=rws)
        else:
            A.route(plan, q, k, p, wl.k_floor, wl.slack, mask=mask, ws=rws)
        if ev is not None:
            ev[1].record(stream)
        if pipeline == "after_route":
            fork.record(stream)            # after routing
            side.wait_event(fork)
            A.attend_relayout(plan, k, v, aws, stream=side)
            join.record(side)
            A.attend_schedule(plan, mask, sched, aws)
            stream.wait_event(join)
        elif pipeline == "beside_route":
            # the schedule kernels need only the mask: they run beside the
            # re-layout's tail, and attention waits for both
            A.attend_schedule(plan, mask, sched, aws)
            stream.wait_event(join)
        elif pipeline == "beside_route_only":
            stream.wait_event(join)
            A.attend_schedule(plan, mask, sched, aws)
        else:
            prepare(mask, sched)
        if ev is not None:
            ev[2].record(stream)
        run(mask, o, sched)
        if ev is not None:
            ev[3].record(stream)

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_step_median = float(np.median([e[0].elapsed_time(e[3]) for e in evs]))
    t_route = np.mean([e[0].elapsed_time(e[1]) for e in evs])
    t_prep = np.mean([e[1].elapsed_time(e[2]) for e in evs])
    t_attn = np.mean([e[2].elapsed_time(e[3]) for e in evs])

    # routing on its own (nothing beside it on the GPU): median of 20 launches
    route_alone = []
    rmask = A.Mask(plan, dev)
    for i in range(23):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if frames:
            A.route_frames(plan, q, k, p, wl.k_floor, p_frame, mask=rmask, ws=rws)
        elif dyn is not None:
            A.route_dynamic(plan, q, k, p, wl.k_floor, args.slack_theta, budget_t, mask=rmask,
                            ws=rws)
        else:
            A.route(plan, q, k, p, wl.k_floor, wl.slack, mask=rmask, ws=rws)
        e1.record(stream)
        torch.cuda.synchronize()
        if i >= 3:
            route_alone.append(e0.elapsed_time(e1))
    del rmask
    t_route_alone = float(np.median(route_alone))

    rp, ci = mask.to_host()
    nnz = int(rp[-1])
    bt, d, nb = plan.block_tokens, wl.head_dim, plan.num_blocks
    flops = 4.0 * bt * bt * d * nnz
    eff_layer = flops / (ms_step * 1e-3) / 1e12
    eff_attn = flops / (t_attn * 1e-3) / 1e12
    dens = np.diff(rp).reshape(-1, nb).sum(1) / nb ** 2

    # valid-pair flops: 4 d * sum over kept pairs of real queries x real keys
    nvalid = block_valid_counts(wl.grid, wl.block)
    rows_i = np.repeat(np.arange(rp.size - 1) % nb, np.diff(rp))
    valid_flops = 4.0 * d * float((nvalid[rows_i] * nvalid[ci]).sum())

    # per-CU balance and kernel time under every schedule (the naive
    # head-major hardware dispatch included)
    if dyn is not None:
        # base and filled masks' attention launches interleaved (each on its own
        # workspace), so that clock drift affects both alike
        dyn["added_pairs"] = nnz - dyn["base_tiles"]
        tb, td = [], []
        for _ in range(6):
            for msk, ws_, acc in ((bmask, bws, tb), (mask, aws, td)):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                run(msk, o2_dyn, sched, ws_=ws_)
                e1.record(stream)
                torch.cuda.synchronize()
                acc.append(e0.elapsed_time(e1))
        dyn["base_ms_attend_kernel"] = round(float(np.median(tb[1:])), 4)
        dyn["ms_attend_kernel"] = round(float(np.median(td[1:])), 4)
        t_tile = dyn["base_ms_attend_kernel"] / dyn["base_tiles"]
        # extra time over what the added tiles cost at the base launch's mean rate
        dyn["fill_cost"] = (round((dyn["ms_attend_kernel"] - dyn["base_ms_attend_kernel"])
                                  / (dyn["added_pairs"] * t_tile), 3)
                            if dyn["added_pairs"] > 0 else None)
        del bws
    bal = {}
    o2 = torch.empty_like(q)
    sweep = {} if (args.timed_only or frames) else A.SCHEDULES
    if split and not args.timed_only:
        sweep = {n: A.SCHEDULES[n] for n in ("nnz_sorted", "head_phased")}
    for name, s in sweep.items():
        try:
            n_wg = A.attend_grid(plan, s)
        except A.AbsError:
            continue
        tel = torch.zeros(n_wg * 4, dtype=torch.int64, device=dev)
        prepare(mask, s)
        run(mask, o2, s, telemetry=tel)
        for _ in range(2):       # settle clocks before timing
            run(mask, o2, s)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(3):
            run(mask, o2, s)
        e1.record(stream)
        torch.cuda.synchronize()
        t = tel.cpu().numpy().reshape(-1, 4)
        assert int(t[:, 2].sum()) == nnz
        bal[name] = imbalance(t)
        bal[name]["ms_attend_kernel"] = round(e0.elapsed_time(e1) / 3, 4)
        bal[name]["xcds_seen"] = int(len(set((t[:, 1] & 0xF).tolist())))
    prepare(mask, sched)   # restore the timed schedule

    # cold steps: L2 and Infinity Cache flushed by writing 512 MB before each;
    # the median of 20
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    cold = []
    for _ in range(0 if args.timed_only else 20):
        flush.fill_(1)
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        step(ev)
        torch.cuda.synchronize()
        cold.append(ev[0].elapsed_time(ev[3]))
    del flush

    # dense comparator: the same layer with every block kept (p = 1), our own
    # kernel; context for the explainer's sparse-over-dense attention speedup
    dense = None
    if not args.timed_only and not frames:
        dmask = A.Mask(plan, dev)
        A.route(plan, q, k, 1.0, 1, 0.0, mask=dmask, ws=rws)
        prepare(dmask, sched)
        run(dmask, o2, sched)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(2):
            run(dmask, o2, sched)
        e1.record(stream)
        torch.cuda.synchronize()
        dense_ms = e0.elapsed_time(e1) / 2
        dense_tiles = int(dmask.row_ptr[-1].item())
        del dmask
        prepare(mask, sched)
        dense = {"ms_attend_kernel": round(dense_ms, 4), "tiles": dense_tiles,
                 "tflops": round(4.0 * bt * bt * d * dense_tiles / (dense_ms * 1e-3) / 1e12, 2),
                 "speedup_sparse_over_dense": round(dense_ms / t_attn, 3)}

    # the bf16 MFMA rate this GPU sustains on its own (power-limited clock),
    # reported beside the data-sheet peak
    probe = mfma_probe(dev) if (not args.timed_only and wl.dtype == "bf16") else None
    # ... and what the attention kernel's inner arithmetic reaches with nothing
    # around it (no copies, barrier, padding or work items)
    loop = attn_loop_probe(dev) if (not args.timed_only and wl.dtype == "bf16") else None

    cpu = None
    parity = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        cb = cpu_baseline(wl, p, inputs, rp, ci)
        if dyn is None:
            parity = mask_parity_counts(cb["route"], p, wl.k_floor, rp, ci)
        cpu = {"value": flops / cb["t_layer_s"] / 1e12, "unit": "TFLOP/s (effective, kept blocks)",
               "cores": cb["cores"], "kind": "oracle", **cb["cpu"],
               "sample": (f"full oracle routing of all {rp.size - 1} rows ({cb['t_route_s']:.1f} s) + "
                          f"oracle attention on {cb['rows']} random rows ({cb['tiles']} of "
                          f"{cb['total_tiles']} kept tiles), extrapolated by kept tiles; "
                          f"layer {cb['t_layer_s']:.1f} s"),
               "ms_per_layer": cb["t_layer_s"] * 1e3}

    frame_stats = None
    if frames:
        fm = fm_t[:nnz].cpu().numpy()
        T = wl.grid[0]
        tblk = wl.block[0]
        per_plane = plan.nblk[1] * plan.nblk[2]
        tl = np.array([min(tblk, T - (j // per_plane) * tblk) for j in range(nb)])
        frame_tok = nvalid / tl                       # real tokens of each frame of a block
        kept_f = np.array([bin(int(x)).count("1") for x in fm])
        tok_frames = kept_f * frame_tok[ci]
        tok_blocks = nvalid[ci]
        valid_flops = 4.0 * d * float((nvalid[rows_i] * tok_frames).sum())
        frame_stats = {"p_frame": p_frame, "kept_frames": int(kept_f.sum()),
                       "frames_of_kept_blocks": int(tl[ci].sum()),
                       "key_tokens_kept": float(tok_frames.sum()),
                       "key_tokens_of_kept_blocks": float(tok_blocks.sum()),
                       "key_fraction_of_block_level": round(float(tok_frames.sum() /
                                                                  tok_blocks.sum()), 4),
                       "blocks_without_frames": int((fm == 0).sum()),
                       "note": "ms_attend_kernel includes the attention prologue (K/V "
                               "re-layout, key-block lists, schedule)"}

    peak = PEAK_BF16_TFLOPS if wl.dtype == "bf16" else PEAK_FP32_TFLOPS
    executed = None if (split or frames) else measured_executed_flop(args.workload, args.sched)
    route_bytes = 2 * wl.tokens * wl.heads * wl.head_dim * (2 if wl.dtype == "bf16" else 4)
    out = {
        "metric": "ms/attn layer + effective TFLOPS (kept blocks) at Wan2.2 480p shape",
        "value": round(eff_layer, 2),
        "unit": "TFLOP/s (effective, kept blocks, whole layer)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": wl.dtype, "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.batch, "heads": wl.heads,
                   "head_dim": wl.head_dim, "grid": list(wl.grid), "block": list(wl.block),
                   "p": p, "k_floor": wl.k_floor, "slack": wl.slack, "sched": args.sched,
                   "split": ({"split_tiles": args.split, "max_parts": max_parts} if split
                             else None),
                   "pipeline": pipeline,
                   "kept_tiles": nnz, "density": round(nnz / (rp.size - 1) / nb, 4),
                   "head_density_min_median_max": [round(float(dens.min()), 4),
                                                   round(float(np.median(dens)), 4),
                                                   round(float(dens.max()), 4)]},
        "ms_per_step_median": round(ms_step_median, 4),
        "ms_route": round(float(t_route), 4),
        "ms_route_alone": round(t_route_alone, 4),
        "ms_attend_prepare": round(float(t_prep), 4),
        "ms_attend_kernel": round(float(t_attn), 4),
        "tflops_attend_kernel": round(eff_attn, 2),
        "tflops_valid_pairs_layer": round(valid_flops / (ms_step * 1e-3) / 1e12, 2),
        "roofline": {"bound": "mfma", "achieved": round(eff_attn, 2), "peak": peak,
                     "unit": "TFLOP/s", "frac": round(eff_attn / peak, 4),
                     "traffic": (None if (split or frames)
                                 else measured_traffic(args.workload, args.sched)),
                     "kernel": ("attn_bf16_kernel<128,128,true,true> + merge_parts_kernel"
                                if split else
                                "attn_bf16_kernel<128,128,true,false,true> (frame masks)"
                                if frames else
                                "attn_bf16_kernel<128,128,false,false>"
                                if args.sched == "head_major"
                                else "attn_bf16_kernel<128,128,true,false>"),
                     "per_unit": "4*Bt^2*d flop per kept tile",
                     "frac_valid_pairs": round(valid_flops / (t_attn * 1e-3) / 1e12 / peak, 4),
                     "frac_executed": (round(executed / (t_attn * 1e-3) / 1e12 / peak, 4)
                                       if executed else None),
                     "probe_peak": probe["tflops"] if probe else None,
                     "loop_probe": loop["tflops"] if loop else None,
                     # executed MFMA rate against what this machine sustains in the
                     # same run (box-independent, unlike the data-sheet fraction)
                     "frac_executed_of_probe": (
                         round(executed / (t_attn * 1e-3) / 1e12 / probe["tflops"], 4)
                         if (executed and probe) else None),
                     "frac_executed_of_loop_probe": (
                         round(executed / (t_attn * 1e-3) / 1e12 / loop["tflops"], 4)
                         if (executed and loop) else None)},
        "mfma_probe_bf16": probe,
        "attn_loop_probe": loop,
        "route_hbm": {"bytes_read_qk": route_bytes,
                      "gbs_algorithmic_alone": round(route_bytes / (t_route_alone * 1e-3) / 1e9, 1),
                      "frac_of_8tbs_alone": round(route_bytes / (t_route_alone * 1e-3) / 1e9
                                                  / PEAK_HBM_GBS, 4),
                      "gbs_algorithmic_in_step": round(route_bytes / (t_route * 1e-3) / 1e9, 1)},
        "mask_parity": parity,
        "imbalance": bal,
        "dynamic_slack": dyn,
        "frames": frame_stats,
        "ms_per_step_cold": round(float(np.median(cold)), 4) if cold else None,
        "dense_p1": dense,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out))


if __name__ == "__main__":
    main()
