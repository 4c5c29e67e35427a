"""The C ABI on the host: the library loads, exports what the header declares,
and rejects bad arguments before touching a device (runs without a GPU)."""
import ctypes
import math
import os
import re

import pytest

import adaptive_block_sparse_amd as A
import oracle as O
import synth_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = ctypes.c_void_p(0x100000)   # never dereferenced: validation fails first


def _lib():
    if not os.path.exists(A.LIB_PATH):
        pytest.skip("libabs.so not built")
    return A.load_library()


def test_exports_match_header():
    lib = _lib()
    header = open(os.path.join(ROOT, "include", "abs.h")).read()
    declared = set(re.findall(r"^\s*(?:abs_status|const char\*)\s+(abs_\w+)\s*\(", header, re.M))
    assert declared == set(A.EXPORTS)
    for name in declared:
        assert hasattr(lib, name)
    assert A.status_string(A.ENOSPACE) == "workspace too small"


def test_probe_library_exports_its_header():
    # the measurement aid (sustained MFMA rate) is a library of its own
    path = os.path.join(ROOT, "adaptive_block_sparse_amd", "libabs_probe.so")
    if not os.path.exists(path):
        pytest.skip("libabs_probe.so not built")
    lib = ctypes.CDLL(path)
    header = open(os.path.join(ROOT, "include", "abs_probe.h")).read()
    declared = set(re.findall(r"^\s*int\s+(abs_probe_\w+)\s*\(", header, re.M))
    assert declared == {"abs_probe_mfma_bf16", "abs_probe_attn_loop", "abs_probe_wall_clock_khz"}
    for name in declared:
        assert hasattr(lib, name)
    f = lib.abs_probe_mfma_bf16
    f.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                  ctypes.c_void_p]
    # invalid arguments are rejected before any launch
    assert f(0, 4, FAKE, FAKE, None) == 1
    assert f(10, 0, FAKE, FAKE, None) == 1
    assert f(10, (1 << 21) + 1, FAKE, FAKE, None) == 1
    g = lib.abs_probe_attn_loop
    g.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                  ctypes.c_void_p, ctypes.c_void_p]
    for qpw, iters, wgs in ((16, 10, 4), (48, 10, 4), (32, 0, 4), (64, 10, 0),
                            (32, 10, (1 << 21) + 1)):
        assert g(qpw, iters, wgs, FAKE, FAKE, None) == 1
    assert f(10, 4, None, FAKE, None) == 1
    assert lib.abs_probe_wall_clock_khz(None) == 1


@pytest.mark.parametrize("cfg", [0, 1, 2, 3, 4])
def test_plan_matches_geometry(cfg):
    _lib()
    wl = si.WORKLOADS[cfg]
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    geo = O.geometry(wl.grid, wl.block)
    assert plan.num_blocks == geo.nb
    assert tuple(plan.padded) == geo.padded and tuple(plan.nblk) == geo.nblk
    assert plan.block_tokens == geo.bt_tokens
    assert plan.rows == wl.batch * wl.heads * geo.nb
    assert plan.col_capacity == plan.rows * geo.nb
    assert plan.tokens == wl.tokens
    assert plan.route_ws_bytes > 0 and plan.attend_ws_bytes > 0
    from parity_utils import pair_groups
    items = plan.rows if wl.dtype == "f32" else len(pair_groups(geo, wl.batch * wl.heads))
    assert A.attend_grid(plan, A.SCHED_HEAD_MAJOR) == items


def _status_of_plan(**kw):
    lib = _lib()
    args = dict(batch=1, heads=2, head_dim=64, grid=(4, 8, 8), block=(2, 4, 4), dtype=A.F32)
    args.update(kw)
    shape = A.Shape(args["batch"], args["heads"], args["head_dim"],
                    (ctypes.c_int32 * 3)(*args["grid"]), (ctypes.c_int32 * 3)(*args["block"]),
                    args["dtype"])
    plan = A.Plan()
    return lib.abs_plan_init(ctypes.byref(shape), ctypes.byref(plan)), plan


@pytest.mark.parametrize("kw,want", [
    (dict(), A.OK),
    (dict(batch=0), A.EINVAL),
    (dict(heads=-1), A.EINVAL),
    (dict(grid=(0, 8, 8)), A.EINVAL),
    (dict(block=(2, 0, 4)), A.EINVAL),
    (dict(head_dim=96), A.ENOTSUP),
    (dict(block=(2, 4, 6)), A.ENOTSUP),        # 48 tokens per block
    (dict(dtype=7), A.ENOTSUP),
    (dict(grid=(200, 200, 200), block=(2, 4, 4)), A.ENOTSUP),   # nb > 8192
    (dict(grid=(31, 125, 250), block=(2, 8, 8)), A.OK),        # nb = 8192, the largest
    (dict(grid=(33, 125, 250), block=(2, 8, 8)), A.ENOTSUP),   # nb = 8704
    # more than 2^31 elements per tensor (64-bit element offsets)
    (dict(grid=(16, 128, 130), block=(2, 8, 8), heads=64, head_dim=128), A.OK),
    # rows * nb >= 2^31 (CSR positions are int32)
    (dict(grid=(31, 125, 250), block=(2, 8, 8), heads=40), A.ENOTSUP),
])
def test_plan_validation(kw, want):
    st, _ = _status_of_plan(**kw)
    assert st == want


def _plan(dtype=A.BF16):
    st, plan = _status_of_plan(head_dim=128, grid=(21, 30, 52), block=(2, 8, 8), heads=4,
                               dtype=dtype)
    assert st == A.OK
    return plan


def _route(plan, q=FAKE, k=FAKE, p=0.9, kf=4, slack=0.0, ws_bytes=None, mask=True, ws=FAKE):
    lib = _lib()
    cm = A.CMask(0x100000, 0x200000, 0x300000)
    ws_bytes = plan.route_ws_bytes if ws_bytes is None else ws_bytes
    return lib.abs_route(ctypes.byref(plan), q, k, p, kf, slack,
                         ctypes.byref(cm) if mask else None, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,want", [
    (dict(p=0.0), A.EINVAL), (dict(p=1.5), A.EINVAL), (dict(p=math.nan), A.EINVAL),
    (dict(p=-0.1), A.EINVAL), (dict(kf=0), A.EINVAL), (dict(slack=1.0), A.EINVAL),
    (dict(slack=-0.5), A.EINVAL), (dict(q=None), A.EINVAL), (dict(mask=False), A.EINVAL),
    (dict(ws=None), A.EINVAL), (dict(ws_bytes=1024), A.ENOSPACE),
])
def test_route_validation(kw, want):
    assert _route(_plan(), **kw) == want


def test_route_slack_needs_its_scratch():
    plan = _plan()
    # the fill needs the probability matrix on top of the means and bitmaps: a
    # workspace of only that matrix's size is refused (before any launch)
    _lib()
    prob_bytes = plan.rows * plan.num_blocks * 4
    assert _route(plan, slack=0.15, ws_bytes=prob_bytes) == A.ENOSPACE


@pytest.mark.parametrize("sched,ws_small,want", [(5, False, A.EINVAL), (-1, False, A.EINVAL),
                                                 (A.SCHED_NNZ_SORTED, True, A.ENOSPACE)])
def test_attend_validation(sched, ws_small, want):
    lib = _lib()
    plan = _plan()
    cm = A.CMask(0x100000, 0x200000, 0x300000)
    nbytes = 1024 if ws_small else plan.attend_ws_bytes
    st = lib.abs_attend_prepare(ctypes.byref(plan), FAKE, FAKE, ctypes.byref(cm), sched, FAKE,
                                nbytes, None)
    assert st == want
    st = lib.abs_attend_run(ctypes.byref(plan), FAKE, FAKE, ctypes.byref(cm), FAKE, sched, FAKE,
                            nbytes, None, None)
    assert st == want
    n = ctypes.c_int32()
    if sched not in (0, 1, 2):
        assert lib.abs_attend_grid(ctypes.byref(plan), sched, ctypes.byref(n)) == A.EINVAL
    st = lib.abs_attend(ctypes.byref(plan), None, FAKE, FAKE, ctypes.byref(cm), FAKE, 0, FAKE,
                        plan.attend_ws_bytes, None, None)
    assert st == A.EINVAL


@pytest.mark.parametrize("kw,want", [
    (dict(), A.OK),
    (dict(sched=A.SCHED_HEAD_PHASED), A.OK),
    (dict(sched=A.SCHED_HEAD_MAJOR), A.EINVAL),
    (dict(sched=A.SCHED_XCD_LOCAL), A.EINVAL),
    (dict(sched=9), A.EINVAL),
    (dict(split=0), A.EINVAL),
    (dict(max_parts=-1), A.EINVAL),
    (dict(max_parts=(1 << 24) + 1), A.EINVAL),
    (dict(dtype=A.F32), A.ENOTSUP),
    (dict(small=True), A.ENOSPACE),
    (dict(q=None), A.EINVAL),
])
def test_attend_split_validation(kw, want):
    lib = _lib()
    plan = _plan(kw.get("dtype", A.BF16))
    sched, split, max_parts = kw.get("sched", 0), kw.get("split", 8), kw.get("max_parts", 16)
    cm = A.CMask(0x100000, 0x200000, 0x300000)
    n = ctypes.c_size_t(0)
    st = lib.abs_attend_split_ws_bytes(ctypes.byref(plan), max_parts, ctypes.byref(n))
    if want == A.OK or kw.get("small") or "q" in kw or "sched" in kw or "split" in kw:
        assert st == A.OK
        need = n.value
    else:
        assert st == want
        need = 1 << 40
    if want == A.OK:
        return   # a valid call would launch: the GPU tests cover it
    nbytes = 1024 if kw.get("small") else need
    q = kw.get("q", FAKE)
    if "q" not in kw:   # prepare takes no q
        st = lib.abs_attend_prepare_split(ctypes.byref(plan), FAKE, FAKE, ctypes.byref(cm), sched,
                                          split, max_parts, FAKE, nbytes, None)
        assert st == want
    if "split" not in kw:   # run takes no split
        st = lib.abs_attend_run_split(ctypes.byref(plan), q, ctypes.byref(cm), FAKE, sched,
                                      max_parts, FAKE, nbytes, None, None)
        assert st == want


def test_attend_split_workspace_size():
    _lib()
    plan = _plan()
    base = A.attend_split_ws_bytes(plan, 0)
    assert base >= plan.attend_ws_bytes
    slot = (2 * plan.block_tokens * plan.s.head_dim + 4 * plan.block_tokens) * 4
    more = A.attend_split_ws_bytes(plan, 100)
    assert more - base >= 100 * slot
    lib = _lib()
    assert lib.abs_attend_split_ws_bytes(ctypes.byref(plan), 4, None) == A.EINVAL


@pytest.mark.parametrize("kw,want", [
    (dict(theta=-0.1), A.EINVAL), (dict(theta=1.5), A.EINVAL), (dict(theta=math.nan), A.EINVAL),
    (dict(budget=None), A.EINVAL), (dict(p=0.0), A.EINVAL), (dict(kf=0), A.EINVAL),
    (dict(ws_bytes=1024), A.ENOSPACE),
])
def test_route_dynamic_validation(kw, want):
    lib = _lib()
    plan = _plan()
    cm = A.CMask(0x100000, 0x200000, 0x300000)
    budget = kw.get("budget", FAKE)
    st = lib.abs_route_dynamic(ctypes.byref(plan), FAKE, FAKE, kw.get("p", 0.9), kw.get("kf", 4),
                               kw.get("theta", 0.01), budget, ctypes.byref(cm), FAKE,
                               kw.get("ws_bytes", plan.route_ws_bytes), None)
    assert st == want


@pytest.mark.parametrize("kw,want", [
    (dict(sched=A.SCHED_HEAD_MAJOR), A.EINVAL), (dict(sched=7), A.EINVAL),
    (dict(fill=1.5), A.EINVAL), (dict(fill=-0.5), A.EINVAL), (dict(fill=math.nan), A.EINVAL),
    (dict(max_pairs=-1), A.EINVAL), (dict(tel=None), A.EINVAL), (dict(out=None), A.EINVAL),
    (dict(dtype=A.F32), A.ENOTSUP),
])
def test_slack_budget_validation(kw, want):
    lib = _lib()
    plan = _plan(kw.get("dtype", A.BF16))
    st = lib.abs_slack_budget(ctypes.byref(plan), kw.get("sched", A.SCHED_XCD_LOCAL),
                              kw.get("tel", FAKE), kw.get("fill", 0.5), kw.get("max_pairs", 100),
                              kw.get("out", FAKE), None)
    assert st == want


def test_relayout_and_schedule_validation():
    lib = _lib()
    plan = _plan()
    cm = A.CMask(0x100000, 0x200000, 0x300000)
    assert lib.abs_attend_relayout(ctypes.byref(plan), None, FAKE, FAKE,
                                   plan.attend_ws_bytes, None) == A.EINVAL
    assert lib.abs_attend_relayout(ctypes.byref(plan), FAKE, FAKE, FAKE, 1024, None) == A.ENOSPACE
    assert lib.abs_attend_schedule(ctypes.byref(plan), ctypes.byref(cm), 9, FAKE,
                                   plan.attend_ws_bytes, None) == A.EINVAL
    assert lib.abs_attend_schedule(ctypes.byref(plan), None, 0, FAKE,
                                   plan.attend_ws_bytes, None) == A.EINVAL
    assert lib.abs_attend_schedule(ctypes.byref(plan), ctypes.byref(cm), 0, FAKE, 1024,
                                   None) == A.ENOSPACE


@pytest.mark.parametrize("cfg,want", [(1, A.SCHED_HEAD_PHASED), (3, A.SCHED_HEAD_PHASED),
                                      (2, A.SCHED_HEAD_PHASED), (4, A.SCHED_HEAD_PHASED),
                                      (0, A.SCHED_HEAD_PHASED)])
def test_default_sched(cfg, want):
    _lib()
    wl = si.WORKLOADS[cfg]
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    assert A.default_sched(plan) == want
    assert _lib().abs_attend_default_sched(ctypes.byref(plan), None) == A.EINVAL


@pytest.mark.parametrize("grid,block", [((21, 30, 52), (2, 8, 8)), ((5, 12, 20), (2, 8, 8)),
                                        ((2, 8, 40), (2, 8, 8)), ((9, 10, 11), (4, 4, 4)),
                                        ((3, 13, 21), (1, 8, 16)), ((2, 8, 8), (2, 8, 8))])
def test_work_items_cover_every_block_once(grid, block):
    # the test-side mirror of the work-item rule: every query block in exactly
    # one item, partners are neighbours along one axis, and the library plans
    # the same number of items
    from parity_utils import pair_groups
    geo = O.geometry(grid, block)
    items = pair_groups(geo, 1)
    seen = [r for pair in items for r in pair if r >= 0]
    assert sorted(seen) == list(range(geo.nb))
    nbt, nbh, nbw = geo.nblk
    for a, b in items:
        if b < 0:
            continue
        ca = (a // (nbh * nbw), (a // nbw) % nbh, a % nbw)
        cb = (b // (nbh * nbw), (b // nbw) % nbh, b % nbw)
        d = [y - x for x, y in zip(ca, cb)]
        assert sorted(d) == [0, 0, 1] and ca[d.index(1)] % 2 == 0
    assert sum(1 for _, b in items if b < 0) <= 1


def _route_noalloc(plan, q=FAKE, k=FAKE, p=0.9, kf=4, slack=0.0, mask=True):
    lib = _lib()
    cm = A.CMask(0x100000, 0x200000, 0x300000)
    return lib.abs_route_noalloc(ctypes.byref(plan), q, k, p, kf, slack,
                                 ctypes.byref(cm) if mask else None, None)


@pytest.mark.parametrize("kw,want", [
    (dict(p=0.0), A.EINVAL), (dict(p=math.nan), A.EINVAL), (dict(kf=0), A.EINVAL),
    (dict(slack=1.0), A.EINVAL), (dict(q=None), A.EINVAL), (dict(mask=False), A.EINVAL),
])
def test_route_noalloc_validation(kw, want):
    assert _route_noalloc(_plan(), **kw) == want


def test_route_noalloc_rejects_plans_beyond_its_scratch():
    # 720p with 40 heads: the route workspace exceeds the 64 MiB static scratch;
    # the call must say so before touching a device
    _lib()
    wl = si.WORKLOADS[2]
    plan = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    assert plan.route_ws_bytes > A.ROUTE_NOALLOC_SCRATCH_BYTES
    assert _route_noalloc(plan, slack=0.15) == A.ETOOBIG
    assert A.status_string(A.ETOOBIG) == "plan too large for the static no-allocation scratch"
    header = open(os.path.join(ROOT, "include", "abs.h")).read()
    assert re.search(r"#define ABS_ROUTE_NOALLOC_SCRATCH_BYTES \(64ull << 20\)", header)


def test_route_frames_validation():
    lib = _lib()
    plan = _plan()
    cm = A.CMask(0x100000, 0x200000, 0x300000)

    def call(q=FAKE, p=0.9, kf=4, pf=0.9, fm=FAKE, ws_bytes=None, plan_=plan):
        nb = plan_.route_ws_bytes if ws_bytes is None else ws_bytes
        return lib.abs_route_frames(ctypes.byref(plan_), q, FAKE, p, kf, pf, ctypes.byref(cm), fm,
                                    FAKE, nb, None)
    assert call(pf=0.0) == A.EINVAL
    assert call(pf=1.5) == A.EINVAL
    assert call(pf=math.nan) == A.EINVAL
    assert call(fm=None) == A.EINVAL
    assert call(q=None) == A.EINVAL
    assert call(kf=0) == A.EINVAL
    assert call(ws_bytes=1024) == A.ENOSPACE
    # 720p: 660 blocks x 2 frames is more than the 1024 frames a row supports
    wl = si.WORKLOADS[2]
    big = A.plan_init(wl.batch, wl.heads, wl.head_dim, wl.grid, wl.block, wl.dtype)
    assert call(plan_=big) == A.ENOTSUP
    # more than 8 frames a block
    st, p9 = _status_of_plan(head_dim=128, grid=(18, 8, 8), block=(16, 2, 4), heads=1,
                             dtype=A.BF16)
    assert st == A.OK and call(plan_=p9) == A.ENOTSUP


def test_attend_frames_validation():
    lib = _lib()
    plan = _plan()
    cm = A.CMask(0x100000, 0x200000, 0x300000)

    def call(plan_=plan, fm=FAKE, sched=0, ws_bytes=None):
        nb = plan_.attend_ws_bytes if ws_bytes is None else ws_bytes
        return lib.abs_attend_frames(ctypes.byref(plan_), FAKE, FAKE, FAKE, ctypes.byref(cm), fm,
                                     FAKE, sched, FAKE, nb, None, None)
    assert call(fm=None) == A.EINVAL
    assert call(sched=9) == A.EINVAL
    assert call(ws_bytes=1024) == A.ENOSPACE
    assert call(plan_=_plan(A.F32)) == A.ENOTSUP
    st, p32 = _status_of_plan(head_dim=128, grid=(8, 8, 8), block=(2, 4, 4), heads=1,
                              dtype=A.BF16)
    assert st == A.OK and call(plan_=p32) == A.ENOTSUP    # 32-token blocks
