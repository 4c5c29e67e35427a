"""Adaptive block-sparse video attention for MI355X (gfx950).

A thin ctypes binding over the C ABI of ``libabs.so`` (declared in
``include/abs.h``).  torch supplies device memory and the stream; every step
of the computation runs in the library's HIP kernels.  There is no fallback:
if the library is not built, every call raises.

Typical use::

    import adaptive_block_sparse_amd as abs_
    plan = abs_.plan_init(batch=1, heads=40, head_dim=128, grid=(21, 30, 52),
                          block=(2, 8, 8), dtype="bf16")
    mask = abs_.route(plan, q, k, p=0.9, k_floor=4)          # per-head CSR
    o = abs_.attend(plan, q, k, v, mask)                      # [B, N, H, d]
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("ABS_LIBRARY") or os.path.join(HERE, "libabs.so")

OK, EINVAL, ENOTSUP, ENOSPACE, EHIP, ETOOBIG = 0, 1, 2, 3, 4, 5
F32, BF16 = 0, 1
SCHED_NNZ_SORTED, SCHED_HEAD_MAJOR, SCHED_HEAD_PHASED, SCHED_XCD_LOCAL = 0, 1, 2, 3
SCHEDULES = {"nnz_sorted": SCHED_NNZ_SORTED, "head_major": SCHED_HEAD_MAJOR,
             "head_phased": SCHED_HEAD_PHASED, "xcd_local": SCHED_XCD_LOCAL}
EXPORTS = ("abs_plan_init", "abs_route", "abs_attend_prepare", "abs_attend_run",
           "abs_attend", "abs_attend_grid", "abs_status_string", "abs_attend_split_ws_bytes",
           "abs_attend_prepare_split", "abs_attend_run_split", "abs_route_dynamic",
           "abs_slack_budget", "abs_attend_relayout", "abs_attend_schedule",
           "abs_attend_default_sched", "abs_route_noalloc", "abs_route_frames",
           "abs_attend_frames")
# bytes of the static device scratch abs_route_noalloc works in (include/abs.h)
ROUTE_NOALLOC_SCRATCH_BYTES = 64 << 20


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("grid", ctypes.c_int32 * 3),
                ("block", ctypes.c_int32 * 3), ("dtype", ctypes.c_int32)]


class Plan(ctypes.Structure):
    _fields_ = [("s", Shape), ("padded", ctypes.c_int32 * 3), ("nblk", ctypes.c_int32 * 3),
                ("num_blocks", ctypes.c_int32), ("block_tokens", ctypes.c_int32),
                ("heads_per_phase", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("tokens", ctypes.c_int64), ("rows", ctypes.c_int64),
                ("col_capacity", ctypes.c_int64), ("route_ws_bytes", ctypes.c_size_t),
                ("attend_ws_bytes", ctypes.c_size_t)]


class CMask(ctypes.Structure):
    _fields_ = [("row_ptr", ctypes.c_void_p), ("col_idx", ctypes.c_void_p),
                ("head_nnz", ctypes.c_void_p)]


class AbsError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {status_string(status)} (status {status})")
        self.status = status


_LIB = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libabs.so (raises if it has not been built)."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(f"HIP library {path} is not built; run "
                           "`python -m adaptive_block_sparse_amd.build`")
    lib = ctypes.CDLL(path)
    P, V, I32, F, SZ = ctypes.POINTER(Plan), ctypes.c_void_p, ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    M = ctypes.POINTER(CMask)
    sig = {
        "abs_plan_init": [ctypes.POINTER(Shape), P],
        "abs_route": [P, V, V, F, I32, F, M, V, SZ, V],
        "abs_attend_prepare": [P, V, V, M, I32, V, SZ, V],
        "abs_attend_run": [P, V, V, M, V, I32, V, SZ, V, V],
        "abs_attend": [P, V, V, V, M, V, I32, V, SZ, V, V],
        "abs_attend_grid": [P, I32, ctypes.POINTER(I32)],
        "abs_attend_default_sched": [P, ctypes.POINTER(I32)],
        "abs_attend_split_ws_bytes": [P, I32, ctypes.POINTER(SZ)],
        "abs_attend_prepare_split": [P, V, V, M, I32, I32, I32, V, SZ, V],
        "abs_attend_run_split": [P, V, M, V, I32, I32, V, SZ, V, V],
        "abs_route_dynamic": [P, V, V, F, I32, F, V, M, V, SZ, V],
        "abs_attend_relayout": [P, V, V, V, SZ, V],
        "abs_attend_schedule": [P, M, I32, V, SZ, V],
        "abs_slack_budget": [P, I32, V, F, ctypes.c_int64, V, V],
        "abs_route_noalloc": [P, V, V, F, I32, F, M, V],
        "abs_route_frames": [P, V, V, F, I32, F, M, V, V, SZ, V],
        "abs_attend_frames": [P, V, V, V, M, V, V, I32, V, SZ, V, V],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.abs_status_string.argtypes = [ctypes.c_int]
    lib.abs_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().abs_status_string(int(status)).decode()


def _check(fn: str, status: int) -> None:
    if status != OK:
        raise AbsError(fn, status)


def plan_init(batch: int, heads: int, head_dim: int, grid: Sequence[int],
              block: Sequence[int], dtype: str = "bf16") -> Plan:
    shape = Shape(batch, heads, head_dim, (ctypes.c_int32 * 3)(*grid),
                  (ctypes.c_int32 * 3)(*block), F32 if dtype == "f32" else BF16)
    plan = Plan()
    _check("abs_plan_init", load_library().abs_plan_init(ctypes.byref(shape), ctypes.byref(plan)))
    return plan


def _torch():
    import torch
    return torch


def _stream(stream) -> ctypes.c_void_p:
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t) -> ctypes.c_void_p:
    return ctypes.c_void_p(t.data_ptr())


def _tensor_dtype(plan: Plan):
    torch = _torch()
    return torch.float32 if plan.s.dtype == F32 else torch.bfloat16


def _check_qkv(plan: Plan, *ts):
    torch = _torch()
    want = (plan.s.batch, int(plan.tokens), plan.s.heads, plan.s.head_dim)
    for t in ts:
        if tuple(t.shape) != want or t.dtype != _tensor_dtype(plan) or not t.is_cuda \
                or not t.is_contiguous():
            raise ValueError(f"expected a contiguous CUDA tensor {want} of {_tensor_dtype(plan)}, "
                             f"got {tuple(t.shape)} {t.dtype} on {t.device}")
    return torch


class Mask:
    """Per-head CSR block mask held in caller-owned torch buffers."""

    def __init__(self, plan: Plan, device):
        torch = _torch()
        self.plan = plan
        self.row_ptr = torch.empty(int(plan.rows) + 1, dtype=torch.int32, device=device)
        self.col_idx = torch.empty(int(plan.col_capacity), dtype=torch.int32, device=device)
        self.head_nnz = torch.empty(plan.s.batch * plan.s.heads, dtype=torch.int32, device=device)

    def c(self) -> CMask:
        return CMask(self.row_ptr.data_ptr(), self.col_idx.data_ptr(), self.head_nnz.data_ptr())

    def nnz(self) -> int:
        return int(self.row_ptr[-1].item())

    def to_host(self):
        """(row_ptr, col_idx) as numpy arrays, col_idx trimmed to nnz."""
        rp = self.row_ptr.cpu().numpy()
        return rp, self.col_idx[: int(rp[-1])].cpu().numpy()


def workspace(nbytes: int, device):
    torch = _torch()
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def route(plan: Plan, q, k, p: float, k_floor: int, slack: float = 0.0,
          mask: Optional[Mask] = None, ws=None, stream=None) -> Mask:
    """Per-head Top-p block routing with a Top-k floor, own-block repair and an
    optional per-head slack budget.  Returns the CSR mask."""
    _check_qkv(plan, q, k)
    mask = Mask(plan, q.device) if mask is None else mask
    ws = workspace(plan.route_ws_bytes, q.device) if ws is None else ws
    cm = mask.c()
    st = load_library().abs_route(ctypes.byref(plan), _ptr(q), _ptr(k), float(p), int(k_floor),
                                  float(slack), ctypes.byref(cm), _ptr(ws), ws.numel(),
                                  _stream(stream))
    _check("abs_route", st)
    return mask


def route_noalloc(plan: Plan, q, k, p: float, k_floor: int, slack: float = 0.0,
                  mask: Optional[Mask] = None, stream=None) -> Mask:
    """route() without a workspace argument: the library works in its static
    per-GPU device scratch and allocates nothing (the mask buffers are the
    caller's; pass `mask` to allocate nothing here either).  Calls that overlap
    on one GPU race."""
    _check_qkv(plan, q, k)
    mask = Mask(plan, q.device) if mask is None else mask
    cm = mask.c()
    st = load_library().abs_route_noalloc(ctypes.byref(plan), _ptr(q), _ptr(k), float(p),
                                          int(k_floor), float(slack), ctypes.byref(cm),
                                          _stream(stream))
    _check("abs_route_noalloc", st)
    return mask


def route_frames(plan: Plan, q, k, p: float, k_floor: int, p_frame: float,
                 mask: Optional[Mask] = None, frame_mask=None, ws=None, stream=None):
    """Block routing, then Top-p over the frames of each row's kept blocks.
    Returns (mask, frame_mask): frame_mask int32 aligned with mask.col_idx,
    bit tau set when frame tau of that block is kept."""
    torch = _check_qkv(plan, q, k)
    mask = Mask(plan, q.device) if mask is None else mask
    if frame_mask is None:
        frame_mask = torch.empty(int(plan.col_capacity), dtype=torch.int32, device=q.device)
    ws = workspace(plan.route_ws_bytes, q.device) if ws is None else ws
    cm = mask.c()
    st = load_library().abs_route_frames(ctypes.byref(plan), _ptr(q), _ptr(k), float(p),
                                         int(k_floor), float(p_frame), ctypes.byref(cm),
                                         _ptr(frame_mask), _ptr(ws), ws.numel(), _stream(stream))
    _check("abs_route_frames", st)
    return mask, frame_mask


def attend_frames(plan: Plan, q, k, v, mask: Mask, frame_mask, sched: Optional[int] = None,
                  o=None, ws=None, telemetry=None, stream=None):
    """Block-sparse attention over the kept frames of the kept blocks; returns
    o [B, N, H, d]."""
    torch = _check_qkv(plan, q, k, v)
    sched = default_sched(plan) if sched is None else sched
    o = torch.empty_like(q) if o is None else o
    ws = workspace(plan.attend_ws_bytes, q.device) if ws is None else ws
    cm = mask.c()
    tp = ctypes.c_void_p(0) if telemetry is None else _ptr(telemetry)
    _check("abs_attend_frames",
           load_library().abs_attend_frames(ctypes.byref(plan), _ptr(q), _ptr(k), _ptr(v),
                                            ctypes.byref(cm), _ptr(frame_mask), _ptr(o),
                                            int(sched), _ptr(ws), ws.numel(), tp,
                                            _stream(stream)))
    return o


def route_dynamic(plan: Plan, q, k, p: float, k_floor: int, theta: float, budget,
                  mask: Optional[Mask] = None, ws=None, stream=None) -> Mask:
    """Routing plus a dynamic slack fill of up to budget[0] pairs (a device
    int64 tensor), candidates P >= theta over the whole batch, highest P first."""
    _check_qkv(plan, q, k)
    mask = Mask(plan, q.device) if mask is None else mask
    ws = workspace(plan.route_ws_bytes, q.device) if ws is None else ws
    cm = mask.c()
    st = load_library().abs_route_dynamic(ctypes.byref(plan), _ptr(q), _ptr(k), float(p),
                                          int(k_floor), float(theta), _ptr(budget),
                                          ctypes.byref(cm), _ptr(ws), ws.numel(), _stream(stream))
    _check("abs_route_dynamic", st)
    return mask


def slack_budget(plan: Plan, sched: int, telemetry, fill: float, max_pairs: int, budget,
                 stream=None) -> None:
    """Write into budget[0] (device int64) the dynamic slack budget derived
    from one persistent launch's telemetry."""
    _check("abs_slack_budget",
           load_library().abs_slack_budget(ctypes.byref(plan), int(sched), _ptr(telemetry),
                                           float(fill), int(max_pairs), _ptr(budget),
                                           _stream(stream)))


def attend_grid(plan: Plan, sched: int = SCHED_NNZ_SORTED) -> int:
    n = ctypes.c_int32(0)
    _check("abs_attend_grid", load_library().abs_attend_grid(ctypes.byref(plan), int(sched),
                                                             ctypes.byref(n)))
    return int(n.value)


def default_sched(plan: Plan) -> int:
    """The schedule measured fastest for this plan's shape."""
    n = ctypes.c_int32(0)
    _check("abs_attend_default_sched",
           load_library().abs_attend_default_sched(ctypes.byref(plan), ctypes.byref(n)))
    return int(n.value)


def attend_prepare(plan: Plan, k, v, mask: Mask, sched: int, ws, stream=None) -> None:
    _check_qkv(plan, k, v)
    cm = mask.c()
    _check("abs_attend_prepare",
           load_library().abs_attend_prepare(ctypes.byref(plan), _ptr(k), _ptr(v), ctypes.byref(cm),
                                             int(sched), _ptr(ws), ws.numel(), _stream(stream)))


def attend_relayout(plan: Plan, k, v, ws, stream=None) -> None:
    """The mask-independent half of attend_prepare (K/V re-layout)."""
    _check_qkv(plan, k, v)
    _check("abs_attend_relayout",
           load_library().abs_attend_relayout(ctypes.byref(plan), _ptr(k), _ptr(v), _ptr(ws),
                                              ws.numel(), _stream(stream)))


def attend_schedule(plan: Plan, mask: Mask, sched: int, ws, stream=None) -> None:
    """The mask-dependent half of attend_prepare (key-block lists, order)."""
    cm = mask.c()
    _check("abs_attend_schedule",
           load_library().abs_attend_schedule(ctypes.byref(plan), ctypes.byref(cm), int(sched),
                                              _ptr(ws), ws.numel(), _stream(stream)))


def attend_run(plan: Plan, q, k, mask: Mask, o, sched: int, ws, telemetry=None,
               stream=None) -> None:
    _check_qkv(plan, q, k, o)
    cm = mask.c()
    tp = ctypes.c_void_p(0) if telemetry is None else _ptr(telemetry)
    _check("abs_attend_run",
           load_library().abs_attend_run(ctypes.byref(plan), _ptr(q), _ptr(k), ctypes.byref(cm),
                                         _ptr(o), int(sched), _ptr(ws), ws.numel(), tp,
                                         _stream(stream)))


def attend(plan: Plan, q, k, v, mask: Mask, sched: Optional[int] = None, o=None, ws=None,
           telemetry=None, stream=None):
    """Block-sparse attention over the kept blocks; returns o [B, N, H, d].
    The default queue is default_sched(plan), the fastest measured for the shape."""
    torch = _check_qkv(plan, q, k, v)
    sched = default_sched(plan) if sched is None else sched
    o = torch.empty_like(q) if o is None else o
    ws = workspace(plan.attend_ws_bytes, q.device) if ws is None else ws
    attend_prepare(plan, k, v, mask, sched, ws, stream)
    attend_run(plan, q, k, mask, o, sched, ws, telemetry, stream)
    return o


def attend_split_ws_bytes(plan: Plan, max_parts: int) -> int:
    """Workspace bytes of the split-and-merge attention with max_parts slots."""
    n = ctypes.c_size_t(0)
    _check("abs_attend_split_ws_bytes",
           load_library().abs_attend_split_ws_bytes(ctypes.byref(plan), int(max_parts),
                                                    ctypes.byref(n)))
    return int(n.value)


def attend_prepare_split(plan: Plan, k, v, mask: Mask, sched: int, split_tiles: int,
                         max_parts: int, ws, stream=None) -> None:
    _check_qkv(plan, k, v)
    cm = mask.c()
    _check("abs_attend_prepare_split",
           load_library().abs_attend_prepare_split(ctypes.byref(plan), _ptr(k), _ptr(v),
                                                   ctypes.byref(cm), int(sched), int(split_tiles),
                                                   int(max_parts), _ptr(ws), ws.numel(),
                                                   _stream(stream)))


def attend_run_split(plan: Plan, q, mask: Mask, o, sched: int, max_parts: int, ws,
                     telemetry=None, stream=None) -> None:
    _check_qkv(plan, q, o)
    cm = mask.c()
    tp = ctypes.c_void_p(0) if telemetry is None else _ptr(telemetry)
    _check("abs_attend_run_split",
           load_library().abs_attend_run_split(ctypes.byref(plan), _ptr(q), ctypes.byref(cm),
                                               _ptr(o), int(sched), int(max_parts), _ptr(ws),
                                               ws.numel(), tp, _stream(stream)))


def attend_split(plan: Plan, q, k, v, mask: Mask, split_tiles: int, max_parts: int,
                 sched: int = SCHED_NNZ_SORTED, o=None, ws=None, telemetry=None, stream=None):
    """Block-sparse attention with heavy work items cut into parts of at most
    about split_tiles union entries (at most max_parts parts in all), merged by
    log-sum-exp; returns o [B, N, H, d]."""
    torch = _check_qkv(plan, q, k, v)
    o = torch.empty_like(q) if o is None else o
    ws = workspace(attend_split_ws_bytes(plan, max_parts), q.device) if ws is None else ws
    attend_prepare_split(plan, k, v, mask, sched, split_tiles, max_parts, ws, stream)
    attend_run_split(plan, q, mask, o, sched, max_parts, ws, telemetry, stream)
    return o
