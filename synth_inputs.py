"""Seeded synthetic Q/K/V for Wan-shaped video self-attention layers.

This module is shared by the tests, the benchmark and the smoke check.  It holds
the workload descriptions (shapes, routing parameters) and the random input
recipe, and nothing of the attention method itself: no blocking, pooling,
scoring, routing or attention arithmetic lives here.

Input recipe (the pages supply no activations; real Wan2.2 / Wan2.1 tensors are
not available, so these stand in for them):

* token coordinates u_n = ((t+1/2)/T, (h+1/2)/H, (w+1/2)/W) over the real grid,
  tokens in row-major (t, h, w) order;
* per head, 16 random Fourier features phi_n = sqrt(2) cos(2 pi Omega u_n + b),
  Omega ~ N(0, 0.5^2) in R^{16x3}, b ~ U[0, 2 pi);
* one projection W ~ N(0, 0.25^2) in R^{16 x d}, shared by Q and K of a head;
* Q~ = phi W + 0.3 eps_q, K~ = phi W + 0.3 eps_k, eps ~ N(0, 1);
* sigma = std of Q~_i . K~_j / sqrt(d) over 65 536 seeded random token pairs
  (all pairs when N <= 4096);
* Q = sqrt(2 / sigma) Q~ / tau_h, K = sqrt(2 / sigma) K~, so logits have a
  standard deviation of about 2 / tau_h; V ~ N(0, 1);
* tau_h = 1 (tiny), U(1, 3) (480p, 720p, long horizon) or log-uniform over
  [0.3, 6] (head-imbalance stress);
* seeds: numpy default_rng([cfg, head, stream]) with stream 0 = Omega, b, W;
  1 = eps_q; 2 = eps_k; 3 = V; 4 = pair sample; batch entry b > 0 uses
  default_rng([cfg, head, 1000 + b, stream]); temperatures use
  default_rng([cfg, 65535]);
* tensors are laid out [B, N, H, d] and cast to the workload dtype with
  round-to-nearest-even (bf16 through torch).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

N_FEATURES = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    cfg: int
    name: str
    batch: int
    heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    grid: tuple                # (T, H, W) latent grid
    block: tuple               # (bt, bh, bw) 3D block
    p: tuple                   # top-p values exercised
    k_floor: int
    slack: float               # per-head budget as a fraction of nb^2 (0 = off)
    tau: str                   # temperature law: "one", "u13", "loguniform"

    @property
    def tokens(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]


WORKLOADS = {
    0: Workload(0, "tiny-4x8x8-d64-f32", 1, 2, 64, "f32", (4, 8, 8), (2, 4, 4),
                (0.9,), 2, 0.0, "one"),
    1: Workload(1, "wan22-14b-480p-21x30x52-h40-d128-bf16", 1, 40, 128, "bf16",
                (21, 30, 52), (2, 8, 8), (0.9,), 4, 0.0, "u13"),
    2: Workload(2, "wan22-14b-720p-21x45x80-h40-d128-bf16", 1, 40, 128, "bf16",
                (21, 45, 80), (2, 8, 8), (0.9, 0.95), 8, 0.0, "u13"),
    3: Workload(3, "wan22-480p-head-imbalance-tau-loguniform", 1, 40, 128, "bf16",
                (21, 30, 52), (2, 8, 8), (0.95,), 4, 0.0, "loguniform"),
    4: Workload(4, "wan21-1.3b-long-81x30x52-h12-d128-bf16-slack15", 1, 12, 128, "bf16",
                (81, 30, 52), (2, 8, 8), (0.9,), 8, 0.15, "u13"),
}


def temperatures(cfg: int, heads: int, law: str) -> np.ndarray:
    rng = np.random.default_rng([cfg, 65535])
    if law == "one":
        return np.ones(heads)
    if law == "u13":
        return rng.uniform(1.0, 3.0, heads)
    if law == "loguniform":
        return np.exp(rng.uniform(math.log(0.3), math.log(6.0), heads))
    raise ValueError(law)


def _coords(grid) -> np.ndarray:
    T, H, W = grid
    t, h, w = np.meshgrid(np.arange(T), np.arange(H), np.arange(W), indexing="ij")
    u = np.stack([(t.ravel() + 0.5) / T, (h.ravel() + 0.5) / H, (w.ravel() + 0.5) / W], 1)
    return u  # [N, 3], row-major (t, h, w)


def head_tensors(cfg: int, head: int, grid, d: int, tau: float,
                 n_pairs: int = 65536, batch: int = 0):
    """Float32 Q, K, V of one head, each [N, d] (before the dtype cast).
    Batch entry b > 0 draws from seeds extended by b."""
    u = _coords(grid)
    N = u.shape[0]
    key = [cfg, head] if batch == 0 else [cfg, head, 1000 + batch]

    def rng(stream):
        return np.random.default_rng(key + [stream])

    r0 = rng(0)
    omega = r0.normal(0.0, 0.5, (N_FEATURES, 3))
    phase = r0.uniform(0.0, 2.0 * math.pi, N_FEATURES)
    proj = r0.normal(0.0, 1.0 / math.sqrt(N_FEATURES), (N_FEATURES, d))
    phi = math.sqrt(2.0) * np.cos(2.0 * math.pi * (u @ omega.T) + phase)
    base = (phi @ proj).astype(np.float32)
    eq = rng(1).standard_normal((N, d), dtype=np.float32)
    ek = rng(2).standard_normal((N, d), dtype=np.float32)
    q = base + np.float32(0.3) * eq
    del eq
    k = base + np.float32(0.3) * ek
    del ek, base
    if N <= 4096:
        lg = (q.astype(np.float64) @ k.astype(np.float64).T) / math.sqrt(d)
        sigma = float(lg.std())
    else:
        idx = rng(4).integers(0, N, (n_pairs, 2))
        lg = np.einsum("ij,ij->i", q[idx[:, 0]].astype(np.float64),
                       k[idx[:, 1]].astype(np.float64)) / math.sqrt(d)
        sigma = float(lg.std())
    s = math.sqrt(2.0 / sigma)
    q *= np.float32(s / tau)
    k *= np.float32(s)
    v = rng(3).standard_normal((N, d), dtype=np.float32)
    return q, k, v


def make_inputs(wl: Workload, heads: Optional[Sequence[int]] = None, device: str = "cpu"):
    """Q, K, V as torch tensors [B, N, H, d] in the workload dtype.

    ``heads`` restricts generation to a subset of head indices (the layout still
    has len(heads) heads, in the given order); the default is all heads.  Each
    batch entry is its own draw (batch entry 0 uses the base seeds).
    """
    import torch

    hs = list(range(wl.heads)) if heads is None else list(heads)
    taus = temperatures(wl.cfg, wl.heads, wl.tau)
    tdt = torch.float32 if wl.dtype == "f32" else torch.bfloat16
    N, d = wl.tokens, wl.head_dim
    out = [torch.empty((wl.batch, N, len(hs), d), dtype=tdt) for _ in range(3)]
    for b in range(wl.batch):
        for slot, h in enumerate(hs):
            qkv = head_tensors(wl.cfg, h, wl.grid, d, float(taus[h]), batch=b)
            for dst, src in zip(out, qkv):
                # round-to-nearest-even cast, done by torch
                dst[b, :, slot, :] = torch.from_numpy(src).to(tdt)
    if device != "cpu":
        out = [t.to(device) for t in out]
    return tuple(out)
