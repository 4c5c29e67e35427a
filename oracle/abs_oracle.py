"""Float64 CPU oracle: 3D video blocking, pooled Top-p routing with a Top-k
floor and own-block repair, slack fill, and block-sparse softmax attention.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Product code must not
import this module.

Sources.  "FVAttn explainer" is the web page titled (in Chinese) "FVAttn:
adaptive sparse attention with runtime load balancing, for video generation",
an explainer of arXiv 2607.16190 "Adaptive Sparse Attention with Runtime Load
Balancing for Video Generation".  Its sections cited here: "The real problem",
"Core method" parts 1 (sparse-routing frontend), 2 (runtime load balancing) and
3 (slack-aware sparse augmentation), "Highlights and limitations", and "Lessons
for engineering".  The pages leave several steps open; each place where this
module picks a reading says so in its docstring ("Reading:").

Conventions.
* Inputs Q, K, V are [B, N, H, d] with tokens in row-major (t, h, w) order over
  the real latent grid (T, H, W).  Values are upcast to float64 on entry.
* Rows of the block mask are indexed r = (b * H + h) * nb + i (query block i).
"""
from __future__ import annotations

import dataclasses
import functools
import math
from typing import Dict, Optional, Sequence

import numpy as np


# --------------------------------------------------------------------------
# 3D video blocks
# --------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Geometry:
    grid: tuple        # (T, H, W) real latent grid
    block: tuple       # (bt, bh, bw)
    nblk: tuple        # blocks along each axis
    padded: tuple      # grid rounded up to whole blocks
    nb: int            # blocks per head
    bt_tokens: int     # tokens per block, bt * bh * bw

    @property
    def tokens(self) -> int:
        return self.grid[0] * self.grid[1] * self.grid[2]


def geometry(grid: Sequence[int], block: Sequence[int]) -> Geometry:
    """Block grid of a (T, H, W) latent video cut into (bt, bh, bw) blocks.

    Source: FVAttn explainer, "Core method" part 1, bullet on video-aware block
    organisation (tokens regrouped into 3D blocks that follow spatio-temporal
    locality) and "Lessons for engineering" item 4 (3D blocks rather than 1D
    chunks).  Reading: each axis is padded up to a whole number of blocks; the
    padding tokens do not exist in the input and never take part in pooling or
    attention.
    """
    grid = tuple(int(x) for x in grid)
    block = tuple(int(x) for x in block)
    nblk = tuple(-(-g // b) for g, b in zip(grid, block))
    padded = tuple(n * b for n, b in zip(nblk, block))
    return Geometry(grid, block, nblk, padded, nblk[0] * nblk[1] * nblk[2],
                    block[0] * block[1] * block[2])


def token_block_slot(t: int, h: int, w: int, geo: Geometry):
    """(block, slot) of latent token (t, h, w).

    Reading: blocks are numbered row-major over the block grid and slots
    row-major inside a block; query and key blocks share this one blocking, so
    "own block" of query block i is key block i.
    """
    bt, bh, bw = geo.block
    _, nbh, nbw = geo.nblk
    blk = ((t // bt) * nbh + h // bh) * nbw + w // bw
    slot = ((t % bt) * bh + h % bh) * bw + w % bw
    return blk, slot


@functools.lru_cache(maxsize=16)
def _members_cached(grid: tuple, block: tuple) -> np.ndarray:
    geo = geometry(grid, block)
    T, H, W = geo.grid
    table = np.full((geo.nb, geo.bt_tokens), -1, dtype=np.int64)
    for t in range(geo.padded[0]):
        for h in range(geo.padded[1]):
            for w in range(geo.padded[2]):
                blk, slot = token_block_slot(t, h, w, geo)
                if t < T and h < H and w < W:
                    table[blk, slot] = (t * H + h) * W + w
    table.setflags(write=False)
    return table


def block_members(geo: Geometry) -> np.ndarray:
    """[nb, bt_tokens] token index n = (t*H + h)*W + w of each block slot, -1 for
    a padding slot.  Built by visiting every padded coordinate once."""
    return _members_cached(geo.grid, geo.block)


# --------------------------------------------------------------------------
# Routing: pooled similarity, Top-p, floor, repair
# --------------------------------------------------------------------------
def pool(X, geo: Geometry) -> np.ndarray:
    """Mean of X over the valid tokens of each block: [B, H, nb, d] float64.

    Source: FVAttn explainer, "Highlights and limitations" (routing scores are
    an approximate similarity computed on a cheap draft) and part 1 (decisions
    are made per 3D block).  Reading: the draft is the block mean of Q and of K
    over the block's real tokens.
    """
    X = np.asarray(X, dtype=np.float64)
    B, N, H, d = X.shape
    members = block_members(geo)
    out = np.empty((B, H, geo.nb, d))
    for blk in range(geo.nb):
        idx = members[blk][members[blk] >= 0]
        out[:, :, blk, :] = X[:, idx, :, :].mean(axis=1)
    return out


def block_probabilities(Qp: np.ndarray, Kp: np.ndarray) -> np.ndarray:
    """P[b, h, i, :] = softmax_j(Qp_i . Kp_j / sqrt(d)) over all key blocks j.

    Source: FVAttn explainer, part 1, Top-p bullet (the kept set is measured by
    cumulative similarity mass).  Reading: the mass is the row softmax of the
    pooled scores, over every key block, with the usual 1/sqrt(d) scale and no
    correction for how many real tokens a block holds.
    """
    d = Qp.shape[-1]
    S = np.einsum("bhid,bhjd->bhij", Qp, Kp) / math.sqrt(d)
    S = S - S.max(axis=-1, keepdims=True)
    E = np.exp(S)
    return E / E.sum(axis=-1, keepdims=True)


def select_row(prow: np.ndarray, i: int, p: float, k_floor: int):
    """Kept key blocks of one query-block row (ascending), plus diagnostics.

    Steps (FVAttn explainer, part 1):
      1. order the key blocks by probability, largest first; equal values keep
         the lower block index first (reading: ties go to the lowest index);
      2. Top-p: m = the smallest count whose cumulative mass reaches p
         (reading: "reaches" means >= p; with p >= 1 every block is kept; if
         rounding keeps every partial sum below p, all nb blocks are kept);
      3. Top-k floor: never fewer than k_floor blocks (reading: the floor counts
         key blocks of each (head, query-block) row; k_floor > nb keeps all);
      4. repair: the query's own block is added if it is not already there
         (reading: the repair works on the materialised set without rescoring,
         and the own block is the hole it fills, so no row or key-block column
         is ever empty).
    """
    prow = np.asarray(prow, dtype=np.float64)
    nb = prow.shape[0]
    order = np.argsort(-prow, kind="stable")
    masses = prow[order]
    if p >= 1.0:
        m = nb
    else:
        csum = np.cumsum(masses)          # sequential running sum in sorted order
        hit = np.nonzero(csum >= p)[0]
        m = int(hit[0]) + 1 if hit.size else nb
    m2 = min(nb, max(m, int(k_floor)))
    kept = set(int(j) for j in order[:m2])
    kept.add(int(i))
    csum = np.concatenate([[0.0], np.cumsum(masses)])
    diag = dict(m=m, m2=m2, c_prev=float(csum[m - 1]), c_at=float(csum[m]),
                p_cut=float(masses[m2 - 1]),
                p_next=float(masses[m2]) if m2 < nb else float("nan"))
    return sorted(kept), diag


def _select_head(P: np.ndarray, p: float, k_floor: int):
    """select_row applied to every row of one head's [nb, nb] matrix at once
    (the same steps, vectorised over rows)."""
    nb = P.shape[0]
    order = np.argsort(-P, axis=1, kind="stable")
    masses = np.take_along_axis(P, order, axis=1)
    csum = np.cumsum(masses, axis=1)
    if p >= 1.0:
        m = np.full(nb, nb, dtype=np.int64)
    else:
        hit = csum >= p
        m = np.where(hit.any(axis=1), hit.argmax(axis=1) + 1, nb).astype(np.int64)
    m2 = np.minimum(nb, np.maximum(m, int(k_floor)))
    keep = np.zeros((nb, nb), dtype=bool)
    rank = np.arange(nb)[None, :]
    np.put_along_axis(keep, order, rank < m2[:, None], axis=1)
    keep[np.arange(nb), np.arange(nb)] = True
    cz = np.concatenate([np.zeros((nb, 1)), csum], axis=1)
    rows = np.arange(nb)
    diag = dict(m=m, m2=m2, c_prev=cz[rows, m - 1], c_at=cz[rows, m],
                p_cut=masses[rows, m2 - 1],
                p_next=np.where(m2 < nb, masses[rows, np.minimum(m2, nb - 1)], np.nan))
    return keep, diag


def row_exemption_causes(diag: Dict[str, np.ndarray], p: float, k_floor: int,
                         gap: float = 1e-4, tie_rel: float = 1e-5):
    """The two reasons a row's kept set is not decided robustly in float32,
    as boolean arrays (close, near_tie):

    close:    the cumulative mass is within ``gap`` of p on one side of the cut
              (and the floor does not decide the count);
    near_tie: the two probabilities straddling the final cut are a near tie,
              0 < |P_cut - P_next| <= tie_rel * P_cut.  Exact ties are not a
              reason: the lowest-index rule decides them on both sides.
    """
    m = np.asarray(diag["m"])
    if p >= 1.0:
        none = np.zeros(m.shape, dtype=bool)
        return none, none.copy()
    close = np.minimum(np.abs(diag["c_prev"] - p), np.abs(diag["c_at"] - p)) <= gap
    close &= ~(m < k_floor)
    dp = np.abs(diag["p_cut"] - diag["p_next"])
    near_tie = (dp > 0) & (dp <= tie_rel * diag["p_cut"])
    near_tie &= ~np.isnan(diag["p_next"])
    return close, near_tie


def row_exemptions(diag: Dict[str, np.ndarray], p: float, k_floor: int,
                   gap: float = 1e-4, tie_rel: float = 1e-5) -> np.ndarray:
    """True for rows whose kept set is not decided robustly in float32: rows
    with either reason of row_exemption_causes.  Every other row is
    exact-checked."""
    close, near_tie = row_exemption_causes(diag, p, k_floor, gap, tie_rel)
    return close | near_tie


def slack_fill(P: np.ndarray, keep: np.ndarray, slack: float):
    """Top up every head to a fixed budget of ceil(slack * nb^2) block pairs.

    Source: FVAttn explainer, part 3 (spare capacity is filled with high-value
    blocks) and "Lessons for engineering" item 5 (filter by score before
    filling).  Reading: the budget is per head over all nb x nb block pairs;
    the unkept pairs with the largest P are added, ties by lowest linear index
    i * nb + j, until the head holds exactly the budget (a head already at or
    above it is unchanged).
    Returns (new_keep, info) where info[(b, h)] gives the budget, the number
    added and the P values of the last added and first skipped candidates.
    """
    B, H, nb, _ = P.shape
    out = keep.copy()
    budget = int(math.ceil(float(slack) * nb * nb))
    info = {}
    for b in range(B):
        for h in range(H):
            flat_keep = out[b, h].reshape(-1)
            nnz = int(flat_keep.sum())
            need = budget - nnz
            rec = dict(budget=budget, nnz=nnz, added=0, last=np.nan, next=np.nan)
            if need > 0:
                cand = np.nonzero(~flat_keep)[0]            # ascending linear index
                vals = P[b, h].reshape(-1)[cand]
                order = np.argsort(-vals, kind="stable")
                take = cand[order[:need]]
                flat_keep[take] = True
                rec.update(added=int(need), last=float(vals[order[need - 1]]),
                           next=float(vals[order[need]]) if need < cand.size else np.nan)
            out[b, h] = flat_keep.reshape(nb, nb)
            info[(b, h)] = rec
    return out, info


def dynamic_slack_fill(P: np.ndarray, keep: np.ndarray, budget: int, theta: float):
    """Add up to `budget` unkept block pairs over the whole batch, highest P first.

    Source: FVAttn explainer, part 3 (capacity that non-critical workers leave
    idle is filled with high-scoring blocks) and "Lessons for engineering"
    item 5 (keep only blocks above a score threshold for the fill; the amount
    injected is the knob to turn down).  Reading on one GPU: the candidates are
    the unkept pairs (b, h, i, j) with P >= theta, over all heads at once (the
    compute units are shared by every head); they are ranked by P descending,
    ties by the lowest linear index ((b*H + h)*nb + i)*nb + j, and the first
    min(budget, number of candidates) are added.
    Returns (new_keep, info): info = dict(added, candidates, last, next), the
    P of the last candidate added and of the first one left out.
    """
    B, H, nb, _ = P.shape
    flat_keep = keep.reshape(-1).copy()
    flat_p = np.asarray(P, dtype=np.float64).reshape(-1)
    cand = np.nonzero(~flat_keep & (flat_p >= theta))[0]      # ascending linear index
    order = np.argsort(-flat_p[cand], kind="stable")
    n = min(max(int(budget), 0), cand.size)
    take = cand[order[:n]]
    flat_keep[take] = True
    info = dict(added=int(n), candidates=int(cand.size),
                last=float(flat_p[take[-1]]) if n > 0 else np.nan,
                next=float(flat_p[cand[order[n]]]) if n < cand.size else np.nan)
    return flat_keep.reshape(B, H, nb, nb), info


def slack_budget(records, fill: float, max_pairs: int) -> int:
    """Pair budget of the dynamic slack fill, from the telemetry of one
    persistent attention launch: records [n, 4] = (hardware id, XCC id, kept
    tiles, busy clock ticks) per workgroup.

    Source: FVAttn explainer, part 3 (after balancing, non-critical workers
    still go idle before the critical path; that slack is filled) and "Lessons
    for engineering" item 1 (watch the tail per worker).  Reading on one GPU:
    the workers are the persistent workgroups; the launch lasts T = max busy;
    the idle capacity is sum_w (T - busy_w) ticks, worth
    idle * sum(tiles) / sum(busy) tiles at the launch's mean cost per tile; the
    budget is floor(fill * that) (the product taken exactly in integers, then
    one float64 multiply and one divide), clamped to [0, max_pairs].
    """
    rec = np.asarray(records, dtype=np.int64).reshape(-1, 4)
    busy = [int(x) for x in rec[:, 3]]
    tiles = int(sum(int(x) for x in rec[:, 2]))
    total = sum(busy)
    if total <= 0 or tiles <= 0:
        return 0
    idle_tiles = (len(busy) * max(busy) - total) * tiles      # exact integer
    val = math.floor(float(fill) * float(idle_tiles) / float(total))
    return max(0, min(int(max_pairs), val))


def keep_to_csr(keep: np.ndarray):
    """CSR of a [B, H, nb, nb] boolean mask: rows (b, h, i) in order, columns
    ascending.  Returns (row_ptr int64 [rows+1], col_idx int64, head_nnz)."""
    B, H, nb, _ = keep.shape
    flat = keep.reshape(B * H * nb, nb)
    counts = flat.sum(axis=1)
    row_ptr = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    col_idx = np.nonzero(flat)[1].astype(np.int64)      # row-major: ascending per row
    head_nnz = keep.reshape(B * H, -1).sum(axis=1).astype(np.int64)
    return row_ptr, col_idx, head_nnz


def csr_to_keep(row_ptr, col_idx, B: int, H: int, nb: int) -> np.ndarray:
    keep = np.zeros((B * H * nb, nb), dtype=bool)
    row_ptr = np.asarray(row_ptr)
    col_idx = np.asarray(col_idx)
    for r in range(B * H * nb):
        keep[r, col_idx[row_ptr[r]:row_ptr[r + 1]]] = True
    return keep.reshape(B, H, nb, nb)


def route(Q, K, geo: Geometry, p: float, k_floor: int, slack: float = 0.0):
    """Pooled Top-p routing of every (batch, head, query-block) row.

    Returns a dict with the CSR arrays, the boolean mask before and after slack
    fill, the block probabilities and the per-row diagnostics used by the
    float32 exemption rule.
    """
    Qp, Kp = pool(Q, geo), pool(K, geo)
    P = block_probabilities(Qp, Kp)
    B, H, nb, _ = P.shape
    keep = np.zeros((B, H, nb, nb), dtype=bool)
    diag = {k: np.empty((B, H, nb)) for k in ("m", "m2", "c_prev", "c_at", "p_cut", "p_next")}
    for b in range(B):
        for h in range(H):
            keep[b, h], dg = _select_head(P[b, h], p, k_floor)
            for key, val in dg.items():
                diag[key][b, h] = val
    base = keep
    info = None
    if slack > 0.0:
        keep, info = slack_fill(P, base, slack)
    row_ptr, col_idx, head_nnz = keep_to_csr(keep)
    return dict(row_ptr=row_ptr, col_idx=col_idx, head_nnz=head_nnz, keep=keep,
                base_keep=base, P=P, Qp=Qp, Kp=Kp, diag=diag, slack_info=info)


# --------------------------------------------------------------------------
# Fine-grained Top-p over frames inside the kept blocks
# --------------------------------------------------------------------------
def frame_members(geo: Geometry) -> np.ndarray:
    """[nb, bt, bh*bw] token index of each slot of each frame, -1 for padding.

    A frame is the part of a 3D block at one temporal offset tau: the tokens
    (t, h, w) of the block with t = (t // bt) * bt + tau.  Slots are row-major
    with t slowest, so frame tau holds slots [tau*bh*bw, (tau+1)*bh*bw).
    """
    bt, bh, bw = geo.block
    return block_members(geo).reshape(geo.nb, bt, bh * bw)


def frame_pool(X, geo: Geometry):
    """Mean of X over the real tokens of each frame: ([B, H, nb, bt, d], counts
    [nb, bt]).  A frame with no real token (a block cut along t) has count 0
    and mean 0."""
    X = np.asarray(X, dtype=np.float64)
    B, N, H, d = X.shape
    fm = frame_members(geo)
    bt = geo.block[0]
    out = np.zeros((B, H, geo.nb, bt, d))
    counts = np.zeros((geo.nb, bt), dtype=np.int64)
    for j in range(geo.nb):
        for tau in range(bt):
            idx = fm[j, tau][fm[j, tau] >= 0]
            counts[j, tau] = idx.size
            if idx.size:
                out[:, :, j, tau, :] = X[:, idx, :, :].mean(axis=1)
    return out, counts


def select_frames_row(scores: np.ndarray, cand: np.ndarray, own: Sequence[int], p_frame: float,
                      k_floor: int):
    """Kept frames of one row, as a boolean array over the row's frame index
    f = j*bt + tau, plus diagnostics.

    Source: FVAttn explainer, "Core method" part 1: Top-p keeps the smallest
    set whose cumulative similarity mass reaches p, and the video-aware 3D
    blocks let block-level decisions be combined with Top-p's fine-grained
    decisions (the fact-check table repeats "block-level decisions combined
    with fine-grained Top-p").  Reading: after the block-level routing, Top-p
    runs again over the frames of the row's kept blocks:
      1. candidates: the frames with real tokens of the kept blocks;
      2. mass: softmax of the frame scores over the candidates only;
      3. order by mass, largest first, equal values to the lower frame index;
      4. m = the smallest count whose cumulative mass reaches p_frame (>=;
         p_frame >= 1 keeps every candidate; if rounding keeps every partial
         sum below p_frame, all candidates are kept);
      5. floor: never fewer than k_floor frames (k_floor beyond the candidate
         count keeps them all);
      6. repair: every candidate frame of the own block is kept.
    """
    scores = np.asarray(scores, dtype=np.float64)
    cand = np.asarray(cand, dtype=bool)
    idx = np.nonzero(cand)[0]
    nc = idx.size
    z = scores[idx] - scores[idx].max()
    e = np.exp(z)
    pc = e / e.sum()
    order = np.argsort(-pc, kind="stable")        # ties: lower frame index first
    masses = pc[order]
    if p_frame >= 1.0:
        m = nc
    else:
        csum = np.cumsum(masses)
        hit = np.nonzero(csum >= p_frame)[0]
        m = int(hit[0]) + 1 if hit.size else nc
    m2 = min(nc, max(m, int(k_floor)))
    keep = np.zeros(scores.shape[0], dtype=bool)
    keep[idx[order[:m2]]] = True
    for f in own:
        if cand[f]:
            keep[f] = True
    csum = np.concatenate([[0.0], np.cumsum(masses)])
    diag = dict(m=m, m2=m2, c_prev=float(csum[m - 1]), c_at=float(csum[m]),
                p_cut=float(masses[m2 - 1]),
                p_next=float(masses[m2]) if m2 < nc else float("nan"))
    return keep, diag


def route_frames(Q, K, geo: Geometry, p: float, k_floor: int, p_frame: float):
    """Block routing (route, no slack fill) followed by the frame-level Top-p
    of select_frames_row in every row.  Scores: the query block's mean of Q
    (as for the blocks) against each frame's mean of K, scale 1/sqrt(d).

    Returns route's dict plus frame_keep [B, H, nb, nb, bt] (kept frames per
    row and key block), frame_mask (int, aligned with col_idx: bit tau set when
    frame tau of that kept block is kept) and frame_diag (per-row
    diagnostics for the exemption rule).
    """
    res = route(Q, K, geo, p, k_floor)
    Kf, counts = frame_pool(K, geo)
    Qp = res["Qp"]
    B, H, nb, d = Qp.shape
    bt = geo.block[0]
    fkeep = np.zeros((B, H, nb, nb, bt), dtype=bool)
    diag = {key: np.empty((B, H, nb)) for key in ("m", "m2", "c_prev", "c_at", "p_cut", "p_next")}
    real = (counts > 0).reshape(-1)
    for b in range(B):
        for h in range(H):
            sc = (np.einsum("id,jtd->ijt", Qp[b, h], Kf[b, h]) / math.sqrt(d)).reshape(nb, nb * bt)
            for i in range(nb):
                cand = np.repeat(res["keep"][b, h, i], bt) & real
                own = range(i * bt, (i + 1) * bt)
                kf, dg = select_frames_row(sc[i], cand, own, p_frame, k_floor)
                fkeep[b, h, i] = kf.reshape(nb, bt)
                for key, val in dg.items():
                    diag[key][b, h, i] = val
    rp, ci = res["row_ptr"], res["col_idx"]
    fmask = np.zeros(ci.size, dtype=np.int64)
    for r in range(B * H * nb):
        b, rem = divmod(r, H * nb)
        h, i = divmod(rem, nb)
        for e in range(rp[r], rp[r + 1]):
            bits = fkeep[b, h, i, ci[e]]
            fmask[e] = int(sum(1 << t for t in range(bt) if bits[t]))
    res.update(frame_keep=fkeep, frame_mask=fmask, frame_diag=diag, frame_counts=counts)
    return res


def sparse_attention_frames(Q, K, V, geo: Geometry, row_ptr, col_idx, frame_mask,
                            rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """sparse_attention restricted to the kept frames: for each real query
    token of block i, one softmax over the real keys of the kept frames of the
    kept blocks of row (b, h, i) (frame_mask aligned with col_idx, bit tau for
    frame tau), scale 1/sqrt(d).  Outputs of rows not computed are NaN."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, N, H, d = Q.shape
    nb = geo.nb
    bt = geo.block[0]
    members = block_members(geo)
    fm = frame_members(geo)
    O = np.full((B, N, H, d), np.nan)
    row_ptr = np.asarray(row_ptr)
    col_idx = np.asarray(col_idx)
    frame_mask = np.asarray(frame_mask)
    todo = range(B * H * nb) if rows is None else rows
    for r in todo:
        b, rem = divmod(int(r), H * nb)
        h, i = divmod(rem, nb)
        qtok = members[i][members[i] >= 0]
        parts = []
        for e in range(row_ptr[r], row_ptr[r + 1]):
            j = int(col_idx[e])
            for tau in range(bt):
                if (int(frame_mask[e]) >> tau) & 1:
                    parts.append(fm[j, tau][fm[j, tau] >= 0])
        ktok = np.concatenate(parts)
        logits = Q[b, qtok, h, :] @ K[b, ktok, h, :].T / math.sqrt(d)
        logits -= logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        w /= w.sum(axis=1, keepdims=True)
        O[b, qtok, h, :] = w @ V[b, ktok, h, :]
    return O


# --------------------------------------------------------------------------
# Attention
# --------------------------------------------------------------------------
def sparse_attention(Q, K, V, geo: Geometry, row_ptr, col_idx,
                     rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Softmax attention of each query block over the union of its kept key
    blocks: O[b, n, h, :] for the real query tokens of the given rows.

    Source: FVAttn explainer, part 1 (the routed mask decides which KV blocks
    each head keeps; attention runs over those) and "The real problem" (the
    quadratic attention is what the sparsity removes).  Reading: one softmax
    over all real keys of all kept blocks, scale 1/sqrt(d), padding keys and
    padding queries absent.  Outputs of rows not computed are NaN.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, N, H, d = Q.shape
    nb = geo.nb
    members = block_members(geo)
    O = np.full((B, N, H, d), np.nan)
    row_ptr = np.asarray(row_ptr)
    col_idx = np.asarray(col_idx)
    todo = range(B * H * nb) if rows is None else rows
    for r in todo:
        b, rem = divmod(int(r), H * nb)
        h, i = divmod(rem, nb)
        qtok = members[i][members[i] >= 0]
        cols = col_idx[row_ptr[r]:row_ptr[r + 1]]
        ktok = np.concatenate([members[j][members[j] >= 0] for j in cols])
        logits = Q[b, qtok, h, :] @ K[b, ktok, h, :].T / math.sqrt(d)
        logits -= logits.max(axis=1, keepdims=True)
        w = np.exp(logits)
        w /= w.sum(axis=1, keepdims=True)
        O[b, qtok, h, :] = w @ V[b, ktok, h, :]
    return O


def dense_attention(Q, K, V) -> np.ndarray:
    """Textbook softmax(Q K^T / sqrt(d)) V per (batch, head), [B, N, H, d]."""
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B, N, H, d = Q.shape
    O = np.empty((B, N, H, d))
    for b in range(B):
        for h in range(H):
            s = Q[b, :, h, :] @ K[b, :, h, :].T / math.sqrt(d)
            s -= s.max(axis=1, keepdims=True)
            w = np.exp(s)
            w /= w.sum(axis=1, keepdims=True)
            O[b, :, h, :] = w @ V[b, :, h, :]
    return O


# --------------------------------------------------------------------------
# Work schedule
# --------------------------------------------------------------------------
def schedule(costs, mode: str, items_per_head: Optional[int] = None,
             heads_per_phase: int = 1, n_queues: int = 8) -> np.ndarray:
    """Order in which work items are processed.

    Source: FVAttn explainer, part 2 (runtime load balancing: measure each
    head's mask size before the kernel runs and hand the heaviest work out
    first; heavy heads go to lighter ranks).  Reading on one GPU: an item is a
    row of the block mask (or a group of rows of one head processed together),
    its cost is its kept-block count, and the compute units pull items from
    one queue.
      "head_major": items in their natural order;
      "nnz_sorted": cost descending, ties by item index;
      "head_phased": heads grouped into consecutive phases of heads_per_phase
         heads; phases in order, inside a phase cost descending, ties by item;
      "xcd_local": one queue per group of compute units (n_queues of them).
         A head's cost is the sum of its items' costs; heads are placed one by
         one, cost descending (ties by head index), each onto the queue with
         the least cost placed so far (ties by queue index).  A queue lists
         its heads in placement order, each head's items in natural order;
         the result is queue 0, then queue 1, and so on.
    """
    costs = np.asarray(costs, dtype=np.int64)
    n = costs.shape[0]
    if mode == "head_major":
        return np.arange(n, dtype=np.int64)
    if mode == "nnz_sorted":
        return np.argsort(-costs, kind="stable").astype(np.int64)
    if mode == "head_phased":
        phase = (np.arange(n) // items_per_head) // heads_per_phase
        return np.array(sorted(range(n), key=lambda r: (phase[r], -costs[r], r)),
                        dtype=np.int64)
    if mode == "xcd_local":
        heads = n // items_per_head
        head_cost = [int(costs[h * items_per_head:(h + 1) * items_per_head].sum())
                     for h in range(heads)]
        load = [0] * n_queues
        queues = [[] for _ in range(n_queues)]
        for h in sorted(range(heads), key=lambda h: (-head_cost[h], h)):
            x = min(range(n_queues), key=lambda x: (load[x], x))
            load[x] += head_cost[h]
            queues[x].append(h)
        return np.array([h * items_per_head + i for x in range(n_queues) for h in queues[x]
                         for i in range(items_per_head)], dtype=np.int64)
    raise ValueError(mode)


# --------------------------------------------------------------------------
# Split-and-merge: heavy work items cut into parts, parts merged by their lse
# --------------------------------------------------------------------------
def split_units(union_counts, split: int, max_parts: int):
    """Cut heavy work items into parts for the split-and-merge attention.

    Source: FVAttn explainer, part 2 (balance the work handed to each worker by
    acting on the heaviest units first: the top-k heavy heads are the ones
    moved) and the APB-V paper notes ("APB-V: Accelerating Long-Video
    Understanding via Sequence-Parallelism-aware Approximate Attention"), key
    design 2: one query block's attention computed in pieces on several hosts
    is joined through FlashAttention's log-sum-exp.  Reading on one GPU: a work
    item walks the ascending union of its rows' kept key blocks
    (union_counts[i] entries); an item with nt > split entries wants
    P = ceil(nt / split) parts, part q taking entries [q nt // P, (q+1) nt // P).
    Items are cut heaviest first (nt descending, ties by item index) while the
    running sum of their P stays within max_parts; the first that does not fit
    ends the cutting.  Result slots are numbered over the cut items in item
    order, consecutively within an item.

    Returns (units, cut): units = [(item, t0, t1, slot)] in item order, slot -1
    for an item left whole; cut = [(item, first_slot, P)] in item order.
    """
    counts = [int(x) for x in union_counts]
    parts = [-(-nt // split) if nt > split else 1 for nt in counts]
    heavy = sorted((i for i, nt in enumerate(counts) if nt > split),
                   key=lambda i: (-counts[i], i))
    chosen, used = set(), 0
    for i in heavy:
        if used + parts[i] > max_parts:
            break
        chosen.add(i)
        used += parts[i]
    units, cut = [], []
    slot = 0
    for item, nt in enumerate(counts):
        if item in chosen:
            P = parts[item]
            cut.append((item, slot, P))
            for q in range(P):
                units.append((item, q * nt // P, (q + 1) * nt // P, slot + q))
            slot += P
        else:
            units.append((item, 0, nt, -1))
    return units, cut


def partial_attention(q, k, v):
    """Softmax attention of queries q [n, d] over one part's keys k, v [m, d]:
    (o [n, d], lse [n]) with o normalised over this part's keys and
    lse = log sum_j exp(q . k_j / sqrt(d)) (natural log).  A part with no keys
    gives o = 0 and lse = -inf.

    Source: the APB-V paper notes, key design 2 (each host's partial attention
    for the query block carries its log-sum-exp for the merge)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    if k.shape[0] == 0:
        return np.zeros((n, v.shape[1])), np.full(n, -np.inf)
    s = q @ k.T / math.sqrt(d)
    mx = s.max(axis=1, keepdims=True)
    w = np.exp(s - mx)
    tot = w.sum(axis=1, keepdims=True)
    return (w / tot) @ v, (mx + np.log(tot))[:, 0]


def merge_partials(parts):
    """Join partial attentions over disjoint key sets: parts = [(o_p, lse_p)].
    With L = log sum_p exp(lse_p), the result is sum_p exp(lse_p - L) o_p,
    the attention over the union of the parts' keys.

    Source: the APB-V paper notes, key design 2 (FlashAttention's log-sum-exp
    merge of a query block's partial results)."""
    lse = np.stack([np.asarray(l, dtype=np.float64) for _, l in parts])     # [P, n]
    top = lse.max(axis=0)
    if not np.isfinite(top).all():
        raise ValueError("every query needs at least one key over the parts")
    wts = np.exp(lse - top)                                                   # [P, n]
    total = wts.sum(axis=0)
    out = sum(w[:, None] * np.asarray(o, dtype=np.float64) for w, (o, _) in zip(wts, parts))
    return out / total[:, None]
