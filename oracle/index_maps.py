"""Index maps of the ring: which global tokens a rank owns, which shard it holds
at each ring step, and which (query, key) blocks the causal mask leaves visible.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Integers only; every
result here is compared bit-exactly with the HIP library's host plan.

Readings of the pages (they give names, not formulas):

* Contiguous sharding -- ringmaster description, "Layout" (``shard.py``, dense
  contiguous sharding): rank r owns global tokens [r*S/P, (r+1)*S/P).
* Zigzag / head-tail load balancing -- ringmaster "Layout" (``balancers.py``,
  head_tail index generation), "Sequence Parallelism IV: ... Load-Balanced
  Rings", the dictionary entry "context parallelism" (causal load imbalance is
  fixed by reordering chunks) and the TASP abstract (Zigzag-Ring Attention):
  the sequence is cut into 2P equal chunks and rank r owns chunk r (its head)
  and chunk 2P-1-r (its tail), stored head first.
* Ring schedule -- DeDLOC guide, "The Geo-Distributed Long-Context Crisis"
  (the static ring 0 -> 1 -> ... -> P-1 -> 0) and "Sequence Parallelism III"
  (queries stay, K/V blocks circulate): rank r receives from r-1, so at step s
  it holds the shard of rank (r - s) mod P.
* Causal mask -- DeDLOC guide, "Best Practices", row "Causal Mask Handling"
  (skip the upper-triangular blocks): key j is visible to query i iff j <= i,
  compared on global positions; the diagonal is visible.
"""
from __future__ import annotations

import numpy as np

ORDERS = ("contiguous", "zigzag")
FULL, DIAG, SKIP = "FULL", "DIAG", "SKIP"


def chunk_length(S: int, P: int, order: str) -> int:
    """Length of one chunk: S/P for contiguous, S/(2P) for zigzag."""
    if order == "contiguous":
        if S % P:
            raise ValueError("S must be divisible by P")
        return S // P
    if order == "zigzag":
        if S % (2 * P):
            raise ValueError("S must be divisible by 2P")
        return S // (2 * P)
    raise ValueError(order)


def rank_spans(S: int, P: int, rank: int, order: str) -> list[tuple[int, int]]:
    """Global (start, length) spans owned by ``rank``, in the rank's local order."""
    if not 0 <= rank < P:
        raise ValueError("rank out of range")
    c = chunk_length(S, P, order)
    if order == "contiguous":
        return [(rank * c, c)]
    return [(rank * c, c), ((2 * P - 1 - rank) * c, c)]


def rank_positions(S: int, P: int, rank: int, order: str) -> np.ndarray:
    """Global position of every local row of ``rank`` (int64), local order."""
    return np.concatenate([np.arange(a, a + n, dtype=np.int64)
                           for a, n in rank_spans(S, P, rank, order)])


def owner(t: int, S: int, P: int, order: str) -> tuple[int, int]:
    """(rank, local row) holding global token ``t`` -- the inverse map, written
    from the chunk definition rather than by inverting ``rank_positions``."""
    c = chunk_length(S, P, order)
    chunk, off = divmod(int(t), c)
    if order == "contiguous":
        return chunk, off
    if chunk < P:
        return chunk, off
    return 2 * P - 1 - chunk, c + off


def ring_source(rank: int, step: int, P: int) -> int:
    """Rank whose K/V shard ``rank`` holds at ring step ``step``."""
    return (rank - step) % P


def visible(qpos: np.ndarray, kpos: np.ndarray, causal: bool) -> np.ndarray:
    """Boolean [len(q), len(k)] visibility matrix on global positions."""
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    if not causal:
        return np.ones((qpos.size, kpos.size), dtype=bool)
    return kpos[None, :] <= qpos[:, None]


def segment_ids(pos, cu_seqlens) -> np.ndarray:
    """Index of the packed sequence holding each position: sequence i covers
    [cu_seqlens[i], cu_seqlens[i+1])."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    return np.searchsorted(cu, np.asarray(pos, dtype=np.int64), side="right") - 1


def visible_masked(qpos, kpos, causal: bool, window: int = 0, cu_seqlens=None) -> np.ndarray:
    """Visibility with the mask variants the tile classifier extends to.

    ringmaster names them only ("Status": sliding-window attention through the
    kernel's window, and packing / varlen).  Readings: a window w > 0 (with
    the causal mask) lets query t see the w most recent keys t-w+1 .. t; packed
    sequences (boundaries 0 = c_0 < c_1 < ... < c_n = S) let a query see only
    keys of its own sequence, under the causal (and window) rule if set.
    """
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    v = visible(qpos, kpos, causal)
    if window:
        v = v & ((qpos[:, None] - kpos[None, :]) < window)
    if cu_seqlens is not None:
        v = v & (segment_ids(qpos, cu_seqlens)[:, None] == segment_ids(kpos, cu_seqlens)[None, :])
    return v


def block_class_bruteforce(qpos, kpos, causal: bool) -> str:
    """Class of a block by enumerating every (query, key) pair."""
    v = visible(qpos, kpos, causal)
    if v.size == 0 or not v.any():
        return SKIP
    return FULL if v.all() else DIAG


def block_class(q0: int, q1: int, k0: int, k1: int, causal: bool) -> str:
    """Class of the block of query positions [q0, q1) x key positions [k0, k1).

    Same answer as the enumeration: with j <= i the test for "every pair
    visible" is the largest key against the smallest query, and "no pair
    visible" is the smallest key against the largest query.
    """
    if q1 <= q0 or k1 <= k0:
        return SKIP
    if not causal:
        return FULL
    if k0 > q1 - 1:
        return SKIP
    if k1 - 1 <= q0:
        return FULL
    return DIAG


def step_pair_classes(S, P, rank, step, order, causal) -> list[list[str]]:
    """Class of each (query span, key span) pair at one ring step."""
    src = ring_source(rank, step, P)
    qs = rank_spans(S, P, rank, order)
    ks = rank_spans(S, P, src, order)
    return [[block_class(a, a + n, b, b + m, causal) for (b, m) in ks]
            for (a, n) in qs]


def _tiles(spans, tile):
    """(start, stop) of every tile; tiles restart at each span, the last one of a
    span may be short."""
    out = []
    for a, n in spans:
        for t in range(0, n, tile):
            out.append((a + t, a + min(n, t + tile)))
    return np.array(out, dtype=np.int64).reshape(-1, 2)


def tile_counts(S, P, rank, step, order, causal, tile_q, tile_k) -> dict:
    """Number of FULL / DIAG / SKIP (query tile, key tile) pairs at one step."""
    src = ring_source(rank, step, P)
    qt = _tiles(rank_spans(S, P, rank, order), tile_q)
    kt = _tiles(rank_spans(S, P, src, order), tile_k)
    if not causal:
        return {FULL: len(qt) * len(kt), DIAG: 0, SKIP: 0}
    q0 = qt[:, 0][:, None]
    q1 = qt[:, 1][:, None]
    k0 = kt[:, 0][None, :]
    k1 = kt[:, 1][None, :]
    skip = k0 > q1 - 1
    full = (k1 - 1 <= q0) & ~skip
    n = qt.shape[0] * kt.shape[0]
    ns, nf = int(skip.sum()), int(full.sum())
    return {FULL: nf, DIAG: n - ns - nf, SKIP: ns}


def visible_pairs(S: int, P: int, rank: int, order: str, causal: bool) -> int:
    """Number of visible (query, key) pairs of one rank over the whole ring, per
    (batch, head): sum over its queries t of |{j : j <= t}| (causal) or S."""
    pos = rank_positions(S, P, rank, order)
    if not causal:
        return int(pos.size) * S
    return int((pos + 1).sum())
