"""Full-softmax attention over the concatenated sequence, per-block partials and
the log-sum-exp merge, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Definition (what every ring schedule must reproduce, up to rounding): for batch
b, query head h, and a query at global position t,

    g      = h // (Hq / Hkv)                      (consecutive GQA grouping)
    V(t)   = {j : j <= t} if causal else {0..S-1}
    s_j    = scale * <Q[b, t, h], K[b, j, g]>     for j in V(t)
    LSE    = m + ln sum_j exp(s_j - m),  m = max_j s_j
    O      = sum_j exp(s_j - LSE) * V[b, j, g]

Sources: the scaled dot product, natural-log log-sum-exp and softmax-weighted
sum are the block computation of the DeDLOC guide, "Step 3" (local attention
returning output and log-sum-exp) and its dense check in "Step 4"; "every query
block sees every key/value block it needs" is "Sequence Parallelism III" and the
dictionary entry "context parallelism"; the mask is the "Causal Mask Handling"
row of the DeDLOC "Best Practices" table; the K/V-head grouping follows the
ringmaster description ("Why": Ulysses is capped by the KV-head count;
"Quickstart": num_kv_heads) read as consecutive groups.

An empty visible set gives the merge identity O = 0, LSE = -inf.
"""
from __future__ import annotations

import numpy as np

from . import index_maps as im

ROW_BLOCK = 256


def attention_rows(q, qpos, k, v, kpos, causal: bool, scale: float, window: int = 0, cu_seqlens=None):
    """Attention of query rows over a set of key rows.

    q: [B, Nq, Hq, D]; k, v: [B, Nk, Hkv, D] (any float dtype, computed in
    float64); qpos [Nq] and kpos [Nk] are global positions; ``window`` and
    ``cu_seqlens`` select the mask variants of ``index_maps.visible_masked``.  Returns
    O [B, Nq, Hq, D] and LSE [B, Nq, Hq] (float64).  With the keys of the whole
    sequence this is the definition; with the keys of one shard it is that
    shard's partial result.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    B, Nq, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    o = np.zeros((B, Nq, Hq, D), dtype=np.float64)
    lse = np.full((B, Nq, Hq), -np.inf, dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            kk = k[b, :, g, :]
            vv = v[b, :, g, :]
            for r0 in range(0, Nq, ROW_BLOCK):
                r1 = min(Nq, r0 + ROW_BLOCK)
                pos = qpos[r0:r1]
                vis = (im.visible(pos, kpos, causal) if not window and cu_seqlens is None
                       else im.visible_masked(pos, kpos, causal, window, cu_seqlens))
                # keys no query of this row block can see carry zero weight
                keep = vis.any(axis=0)
                if not keep.any():
                    continue
                vis = vis[:, keep]
                s = scale * (q[b, r0:r1, h, :] @ kk[keep].T)
                s = np.where(vis, s, -np.inf)
                m = s.max(axis=1)
                has = np.isfinite(m)
                msafe = np.where(has, m, 0.0)
                l = np.exp(s - msafe[:, None]).sum(axis=1)
                with np.errstate(divide="ignore"):
                    row_lse = np.where(has, msafe + np.log(l), -np.inf)
                w = np.exp(s - np.where(has, row_lse, 0.0)[:, None])
                w[~has] = 0.0
                o[b, r0:r1, h, :] = w @ vv[keep]
                lse[b, r0:r1, h] = row_lse
    return o, lse


def lse_merge(o_a, lse_a, o_b, lse_b):
    """Merge two partial results of the same rows.

    DeDLOC guide, "3. Online Softmax Rescaling Across Decentralized Ranks" and
    the merge routine of "Step 3": with m = max(lse_a, lse_b) and weights
    w = exp(lse - m), O = (w_a O_a + w_b O_b) / (w_a + w_b) and
    LSE = m + ln(w_a + w_b).  The pages leave the empty case open (their formula
    gives NaN when both are -inf); reading: (O = 0, LSE = -inf) is the identity,
    merge(identity, x) = x exactly and merge(identity, identity) = identity.
    o_*: [..., D]; lse_*: [...].
    """
    o_a = np.asarray(o_a, dtype=np.float64)
    o_b = np.asarray(o_b, dtype=np.float64)
    lse_a = np.asarray(lse_a, dtype=np.float64)
    lse_b = np.asarray(lse_b, dtype=np.float64)
    a_empty = np.isneginf(lse_a)
    b_empty = np.isneginf(lse_b)
    both = a_empty & b_empty
    m = np.maximum(lse_a, lse_b)
    m = np.where(both, 0.0, m)
    w_a = np.where(a_empty, 0.0, np.exp(lse_a - m))
    w_b = np.where(b_empty, 0.0, np.exp(lse_b - m))
    den = w_a + w_b
    den_safe = np.where(both, 1.0, den)
    o = (w_a[..., None] * o_a + w_b[..., None] * o_b) / den_safe[..., None]
    with np.errstate(divide="ignore"):
        lse = np.where(both, -np.inf, m + np.log(den_safe))
    # exact pass-through of the non-empty side when the other is the identity
    o = np.where(a_empty[..., None] & ~both[..., None], o_b, o)
    o = np.where(b_empty[..., None] & ~both[..., None], o_a, o)
    lse = np.where(a_empty & ~both, lse_b, lse)
    lse = np.where(b_empty & ~both, lse_a, lse)
    o = np.where(both[..., None], 0.0, o)
    return o, lse


def identity(shape_o):
    """The merge identity (O = 0, LSE = -inf) for O of the given shape."""
    return np.zeros(shape_o, dtype=np.float64), np.full(shape_o[:-1], -np.inf)


def rank_reference(Qg, Kg, Vg, S, P, rank, order, causal, scale, rows=None):
    """Definition for one rank's rows, from the global [B, S, H, D] tensors.

    ``Qg`` may instead hold only the rank's rows in local order (shape
    [B, S/P, Hq, D]).  ``rows`` optionally selects local rows.  Returns O and
    LSE in the rank's local row order.
    """
    qpos = im.rank_positions(S, P, rank, order)
    q = Qg if Qg.shape[1] == qpos.size else Qg[:, qpos]
    if rows is not None:
        rows = np.asarray(rows, dtype=np.int64)
        q = q[:, rows]
        qpos = qpos[rows]
    return attention_rows(q, qpos, Kg, Vg, np.arange(S, dtype=np.int64),
                          causal, scale)


def ring_forward(q_local, k_shards, v_shards, S, P, rank, order, causal, scale,
                 steps=None):
    """The oracle's own ring decomposition (for the invariant only).

    ``k_shards``/``v_shards``: [P, B, S/P, Hkv, D], shard p in rank p's local
    order.  The rank merges the partial of each source shard in ``steps`` order
    (default: the ring schedule (rank - s) mod P).
    """
    qpos = im.rank_positions(S, P, rank, order)
    B, Nq, Hq, D = q_local.shape
    o, lse = identity((B, Nq, Hq, D))
    order_src = ([im.ring_source(rank, s, P) for s in range(P)]
                 if steps is None else list(steps))
    for src in order_src:
        kpos = im.rank_positions(S, P, src, order)
        o_s, lse_s = attention_rows(q_local, qpos, k_shards[src], v_shards[src],
                                    kpos, causal, scale)
        o, lse = lse_merge(o, lse, o_s, lse_s)
    return o, lse
