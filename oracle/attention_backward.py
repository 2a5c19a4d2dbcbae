"""Gradients of the attention definition, in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages ask for the backward pass without writing it out: ringmaster's
description lists forward and backward for the p2p ring and the all-gather
path ("Status", Ring row) and calls the p2p backward a flash-style reverse
ring (the note under "Why" on the two Ring paths).  What any such backward
must produce is the exact derivative of the definition in ``attention.py``;
for one (batch, query head h, kv head g = h // G) and the loss gradient dO:

    P[i, j] = exp(s_ij - LSE_i)  on visible pairs, 0 elsewhere,
              s_ij = scale * <Q_i, K_j>
    dV_j   += sum_i P[i, j] dO_i
    dP_ij   = <dO_i, V_j>
    D_i     = <dO_i, O_i> = sum_j P[i, j] dP_ij
    dS_ij   = P[i, j] (dP_ij - D_i)
    dQ_i    = scale * sum_j dS_ij K_j
    dK_j   += scale * sum_i dS_ij Q_i

(sums over the G query heads of a group accumulate into the shared dK, dV).
These are the chain rule through the softmax; they are pinned against central
finite differences of the forward definition.  Rows with no visible key have
O = 0 and contribute nothing.
"""
from __future__ import annotations

import numpy as np

from . import index_maps as im


def _row_block(qb, qpos, kk, vv, dob, kpos, causal, scale, window=0, cu_seqlens=None):
    """P, dS of a block of query rows of one head against keys kk, vv."""
    vis = im.visible_masked(qpos, kpos, causal, window, cu_seqlens)
    s = scale * (qb @ kk.T)
    s = np.where(vis, s, -np.inf)
    m = s.max(axis=1)
    has = np.isfinite(m)
    msafe = np.where(has, m, 0.0)
    p = np.exp(s - msafe[:, None])
    p = np.where(vis, p, 0.0)
    den = p.sum(axis=1)
    p = p / np.where(has, den, 1.0)[:, None]
    o = p @ vv
    dp = dob @ vv.T
    d = (dob * o).sum(axis=1)
    ds = p * (dp - d[:, None])
    return p, ds


def attention_grads(Q, K, V, dO, causal: bool, scale: float, qpos=None, kpos=None, window: int = 0,
                    cu_seqlens=None):
    """dQ, dK, dV of sum(dO * O) for O = attention(Q, K, V).

    Q, dO: [B, Nq, Hq, D]; K, V: [B, Nk, Hkv, D]; positions default to
    0..N-1.  With ``Q`` holding only some query rows (``qpos`` their global
    positions), dK and dV are those rows' contributions.  ``window`` and
    ``cu_seqlens`` select the mask variants of ``index_maps.visible_masked``.
    """
    Q = np.asarray(Q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    B, Nq, Hq, D = Q.shape
    Nk, Hkv = K.shape[1], K.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    qpos = np.arange(Nq, dtype=np.int64) if qpos is None else np.asarray(qpos, dtype=np.int64)
    kpos = np.arange(Nk, dtype=np.int64) if kpos is None else np.asarray(kpos, dtype=np.int64)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(K)
    dV = np.zeros_like(V)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            p, ds = _row_block(Q[b, :, h], qpos, K[b, :, g], V[b, :, g], dO[b, :, h], kpos, causal, scale,
                               window, cu_seqlens)
            dV[b, :, g] += p.T @ dO[b, :, h]
            dQ[b, :, h] = scale * (ds @ K[b, :, g])
            dK[b, :, g] += scale * (ds.T @ Q[b, :, h])
    return dQ, dK, dV


def dq_rows(q, qpos, K, V, do, causal: bool, scale: float, kpos=None):
    """dQ of the given query rows only (q, do: [B, Nq, Hq, D], any rows of the
    sequence; K, V: the keys they attend to, global positions ``kpos``)."""
    dq, _, _ = attention_grads(q, K, V, do, causal, scale, qpos=qpos, kpos=kpos)
    return dq
