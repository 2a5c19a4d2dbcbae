"""Ulysses sequence <-> head regrouping (the local pack and unpack around the
all-to-all).

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Sequence Parallelism II: DeepSpeed Ulysses and All-to-All Attention" and the
dictionary entry "context parallelism": before attention each rank holds every
head of its own tokens; after the all-to-all it holds every token of a subset of
the heads.  Reading: destination j of P_u owns the contiguous head block
[j*H/P_u, (j+1)*H/P_u).  The pack lays out one piece per destination:

    SEQ2HEAD:  out[j, b, t, h', :] = x[b, t, j*H/P_u + h', :]
    HEAD2SEQ:  its exact inverse.
"""
from __future__ import annotations

import numpy as np


def seq2head(x: np.ndarray, P_u: int) -> np.ndarray:
    """x [B, s_loc, H, D] -> [P_u, B, s_loc, H/P_u, D], piece j = head block j."""
    B, s_loc, H, D = x.shape
    if H % P_u:
        raise ValueError("H must be divisible by P_u")
    hp = H // P_u
    out = np.empty((P_u, B, s_loc, hp, D), dtype=x.dtype)
    for j in range(P_u):
        out[j] = x[:, :, j * hp:(j + 1) * hp, :]
    return out


def head2seq(y: np.ndarray) -> np.ndarray:
    """[P_u, B, s_loc, H/P_u, D] -> [B, s_loc, H, D]; inverse of ``seq2head``."""
    P_u, B, s_loc, hp, D = y.shape
    out = np.empty((B, s_loc, P_u * hp, D), dtype=y.dtype)
    for j in range(P_u):
        out[:, :, j * hp:(j + 1) * hp, :] = y[j]
    return out
