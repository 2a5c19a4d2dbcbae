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


# ---------------------------------------------------------------------------
# Messages of one all-to-all for several tensors (the fused exchange of
# ringmaster's Ulysses leg: one collective carries K and V, or Q, K and V).
# A piece is the message between one pair of ranks: one section per tensor.

def to_pieces(tensors, P_u: int, group: str):
    """Sender side ("heads": tensors [B, s_loc, H_i, D_i], piece j section i =
    head block j) or receiver side ("seq": tensors [B, P_u*s_loc, Hp_i, D_i],
    piece u section i = tokens [u*s_loc, (u+1)*s_loc)).  Returns a list of
    P_u pieces, each a list of sections."""
    out = []
    for j in range(P_u):
        piece = []
        for x in tensors:
            if group == "heads":
                hp = x.shape[2] // P_u
                if x.shape[2] % P_u:
                    raise ValueError("heads must be divisible by P_u")
                piece.append(x[:, :, j * hp:(j + 1) * hp, :].copy())
            else:
                s_loc = x.shape[1] // P_u
                piece.append(x[:, j * s_loc:(j + 1) * s_loc].copy())
        out.append(piece)
    return out


def from_pieces(pieces, group: str):
    """Inverse of ``to_pieces``: the tensors back from P_u pieces."""
    P_u = len(pieces)
    out = []
    for i in range(len(pieces[0])):
        secs = [pieces[j][i] for j in range(P_u)]
        if group == "heads":
            out.append(np.concatenate(secs, axis=2))
        else:
            out.append(np.concatenate(secs, axis=1))
    return out


def piece_bytes(pieces) -> np.ndarray:
    """The pieces as one byte buffer: piece after piece, section after
    section, each in C order."""
    return np.concatenate([np.ascontiguousarray(sec).view(np.uint8).ravel()
                           for piece in pieces for sec in piece])


def exchange(sends):
    """The all-to-all itself: rank u's piece j goes to rank j, which files
    it as its piece u.  ``sends[u]`` is rank u's list of P_u pieces."""
    P_u = len(sends)
    return [[sends[u][j] for u in range(P_u)] for j in range(P_u)]
