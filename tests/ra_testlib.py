"""Shared helpers of the GPU parity tests: seeded inputs on the device, oracle
references, comparisons.  Inputs come from ``seeded_inputs``; references come
from ``oracle``; the HIP path is reached only through the C ABI binding."""
from __future__ import annotations

import sys

import numpy as np

import seeded_inputs as si
from oracle import attention as oa
from oracle import index_maps as im

# Tolerances: max abs error on O and LSE, fp32 inputs and bf16 inputs with fp32
# accumulation.
TOL = {"f32": 1e-5, "bf16": 2e-2}


def say(*args):
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def torch_dtype(dtype):
    import torch
    return torch.float32 if dtype == "f32" else torch.bfloat16


def to_device(x: np.ndarray, dtype: str):
    """numpy float32 or bf16 bit pattern array -> GPU tensor of that dtype."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


class RankCase:
    """Seeded tensors of a ring: the global K and V (every shard is cut from
    them), and per-rank queries generated on demand."""

    def __init__(self, seed_id, dtype, B, Hq, Hkv, D, S, P, order, causal, k_scale=1.0):
        self.seed_id, self.dtype = seed_id, dtype
        self.B, self.Hq, self.Hkv, self.D, self.S, self.P = B, Hq, Hkv, D, S, P
        self.order, self.causal, self.k_scale = order, causal, k_scale
        self.scale = 1.0 / np.sqrt(D)
        whole = [(0, S)]
        self.Kg = si.tokens(seed_id, si.TENSOR_K, B, S, Hkv, D, whole, dtype, scale=k_scale)
        self.Vg = si.tokens(seed_id, si.TENSOR_V, B, S, Hkv, D, whole, dtype)
        self._kv = None

    @classmethod
    def from_workload(cls, w, S=None, P=None):
        return cls(w.seed_id, w.dtype, w.B, w.Hq, w.Hkv, w.D, S or w.S, P or w.P, w.order, w.causal,
                   w.k_scale)

    def q_rows(self, spans):
        return si.tokens(self.seed_id, si.TENSOR_Q, self.B, self.S, self.Hq, self.D, spans, self.dtype)

    def device_shards(self, ra):
        """[P, B, S/P, Hkv, D] K and V on the GPU, gathered with the library's
        own rank spans."""
        import torch
        if self._kv is None:
            out = []
            for X in (self.Kg, self.Vg):
                xg = to_device(X, self.dtype)
                shards = torch.empty((self.P, self.B, self.S // self.P, self.Hkv, self.D),
                                     dtype=xg.dtype, device="cuda")
                for p in range(self.P):
                    off = 0
                    for a, n in ra.rank_spans(self.order, self.S, self.P, p):
                        shards[p, :, off:off + n] = xg[:, a:a + n]
                        off += n
                del xg
                out.append(shards)
            self._kv = tuple(out)
        return self._kv

    def release(self):
        self._kv = None

    def run_rank(self, ra, rank, poison=True):
        import torch
        q = to_device(self.q_rows(ra.rank_spans(self.order, self.S, self.P, rank)), self.dtype)
        ks, vs = self.device_shards(ra)
        s_loc = self.S // self.P
        o = torch.empty(self.B, s_loc, self.Hq, self.D, device="cuda", dtype=torch.float32)
        lse = torch.empty(self.B, s_loc, self.Hq, device="cuda", dtype=torch.float32)
        if poison:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
        ra.ra_rank_forward(q, ks, vs, o, lse, S=self.S, P=self.P, rank=rank, order=self.order,
                           causal=self.causal, scale=self.scale)
        torch.cuda.synchronize()
        return o.cpu().numpy(), lse.cpu().numpy()

    def run_allgather(self, ra, rank, poison=True):
        """ra_allgather_forward of ``rank``: the global K and V resident at once."""
        import torch
        q = to_device(self.q_rows(ra.rank_spans(self.order, self.S, self.P, rank)), self.dtype)
        kg, vg = to_device(self.Kg, self.dtype), to_device(self.Vg, self.dtype)
        s_loc = self.S // self.P
        o = torch.empty(self.B, s_loc, self.Hq, self.D, device="cuda", dtype=torch.float32)
        lse = torch.empty(self.B, s_loc, self.Hq, device="cuda", dtype=torch.float32)
        if poison:
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
        ra.ra_allgather_forward(q, kg, vg, o, lse, S=self.S, P=self.P, rank=rank, order=self.order,
                                causal=self.causal, scale=self.scale)
        torch.cuda.synchronize()
        return o.cpu().numpy(), lse.cpu().numpy()

    def reference(self, rank, rows=None):
        """Oracle (definition over the concatenated sequence), float64, for the
        rank's local rows ``rows`` (all rows if None)."""
        pos = im.rank_positions(self.S, self.P, rank, self.order)
        qsel = pos if rows is None else pos[np.asarray(rows)]
        q = si.to_f64(self.q_rows([(int(t), 1) for t in qsel]) if rows is not None
                      else self.q_rows(im.rank_spans(self.S, self.P, rank, self.order)), self.dtype)
        kmax = int(qsel.max()) + 1 if self.causal else self.S
        return oa.attention_rows(q, qsel, si.to_f64(self.Kg[:, :kmax], self.dtype),
                                 si.to_f64(self.Vg[:, :kmax], self.dtype), np.arange(kmax),
                                 self.causal, self.scale)


def sample_rows(S, P, rank, order, n_random, seed, per_tile=0):
    """Local rows at every span boundary plus seeded random rows; with
    ``per_tile`` > 0 also one seeded row inside every run of ``per_tile``
    consecutive rows of each span (the forward kernel's work items are 256
    rows of one head, and every head of a sampled row is compared)."""
    spans = im.rank_spans(S, P, rank, order)
    rows = set()
    rng = np.random.default_rng(seed)
    off = 0
    for _, n in spans:
        for r in (off, off + 1, off + n // 2, off + n - 2, off + n - 1):
            if off <= r < off + n:
                rows.add(r)
        if per_tile:
            for a in range(0, n, per_tile):
                rows.add(off + a + int(rng.integers(0, min(per_tile, n - a))))
        off += n
    rows.update(int(x) for x in rng.integers(0, S // P, n_random))
    return np.array(sorted(rows), dtype=np.int64)


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nanmax(np.where(np.isnan(d), np.inf, d))) if d.size else 0.0


def assert_close(o, lse, o_ref, lse_ref, dtype, what=""):
    eo, el = max_err(o, o_ref), max_err(lse, lse_ref)
    say(f"{what} max|dO| = {eo:.3e}  max|dLSE| = {el:.3e}  (tol {TOL[dtype]:.0e})")
    assert np.isfinite(o).all() or np.isnan(o_ref).any(), "non-finite output"
    assert eo <= TOL[dtype], f"O error {eo} > {TOL[dtype]}"
    assert el <= TOL[dtype], f"LSE error {el} > {TOL[dtype]}"
