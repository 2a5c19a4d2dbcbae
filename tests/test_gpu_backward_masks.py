"""ra_rank_backward_masked (sliding window, packed sequences) against the
oracle's gradients of the attention definition under the same masks.  GPU
tests."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_backward as ob
from oracle import index_maps as im
from seeded_inputs import workload
from ra_testlib import RankCase, say, to_device

pytestmark = pytest.mark.gpu

# Bound on max |GPU - oracle| / max |oracle| per gradient tensor, as for the
# unmasked backward (bf16 inputs, P and dS rounded to bf16 before their
# products, fp32 accumulation).
GRAD_TOL = 2e-2


@pytest.fixture(scope="module")
def ra():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return ra


class MaskedBwdCase(RankCase):
    """A ring with a seeded loss gradient dO and a mask (window, boundaries)."""

    def __init__(self, *a, window=0, cu=None, **kw):
        super().__init__(*a, **kw)
        self.window, self.cu = window, cu

    def dout_rows(self, spans):
        return si.tokens(self.seed_id, si.TENSOR_DO, self.B, self.S, self.Hq, self.D, spans, self.dtype)

    def run_backward(self, ra, rank, dk, dv):
        """Masked forward then masked backward of ``rank``; returns dq (local
        order) and adds the rank's contributions into dk, dv."""
        import torch
        spans = ra.rank_spans(self.order, self.S, self.P, rank)
        q = to_device(self.q_rows(spans), self.dtype)
        do = to_device(self.dout_rows(spans), self.dtype)
        ks, vs = self.device_shards(ra)
        s_loc = self.S // self.P
        o = torch.full((self.B, s_loc, self.Hq, self.D), float("nan"), device="cuda")
        lse = torch.full((self.B, s_loc, self.Hq), float("nan"), device="cuda")
        kw = dict(S=self.S, P=self.P, rank=rank, order=self.order, causal=self.causal, scale=self.scale,
                  window=self.window, cu_seqlens=self.cu)
        ra.ra_rank_forward_masked(q, ks, vs, o, lse, **kw)
        dq = torch.full((self.B, s_loc, self.Hq, self.D), float("nan"), device="cuda")
        delta = torch.empty((self.B, s_loc, self.Hq), device="cuda")
        ra.ra_rank_backward_masked(q, ks, vs, o, lse, do, dq, dk, dv, delta, **kw)
        torch.cuda.synchronize()
        return dq.cpu().numpy()


def _rel_err(x, ref, floor=1e-30):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), floor))


def _term_floor(scale, dO, V, X):
    """A size of the terms of dQ (X = K) or dK (X = Q): scale |dP| |X| with
    |dP_ij| <= |dO_i| |V_j|, times 1e-3.  Where the exact gradient vanishes
    (a window of one key: dS = P (dP - delta) = 0) it bounds the relative
    error's denominator from below; elsewhere the gradient is far larger."""
    n_do = np.sqrt((dO ** 2).sum(axis=-1)).max()
    n_v = np.sqrt((V ** 2).sum(axis=-1)).max()
    return 1e-3 * scale * n_do * n_v * np.abs(X).max()


CASES = [
    # (label, B, Hq, Hkv, S, P, order, causal, window, cu)
    ("window100_zigzag_p4", 1, 8, 2, 1024, 4, "zigzag", True, 100, None),
    ("window1_contig_p2", 1, 4, 2, 512, 2, "contiguous", True, 1, None),
    ("window300_zigzag_p8", 1, 4, 2, 2048, 8, "zigzag", True, 300, None),
    ("packed_zigzag_p4", 1, 8, 2, 1024, 4, "zigzag", True, 0, [0, 300, 301, 700, 1024]),
    ("packed_noncausal_p4", 2, 4, 1, 512, 4, "contiguous", False, 0, [0, 100, 320, 321, 512]),
    ("packed_window_zigzag", 1, 4, 2, 1024, 4, "zigzag", True, 90, [0, 257, 600, 800, 1024]),
    ("ragged_packed_window", 1, 4, 2, 1400, 4, "zigzag", True, 77, [0, 9, 700, 1399, 1400]),
    ("single_rank_packed", 1, 4, 1, 384, 1, "zigzag", True, 0, [0, 200, 384]),
    # more key tiles with work than the GPU has CUs on each rank's first step:
    # the fused masked dK/dV kernel (later steps, with few tiles, the split ones)
    ("fused_window600_packed_b3", 3, 16, 16, 2048, 2, "zigzag", True, 600, [0, 700, 701, 1500, 2048]),
    # GQA 32/8 through the fused masked kernel (step 0 of each rank)
    ("fused_gqa32x8_window300_b8", 8, 32, 8, 2048, 2, "zigzag", True, 300, None),
    # non-causal packed sequences through the fused masked kernel: rows see
    # keys after them, so query tiles sit before the wave's keys
    ("fused_gqa32x8_packed_noncausal_b8", 8, 32, 8, 2048, 2, "contiguous", False, 0, [0, 700, 701, 1500, 2048]),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c[0] for c in CASES])
def test_small_rings_all_ranks(ra, cfg):
    """Every rank's masked backward into shared dK/dV: dQ of each rank and
    the summed dK, dV equal the oracle's masked gradients of the whole
    sequence."""
    import torch
    label, B, Hq, Hkv, S, P, order, causal, window, cu = cfg
    D = 128
    case = MaskedBwdCase(500 + len(label), "bf16", B, Hq, Hkv, D, S, P, order, causal, window=window, cu=cu)
    if label.startswith("fused"):
        plan = ra.ra_rank_launches(dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, P=P, rank=0, order=order,
                                   causal=causal, backward=True, n_cus=0, window=window, cu_seqlens=cu)
        say(label, "rank 0 backward kernels", [(s_["kernel"], s_["masked"]) for s_ in plan])
        assert plan[0]["kernel"] == "bwd_fused" and plan[0]["masked"]
    s_loc = S // P
    dk = torch.zeros((P, B, s_loc, Hkv, D), device="cuda")
    dv = torch.zeros_like(dk)
    dqs = []
    for r in range(P):
        say(label, "masked backward rank", r)
        dqs.append(case.run_backward(ra, r, dk, dv))
    Qg = si.to_f64(case.q_rows([(0, S)]), "bf16")
    Kg, Vg = si.to_f64(case.Kg, "bf16"), si.to_f64(case.Vg, "bf16")
    dOg = si.to_f64(case.dout_rows([(0, S)]), "bf16")
    dQ, dK, dV = ob.attention_grads(Qg, Kg, Vg, dOg, causal, case.scale, window=window, cu_seqlens=cu)
    dkh, dvh = dk.cpu().numpy(), dv.cpu().numpy()
    fq = _term_floor(case.scale, dOg, Vg, Kg)
    fk = _term_floor(case.scale, dOg, Vg, Qg)
    for r in range(P):
        pos = im.rank_positions(S, P, r, order)
        e_q = _rel_err(dqs[r], dQ[:, pos], fq)
        e_k = _rel_err(dkh[r], dK[:, pos], fk)
        e_v = _rel_err(dvh[r], dV[:, pos])
        say(f"{label} rank {r}: rel err dQ {e_q:.2e} dK {e_k:.2e} dV {e_v:.2e}")
        assert np.isfinite(dqs[r]).all() and np.isfinite(dkh[r]).all() and np.isfinite(dvh[r]).all()
        assert e_q <= GRAD_TOL and e_k <= GRAD_TOL and e_v <= GRAD_TOL
    case.release()


F32_CASES = [
    # (label, D, B, Hq, Hkv, S, P, order, causal, window, cu): the SIMT backward
    ("f32_window40_zigzag_p4", 64, 1, 2, 2, 512, 4, "zigzag", True, 40, None),
    ("f32_packed_window_contig_p4", 64, 1, 4, 2, 512, 4, "contiguous", True, 30, [0, 100, 101, 400, 512]),
    ("f32_packed_noncausal_d128", 128, 1, 2, 1, 256, 2, "contiguous", False, 0, [0, 90, 256]),
]


@pytest.mark.parametrize("cfg", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_f32_masked_rings_all_ranks(ra, cfg):
    """The masks through the float32 (SIMT) backward, to 1e-5."""
    import torch
    label, D, B, Hq, Hkv, S, P, order, causal, window, cu = cfg
    case = MaskedBwdCase(540 + len(label), "f32", B, Hq, Hkv, D, S, P, order, causal, window=window, cu=cu)
    s_loc = S // P
    dk = torch.zeros((P, B, s_loc, Hkv, D), device="cuda")
    dv = torch.zeros_like(dk)
    dqs = [case.run_backward(ra, r, dk, dv) for r in range(P)]
    Qg = si.to_f64(case.q_rows([(0, S)]), "f32")
    Kg, Vg = si.to_f64(case.Kg, "f32"), si.to_f64(case.Vg, "f32")
    dOg = si.to_f64(case.dout_rows([(0, S)]), "f32")
    dQ, dK, dV = ob.attention_grads(Qg, Kg, Vg, dOg, causal, case.scale, window=window, cu_seqlens=cu)
    dkh, dvh = dk.cpu().numpy(), dv.cpu().numpy()
    for r in range(P):
        pos = im.rank_positions(S, P, r, order)
        e = [_rel_err(dqs[r], dQ[:, pos]), _rel_err(dkh[r], dK[:, pos]), _rel_err(dvh[r], dV[:, pos])]
        say(f"{label} rank {r}: rel err dQ {e[0]:.2e} dK {e[1]:.2e} dV {e[2]:.2e}")
        assert max(e) <= 1e-5
    case.release()


def test_no_mask_equals_unmasked_backward(ra):
    """With neither a window nor boundaries the masked entry point is
    ra_rank_backward: the same kernels, so the same bits."""
    import torch
    case = MaskedBwdCase(77, "bf16", 1, 8, 2, 128, 1024, 4, "zigzag", True)
    s_loc = case.S // case.P
    shape = (case.P, case.B, s_loc, case.Hkv, case.D)
    dk_a, dv_a = torch.zeros(shape, device="cuda"), torch.zeros(shape, device="cuda")
    dk_b, dv_b = torch.zeros(shape, device="cuda"), torch.zeros(shape, device="cuda")
    spans = ra.rank_spans(case.order, case.S, case.P, 2)
    q = to_device(case.q_rows(spans), "bf16")
    do = to_device(case.dout_rows(spans), "bf16")
    ks, vs = case.device_shards(ra)
    kw = dict(S=case.S, P=case.P, rank=2, order=case.order, causal=True, scale=case.scale)
    o = torch.empty((case.B, s_loc, case.Hq, case.D), device="cuda")
    lse = torch.empty((case.B, s_loc, case.Hq), device="cuda")
    ra.ra_rank_forward(q, ks, vs, o, lse, **kw)
    dq_a, dq_b = torch.empty_like(o), torch.empty_like(o)
    delta = torch.empty_like(lse)
    ra.ra_rank_backward(q, ks, vs, o, lse, do, dq_a, dk_a, dv_a, delta, **kw)
    ra.ra_rank_backward_masked(q, ks, vs, o, lse, do, dq_b, dk_b, dv_b, delta, **kw)
    torch.cuda.synchronize()
    assert torch.equal(dq_a, dq_b) and torch.equal(dk_a, dk_b) and torch.equal(dv_a, dv_b)
    case.release()


@pytest.mark.parametrize("which", ["window4096_first", "window4096_last", "packed_first", "packed_last"])
def test_full_size_131k_sampled_and_conserved(ra, which):
    """131k-token zigzag ring of 16, GQA 32/8, under a 4096-token window or
    packed sequences: dQ of sampled rows against the oracle, and over all keys
    dK sums to zero and dV to the sum of the rank's dO."""
    import torch
    w = workload("bf16_gqa32x8_d128_s128k_ring16_zigzag_causal")
    r = 0 if which.endswith("first") else w.P - 1
    if which.startswith("window"):
        window, cu = 4096, None
    else:
        window = 0
        rng = np.random.default_rng(11)
        cuts = np.sort(rng.choice(np.arange(1, w.S), 23, replace=False))
        cu = [0] + [int(c) for c in cuts] + [w.S]
    case = MaskedBwdCase(w.seed_id, w.dtype, w.B, w.Hq, w.Hkv, w.D, w.S, w.P, w.order, w.causal,
                         k_scale=w.k_scale, window=window, cu=cu)
    s_loc = w.S // w.P
    dk = torch.zeros((w.P, w.B, s_loc, w.Hkv, w.D), device="cuda")
    dv = torch.zeros_like(dk)
    say("masked backward full size", which)
    dq = case.run_backward(ra, r, dk, dv)
    assert np.isfinite(dq).all()
    spans = im.rank_spans(w.S, w.P, r, w.order)
    pos = im.rank_positions(w.S, w.P, r, w.order)
    rng = np.random.default_rng(60 + r)
    rows = np.unique(np.concatenate([[0, 1, s_loc // 2 - 1, s_loc // 2, s_loc - 1],
                                     rng.choice(s_loc, 6, replace=False)]))
    qsel = pos[rows]
    q = si.to_f64(case.q_rows([(int(t), 1) for t in qsel]), "bf16")
    do = si.to_f64(case.dout_rows([(int(t), 1) for t in qsel]), "bf16")
    kmax = int(qsel.max()) + 1
    ref, _, _ = ob.attention_grads(q, si.to_f64(case.Kg[:, :kmax], "bf16"), si.to_f64(case.Vg[:, :kmax], "bf16"),
                                   do, True, case.scale, qpos=qsel, kpos=np.arange(kmax), window=window,
                                   cu_seqlens=cu)
    e_q = _rel_err(dq[:, rows], ref)
    say(f"{which}: sampled dQ rel err {e_q:.2e}")
    assert e_q <= GRAD_TOL
    dks = dk.sum(dim=(0, 2), dtype=torch.float64).cpu().numpy()       # [B, Hkv, D]
    dvs = dv.sum(dim=(0, 2), dtype=torch.float64).cpu().numpy()
    dO_all = si.to_f64(case.dout_rows(spans), "bf16")                  # [B, s_loc, Hq, D]
    G = w.Hq // w.Hkv
    want_v = dO_all.sum(axis=1).reshape(w.B, w.Hkv, G, w.D).sum(axis=2)
    scale_v = np.abs(want_v).max()
    e_v = float(np.abs(dvs - want_v).max() / scale_v)
    e_k = float(np.abs(dks).max() / scale_v)
    say(f"{which}: sum dV rel err {e_v:.2e}, |sum dK| / |sum dO| {e_k:.2e}")
    assert e_v <= GRAD_TOL and e_k <= GRAD_TOL
    case.release()
