"""ra_rank_backward (the reverse ring of one rank, simulated on one GPU)
against the oracle's gradients of the attention definition.  GPU tests."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention_backward as ob
from oracle import index_maps as im
from seeded_inputs import workload
from ra_testlib import RankCase, say, to_device

pytestmark = pytest.mark.gpu

# Bound on max |GPU - oracle| / max |oracle| per gradient tensor (bf16 inputs,
# P and dS rounded to bf16 before their products, fp32 accumulation).
GRAD_TOL = 2e-2


@pytest.fixture(scope="module")
def ra():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return ra


class BwdCase(RankCase):
    """A ring with a seeded loss gradient dO of the whole sequence."""

    def dout_rows(self, spans):
        return si.tokens(self.seed_id, si.TENSOR_DO, self.B, self.S, self.Hq, self.D, spans, self.dtype)

    def run_backward(self, ra, rank, dk, dv):
        """Forward then backward of ``rank``; returns dq (local order) and adds
        the rank's contributions into the device tensors dk, dv."""
        import torch
        o, lse = self.run_rank(ra, rank, poison=False)
        spans = ra.rank_spans(self.order, self.S, self.P, rank)
        q = to_device(self.q_rows(spans), self.dtype)
        do = to_device(self.dout_rows(spans), self.dtype)
        ks, vs = self.device_shards(ra)
        o_d, lse_d = torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda()
        s_loc = self.S // self.P
        dq = torch.full((self.B, s_loc, self.Hq, self.D), float("nan"), device="cuda")
        delta = torch.empty((self.B, s_loc, self.Hq), device="cuda")
        ra.ra_rank_backward(q, ks, vs, o_d, lse_d, do, dq, dk, dv, delta, S=self.S, P=self.P, rank=rank,
                            order=self.order, causal=self.causal, scale=self.scale)
        torch.cuda.synchronize()
        return dq.cpu().numpy()


def _rel_err(x, ref):
    return float(np.abs(x - ref).max() / max(np.abs(ref).max(), 1e-30))


SMALL = [
    # (label, B, Hq, Hkv, S, P, order, causal)
    ("zigzag_gqa_p4", 1, 8, 2, 1024, 4, "zigzag", True),
    ("gqa_zigzag_p8", 1, 8, 2, 2048, 8, "zigzag", True),
    ("contig_causal_p3", 1, 4, 4, 768, 3, "contiguous", True),
    ("noncausal_b2", 2, 4, 1, 512, 4, "contiguous", False),
    ("ragged_zigzag", 1, 4, 2, 1400, 4, "zigzag", True),
    ("single_rank", 1, 4, 1, 384, 1, "zigzag", True),
    # more key tiles with work than the GPU has CUs (B x Hkv x active tiles >
    # 256): the fused dK/dV kernel; rank 1's second step (192 tiles) takes the
    # split kernels
    ("fused_dkdv_zigzag_b3", 3, 16, 16, 2048, 2, "zigzag", True),
    ("fused_dkdv_noncausal_b5", 5, 16, 16, 1024, 2, "contiguous", False),
    # GQA 32/8 like the 131k workload: the fused kernel's dK waves walk the
    # four query heads of each key tile's group and the dV waves replay that
    # walk to take P from LDS; both of rank 0's steps and rank 1's first step
    # (512 key tiles with work) take it, rank 1's second step the split ones
    ("fused_dkdv_gqa32x8_b8", 8, 32, 8, 2048, 2, "zigzag", True),
]

# which backward kernel must carry some step of rank 0 in the rings above
FUSED = {"fused_dkdv_zigzag_b3", "fused_dkdv_noncausal_b5", "fused_dkdv_gqa32x8_b8"}


@pytest.mark.parametrize("cfg", SMALL, ids=[c[0] for c in SMALL])
def test_small_rings_all_ranks(ra, cfg):
    """Every rank's backward into shared dK/dV: dQ of each rank and the summed
    dK, dV equal the oracle's gradients of the whole sequence."""
    import torch
    label, B, Hq, Hkv, S, P, order, causal = cfg
    D = 128
    case = BwdCase(300 + len(label), "bf16", B, Hq, Hkv, D, S, P, order, causal)
    if label in FUSED:
        plan = ra.ra_rank_launches(dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, D=D, S=S, P=P, rank=0, order=order,
                                   causal=causal, backward=True, n_cus=0)
        say(label, "rank 0 backward kernels", [s_["kernel"] for s_ in plan])
        assert plan[0]["kernel"] == "bwd_fused"
    s_loc = S // P
    dk = torch.zeros((P, B, s_loc, Hkv, D), device="cuda")
    dv = torch.zeros_like(dk)
    dqs = []
    for r in range(P):
        say(label, "backward rank", r)
        dqs.append(case.run_backward(ra, r, dk, dv))
    Qg = si.to_f64(case.q_rows([(0, S)]), "bf16")
    Kg, Vg = si.to_f64(case.Kg, "bf16"), si.to_f64(case.Vg, "bf16")
    dOg = si.to_f64(case.dout_rows([(0, S)]), "bf16")
    dQ, dK, dV = ob.attention_grads(Qg, Kg, Vg, dOg, causal, case.scale)
    dkh, dvh = dk.cpu().numpy(), dv.cpu().numpy()
    for r in range(P):
        pos = im.rank_positions(S, P, r, order)
        e_q = _rel_err(dqs[r], dQ[:, pos])
        e_k = _rel_err(dkh[r], dK[:, pos])
        e_v = _rel_err(dvh[r], dV[:, pos])
        say(f"{label} rank {r}: rel err dQ {e_q:.2e} dK {e_k:.2e} dV {e_v:.2e}")
        assert np.isfinite(dqs[r]).all() and np.isfinite(dkh[r]).all() and np.isfinite(dvh[r]).all()
        assert e_q <= GRAD_TOL and e_k <= GRAD_TOL and e_v <= GRAD_TOL


# Float32 inputs or D = 64 take the plain SIMT backward (float32 throughout,
# no bf16 rounding of P or dS): float32 inputs to 1e-5 of the gradient scale
# (observed <= 1.3e-6), bf16 inputs to the bf16 bound.
SIMT_TOL = {"f32": 1e-5, "bf16": GRAD_TOL}

SIMT = [
    # (label, dtype, B, Hq, Hkv, D, S, P, order, causal)
    ("f32_mha2_d64_s512_ring4_contig", "f32", 1, 2, 2, 64, 512, 4, "contiguous", True),
    ("f32_gqa_d128_zigzag_p4", "f32", 1, 4, 2, 128, 512, 4, "zigzag", True),
    ("f32_noncausal_b2_d64", "f32", 2, 2, 1, 64, 256, 2, "contiguous", False),
    ("bf16_gqa_d64_zigzag_p4", "bf16", 1, 8, 2, 64, 1024, 4, "zigzag", True),
]


@pytest.mark.parametrize("cfg", SIMT, ids=[c[0] for c in SIMT])
def test_simt_rings_all_ranks(ra, cfg):
    """Float32 inputs and D = 64: every rank's backward into shared dK/dV
    against the oracle's gradients of the whole sequence."""
    import torch
    label, dtype, B, Hq, Hkv, D, S, P, order, causal = cfg
    case = BwdCase(320 + len(label), dtype, B, Hq, Hkv, D, S, P, order, causal)
    s_loc = S // P
    dk = torch.zeros((P, B, s_loc, Hkv, D), device="cuda")
    dv = torch.zeros_like(dk)
    dqs = []
    for r in range(P):
        say(label, "backward rank", r)
        dqs.append(case.run_backward(ra, r, dk, dv))
    Qg = si.to_f64(case.q_rows([(0, S)]), dtype)
    Kg, Vg = si.to_f64(case.Kg, dtype), si.to_f64(case.Vg, dtype)
    dOg = si.to_f64(case.dout_rows([(0, S)]), dtype)
    dQ, dK, dV = ob.attention_grads(Qg, Kg, Vg, dOg, causal, case.scale)
    dkh, dvh = dk.cpu().numpy(), dv.cpu().numpy()
    tol = SIMT_TOL[dtype]
    for r in range(P):
        pos = im.rank_positions(S, P, r, order)
        e_q = _rel_err(dqs[r], dQ[:, pos])
        e_k = _rel_err(dkh[r], dK[:, pos])
        e_v = _rel_err(dvh[r], dV[:, pos])
        say(f"{label} rank {r}: rel err dQ {e_q:.2e} dK {e_k:.2e} dV {e_v:.2e}")
        assert np.isfinite(dqs[r]).all() and np.isfinite(dkh[r]).all() and np.isfinite(dvh[r]).all()
        assert e_q <= tol and e_k <= tol and e_v <= tol
    case.release()


def _full_size_check(ra, name, r, seed):
    """Rank r of a full-size workload: dQ of sampled rows against the oracle,
    and over all keys dK sums to zero and dV to the sum of the rank's dO (each
    row's weights sum to one, its dS to zero)."""
    import torch
    w = workload(name)
    case = BwdCase.from_workload(w)
    s_loc = w.S // w.P
    dk = torch.zeros((w.P, w.B, s_loc, w.Hkv, w.D), device="cuda")
    dv = torch.zeros_like(dk)
    say("backward full size", name, "rank", r)
    dq = case.run_backward(ra, r, dk, dv)
    assert np.isfinite(dq).all()
    spans = im.rank_spans(w.S, w.P, r, w.order)
    pos = im.rank_positions(w.S, w.P, r, w.order)
    rng = np.random.default_rng(seed + r)
    rows = np.unique(np.concatenate([[0, 1, s_loc // 2 - 1, s_loc // 2, s_loc - 1],
                                     rng.choice(s_loc, 6, replace=False)]))
    qsel = pos[rows]
    q = si.to_f64(case.q_rows([(int(t), 1) for t in qsel]), "bf16")
    do = si.to_f64(case.dout_rows([(int(t), 1) for t in qsel]), "bf16")
    kmax = int(qsel.max()) + 1 if w.causal else w.S
    ref = ob.dq_rows(q, qsel, si.to_f64(case.Kg[:, :kmax], "bf16"), si.to_f64(case.Vg[:, :kmax], "bf16"), do,
                     w.causal, case.scale, kpos=np.arange(kmax))
    e_q = _rel_err(dq[:, rows], ref)
    say(f"{name} rank {r}: sampled dQ rel err {e_q:.2e}")
    assert e_q <= GRAD_TOL
    # conservation over every key of every shard
    dks = dk.sum(dim=(0, 2), dtype=torch.float64).cpu().numpy()       # [B, Hkv, D]
    dvs = dv.sum(dim=(0, 2), dtype=torch.float64).cpu().numpy()
    dO_all = si.to_f64(case.dout_rows(spans), "bf16")                  # [B, s_loc, Hq, D]
    G = w.Hq // w.Hkv
    want_v = dO_all.sum(axis=1).reshape(w.B, w.Hkv, G, w.D).sum(axis=2)
    scale_v = np.abs(want_v).max()
    e_v = float(np.abs(dvs - want_v).max() / scale_v)
    e_k = float(np.abs(dks).max() / scale_v)
    say(f"{name} rank {r}: sum dV rel err {e_v:.2e}, |sum dK| / |sum dO| {e_k:.2e}")
    assert e_v <= GRAD_TOL and e_k <= GRAD_TOL
    case.release()


@pytest.mark.parametrize("which", ["first", "last"])
def test_full_size_131k_sampled_and_conserved(ra, which):
    """131k-token zigzag ring of 16, GQA 32/8, first and last rank."""
    name = "bf16_gqa32x8_d128_s128k_ring16_zigzag_causal"
    _full_size_check(ra, name, 0 if which == "first" else workload(name).P - 1, 40)


@pytest.mark.parametrize("name,r", [
    ("bf16_gqa32x8_d128_s32k_ring8_zigzag_causal", 3),
    ("bf16_mha16_b2_d128_s64k_ring8_contiguous_full", 5),
])
def test_full_size_other_workloads(ra, name, r):
    """The 32k zigzag ring of 8 and the non-causal contiguous ring of 8 (batch
    2, 16 heads without grouping) at full size."""
    _full_size_check(ra, name, r, 70)
