"""ra_rank_forward_masked (sliding window, packed sequences) against the
oracle's attention under the same masks.  GPU tests."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention as oa
from oracle import index_maps as im
from seeded_inputs import workload
from ra_testlib import RankCase, assert_close, sample_rows, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return ra


def run_masked(ra, case, rank, window, cu):
    import torch
    q = to_device(case.q_rows(ra.rank_spans(case.order, case.S, case.P, rank)), case.dtype)
    ks, vs = case.device_shards(ra)
    s_loc = case.S // case.P
    o = torch.full((case.B, s_loc, case.Hq, case.D), float("nan"), device="cuda")
    lse = torch.full((case.B, s_loc, case.Hq), float("nan"), device="cuda")
    ra.ra_rank_forward_masked(q, ks, vs, o, lse, S=case.S, P=case.P, rank=rank, order=case.order,
                              causal=case.causal, scale=case.scale, window=window, cu_seqlens=cu)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def reference(case, rank, window, cu, rows=None):
    pos = im.rank_positions(case.S, case.P, rank, case.order)
    qsel = pos if rows is None else pos[np.asarray(rows)]
    q = si.to_f64(case.q_rows([(int(t), 1) for t in qsel]), case.dtype)
    kmax = int(qsel.max()) + 1 if case.causal else case.S
    return oa.attention_rows(q, qsel, si.to_f64(case.Kg[:, :kmax], case.dtype),
                             si.to_f64(case.Vg[:, :kmax], case.dtype), np.arange(kmax), case.causal,
                             case.scale, window=window, cu_seqlens=cu)


CASES = [
    # (label, B, Hq, Hkv, S, P, order, causal, window, cu)
    ("window100_zigzag_p4", 1, 8, 2, 2048, 4, "zigzag", True, 100, None),
    ("window1_contig_p2", 1, 4, 2, 512, 2, "contiguous", True, 1, None),
    ("window700_zigzag_p8", 1, 8, 2, 4096, 8, "zigzag", True, 700, None),
    ("window32_contig_p4", 2, 4, 4, 1024, 4, "contiguous", True, 32, None),
    ("packed_zigzag_p4", 1, 8, 2, 2048, 4, "zigzag", True, 0, [0, 300, 301, 1000, 2048]),
    ("packed_noncausal_p4", 2, 4, 1, 1024, 4, "contiguous", False, 0, [0, 100, 640, 641, 1024]),
    ("packed_window_zigzag", 1, 4, 2, 2048, 4, "zigzag", True, 200, [0, 513, 1200, 1600, 2048]),
    ("ragged_packed_window", 1, 4, 2, 1400, 4, "zigzag", True, 77, [0, 9, 700, 1399, 1400]),
    ("single_rank_packed", 1, 4, 1, 384, 1, "zigzag", True, 0, [0, 200, 384]),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c[0] for c in CASES])
def test_small_rings_every_row(ra, cfg):
    label, B, Hq, Hkv, S, P, order, causal, window, cu = cfg
    case = RankCase(600 + len(label), "bf16", B, Hq, Hkv, 128, S, P, order, causal)
    for r in range(P):
        say(label, "rank", r)
        o, lse = run_masked(ra, case, r, window, cu)
        o_ref, l_ref = reference(case, r, window, cu)
        assert_close(o, lse, o_ref, l_ref, "bf16", f"{label} rank {r}")


F32_CASES = [
    # (label, B, Hq, Hkv, D, S, P, order, causal, window, cu): float32 inputs,
    # the float32 kernel's tiles (ragged tails, both key-span edges)
    ("f32_window50_contig_p4", 1, 2, 2, 64, 512, 4, "contiguous", True, 50, None),
    ("f32_window7_zigzag_p4", 1, 4, 2, 64, 512, 4, "zigzag", True, 7, None),
    ("f32_packed_zigzag_p4", 1, 2, 1, 64, 512, 4, "zigzag", True, 0, [0, 77, 78, 300, 512]),
    ("f32_packed_noncausal_p2", 2, 2, 2, 64, 256, 2, "contiguous", False, 0, [0, 31, 200, 256]),
    ("f32_packed_window_d128", 1, 2, 2, 128, 384, 3, "zigzag", True, 40, [0, 100, 250, 384]),
]


@pytest.mark.parametrize("cfg", F32_CASES, ids=[c[0] for c in F32_CASES])
def test_f32_small_rings_every_row(ra, cfg):
    """The masks through the float32 kernel, every row of every rank, to the
    float32 tolerance."""
    label, B, Hq, Hkv, D, S, P, order, causal, window, cu = cfg
    case = RankCase(660 + len(label), "f32", B, Hq, Hkv, D, S, P, order, causal)
    for r in range(P):
        say(label, "rank", r)
        o, lse = run_masked(ra, case, r, window, cu)
        o_ref, l_ref = reference(case, r, window, cu)
        assert_close(o, lse, o_ref, l_ref, "f32", f"{label} rank {r}")


def test_f32_no_mask_equals_the_ring(ra):
    """The float32 kernel's masked entry with no mask gives the plain ring's
    bits."""
    case = RankCase(641, "f32", 1, 2, 2, 64, 512, 4, "contiguous", True)
    o_m, l_m = run_masked(ra, case, 3, 0, None)
    o_r, l_r = case.run_rank(ra, 3)
    np.testing.assert_array_equal(o_m, o_r)
    np.testing.assert_array_equal(l_m, l_r)


def test_no_mask_equals_the_ring(ra):
    """With neither a window nor packed sequences the masked driver is the
    plain one, bit for bit."""
    case = RankCase(640, "bf16", 1, 8, 2, 128, 2048, 4, "zigzag", True)
    o_m, l_m = run_masked(ra, case, 1, 0, None)
    o_r, l_r = case.run_rank(ra, 1)
    np.testing.assert_array_equal(o_m, o_r)
    np.testing.assert_array_equal(l_m, l_r)


@pytest.mark.parametrize("which", ["window4096_first", "window4096_last", "packed_first", "packed_last"])
def test_full_size_131k_sampled(ra, which):
    w = workload("bf16_gqa32x8_d128_s128k_ring16_zigzag_causal")
    r = 0 if which.endswith("first") else w.P - 1
    if which.startswith("window"):
        window, cu = 4096, None
    else:
        rng = np.random.default_rng(7)
        cu = [0] + sorted(rng.choice(np.arange(1, w.S), 9, replace=False).tolist()) + [w.S]
        window = 0
    say("masked full size", which, "rank", r)
    case = RankCase.from_workload(w)
    o, lse = run_masked(ra, case, r, window, cu)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = sample_rows(w.S, w.P, r, w.order, n_random=12, seed=200 + r)
    o_ref, l_ref = reference(case, r, window, cu, rows)
    assert_close(o[:, rows], lse[:, rows], o_ref, l_ref, "bf16", f"{which} rank {r}")
    case.release()
