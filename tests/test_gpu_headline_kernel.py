"""Every-row parity of the kernels that produce the benchmark figures.

The full-size rings run the bf16 D = 128 four-wave step kernel, which the host
picks for launches with many work items (at least two query tiles per CU).  The
reduced rings below are sized so that the host picks that same kernel, and
each test first asks the library (``ra_rank_launches``, with the device's own
compute-unit count) which kernel every step launches and asserts it, so a
different device or a changed rule cannot silently reroute the test.  Then
every output row of every listed rank is compared with the oracle, dense
attention over the concatenated sequence, the check the DeDLOC guide's
"Step 4: Verification and Benchmarking Test Harness" makes on every output.
GPU tests.
"""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention as oa
from oracle import index_maps as im
from ra_testlib import RankCase, assert_close, say, to_device

pytestmark = pytest.mark.gpu

FOUR_WAVE = "step_bf16"


@pytest.fixture(scope="module")
def ra():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return ra


def launches(ra, case, rank, window=0, cu=None):
    return ra.ra_rank_launches(dtype=case.dtype, B=case.B, Hq=case.Hq, Hkv=case.Hkv, D=case.D, S=case.S,
                               P=case.P, rank=rank, order=case.order, causal=case.causal, n_cus=0,
                               window=window, cu_seqlens=cu)


def run_masked(ra, case, rank, window, cu):
    import torch
    q = to_device(case.q_rows(ra.rank_spans(case.order, case.S, case.P, rank)), case.dtype)
    ks, vs = case.device_shards(ra)
    s_loc = case.S // case.P
    o = torch.full((case.B, s_loc, case.Hq, case.D), float("nan"), device="cuda")
    lse = torch.full((case.B, s_loc, case.Hq), float("nan"), device="cuda")
    cu_dev = torch.tensor(cu, dtype=torch.int64, device="cuda") if cu is not None else None
    ra.ra_rank_forward_masked(q, ks, vs, o, lse, S=case.S, P=case.P, rank=rank, order=case.order,
                              causal=case.causal, scale=case.scale, window=window, cu_seqlens=cu,
                              cu_seqlens_dev=cu_dev)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def masked_reference(case, rank, window, cu):
    pos = im.rank_positions(case.S, case.P, rank, case.order)
    q = si.to_f64(case.q_rows(im.rank_spans(case.S, case.P, rank, case.order)), case.dtype)
    kmax = int(pos.max()) + 1 if case.causal else case.S
    return oa.attention_rows(q, pos, si.to_f64(case.Kg[:, :kmax], case.dtype),
                             si.to_f64(case.Vg[:, :kmax], case.dtype), np.arange(kmax), case.causal,
                             case.scale, window=window, cu_seqlens=cu)


RINGS = [
    # (label, B, Hq, Hkv, S, P, order, causal, k_scale, window, cu, ranks)
    # GQA 16/4, zigzag: diagonal step 0 and the full step 1 (1024 and 512 items)
    ("gqa_zigzag_b8", 8, 16, 4, 4096, 2, "zigzag", True, 1.0, 0, None, (0, 1)),
    # chunks of 1000 rows: ragged query tiles (232 rows) and key tiles (8 keys)
    ("ragged_zigzag_b8", 8, 16, 4, 4000, 2, "zigzag", True, 1.0, 0, None, (0, 1)),
    # contiguous causal ring of 4: rank 3 takes four launches, rank 0 one;
    # K x 0.5 flattens the softmax as in the 524k workload
    ("khalf_contig_causal_p4_b8", 8, 16, 4, 8192, 4, "contiguous", True, 0.5, 0, None, (0, 3)),
    # batch 4, 16 heads without grouping, bidirectional: every tile unmasked
    ("mha_noncausal_b4", 4, 16, 16, 4096, 2, "contiguous", False, 1.0, 0, None, (0, 1)),
    # the masked instantiation: a window over both steps, packed sequences
    ("window1500_zigzag_b16", 16, 16, 4, 4096, 2, "zigzag", True, 1.0, 1500, None, (0, 1)),
    ("packed_zigzag_b8", 8, 16, 4, 4096, 2, "zigzag", True, 1.0, 0, [0, 700, 701, 2500, 4096], (0, 1)),
    ("packed_noncausal_b8", 8, 16, 4, 4096, 2, "contiguous", False, 1.0, 0, [0, 700, 701, 2500, 4096],
     (0,)),
]


@pytest.mark.parametrize("cfg", RINGS, ids=[c[0] for c in RINGS])
def test_four_wave_kernel_every_row(ra, cfg):
    label, B, Hq, Hkv, S, P, order, causal, k_scale, window, cu, ranks = cfg
    case = RankCase(900 + len(label), "bf16", B, Hq, Hkv, 128, S, P, order, causal, k_scale)
    for r in ranks:
        plan = launches(ra, case, r, window, cu)
        kinds = [s["kernel"] for s in plan]
        say(label, "rank", r, "kernels", kinds)
        launched = [k for k in kinds if k != "none"]
        assert launched and all(k == FOUR_WAVE for k in launched), kinds
        assert all(s["masked"] == bool(window or cu) for s in plan if s["kernel"] != "none")
        if window or cu is not None:
            o, lse = run_masked(ra, case, r, window, cu)
            o_ref, l_ref = masked_reference(case, r, window, cu)
        else:
            o, lse = case.run_rank(ra, r)
            o_ref, l_ref = case.reference(r)
        assert_close(o, lse, o_ref, l_ref, "bf16", f"{label} rank {r}")
    case.release()


def test_allgather_form_every_row(ra):
    """The all-gather form: one launch of the same kernel over the whole
    resident sequence (1024 items), every row of rank 1."""
    case = RankCase(951, "bf16", 8, 16, 4, 128, 4096, 2, "zigzag", True)
    o, lse = case.run_allgather(ra, 1)
    o_ref, l_ref = case.reference(1)
    assert_close(o, lse, o_ref, l_ref, "bf16", "allgather gqa_zigzag_b8 rank 1")


def test_masked_graph_capture_with_device_boundaries(ra):
    """With the caller's device copy of the packed-sequence boundaries the
    masked ring makes no allocation or copy of its own, so it can be captured
    as a graph; three replays (eager work between them) match the eager
    call bit for bit."""
    import torch
    cu = [0, 700, 701, 2500, 4096]
    case = RankCase(952, "bf16", 8, 16, 4, 128, 4096, 2, "zigzag", True)
    q = to_device(case.q_rows(ra.rank_spans("zigzag", 4096, 2, 1)), "bf16")
    ks, vs = case.device_shards(ra)
    cu_dev = torch.tensor(cu, dtype=torch.int64, device="cuda")
    o = torch.empty((8, 2048, 16, 128), device="cuda")
    lse = torch.empty((8, 2048, 16), device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    kw = dict(S=4096, P=2, rank=1, order="zigzag", causal=True, cu_seqlens=cu, cu_seqlens_dev=cu_dev,
              stream=stream)
    with torch.cuda.stream(stream):
        ra.ra_rank_forward_masked(q, ks, vs, o, lse, **kw)
        stream.synchronize()
        o_e, l_e = o.clone(), lse.clone()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            ra.ra_rank_forward_masked(q, ks, vs, o, lse, **kw)
        for i in range(3):
            o.fill_(float("nan"))
            lse.fill_(float("nan"))
            g.replay()
            stream.synchronize()
            say("masked graph replay", i)
            assert torch.equal(o, o_e) and torch.equal(lse, l_e)
    torch.cuda.synchronize()
    o_ref, l_ref = masked_reference(case, 1, 0, cu)
    assert_close(o_e.cpu().numpy(), l_e.cpu().numpy(), o_ref, l_ref, "bf16", "packed graph rank 1")
