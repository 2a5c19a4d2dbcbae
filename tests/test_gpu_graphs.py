"""The rank drivers under HIP graph capture: the library allocates nothing,
never synchronizes and records no memset, so a caller can capture a whole
ring (forward or backward) and replay it.  Each replay, with eager work of
the program in between, must give the eager call's bits.  GPU tests."""
import numpy as np
import pytest

import seeded_inputs as si
from ra_testlib import RankCase, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return ra


CASES = [
    # (label, dtype, B, Hq, Hkv, D, S, P, order, causal, rank)
    ("bf16_zigzag_p4", "bf16", 1, 8, 2, 128, 2048, 4, "zigzag", True, 2),
    ("f32_contig_p4", "f32", 1, 2, 2, 64, 512, 4, "contiguous", True, 3),
]


def _inputs(ra, case, rank):
    spans = ra.rank_spans(case.order, case.S, case.P, rank)
    q = to_device(case.q_rows(spans), case.dtype)
    do = to_device(si.tokens(case.seed_id, si.TENSOR_DO, case.B, case.S, case.Hq, case.D, spans, case.dtype),
                   case.dtype)
    ks, vs = case.device_shards(ra)
    return q, do, ks, vs


@pytest.mark.parametrize("cfg", CASES, ids=[c[0] for c in CASES])
def test_forward_graph_replays_match_eager(ra, cfg):
    import torch
    label, dtype, B, Hq, Hkv, D, S, P, order, causal, rank = cfg
    case = RankCase(900 + len(label), dtype, B, Hq, Hkv, D, S, P, order, causal)
    q, _, ks, vs = _inputs(ra, case, rank)
    s_loc = S // P
    kw = dict(S=S, P=P, rank=rank, order=order, causal=causal, scale=case.scale)
    o_e = torch.empty((B, s_loc, Hq, D), device="cuda")
    l_e = torch.empty((B, s_loc, Hq), device="cuda")
    ra.ra_rank_forward(q, ks, vs, o_e, l_e, **kw)
    torch.cuda.synchronize()

    o = torch.empty_like(o_e)
    lse = torch.empty_like(l_e)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        ra.ra_rank_forward(q, ks, vs, o, lse, stream=stream, **kw)
    torch.cuda.synchronize()
    for i in range(3):
        o.fill_(float("nan"))              # eager work between the replays
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(label, "forward replay", i)
        assert torch.equal(o, o_e) and torch.equal(lse, l_e)
    case.release()


@pytest.mark.parametrize("cfg", CASES, ids=[c[0] for c in CASES])
def test_backward_graph_replays_match_eager(ra, cfg):
    import torch
    label, dtype, B, Hq, Hkv, D, S, P, order, causal, rank = cfg
    case = RankCase(920 + len(label), dtype, B, Hq, Hkv, D, S, P, order, causal)
    q, do, ks, vs = _inputs(ra, case, rank)
    s_loc = S // P
    kw = dict(S=S, P=P, rank=rank, order=order, causal=causal, scale=case.scale)
    o = torch.empty((B, s_loc, Hq, D), device="cuda")
    lse = torch.empty((B, s_loc, Hq), device="cuda")
    ra.ra_rank_forward(q, ks, vs, o, lse, **kw)
    shard = (P, B, s_loc, Hkv, D)
    dq_e = torch.empty_like(o)
    dk_e, dv_e = torch.zeros(shard, device="cuda"), torch.zeros(shard, device="cuda")
    delta = torch.empty_like(lse)
    ra.ra_rank_backward(q, ks, vs, o, lse, do, dq_e, dk_e, dv_e, delta, **kw)
    torch.cuda.synchronize()

    dq = torch.empty_like(o)
    dk, dv = torch.zeros(shard, device="cuda"), torch.zeros(shard, device="cuda")
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        ra.ra_rank_backward(q, ks, vs, o, lse, do, dq, dk, dv, delta, stream=stream, **kw)
    torch.cuda.synchronize()
    for i in range(3):
        dq.fill_(float("nan"))             # dQ is written; dK and dV are added to
        dk.zero_()
        dv.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        say(label, "backward replay", i)
        assert torch.equal(dq, dq_e) and torch.equal(dk, dk_e) and torch.equal(dv, dv_e)
    case.release()
