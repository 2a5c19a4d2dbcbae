"""ra_rank_backward_noalloc (the backward with the library's own device
scratch for its delta workspace) against ra_rank_backward (the same kernels
with a caller-provided workspace), through the C ABI binding.  The backward
kernels add no partial sums with atomics, so the two must agree bit for bit.
Two calls in a row, the second on a smaller ring, show that the shared
scratch carries nothing from one call to the next.  GPU test."""
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


def _inputs(ra, case, rank):
    import torch
    o, lse = case.run_rank(ra, rank, poison=False)
    spans = ra.rank_spans(case.order, case.S, case.P, rank)
    q = to_device(case.q_rows(spans), case.dtype)
    do = to_device(si.tokens(case.seed_id, si.TENSOR_DO, case.B, case.S, case.Hq, case.D, spans, case.dtype),
                   case.dtype)
    ks, vs = case.device_shards(ra)
    return q, ks, vs, torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(), do


def _grads(ra, case, rank, args, noalloc):
    """dq, dk, dv of rank `rank`, from the workspace call or the scratch call."""
    import torch
    q, ks, vs, o, lse, do = args
    s_loc = case.S // case.P
    kw = dict(S=case.S, P=case.P, rank=rank, order=case.order, causal=case.causal, scale=case.scale)
    dq = torch.full((case.B, s_loc, case.Hq, case.D), float("nan"), device="cuda")
    dk = torch.zeros((case.P, case.B, s_loc, case.Hkv, case.D), device="cuda")
    dv = torch.zeros_like(dk)
    if noalloc:
        ra.ra_rank_backward_noalloc(q, ks, vs, o, lse, do, dq, dk, dv, **kw)
    else:
        delta = torch.empty((case.B, s_loc, case.Hq), device="cuda")
        ra.ra_rank_backward(q, ks, vs, o, lse, do, dq, dk, dv, delta, **kw)
    return dq, dk, dv


def test_noalloc_matches_workspace_backward_twice(ra):
    """The workspace call on two rings first, then the scratch call twice in
    a row (the larger ring, then the smaller one), each against the
    workspace call's gradients on the same inputs."""
    import torch
    cases = [
        # (label, B, Hq, Hkv, S, P, order, causal, rank): a GQA zigzag ring
        # whose backward takes the fused dK/dV kernel, then a smaller one
        ("gqa32x8_zigzag_b8", 8, 32, 8, 2048, 2, "zigzag", True, 0),
        ("mqa_contig_small", 1, 4, 1, 512, 4, "contiguous", True, 2),
    ]
    runs = []
    for label, B, Hq, Hkv, S, P, order, causal, rank in cases:
        case = RankCase(970 + len(label), "bf16", B, Hq, Hkv, 128, S, P, order, causal)
        args = _inputs(ra, case, rank)
        say("workspace backward", label, "rank", rank)
        ref = _grads(ra, case, rank, args, False)
        runs.append((label, case, rank, args, ref, B * (S // P) * Hq))
    assert runs[1][5] < runs[0][5]
    got = []
    for label, case, rank, args, _, _ in runs:
        say("noalloc backward", label, "rank", rank)
        got.append(_grads(ra, case, rank, args, True))
    torch.cuda.synchronize()
    for (label, case, _, _, ref, _), g in zip(runs, got):
        for name, a, b in zip(("dq", "dk", "dv"), g, ref):
            a, b = a.cpu().numpy(), b.cpu().numpy()
            assert np.isfinite(b).all(), (label, name)
            np.testing.assert_array_equal(a, b, err_msg=f"{label} {name}")
        case.release()
