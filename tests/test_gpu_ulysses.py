"""The Ulysses path on one GPU: multi-tensor messages of the all-to-all
(ra_ulysses_pieces) bit-exact against the oracle, and the whole path (pack,
exchange, regroup, attention over all tokens of a head block, and back)
against the oracle's attention.  The exchange itself, which a real run does
with one collective, is a plain copy between the simulated ranks' buffers
here.  GPU tests."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention as oa
from oracle import relayout as rl
from ra_testlib import assert_close, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return ra


def _dev(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def _buf(nbytes):
    import torch
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda")


SHAPES = [
    # (label, P_u, B, s_loc, [(H, D, numpy dtype), ...])
    ("qkv_bf16_gqa", 4, 2, 64, [(8, 128, np.uint16), (4, 128, np.uint16), (4, 128, np.uint16)]),
    ("o_lse_f32", 4, 1, 96, [(8, 128, np.float32), (8, 1, np.float32)]),
    ("odd_bytes", 3, 2, 10, [(6, 3, np.float32), (3, 5, np.uint16), (3, 1, np.uint8)]),
    ("single", 1, 1, 33, [(2, 16, np.float32)]),
    ("mha_64k_shard", 8, 2, 8192, [(16, 128, np.uint16)] * 3),
]


@pytest.mark.parametrize("group", ["heads", "seq"])
@pytest.mark.parametrize("cfg", SHAPES, ids=[c[0] for c in SHAPES])
def test_pieces_bit_exact_both_directions(ra, cfg, group):
    label, P_u, B, s_loc, specs = cfg
    rng = np.random.default_rng(len(label) + 3)
    xs = []
    for H, D, dt in specs:
        if group == "seq":
            shape = (B, P_u * s_loc, H, D)
        else:
            shape = (B, s_loc, H, D)
        xs.append(rng.integers(0, 255, size=shape, dtype=np.uint8).view(np.uint8).astype(dt)
                  if dt == np.uint8 else rng.integers(0, 65535, size=shape).astype(dt) if dt == np.uint16
                  else rng.standard_normal(shape).astype(dt))
    say(label, group, [x.shape for x in xs])
    ref = rl.piece_bytes(rl.to_pieces(xs, P_u, group))
    dev = [_dev(x) for x in xs]
    pieces = _buf(ref.size)
    gid = ra.RA_GROUP_HEADS if group == "heads" else ra.RA_GROUP_SEQ
    ra.ra_ulysses_pieces(dev, pieces, P_u, to_pieces=True, group=gid)
    np.testing.assert_array_equal(pieces.cpu().numpy(), ref)
    outs = [d.clone().fill_(0) for d in dev]
    ra.ra_ulysses_pieces(outs, pieces, P_u, to_pieces=False, group=gid)
    for a, b in zip(outs, xs):
        np.testing.assert_array_equal(a.cpu().numpy(), b)


PATHS = [
    # (label, P_u, B, S, Hq, Hkv, causal)
    ("gqa_causal_pu4", 4, 2, 1024, 8, 4, True),
    ("mha_full_pu8", 8, 2, 2048, 16, 16, False),
    ("gqa_causal_pu2_ragged", 2, 1, 1200, 4, 2, True),
]


@pytest.mark.parametrize("cfg", PATHS, ids=[c[0] for c in PATHS])
def test_ulysses_attention_path(ra, cfg):
    """Every simulated rank: fused Q/K/V pack, exchange, regroup into all
    tokens of a head block, attention, fused O/LSE back, exchange, unpack;
    each rank's output equals the definition for its tokens and all heads."""
    import torch
    label, P_u, B, S, Hq, Hkv, causal = cfg
    D, seed = 128, 500 + len(label)
    s_loc, hq, hk = S // P_u, Hq // P_u, Hkv // P_u
    scale = D ** -0.5
    Qg = si.tokens(seed, si.TENSOR_Q, B, S, Hq, D, [(0, S)], "bf16")
    Kg = si.tokens(seed, si.TENSOR_K, B, S, Hkv, D, [(0, S)], "bf16")
    Vg = si.tokens(seed, si.TENSOR_V, B, S, Hkv, D, [(0, S)], "bf16")
    H, SEQ = ra.RA_GROUP_HEADS, ra.RA_GROUP_SEQ
    piece_in = B * s_loc * (hq + 2 * hk) * D * 2
    sends = []
    for u in range(P_u):
        sh = [to_device(X[:, u * s_loc:(u + 1) * s_loc], "bf16") for X in (Qg, Kg, Vg)]
        buf = _buf(P_u * piece_in)
        ra.ra_ulysses_pieces(sh, buf, P_u, to_pieces=True, group=H)
        sends.append(buf.view(P_u, piece_in))
    piece_out = B * s_loc * hq * (D + 1) * 4
    back = []
    for j in range(P_u):
        recv = torch.stack([sends[u][j] for u in range(P_u)])      # the all-to-all
        q = torch.empty((B, S, hq, D), dtype=torch.bfloat16, device="cuda")
        k = torch.empty((B, S, hk, D), dtype=torch.bfloat16, device="cuda")
        v = torch.empty_like(k)
        ra.ra_ulysses_pieces([q, k, v], recv, P_u, to_pieces=False, group=SEQ)
        o = torch.empty((B, S, hq, D), device="cuda")
        lse = torch.empty((B, S, hq, 1), device="cuda")
        ra.ra_step(q, k, v, o, lse.view(B, S, hq), [(0, S)], [(0, S)], causal=causal, scale=scale)
        buf = _buf(P_u * piece_out)
        ra.ra_ulysses_pieces([o, lse], buf, P_u, to_pieces=True, group=SEQ)
        back.append(buf.view(P_u, piece_out))
    for u in range(P_u):
        recv = torch.stack([back[j][u] for j in range(P_u)])        # the way back
        o_u = torch.empty((B, s_loc, Hq, D), device="cuda")
        lse_u = torch.empty((B, s_loc, Hq, 1), device="cuda")
        ra.ra_ulysses_pieces([o_u, lse_u], recv, P_u, to_pieces=False, group=H)
        pos = np.arange(u * s_loc, (u + 1) * s_loc)
        o_ref, l_ref = oa.attention_rows(si.to_f64(Qg[:, pos], "bf16"), pos, si.to_f64(Kg, "bf16"),
                                         si.to_f64(Vg, "bf16"), np.arange(S), causal, scale)
        assert_close(o_u.cpu().numpy(), lse_u.cpu().numpy()[..., 0], o_ref, l_ref, "bf16", f"{label} rank {u}")
