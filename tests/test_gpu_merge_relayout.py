"""ra_lse_merge and ra_ulysses_relayout against the oracle.  GPU tests."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention as oa
from oracle import relayout as orl
from ra_testlib import say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return torch, ra


def _partials(rows, D, seed, empty_frac=0.15):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(2):
        o = rng.standard_normal((rows, D)).astype(np.float32)
        lse = (rng.standard_normal(rows) * 4).astype(np.float32)
        e = rng.random(rows) < empty_frac
        lse[e] = -np.inf
        o[e] = 0.0
        out.append((o, lse))
    return out


@pytest.mark.parametrize("rows,D", [(1, 128), (1000, 128), (4099, 64), (517, 7), (33, 1)])
def test_merge_matches_oracle(env, rows, D):
    torch, ra = env
    say("ra_lse_merge", rows, D)
    (oa_, la), (ob, lb) = _partials(rows, D, rows + D)
    # force every -inf combination
    if rows >= 4:
        la[0] = lb[0] = -np.inf
        oa_[0] = ob[0] = 0
        la[1] = -np.inf
        oa_[1] = 0
        lb[2] = -np.inf
        ob[2] = 0
    t = lambda x: torch.from_numpy(x).cuda()  # noqa: E731
    oo = torch.full((rows, D), float("nan"), device="cuda")
    lo = torch.full((rows,), float("nan"), device="cuda")
    ra.ra_lse_merge(t(oa_), t(la), t(ob), t(lb), oo, lo)
    torch.cuda.synchronize()
    ro, rl = oa.lse_merge(oa_.astype(np.float64), la.astype(np.float64), ob.astype(np.float64),
                          lb.astype(np.float64))
    got_o, got_l = oo.cpu().numpy(), lo.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert np.abs(got_o - ro).max() <= 1e-5
    assert np.abs(got_l[fin] - rl[fin]).max() <= 1e-5
    # identity passes the other side through bit-exactly
    a_id, b_id = np.isneginf(la), np.isneginf(lb)
    assert np.array_equal(got_o[a_id & ~b_id], ob[a_id & ~b_id])
    assert np.array_equal(got_l[a_id & ~b_id], lb[a_id & ~b_id])
    assert np.array_equal(got_o[b_id & ~a_id], oa_[b_id & ~a_id])
    assert (got_o[a_id & b_id] == 0).all()


def test_merge_full_size_every_row(env):
    """The merge at the size the benchmark times: the 131k rank's 262,144 rows
    of 128 (8192 local rows x 32 heads), every row against the oracle."""
    torch, ra = env
    rows, D = 262144, 128
    say("ra_lse_merge full size", rows, D)
    (oa_, la), (ob, lb) = _partials(rows, D, 77)
    t = lambda x: torch.from_numpy(x).cuda()  # noqa: E731
    oo = torch.full((rows, D), float("nan"), device="cuda")
    lo = torch.full((rows,), float("nan"), device="cuda")
    ra.ra_lse_merge(t(oa_), t(la), t(ob), t(lb), oo, lo)
    torch.cuda.synchronize()
    ro, rl = oa.lse_merge(oa_.astype(np.float64), la.astype(np.float64), ob.astype(np.float64),
                          lb.astype(np.float64))
    got_o, got_l = oo.cpu().numpy(), lo.cpu().numpy()
    assert np.array_equal(np.isneginf(got_l), np.isneginf(rl))
    fin = np.isfinite(rl)
    eo, el = float(np.abs(got_o - ro).max()), float(np.abs(got_l[fin] - rl[fin]).max())
    say(f"max|dO| {eo:.2e} max|dLSE| {el:.2e}")
    assert eo <= 1e-5 and el <= 1e-5
    a_id, b_id = np.isneginf(la), np.isneginf(lb)
    assert np.array_equal(got_o[a_id & ~b_id], ob[a_id & ~b_id])
    assert np.array_equal(got_o[b_id & ~a_id], oa_[b_id & ~a_id])


def test_merge_in_place(env):
    torch, ra = env
    (oa_, la), (ob, lb) = _partials(2048, 128, 3)
    ta, tla = torch.from_numpy(oa_).cuda(), torch.from_numpy(la).cuda()
    tb, tlb = torch.from_numpy(ob).cuda(), torch.from_numpy(lb).cuda()
    ra.ra_lse_merge(ta, tla, tb, tlb, ta, tla)   # out aliases a
    torch.cuda.synchronize()
    ro, rl = oa.lse_merge(oa_.astype(np.float64), la.astype(np.float64), ob.astype(np.float64),
                          lb.astype(np.float64))
    assert np.abs(ta.cpu().numpy() - ro).max() <= 1e-5
    fin = np.isfinite(rl)
    assert np.abs(tla.cpu().numpy()[fin] - rl[fin]).max() <= 1e-5


RELAYOUT = [
    # (B, s_loc, H, D, P_u, dtype)
    (1, 64, 16, 128, 8, np.uint16),
    (2, 100, 12, 8, 3, np.uint16),
    (1, 37, 6, 7, 3, np.uint8),     # 14-byte runs of odd-length elements
    (2, 50, 8, 5, 8, np.uint8),     # 5-byte runs: byte copies
    (1, 33, 4, 16, 1, np.float32),
    (3, 17, 16, 64, 16, np.float32),
    (1, 8, 4, 4, 2, np.uint64),
]


@pytest.mark.parametrize("case", RELAYOUT)
def test_relayout_bit_exact_and_round_trip(env, case):
    torch, ra = env
    B, s_loc, H, D, P_u, dt = case
    say("ra_ulysses_relayout", case)
    rng = np.random.default_rng(sum(case[:5]))
    x = rng.integers(0, np.iinfo(np.int64).max, (B, s_loc, H, D), dtype=np.int64).astype(dt)
    xt = torch.from_numpy(x.view(np.int8)).cuda()  # raw bytes
    want = orl.seq2head(x, P_u)
    out = torch.zeros(want.nbytes, dtype=torch.int8, device="cuda")
    eb = x.itemsize
    rc = ra.lib.ra_ulysses_relayout(ra.RA_SEQ2HEAD, eb, B, s_loc, H, D, P_u, ra._ptr(xt), ra._ptr(out),
                                    ra._stream(None))
    assert rc == 0, ra.ra_last_error()
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(dt).reshape(want.shape)
    assert np.array_equal(got, want)
    back = torch.zeros_like(xt)
    rc = ra.lib.ra_ulysses_relayout(ra.RA_HEAD2SEQ, eb, B, s_loc, H, D, P_u, ra._ptr(out), ra._ptr(back),
                                    ra._stream(None))
    assert rc == 0, ra.ra_last_error()
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy().view(dt).reshape(x.shape), x)
    assert np.array_equal(orl.head2seq(want), x)


def test_relayout_full_size_mha_shard(env):
    """The 16-head MHA shard of 8192 tokens, batch 2, regrouped for 8 destinations
    (bf16, the relayout the benchmark times)."""
    torch, ra = env
    B, s_loc, H, D, P_u = 2, 8192, 16, 128, 8
    say("ra_ulysses_relayout full size", (B, s_loc, H, D, P_u))
    x = si.tokens(4, si.TENSOR_Q, B, 65536, H, D, [(0, s_loc)], "bf16")
    xd = to_device(x, "bf16")
    out = torch.empty(P_u, B, s_loc, H // P_u, D, dtype=torch.bfloat16, device="cuda")
    ra.ra_ulysses_relayout(xd, out, P_u, ra.RA_SEQ2HEAD)
    back = torch.empty_like(xd)
    ra.ra_ulysses_relayout(out, back, P_u, ra.RA_HEAD2SEQ)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, orl.seq2head(x, P_u))
    assert torch.equal(back.view(torch.int16), xd.view(torch.int16))
