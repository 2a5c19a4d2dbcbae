"""ra_step (one ring step, fused merge) against the oracle, element by element.
GPU tests: they call the HIP kernels through the C ABI."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention as oa
from ra_testlib import TOL, assert_close, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return torch, ra


def _span_pos(spans):
    return np.concatenate([np.arange(a, a + n) for a, n in spans]) if spans else np.zeros(0, np.int64)


def make_step(dtype, B, Hq, Hkv, D, qspans, kspans, seed, k_scale=1.0):
    S = max([a + n for a, n in list(qspans) + list(kspans)] + [1])
    q = si.tokens(seed, si.TENSOR_Q, B, S, Hq, D, qspans, dtype)
    k = si.tokens(seed, si.TENSOR_K, B, S, Hkv, D, kspans, dtype, scale=k_scale)
    v = si.tokens(seed, si.TENSOR_V, B, S, Hkv, D, kspans, dtype)
    return q, k, v


def run_step(env, dtype, q, k, v, qspans, kspans, causal, accum=False, o0=None, lse0=None):
    torch, ra = env
    B, Sq, Hq, D = q.shape
    qd, kd, vd = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    if o0 is None:
        o = torch.full((B, Sq, Hq, D), float("nan"), device="cuda")
        lse = torch.full((B, Sq, Hq), float("nan"), device="cuda")
    else:
        o = torch.from_numpy(o0.astype(np.float32)).cuda()
        lse = torch.from_numpy(lse0.astype(np.float32)).cuda()
    ra.ra_step(qd, kd, vd, o, lse, qspans, kspans, causal=causal, scale=D ** -0.5, accum=accum)
    torch.cuda.synchronize()
    return o.cpu().numpy(), lse.cpu().numpy()


def oracle_partial(dtype, q, k, v, qspans, kspans, causal):
    f = lambda x: si.to_f64(x, dtype)  # noqa: E731
    D = q.shape[-1]
    return oa.attention_rows(f(q), _span_pos(qspans), f(k), f(v), _span_pos(kspans), causal, D ** -0.5)


CASES = {
    # name: (qspans, kspans, causal)
    "full": ([(1024, 256)], [(0, 512)], True),
    "diag": ([(512, 256)], [(512, 256)], True),
    "skip": ([(0, 256)], [(512, 256)], True),
    "zigzag_step0": ([(0, 128), (896, 128)], [(0, 128), (896, 128)], True),
    "zigzag_later": ([(128, 128), (768, 128)], [(0, 128), (896, 128)], True),
    "ragged_causal": ([(100, 77), (500, 131)], [(37, 203), (400, 91)], True),
    "ragged_full": ([(5, 199)], [(300, 70), (11, 3)], False),
    "one_key": ([(64, 130)], [(64, 1)], True),
}


@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("bf16", 128), ("bf16", 64)])
@pytest.mark.parametrize("name", list(CASES))
def test_step_init_and_accum(env, dtype, D, name):
    qspans, kspans, causal = CASES[name]
    B, Hq, Hkv = 2, 4, 2
    say("ra_step", name, dtype, f"D={D}", f"B={B} Hq={Hq} Hkv={Hkv}", qspans, kspans)
    q, k, v = make_step(dtype, B, Hq, Hkv, D, qspans, kspans, seed=100 + D)
    o_ref, l_ref = oracle_partial(dtype, q, k, v, qspans, kspans, causal)
    o, lse = run_step(env, dtype, q, k, v, qspans, kspans, causal)
    assert not np.isnan(o).any() and not np.isnan(lse).any(), "INIT left rows unwritten"
    empty = np.isneginf(l_ref)
    assert np.array_equal(np.isneginf(lse), empty)
    assert (o[empty] == 0).all()
    assert_close(o, lse, o_ref, l_ref, dtype, f"INIT {name}")

    # ACCUM onto a running state that is itself a partial over other keys
    k2spans = [(7, 150)]
    _, k2, v2 = make_step(dtype, B, Hq, Hkv, D, qspans, k2spans, seed=200 + D)
    run_o, run_l = oracle_partial(dtype, q, k2, v2, qspans, k2spans, causal)
    run_o32, run_l32 = run_o.astype(np.float32), run_l.astype(np.float32)
    o2, l2 = run_step(env, dtype, q, k, v, qspans, kspans, causal, accum=True, o0=run_o32, lse0=run_l32)
    mo, ml = oa.lse_merge(run_o32.astype(np.float64), run_l32.astype(np.float64), o_ref, l_ref)
    assert_close(o2, l2, mo, ml, dtype, f"ACCUM {name}")
    # rows whose partial is empty are left bit-identical
    assert np.array_equal(o2[empty], run_o32[empty])
    assert np.array_equal(l2[empty], run_l32[empty])
    # rows whose running state is the identity receive the partial bit-exactly
    ident = np.isneginf(run_l32) & ~empty
    if ident.any():
        assert np.array_equal(o2[ident], o[ident]) and np.array_equal(l2[ident], lse[ident])


@pytest.mark.parametrize("Hq,Hkv", [(8, 8), (8, 4), (8, 2), (8, 1), (32, 8)])
def test_step_gqa_ratios(env, Hq, Hkv):
    qspans, kspans = [(300, 260)], [(0, 520)]
    for dtype in ("bf16", "f32"):
        say("ra_step GQA", dtype, Hq, Hkv)
        q, k, v = make_step(dtype, 1, Hq, Hkv, 128, qspans, kspans, seed=Hq * 10 + Hkv)
        o_ref, l_ref = oracle_partial(dtype, q, k, v, qspans, kspans, True)
        o, lse = run_step(env, dtype, q, k, v, qspans, kspans, True)
        assert_close(o, lse, o_ref, l_ref, dtype, f"GQA {Hq}/{Hkv} {dtype}")


def test_step_sharp_softmax_and_large_scores(env):
    """Scores spread over a wide range move the running maximum many times."""
    qspans, kspans = [(2048, 256)], [(0, 2304)]
    q, k, v = make_step("f32", 1, 2, 1, 64, qspans, kspans, seed=9, k_scale=8.0)
    o_ref, l_ref = oracle_partial("f32", q, k, v, qspans, kspans, True)
    o, lse = run_step(env, "f32", q, k, v, qspans, kspans, True)
    say("sharp f32: max|O-ref| =", float(np.abs(o - o_ref).max()))
    assert np.abs(o - o_ref).max() <= TOL["f32"]
    assert np.abs(lse - l_ref).max() <= 1e-5 * max(1.0, float(np.abs(l_ref).max()))


def test_step_empty_key_block(env):
    torch, ra = env
    qspans = [(0, 130)]
    q, _, _ = make_step("bf16", 1, 2, 2, 128, qspans, [(0, 1)], seed=1)
    k = np.zeros((1, 0, 2, 128), np.uint16)
    o, lse = run_step(env, "bf16", q, k, k.copy(), qspans, [(0, 0)], True)
    assert (o == 0).all() and np.isneginf(lse).all()
    run_o = np.random.default_rng(0).standard_normal(o.shape).astype(np.float32)
    run_l = np.random.default_rng(1).standard_normal(lse.shape).astype(np.float32)
    o2, l2 = run_step(env, "bf16", q, k, k.copy(), qspans, [(0, 0)], True, accum=True, o0=run_o, lse0=run_l)
    assert np.array_equal(o2, run_o) and np.array_equal(l2, run_l)


def test_step_is_deterministic(env):
    qspans, kspans = [(0, 384), (1000, 128)], [(0, 512), (900, 200)]
    q, k, v = make_step("bf16", 1, 8, 2, 128, qspans, kspans, seed=5)
    a = run_step(env, "bf16", q, k, v, qspans, kspans, True)
    b = run_step(env, "bf16", q, k, v, qspans, kspans, True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_step_error_leaves_outputs_untouched(env):
    torch, ra = env
    q = torch.zeros(1, 128, 6, 128, device="cuda", dtype=torch.bfloat16)
    k = torch.zeros(1, 128, 4, 128, device="cuda", dtype=torch.bfloat16)  # 6 % 4 != 0
    o = torch.full((1, 128, 6, 128), float("nan"), device="cuda")
    lse = torch.full((1, 128, 6), float("nan"), device="cuda")
    with pytest.raises(ra.RaError) as e:
        ra.ra_step(q, k, k, o, lse, [(0, 128)], [(0, 128)], causal=True)
    assert e.value.status == ra.RA_E_INVAL
    torch.cuda.synchronize()
    assert torch.isnan(o).all() and torch.isnan(lse).all()
