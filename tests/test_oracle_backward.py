"""Pins of the backward oracle (gradients of the attention definition)
against things other than its own formulas: central finite differences of
the forward definition, closed forms and conservation laws."""
import numpy as np
import pytest

from oracle import attention as oa
from oracle import attention_backward as ob
from oracle import index_maps as im


def _loss_fn(dO, causal, scale, window=0, cu=None):
    def loss(Q, K, V):
        pos_q = np.arange(Q.shape[1])
        pos_k = np.arange(K.shape[1])
        o, _ = oa.attention_rows(Q, pos_q, K, V, pos_k, causal, scale, window=window, cu_seqlens=cu)
        return float((o * dO).sum())
    return loss


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (3, 1)])
def test_gradients_match_finite_differences(causal, Hq, Hkv):
    rng = np.random.default_rng(7 + Hq + 10 * causal)
    B, S, D = 2, 6, 3
    Q = rng.standard_normal((B, S, Hq, D))
    K = rng.standard_normal((B, S, Hkv, D))
    V = rng.standard_normal((B, S, Hkv, D))
    dO = rng.standard_normal((B, S, Hq, D))
    scale = 0.8
    dQ, dK, dV = ob.attention_grads(Q, K, V, dO, causal, scale)
    loss = _loss_fn(dO, causal, scale)
    eps = 1e-6
    for which, X, dX in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            args = {"Q": Q, "K": K, "V": V}
            xp, xm = X.copy(), X.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num[idx] = (loss(**{**args, which: xp}) - loss(**{**args, which: xm})) / (2 * eps)
        assert np.abs(num - dX).max() < 1e-7, which


def test_single_key_closed_form():
    """One key: every row's softmax is 1, so dV_0 = sum of dO over the rows and
    heads of its group and dQ = dK = 0."""
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((1, 1, 4, 5))
    K = rng.standard_normal((1, 1, 2, 5))
    V = rng.standard_normal((1, 1, 2, 5))
    dO = rng.standard_normal((1, 1, 4, 5))
    dQ, dK, dV = ob.attention_grads(Q, K, V, dO, True, 0.5)
    assert np.abs(dQ).max() < 1e-15 and np.abs(dK).max() < 1e-15
    np.testing.assert_allclose(dV[0, 0, 0], dO[0, 0, 0] + dO[0, 0, 1], rtol=0, atol=1e-15)
    np.testing.assert_allclose(dV[0, 0, 1], dO[0, 0, 2] + dO[0, 0, 3], rtol=0, atol=1e-15)


@pytest.mark.parametrize("causal", [True, False])
def test_conservation_laws(causal):
    """Each row's weights sum to 1 and its dS to 0, so summed over all keys
    dV equals the sum of dO over the group's rows and dK sums to zero."""
    rng = np.random.default_rng(11)
    B, S, Hq, Hkv, D = 2, 40, 4, 2, 8
    Q, dO = rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, S, Hq, D))
    K, V = rng.standard_normal((B, S, Hkv, D)), rng.standard_normal((B, S, Hkv, D))
    _, dK, dV = ob.attention_grads(Q, K, V, dO, causal, 0.3)
    for g in range(Hkv):
        np.testing.assert_allclose(dV[:, :, g].sum(axis=1), dO[:, :, 2 * g:2 * g + 2].sum(axis=(1, 2)),
                                   rtol=0, atol=1e-11)
        assert np.abs(dK[:, :, g].sum(axis=1)).max() < 1e-11


def test_rank_contributions_add_up_and_rows_are_independent():
    """dK, dV are sums over query rows: the contributions of the ranks' rows
    (zigzag ring of 4) add up to the whole; dQ of a row depends on that row only."""
    rng = np.random.default_rng(5)
    B, S, Hq, Hkv, D, P = 1, 32, 2, 1, 4, 4
    Q, dO = rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, S, Hq, D))
    K, V = rng.standard_normal((B, S, Hkv, D)), rng.standard_normal((B, S, Hkv, D))
    dQ, dK, dV = ob.attention_grads(Q, K, V, dO, True, 0.6)
    sk, sv = np.zeros_like(dK), np.zeros_like(dV)
    for r in range(P):
        pos = im.rank_positions(S, P, r, "zigzag")
        dq_r, dk_r, dv_r = ob.attention_grads(Q[:, pos], K, V, dO[:, pos], True, 0.6, qpos=pos)
        np.testing.assert_allclose(dq_r, dQ[:, pos], rtol=0, atol=1e-13)
        sk += dk_r
        sv += dv_r
    np.testing.assert_allclose(sk, dK, rtol=0, atol=1e-12)
    np.testing.assert_allclose(sv, dV, rtol=0, atol=1e-12)
    rows = np.array([3, 17, 30])
    np.testing.assert_allclose(ob.dq_rows(Q[:, rows], rows, K, V, dO[:, rows], True, 0.6), dQ[:, rows],
                               rtol=0, atol=1e-13)


@pytest.mark.parametrize("causal,window,cu", [(True, 3, None), (True, 0, [0, 2, 6]), (False, 0, [0, 4, 6]),
                                              (True, 2, [0, 3, 6])])
def test_masked_gradients_match_finite_differences(causal, window, cu):
    rng = np.random.default_rng(17 + window)
    B, S, Hq, Hkv, D = 1, 6, 2, 1, 3
    Q = rng.standard_normal((B, S, Hq, D))
    K = rng.standard_normal((B, S, Hkv, D))
    V = rng.standard_normal((B, S, Hkv, D))
    dO = rng.standard_normal((B, S, Hq, D))
    dQ, dK, dV = ob.attention_grads(Q, K, V, dO, causal, 0.9, window=window, cu_seqlens=cu)
    loss = _loss_fn(dO, causal, 0.9, window, cu)
    eps = 1e-6
    for which, X, dX in (("Q", Q, dQ), ("K", K, dK), ("V", V, dV)):
        num = np.zeros_like(X)
        for idx in np.ndindex(X.shape):
            args = {"Q": Q, "K": K, "V": V}
            xp, xm = X.copy(), X.copy()
            xp[idx] += eps
            xm[idx] -= eps
            num[idx] = (loss(**{**args, which: xp}) - loss(**{**args, which: xm})) / (2 * eps)
        assert np.abs(num - dX).max() < 1e-7, which
