"""Pins of the CPU oracle against things other than itself: hand-derived
fixtures, brute-force enumeration, closed forms, a library routine and exact
invariants.  CPU only."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import attention as oa
from oracle import index_maps as im
from oracle import relayout as orl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# brute force: pure-Python loops, independent of numpy's vector code paths


def brute_attention(q, k, v, qpos, kpos, causal, scale):
    """Triple loops with math.exp/log; returns O and LSE as nested lists."""
    B, Nq, Hq, D = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Nq, Hq, D))
    L = np.full((B, Nq, Hq), -math.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // G
            for i in range(Nq):
                scores = []
                for j in range(k.shape[1]):
                    if causal and kpos[j] > qpos[i]:
                        continue
                    s = 0.0
                    for d in range(D):
                        s += float(q[b, i, h, d]) * float(k[b, j, g, d])
                    scores.append((scale * s, j))
                if not scores:
                    continue
                m = max(s for s, _ in scores)
                tot = sum(math.exp(s - m) for s, _ in scores)
                lse = m + math.log(tot)
                L[b, i, h] = lse
                for d in range(D):
                    O[b, i, h, d] = sum(math.exp(s - lse) * float(v[b, j, g, d])
                                        for s, j in scores)
    return O, L


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("order", im.ORDERS)
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("P", [1, 2, 4])
@pytest.mark.parametrize("Hq,Hkv", [(2, 2), (4, 2), (4, 1)])
def test_definition_matches_brute_force(order, causal, P, Hq, Hkv):
    S, D, B = 16, 8, 2
    seed = hash((order, causal, P, Hq, Hkv)) % 2**32
    Q, K, V = (_rand((B, S, Hq if i == 0 else Hkv, D), seed + i) for i in range(3))
    scale = 1 / math.sqrt(D)
    for r in range(P):
        pos = im.rank_positions(S, P, r, order)
        o, l = oa.rank_reference(Q, K, V, S, P, r, order, causal, scale)
        ob, lb = brute_attention(Q[:, pos], K, V, pos, np.arange(S), causal, scale)
        np.testing.assert_allclose(o, ob, rtol=0, atol=1e-12)
        np.testing.assert_allclose(l, lb, rtol=0, atol=1e-12)


def test_single_rank_matches_library_sdpa():
    """P = 1 reduces to ordinary attention: CPU torch SDPA in float64."""
    torch = pytest.importorskip("torch")
    B, S, Hq, Hkv, D = 2, 96, 8, 2, 32
    Q, K, V = (_rand((B, S, h, D), 7 + i) for i, h in enumerate((Hq, Hkv, Hkv)))
    scale = 1 / math.sqrt(D)
    for causal in (True, False):
        o, lse = oa.rank_reference(Q, K, V, S, 1, 0, "contiguous", causal, scale)
        tq = torch.from_numpy(Q).permute(0, 2, 1, 3)
        tk = torch.from_numpy(K).permute(0, 2, 1, 3)
        tv = torch.from_numpy(V).permute(0, 2, 1, 3)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=scale, enable_gqa=True)
        np.testing.assert_allclose(o, ref.permute(0, 2, 1, 3).numpy(), atol=1e-12)
        # LSE via the library's logsumexp over explicitly masked scores
        kk = np.repeat(K, Hq // Hkv, axis=2)
        s = scale * np.einsum("bihd,bjhd->bhij", Q, kk)
        if causal:
            s = np.where(np.tril(np.ones((S, S), bool))[None, None], s, -np.inf)
        ref_lse = torch.logsumexp(torch.from_numpy(s), dim=-1).permute(0, 2, 1).numpy()
        np.testing.assert_allclose(lse, ref_lse, atol=1e-12)


def test_gqa_equals_mha_with_repeated_heads():
    """Consecutive grouping: Hkv heads shared by Hq/Hkv query heads each equals
    MHA on K/V heads repeated in place."""
    B, S, Hq, Hkv, D = 1, 32, 8, 2, 16
    Q, K, V = (_rand((B, S, h, D), 70 + i) for i, h in enumerate((Hq, Hkv, Hkv)))
    o1, l1 = oa.rank_reference(Q, K, V, S, 2, 1, "zigzag", True, 0.3)
    o2, l2 = oa.rank_reference(Q, np.repeat(K, 4, axis=2), np.repeat(V, 4, axis=2),
                               S, 2, 1, "zigzag", True, 0.3)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


# ----------------------------------------------------------------------------
# closed forms


@pytest.mark.parametrize("causal", [True, False])
def test_zero_queries_give_uniform_weights(causal):
    B, S, H, D, P = 1, 64, 2, 8, 4
    Q = np.zeros((B, S, H, D))
    K, V = _rand((B, S, H, D), 1), _rand((B, S, H, D), 2)
    for r in range(P):
        pos = im.rank_positions(S, P, r, "zigzag")
        o, l = oa.rank_reference(Q, K, V, S, P, r, "zigzag", causal, 0.5)
        for i, t in enumerate(pos):
            n = t + 1 if causal else S
            np.testing.assert_allclose(l[0, i], math.log(n), atol=1e-12)
            np.testing.assert_allclose(o[0, i], V[0, :n].mean(axis=0), atol=1e-12)


def test_constant_values_pass_through():
    B, S, H, D = 1, 32, 2, 4
    Q, K = _rand((B, S, H, D), 3) * 3, _rand((B, S, H, D), 4) * 3
    vrow = np.array([0.5, -2.0, 3.25, 7.0])
    V = np.broadcast_to(vrow, (B, S, H, D)).copy()
    o, _ = oa.rank_reference(Q, K, V, S, 2, 0, "zigzag", True, 1.0)
    np.testing.assert_allclose(o, np.broadcast_to(vrow, o.shape), atol=1e-12)


def test_first_row_causal():
    B, S, H, D = 1, 16, 1, 8
    Q, K, V = (_rand((B, S, H, D), 10 + i) for i in range(3))
    o, l = oa.rank_reference(Q, K, V, S, 1, 0, "contiguous", True, 0.25)
    np.testing.assert_allclose(o[0, 0, 0], V[0, 0, 0], atol=1e-15)
    np.testing.assert_allclose(l[0, 0, 0], 0.25 * Q[0, 0, 0] @ K[0, 0, 0], atol=1e-15)


def test_golden_rational_attention():
    g = _golden("attention_rational.json")
    w = np.array(g["w"], dtype=np.float64)
    n = w.size
    Q = np.ones((1, n, 1, 1))
    K = np.log(w).reshape(1, n, 1, 1)
    V = np.array(g["v"], dtype=np.float64).reshape(1, n, 1, 1)
    o, l = oa.rank_reference(Q, K, V, n, 1, 0, "contiguous", True, 1.0)
    for t in range(n):
        num, den = g["O"][t]
        assert abs(o[0, t, 0, 0] - num / den) < 1e-12
        assert abs(l[0, t, 0] - math.log(g["LSE_of"][t])) < 1e-12
    # exact rational check of the derivation itself
    for t in range(n):
        frac = sum(Fraction(int(a)) * b for a, b in zip(w[:t + 1], g["v"][:t + 1])) / int(w[:t + 1].sum())
        assert frac == Fraction(*g["O"][t])


# ----------------------------------------------------------------------------
# LSE merge


def test_golden_merge():
    g = _golden("merge_worked.json")
    o, l = oa.lse_merge(np.array([g["o_a"]], float), np.array([math.log(g["lse_a_of"])]),
                        np.array([g["o_b"]], float), np.array([math.log(g["lse_b_of"])]))
    np.testing.assert_allclose(o[0], [a / b for a, b in g["o"]], atol=1e-15)
    np.testing.assert_allclose(l[0], math.log(g["lse_of"]), atol=1e-15)


def _partials(n, D, seed):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        o = rng.standard_normal((n, D))
        lse = rng.standard_normal(n) * 3
        lse[rng.random(n) < 0.2] = -np.inf
        o[np.isneginf(lse)] = 0.0
        out.append((o, lse))
    return out


def test_merge_identity_is_exact():
    (o, l), _, _ = _partials(64, 8, 0)
    io, il = oa.identity(o.shape)
    for a, b in (((io, il), (o, l)), ((o, l), (io, il))):
        mo, ml = oa.lse_merge(*a, *b)
        np.testing.assert_array_equal(mo, o)
        np.testing.assert_array_equal(ml, l)
    mo, ml = oa.lse_merge(io, il, io, il)
    np.testing.assert_array_equal(mo, io)
    np.testing.assert_array_equal(ml, il)


def test_merge_commutative_associative_and_doubling():
    a, b, c = _partials(128, 8, 1)
    ab = oa.lse_merge(*a, *b)
    ba = oa.lse_merge(*b, *a)
    np.testing.assert_allclose(ab[0], ba[0], atol=1e-13)
    np.testing.assert_array_equal(np.isneginf(ab[1]), np.isneginf(ba[1]))
    np.testing.assert_allclose(ab[1], ba[1], atol=1e-13)
    left = oa.lse_merge(*ab, *c)
    right = oa.lse_merge(*a, *oa.lse_merge(*b, *c))
    np.testing.assert_allclose(left[0], right[0], atol=1e-12)
    np.testing.assert_allclose(left[1], right[1], atol=1e-12)
    aa = oa.lse_merge(*a, *a)
    np.testing.assert_allclose(aa[0], a[0], atol=1e-14)
    np.testing.assert_allclose(aa[1], a[1] + math.log(2), atol=1e-14)


def test_merge_is_softmax_over_union():
    """Two partials over disjoint key sets merge to the attention over the union
    (the DeDLOC Step 4 check, in float64)."""
    B, N, H, D = 1, 8, 2, 16
    rng = np.random.default_rng(5)
    q = rng.standard_normal((B, N, H, D))
    k = rng.standard_normal((B, 2 * N, H, D))
    v = rng.standard_normal((B, 2 * N, H, D))
    pos = np.arange(2 * N)
    full = oa.attention_rows(q, pos[:N] + 100, k, v, pos, False, 0.125)
    p0 = oa.attention_rows(q, pos[:N] + 100, k[:, :N], v[:, :N], pos[:N], False, 0.125)
    p1 = oa.attention_rows(q, pos[:N] + 100, k[:, N:], v[:, N:], pos[N:], False, 0.125)
    m = oa.lse_merge(*p0, *p1)
    np.testing.assert_allclose(m[0], full[0], atol=1e-13)
    np.testing.assert_allclose(m[1], full[1], atol=1e-13)


# ----------------------------------------------------------------------------
# ring decomposition = definition


def _shards(X, S, P, order):
    return np.stack([X[:, im.rank_positions(S, P, p, order)] for p in range(P)])


@pytest.mark.parametrize("order", im.ORDERS)
@pytest.mark.parametrize("causal", [True, False])
def test_ring_equals_definition_all_step_orders_P4(order, causal):
    S, P, B, Hq, Hkv, D = 32, 4, 1, 4, 2, 8
    Q, K, V = (_rand((B, S, h, D), 20 + i) for i, h in enumerate((Hq, Hkv, Hkv)))
    ks, vs = _shards(K, S, P, order), _shards(V, S, P, order)
    for r in range(P):
        ref = oa.rank_reference(Q, K, V, S, P, r, order, causal, 0.3)
        ql = Q[:, im.rank_positions(S, P, r, order)]
        for perm in itertools.permutations(range(P)):
            o, l = oa.ring_forward(ql, ks, vs, S, P, r, order, causal, 0.3, steps=perm)
            np.testing.assert_allclose(o, ref[0], atol=1e-12)
            np.testing.assert_allclose(l, ref[1], atol=1e-12)


@pytest.mark.parametrize("P", [8, 16, 32])
@pytest.mark.parametrize("order", im.ORDERS)
def test_ring_equals_definition_random_orders(P, order):
    S = 4 * P
    B, Hq, Hkv, D = 1, 2, 1, 4
    Q, K, V = (_rand((B, S, h, D), 30 + P + i) for i, h in enumerate((Hq, Hkv, Hkv)))
    ks, vs = _shards(K, S, P, order), _shards(V, S, P, order)
    rng = np.random.default_rng(P)
    for r in (0, P // 2, P - 1):
        ref = oa.rank_reference(Q, K, V, S, P, r, order, True, 0.5)
        ql = Q[:, im.rank_positions(S, P, r, order)]
        for steps in (None, rng.permutation(P)):
            o, l = oa.ring_forward(ql, ks, vs, S, P, r, order, True, 0.5, steps=steps)
            np.testing.assert_allclose(o, ref[0], atol=1e-12)
            np.testing.assert_allclose(l, ref[1], atol=1e-12)


# ----------------------------------------------------------------------------
# index maps


def test_golden_index_maps():
    g = _golden("index_maps_small.json")
    for key, ranks in g["zigzag"].items():
        S, P = (int(x[1:]) for x in key.split("_"))
        for r, pos in enumerate(ranks):
            assert im.rank_positions(S, P, r, "zigzag").tolist() == pos
    for key, ranks in g["contiguous"].items():
        S, P = (int(x[1:]) for x in key.split("_"))
        for r, pos in enumerate(ranks):
            assert im.rank_positions(S, P, r, "contiguous").tolist() == pos
    for r, srcs in enumerate(g["ring_sources_P4"]):
        assert [im.ring_source(r, s, 4) for s in range(4)] == srcs
    for rk, steps in g["zigzag_S16_P2_classes"].items():
        r = int(rk[4:])
        for sk, table in steps.items():
            assert im.step_pair_classes(16, 2, r, int(sk[4:]), "zigzag", True) == table


@pytest.mark.parametrize("order", im.ORDERS)
@pytest.mark.parametrize("S,P", [(64, 4), (128, 8), (512, 16), (96, 3)])
def test_maps_are_permutations_and_invert(order, S, P):
    allpos = np.concatenate([im.rank_positions(S, P, r, order) for r in range(P)])
    assert sorted(allpos.tolist()) == list(range(S))
    for r in range(P):
        for i, t in enumerate(im.rank_positions(S, P, r, order)):
            assert im.owner(int(t), S, P, order) == (r, i)


@pytest.mark.parametrize("S,P", [(64, 4), (128, 8), (512, 16), (32768, 8), (131072, 16),
                                 (524288, 32)])
def test_balance_closed_forms(S, P):
    c = S // (2 * P)
    s_loc = S // P
    for r in range(P):
        assert im.visible_pairs(S, P, r, "zigzag", True) == c * (S + 1)
        assert im.visible_pairs(S, P, r, "contiguous", True) == s_loc * s_loc * r + s_loc * (s_loc + 1) // 2
        assert im.visible_pairs(S, P, r, "contiguous", False) == s_loc * S


@pytest.mark.parametrize("order", im.ORDERS)
def test_block_class_matches_enumeration(order):
    rng = np.random.default_rng(3)
    for _ in range(400):
        q0, k0 = (int(x) for x in rng.integers(0, 40, 2))
        q1, k1 = q0 + int(rng.integers(0, 9)), k0 + int(rng.integers(0, 9))
        for causal in (True, False):
            assert im.block_class(q0, q1, k0, k1, causal) == im.block_class_bruteforce(
                np.arange(q0, q1), np.arange(k0, k1), causal)


@pytest.mark.parametrize("order", im.ORDERS)
@pytest.mark.parametrize("S,P,tq,tk", [(64, 4, 4, 4), (96, 3, 8, 4), (80, 2, 6, 5), (128, 8, 8, 8)])
def test_tile_counts_match_enumeration(order, S, P, tq, tk):
    for r in range(P):
        for s in range(P):
            src = im.ring_source(r, s, P)
            qpos = im.rank_positions(S, P, r, order)
            kpos = im.rank_positions(S, P, src, order)
            want = {im.FULL: 0, im.DIAG: 0, im.SKIP: 0}
            # tiles restart at each span of the rank's local order
            def tiles(spans, pos, t):
                off = 0
                out = []
                for _, n in spans:
                    for a in range(0, n, t):
                        out.append(pos[off + a: off + min(n, a + t)])
                    off += n
                return out
            for qt in tiles(im.rank_spans(S, P, r, order), qpos, tq):
                for kt in tiles(im.rank_spans(S, P, src, order), kpos, tk):
                    want[im.block_class_bruteforce(qt, kt, True)] += 1
            assert im.tile_counts(S, P, r, s, order, True, tq, tk) == want


def test_zigzag_step_classes_closed_form():
    """Zigzag, step 0: one FULL, two DIAG, one SKIP; every later step: two FULL,
    two SKIP (src < r: both query chunks see key chunk src; src > r: only the
    tail query chunk sees both key chunks)."""
    for S, P in [(64, 4), (32768, 8), (131072, 16), (524288, 32)]:
        for r in range(P):
            for s in range(P):
                t = im.step_pair_classes(S, P, r, s, "zigzag", True)
                flat = sum(t, [])
                if s == 0:
                    assert sorted(flat) == ["DIAG", "DIAG", "FULL", "SKIP"]
                    continue
                src = im.ring_source(r, s, P)
                assert sorted(flat) == ["FULL", "FULL", "SKIP", "SKIP"]
                if src < r:
                    assert t == [["FULL", "SKIP"], ["FULL", "SKIP"]]
                else:
                    assert t == [["SKIP", "SKIP"], ["FULL", "FULL"]]


# ----------------------------------------------------------------------------
# relayout


@pytest.mark.parametrize("P_u", [1, 2, 4, 8, 16])
def test_relayout_matches_reshape_and_round_trips(P_u):
    B, s_loc, H, D = 2, 12, 16, 8
    x = np.random.default_rng(P_u).integers(0, 2**16, (B, s_loc, H, D)).astype(np.uint16)
    y = orl.seq2head(x, P_u)
    ref = x.reshape(B, s_loc, P_u, H // P_u, D).transpose(2, 0, 1, 3, 4)
    np.testing.assert_array_equal(y, ref)
    np.testing.assert_array_equal(orl.head2seq(y), x)


# ---------------------------------------------------------------------------
# Multi-tensor Ulysses messages

def test_pieces_one_tensor_heads_is_seq2head():
    rng = np.random.default_rng(21)
    x = rng.standard_normal((2, 5, 8, 3)).astype(np.float32)
    from oracle import relayout as rl
    pcs = rl.to_pieces([x], 4, "heads")
    np.testing.assert_array_equal(np.stack([p[0] for p in pcs]), rl.seq2head(x, 4))
    np.testing.assert_array_equal(rl.piece_bytes(pcs), np.ascontiguousarray(rl.seq2head(x, 4)).view(np.uint8).ravel())


@pytest.mark.parametrize("group", ["heads", "seq"])
def test_pieces_round_trip(group):
    from oracle import relayout as rl
    rng = np.random.default_rng(22)
    xs = [rng.standard_normal((2, 12, 6, 4)).astype(np.float32),
          rng.integers(0, 65535, (2, 12, 3, 8), dtype=np.uint16)]
    back = rl.from_pieces(rl.to_pieces(xs, 3, group), group)
    for a, b in zip(xs, back):
        np.testing.assert_array_equal(a, b)


def test_ulysses_exchange_gives_each_rank_all_tokens_of_its_heads():
    """Sequence Parallelism II: before the all-to-all rank u holds all heads
    of tokens [u s, (u+1) s); after it rank j holds all tokens of head block
    j.  Pack, exchange and the receiver's regrouping must give exactly the
    global tensor's head block, and the way back must restore the shards."""
    from oracle import relayout as rl
    rng = np.random.default_rng(23)
    P_u, B, S = 4, 2, 16
    Q = rng.standard_normal((B, S, 8, 5))
    K = rng.standard_normal((B, S, 4, 5))
    s_loc = S // P_u
    shards = [[Q[:, u * s_loc:(u + 1) * s_loc], K[:, u * s_loc:(u + 1) * s_loc]] for u in range(P_u)]
    recv = rl.exchange([rl.to_pieces(sh, P_u, "heads") for sh in shards])
    for j in range(P_u):
        q_j, k_j = rl.from_pieces(recv[j], "seq")
        np.testing.assert_array_equal(q_j, Q[:, :, 2 * j:2 * j + 2])
        np.testing.assert_array_equal(k_j, K[:, :, j:j + 1])
    # the way back (outputs of the head blocks to their token owners)
    outs = [[Q[:, :, 2 * j:2 * j + 2]] for j in range(P_u)]
    back = rl.exchange([rl.to_pieces(o, P_u, "seq") for o in outs])
    for u in range(P_u):
        (o_u,) = rl.from_pieces(back[u], "heads")
        np.testing.assert_array_equal(o_u, Q[:, u * s_loc:(u + 1) * s_loc])


# ---------------------------------------------------------------------------
# Mask variants: sliding window and packed sequences

def _brute_visible(qpos, kpos, causal, window, cu):
    out = np.zeros((len(qpos), len(kpos)), dtype=bool)
    for a, t in enumerate(qpos):
        st = max(c for c in cu[:-1] if c <= t) if cu is not None else None
        for b, j in enumerate(kpos):
            ok = (not causal) or j <= t
            if window:
                ok = ok and t - j < window
            if cu is not None:
                sj = max(c for c in cu[:-1] if c <= j)
                ok = ok and sj == st
            out[a, b] = ok
    return out


@pytest.mark.parametrize("causal,window,cu", [
    (True, 5, None), (True, 1, None), (True, 0, [0, 7, 9, 20, 32]), (False, 0, [0, 3, 32]),
    (True, 4, [0, 11, 12, 30, 32]),
])
def test_masked_visibility_matches_enumeration(causal, window, cu):
    pos = np.arange(32)
    rng = np.random.default_rng(8)
    qpos = rng.permutation(pos)[:20]
    np.testing.assert_array_equal(im.visible_masked(qpos, pos, causal, window, cu),
                                  _brute_visible(qpos, pos, causal, window, cu))


def test_window_of_one_returns_own_value():
    """Window 1: each query sees only itself, so O_t = V_t and LSE_t = s_tt."""
    rng = np.random.default_rng(9)
    B, S, H, D = 1, 12, 2, 4
    Q, K, V = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    pos = np.arange(S)
    o, lse = oa.attention_rows(Q, pos, K, V, pos, True, 0.7, window=1)
    np.testing.assert_allclose(o, V, rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, 0.7 * (Q * K).sum(-1), rtol=0, atol=1e-14)


def test_full_window_and_single_sequence_are_the_causal_mask():
    rng = np.random.default_rng(10)
    B, S, H, D = 1, 24, 2, 4
    Q, K, V = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    pos = np.arange(S)
    ref = oa.attention_rows(Q, pos, K, V, pos, True, 0.5)
    for kw in (dict(window=S), dict(cu_seqlens=[0, S])):
        o, lse = oa.attention_rows(Q, pos, K, V, pos, True, 0.5, **kw)
        np.testing.assert_allclose(o, ref[0], rtol=0, atol=1e-14)
        np.testing.assert_allclose(lse, ref[1], rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [True, False])
def test_packed_sequences_are_independent(causal):
    """Packing is only a layout: each sequence of the pack gives what it gives
    alone (plain attention over its own tokens)."""
    rng = np.random.default_rng(11)
    B, H, D = 2, 2, 4
    cu = [0, 5, 6, 19, 30]
    S = cu[-1]
    Q, K, V = (rng.standard_normal((B, S, H, D)) for _ in range(3))
    pos = np.arange(S)
    o, lse = oa.attention_rows(Q, pos, K, V, pos, causal, 0.6, cu_seqlens=cu)
    for a, b in zip(cu[:-1], cu[1:]):
        p = np.arange(b - a)
        o_s, l_s = oa.attention_rows(Q[:, a:b], p, K[:, a:b], V[:, a:b], p, causal, 0.6)
        np.testing.assert_allclose(o[:, a:b], o_s, rtol=0, atol=1e-13)
        np.testing.assert_allclose(lse[:, a:b], l_s, rtol=0, atol=1e-13)
