"""The library's host plan (ra_plan) against the oracle's index maps, bit-exact.
CPU only: ra_plan does integer work on the host and touches no GPU."""
import numpy as np
import pytest

from oracle import index_maps as im
from seeded_inputs import WORKLOADS

ra = pytest.importorskip("ring_attention_blockwise_amd")

KERNEL_TILES = (128, 64)


def _check(order, S, P, r, s, causal, tq, tk, with_tiles=True):
    got = ra.ra_plan(order, S, P, r, s, causal, tq, tk)
    src = im.ring_source(r, s, P)
    assert got["src"] == src
    assert got["qspans"] == im.rank_spans(S, P, r, order)
    assert got["kspans"] == im.rank_spans(S, P, src, order)
    classes = [[im.block_class(a, a + n, b, b + m, causal) for (b, m) in got["kspans"]]
               for (a, n) in got["qspans"]]
    assert got["classes"] == classes
    assert got["classes"] == im.step_pair_classes(S, P, r, s, order, causal)
    if with_tiles:
        assert got["tiles"] == im.tile_counts(S, P, r, s, order, causal, tq, tk)


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_plan_matches_oracle_on_workloads(name):
    w = WORKLOADS[name]
    ranks = range(w.P) if w.P <= 16 else (0, 1, w.P // 2, w.P - 2, w.P - 1)
    for r in ranks:
        for s in range(w.P):
            _check(w.order, w.S, w.P, r, s, w.causal, *KERNEL_TILES,
                   with_tiles=(w.S <= 131072 or s % 8 == 0))


@pytest.mark.parametrize("order", ["contiguous", "zigzag"])
def test_plan_matches_oracle_random_small(order):
    rng = np.random.default_rng(11)
    for _ in range(150):
        P = int(rng.integers(1, 9))
        c = int(rng.integers(1, 40))
        S = c * (2 * P if order == "zigzag" else P)
        r, s = int(rng.integers(0, P)), int(rng.integers(0, P))
        tq, tk = int(rng.integers(1, 50)), int(rng.integers(1, 50))
        _check(order, S, P, r, s, bool(rng.integers(0, 2)), tq, tk)


def test_rank_spans_are_the_oracle_map():
    for order in ("contiguous", "zigzag"):
        for S, P in ((64, 4), (131072, 16), (524288, 32)):
            for r in range(P):
                spans = ra.rank_spans(order, S, P, r)
                pos = np.concatenate([np.arange(a, a + n) for a, n in spans])
                np.testing.assert_array_equal(pos, im.rank_positions(S, P, r, order))


@pytest.mark.parametrize("args", [
    ("zigzag", 100, 8, 0, 0),      # S not divisible by 2P
    ("contiguous", 10, 4, 0, 0),   # S not divisible by P
    ("zigzag", 64, 4, 4, 0),       # rank out of range
    ("zigzag", 64, 4, 0, 4),       # step out of range
    ("zigzag", 64, 0, 0, 0),       # P < 1
])
def test_plan_rejects_bad_rings(args):
    order, S, P, r, s = args
    with pytest.raises(ra.RaError) as e:
        ra.ra_plan(order, S, P, r, s, True, 64, 64)
    assert e.value.status == ra.RA_E_INVAL
    assert ra.ra_last_error()


# ---------------------------------------------------------------------------
# ra_rank_launches: which kernel each step launches (host-only, planned for
# the 256 compute units of an MI355X)

@pytest.mark.parametrize("name", list(WORKLOADS))
def test_launches_follow_the_pair_classes(name):
    """A step launches iff some (query span, key span) pair of it is not
    SKIP in the oracle's classes (step 0 always launches: it writes every
    row)."""
    w = WORKLOADS[name]
    ranks = range(w.P) if w.P <= 8 else (0, w.P // 2, w.P - 1)
    for r in ranks:
        for backward in (False, True):
            plan = ra.ra_rank_launches(dtype=w.dtype, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, S=w.S, P=w.P, rank=r,
                                       order=w.order, causal=w.causal, backward=backward, n_cus=256)
            assert len(plan) == w.P
            for s in range(w.P):
                classes = im.step_pair_classes(w.S, w.P, r, s, w.order, w.causal)
                sees = any(c != "SKIP" for row in classes for c in row)
                assert (plan[s]["kernel"] != "none") == (sees or (s == 0 and not backward)), (r, s, classes)


def test_benchmark_workloads_take_the_four_wave_kernel():
    """The 131k, 64k and 524k rings launch the four-wave step kernel on
    every step, and the fused dK/dV backward; the 32k ring's steps (256
    query tiles with work: one per CU) take the key-split kernel."""
    for name in ("bf16_gqa32x8_d128_s128k_ring16_zigzag_causal", "bf16_mha16_b2_d128_s64k_ring8_contiguous_full",
                 "bf16_gqa32x8_d128_s512k_ring32_zigzag_causal_khalf"):
        w = WORKLOADS[name]
        kw = dict(dtype=w.dtype, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, S=w.S, P=w.P, rank=0, order=w.order,
                  causal=w.causal, n_cus=256)
        assert {s["kernel"] for s in ra.ra_rank_launches(**kw)} == {"step_bf16"}, name
        assert {s["kernel"] for s in ra.ra_rank_launches(backward=True, **kw)} == {"bwd_fused"}, name
    w = WORKLOADS["bf16_gqa32x8_d128_s32k_ring8_zigzag_causal"]
    plan = ra.ra_rank_launches(dtype=w.dtype, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, S=w.S, P=w.P, rank=0,
                               order=w.order, causal=w.causal, n_cus=256)
    assert {s["kernel"] for s in plan} == {"step_bf16_ksplit"}
    w = WORKLOADS["f32_mha2_d64_s512_ring4_contiguous_causal"]
    plan = ra.ra_rank_launches(dtype=w.dtype, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D, S=w.S, P=w.P, rank=3,
                               order=w.order, causal=w.causal, backward=True, n_cus=256)
    assert {s["kernel"] for s in plan} == {"bwd_simt"}


def test_launches_masked_instantiation():
    kw = dict(dtype="bf16", B=16, Hq=16, Hkv=4, D=128, S=4096, P=2, rank=0, order="zigzag", causal=True,
              n_cus=256)
    plan = ra.ra_rank_launches(window=1500, **kw)
    assert [(s["kernel"], s["masked"]) for s in plan] == [("step_bf16", True)] * 2
    plan = ra.ra_rank_launches(**kw)
    assert [(s["kernel"], s["masked"]) for s in plan] == [("step_bf16", False)] * 2
    # a one-key window cannot reach the held block of step 1 (keys
    # [1024, 3072), rank 0 holds rows [0, 1024) and [3072, 4096)): no launch
    plan = ra.ra_rank_launches(window=1, **kw)
    assert plan[1]["kernel"] == "none"


@pytest.mark.parametrize("bad", [dict(n_cus=-1), dict(S=4094), dict(rank=2), dict(window=-3),
                                 dict(causal=False, window=8), dict(cu_seqlens=[0, 5, 5, 4096])])
def test_launches_reject_bad_arguments(bad):
    kw = dict(dtype="bf16", B=1, Hq=8, Hkv=2, D=128, S=4096, P=2, rank=0, order="zigzag", causal=True, n_cus=256)
    kw.update(bad)
    with pytest.raises(ra.RaError) as e:
        ra.ra_rank_launches(**kw)
    assert e.value.status == ra.RA_E_INVAL
