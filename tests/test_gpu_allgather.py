"""ra_allgather_forward (the rank's queries against the whole resident
sequence in one launch) against the oracle's full attention.  GPU tests."""
import numpy as np
import pytest

from seeded_inputs import WORKLOADS, workload
from seeded_inputs.workloads import SMALL
from ra_testlib import RankCase, assert_close, sample_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return ra


RINGS = [
    # (label, dtype, B, Hq, Hkv, D, S, P, order, causal, k_scale, ranks)
    ("small_f32_contig", "f32", 1, 2, 2, 64, 512, 4, "contiguous", True, 1.0, range(4)),
    ("gqa_zigzag_p8", "bf16", 1, 32, 8, 128, 4096, 8, "zigzag", True, 1.0, (0, 4, 7)),
    ("ragged_zigzag", "bf16", 1, 8, 2, 128, 1600, 4, "zigzag", True, 1.0, range(4)),
    ("ragged_zigzag_f32", "f32", 1, 4, 1, 64, 1400, 4, "zigzag", True, 1.0, (0, 3)),
    ("mha_contig_full_b2", "bf16", 2, 16, 16, 128, 2048, 8, "contiguous", False, 1.0, (0, 5)),
    ("single_rank_causal", "bf16", 1, 4, 1, 128, 384, 1, "zigzag", True, 1.0, (0,)),
    ("mqa_d64", "bf16", 1, 8, 1, 64, 2048, 4, "zigzag", True, 1.0, (0, 3)),
]


@pytest.mark.parametrize("cfg", RINGS, ids=[c[0] for c in RINGS])
def test_small_rings_every_row(ra, cfg):
    label, dtype, B, Hq, Hkv, D, S, P, order, causal, k_scale, ranks = cfg
    case = RankCase(70 + len(label), dtype, B, Hq, Hkv, D, S, P, order, causal, k_scale)
    for r in ranks:
        say(label, "allgather rank", r)
        o, lse = case.run_allgather(ra, r)
        o_ref, l_ref = case.reference(r)
        assert_close(o, lse, o_ref, l_ref, dtype, f"{label} allgather rank {r}")


def test_allgather_matches_the_ring(ra):
    """Same definition, different summation order: the one-launch result and
    the P-step ring agree to the bf16 bound on every row."""
    case = RankCase(91, "bf16", 1, 8, 2, 128, 4096, 8, "zigzag", True)
    for r in (0, 7):
        o_a, l_a = case.run_allgather(ra, r)
        o_r, l_r = case.run_rank(ra, r)
        assert_close(o_a, l_a, o_r.astype(np.float64), l_r.astype(np.float64), "bf16", f"ring vs allgather {r}")


FULL = [n for n in WORKLOADS if n != SMALL]


@pytest.mark.parametrize("name", FULL)
@pytest.mark.parametrize("which", ["first", "last"])
def test_full_size_workloads_sampled(ra, name, which):
    w = workload(name)
    r = {"first": 0, "last": w.P - 1}[which]
    say("allgather full size", name, "rank", r)
    case = RankCase.from_workload(w)
    o, lse = case.run_allgather(ra, r)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = sample_rows(w.S, w.P, r, w.order, n_random=8 if w.S > 200000 else 16, seed=100 + r)
    o_ref, l_ref = case.reference(r, rows)
    assert_close(o[:, rows], lse[:, rows], o_ref, l_ref, w.dtype, f"{name} allgather rank {r}")
