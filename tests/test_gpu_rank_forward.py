"""ra_rank_forward (one rank's whole ring, simulated on one GPU) against the
oracle's full attention over the concatenated sequence.  GPU tests."""
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


def _full_check(ra, case, ranks, what):
    for r in ranks:
        say(what, "rank", r)
        o, lse = case.run_rank(ra, r)
        o_ref, l_ref = case.reference(r)
        assert_close(o, lse, o_ref, l_ref, case.dtype, f"{what} rank {r}")


def test_small_fp32_workload_every_rank(ra):
    """fp32, batch 1, 2 heads, D 64, 512 tokens on a contiguous causal ring of 4:
    every rank, every row, to 1e-5."""
    w = workload(SMALL)
    _full_check(ra, RankCase.from_workload(w), range(w.P), w.name)


SMALL_RINGS = [
    # (label, dtype, B, Hq, Hkv, D, S, P, order, causal, k_scale, ranks)
    ("gqa_zigzag_p8", "bf16", 1, 32, 8, 128, 4096, 8, "zigzag", True, 1.0, (0, 4, 7)),
    ("gqa_zigzag_p8_f32", "f32", 1, 8, 2, 128, 4096, 8, "zigzag", True, 1.0, (0, 3, 7)),
    ("ragged_zigzag", "bf16", 1, 8, 2, 128, 1600, 4, "zigzag", True, 1.0, range(4)),
    ("ragged_zigzag_f32", "f32", 1, 4, 1, 64, 1400, 4, "zigzag", True, 1.0, range(4)),
    ("mha_contig_full_b2", "bf16", 2, 16, 16, 128, 2048, 8, "contiguous", False, 1.0, (0, 5)),
    ("contig_causal_f32", "f32", 2, 4, 2, 128, 1024, 4, "contiguous", True, 1.0, range(4)),
    ("khalf_zigzag_p16", "bf16", 1, 8, 2, 128, 8192, 16, "zigzag", True, 0.5, (0, 8, 15)),
    ("single_rank_causal", "bf16", 1, 4, 1, 128, 384, 1, "zigzag", True, 1.0, (0,)),
    ("single_rank_contig_f32", "f32", 1, 2, 2, 64, 200, 1, "contiguous", True, 1.0, (0,)),
    ("mqa_d64", "bf16", 1, 8, 1, 64, 2048, 4, "zigzag", True, 1.0, (0, 3)),
]


@pytest.mark.parametrize("cfg", SMALL_RINGS, ids=[c[0] for c in SMALL_RINGS])
def test_small_rings(ra, cfg):
    label, dtype, B, Hq, Hkv, D, S, P, order, causal, k_scale, ranks = cfg
    case = RankCase(50 + len(label), dtype, B, Hq, Hkv, D, S, P, order, causal, k_scale)
    _full_check(ra, case, ranks, label)


_CACHE = {}


def _case(name):
    if name not in _CACHE:
        _CACHE.clear()
        _CACHE[name] = RankCase.from_workload(workload(name))
    return _CACHE[name]


FULL = [n for n in WORKLOADS if n != SMALL]


@pytest.mark.parametrize("name", FULL)
@pytest.mark.parametrize("which", ["first", "middle", "last"])
def test_full_size_workloads_sampled(ra, name, which):
    """Full-size workloads in the benchmark's launch configuration; outputs at
    span boundaries, one seeded row in every 256-row work item of each span
    (all heads) and seeded random rows are compared with the oracle."""
    w = workload(name)
    r = {"first": 0, "middle": w.P // 2, "last": w.P - 1}[which]
    say("full size", name, "rank", r)
    case = _case(name)
    o, lse = case.run_rank(ra, r)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    rows = sample_rows(w.S, w.P, r, w.order, n_random=4 if w.S > 200000 else 8, seed=r, per_tile=256)
    o_ref, l_ref = case.reference(r, rows)
    assert_close(o[:, rows], lse[:, rows], o_ref, l_ref, w.dtype, f"{name} rank {r}")
    if which == "last":
        case.release()
