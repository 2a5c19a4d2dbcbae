"""The bf16 step kernels' online softmax where its reference has to move
after a row's first tile.  On N(0, 1) inputs a row's first visible tile
almost always sets a reference that later tiles never exceed by 2^8 in
probability, so the path that rescales O and the row sum (the scores formed
again from the K tile, the tile maximum, the rescale, the probabilities taken
again) runs at full strength mostly on first tiles.  These rings shape K so
that it runs on many later tiles too:

- ``grow``: key j's row scaled by 1 + 6 j / S, so each row's scores rise
  along the keys and its maximum keeps moving (steps 0..P-1 of the ring
  bring later blocks);
- ``spikes``: every 97th key scaled by 12, large isolated scores that move
  the reference by far more than 2^8 at once;
- ``wide``: K scaled by 8, scores with a standard deviation of 8 (very
  peaked rows, most probabilities far below one);
- ``shrink``: key j's row scaled by 7 - 6 j / S, the maximum early and the
  later tiles' probabilities small.

Every output row of the listed ranks is compared with the oracle, dense
attention over the concatenated sequence in float64, as the DeDLOC guide's
"Step 4: Verification and Benchmarking Test Harness" compares dense and ring
outputs; the library's launch plan is asserted first, so each ring is known
to run the kernel it is meant for.  GPU tests."""
import numpy as np
import pytest

import seeded_inputs as si
from oracle import attention as oa
from oracle import index_maps as im
from ra_testlib import RankCase, assert_close, say, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def ra():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import ring_attention_blockwise_amd as ra
    return ra


def shaped(case, profile):
    """Scale each key's row of the case's global K by the profile's factor,
    rounded back to bf16 (both the GPU and the oracle then read these
    values)."""
    j = np.arange(case.S, dtype=np.float64)
    if profile == "grow":
        f = 1.0 + 6.0 * j / case.S
    elif profile == "shrink":
        f = 7.0 - 6.0 * j / case.S
    elif profile == "spikes":
        f = np.where(j % 97 == 13, 12.0, 1.0)
    elif profile == "wide":
        f = np.full(case.S, 8.0)
    else:
        raise ValueError(profile)
    k = si.bf16_bits_to_f32(case.Kg) * f.astype(np.float32)[None, :, None, None]
    case.Kg = si.f32_to_bf16_bits(k.astype(np.float32))
    return case


def launches(ra, case, rank, window=0):
    return ra.ra_rank_launches(dtype="bf16", B=case.B, Hq=case.Hq, Hkv=case.Hkv, D=128, S=case.S, P=case.P,
                               rank=rank, order=case.order, causal=case.causal, n_cus=0, window=window)


CASES = [
    # (label, B, Hq, Hkv, S, P, order, causal, profile, window, kernels the
    # steps may launch (the first one at least once), ranks)
    ("grow_zigzag_b8", 8, 16, 4, 4096, 2, "zigzag", True, "grow", 0, ("step_bf16",), (0, 1)),
    ("spikes_zigzag_b8", 8, 16, 4, 4096, 2, "zigzag", True, "spikes", 0, ("step_bf16",), (1,)),
    ("wide_zigzag_b8", 8, 16, 4, 4096, 2, "zigzag", True, "wide", 0, ("step_bf16",), (1,)),
    ("shrink_zigzag_b8", 8, 16, 4, 4096, 2, "zigzag", True, "shrink", 0, ("step_bf16",), (0,)),
    ("grow_noncausal_b4", 4, 16, 16, 4096, 2, "contiguous", False, "grow", 0, ("step_bf16",), (0,)),
    # the eight-wave key split (few work items), both wave sets' references
    # merged at the end
    ("grow_ksplit_p4", 1, 8, 2, 2048, 4, "zigzag", True, "grow", 0, ("step_bf16_ksplit",), (0, 3)),
    ("spikes_ksplit_p4", 1, 8, 2, 2048, 4, "zigzag", True, "spikes", 0, ("step_bf16_ksplit",), (2,)),
    # the masked instantiations: a window over the growing keys (its second
    # step has few items and takes the key split)
    ("grow_window700_b8", 8, 16, 4, 4096, 2, "zigzag", True, "grow", 700, ("step_bf16", "step_bf16_ksplit"),
     (1,)),
]


@pytest.mark.parametrize("cfg", CASES, ids=[c[0] for c in CASES])
def test_reference_moves_every_row(ra, cfg):
    import torch
    label, B, Hq, Hkv, S, P, order, causal, profile, window, kernels, ranks = cfg
    case = shaped(RankCase(700 + len(label), "bf16", B, Hq, Hkv, 128, S, P, order, causal), profile)
    for r in ranks:
        kinds = [s["kernel"] for s in launches(ra, case, r, window)]
        say(label, "rank", r, "kernels", kinds)
        assert all(k in kernels + ("none",) for k in kinds) and kernels[0] in kinds, kinds
        if window:
            q = to_device(case.q_rows(ra.rank_spans(order, S, P, r)), "bf16")
            ks, vs = case.device_shards(ra)
            o = torch.full((B, S // P, Hq, 128), float("nan"), device="cuda")
            lse = torch.full((B, S // P, Hq), float("nan"), device="cuda")
            ra.ra_rank_forward_masked(q, ks, vs, o, lse, S=S, P=P, rank=r, order=order, causal=causal,
                                      scale=case.scale, window=window)
            torch.cuda.synchronize()
            o, lse = o.cpu().numpy(), lse.cpu().numpy()
            pos = im.rank_positions(S, P, r, order)
            qf = si.to_f64(case.q_rows(im.rank_spans(S, P, r, order)), "bf16")
            kmax = int(pos.max()) + 1
            o_ref, l_ref = oa.attention_rows(qf, pos, si.to_f64(case.Kg[:, :kmax], "bf16"),
                                             si.to_f64(case.Vg[:, :kmax], "bf16"), np.arange(kmax), causal,
                                             case.scale, window=window)
        else:
            o, lse = case.run_rank(ra, r)
            o_ref, l_ref = case.reference(r)
        assert_close(o, lse, o_ref, l_ref, "bf16", f"{label} rank {r}")
    case.release()
