"""The C ABI itself, without a GPU: the library loads, exports every function
include/ra.h declares, and rejects bad arguments before touching a pointer or
the HIP runtime."""
import ctypes
import os
import re

import pytest

ra = pytest.importorskip("ring_attention_blockwise_amd")

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "ra.h")
# never dereferenced: every call below fails validation first
FAKE = ctypes.c_void_p(0x100000)


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(ra_\w+)\s*\(", text, re.M)))


def test_header_declares_the_boundary():
    assert _declared() == sorted(ra.EXPORTS)


def test_every_declared_symbol_is_exported():
    for name in _declared():
        assert hasattr(ra.lib, name), name


def test_abi_version_matches_header():
    m = re.search(r"#define RA_ABI_VERSION (\d+)", open(HEADER).read())
    assert ra.ra_abi_version() == int(m.group(1))


def _desc(**kw):
    qs = kw.pop("qspans", [(0, 256)])
    ks = kw.pop("kspans", [(0, 256)])
    d = dict(dtype=ra.RA_DTYPE_BF16, B=1, Hq=8, Hkv=2, D=128, Sq=256, Sk=256, causal=1, scale=0.088,
             n_qspans=1, n_kspans=1)
    d.update(kw)
    return ra.ra_step_desc(d["dtype"], d["B"], d["Hq"], d["Hkv"], d["D"], d["Sq"], d["Sk"], d["causal"],
                           d["scale"], d["n_qspans"], d["n_kspans"], ra._spans(qs), ra._spans(ks))


@pytest.mark.parametrize("kw,status", [
    (dict(Hq=6, Hkv=4), ra.RA_E_INVAL),
    (dict(D=96), ra.RA_E_UNSUPPORTED),
    (dict(dtype=7), ra.RA_E_UNSUPPORTED),
    (dict(scale=0.0), ra.RA_E_INVAL),
    (dict(scale=float("nan")), ra.RA_E_INVAL),
    (dict(n_qspans=3), ra.RA_E_INVAL),
    (dict(Sq=255), ra.RA_E_INVAL),                        # spans do not sum to Sq
    (dict(qspans=[(0, -1)], Sq=-1), ra.RA_E_INVAL),
    (dict(B=0), ra.RA_E_INVAL),
])
def test_step_rejects_bad_descriptors(kw, status):
    d = _desc(**kw)
    rc = ra.lib.ra_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, ra.RA_STEP_INIT, None)
    assert rc == status
    assert ra.ra_last_error()


def test_step_rejects_bad_flags_null_and_misaligned():
    d = _desc()
    assert ra.lib.ra_step(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, 5, None) == ra.RA_E_INVAL
    assert ra.lib.ra_step(ctypes.byref(d), None, FAKE, FAKE, FAKE, FAKE, 0, None) == ra.RA_E_INVAL
    odd = ctypes.c_void_p(0x100008)
    assert ra.lib.ra_step(ctypes.byref(d), odd, FAKE, FAKE, FAKE, FAKE, 0, None) == ra.RA_E_INVAL
    assert ra.lib.ra_step(None, FAKE, FAKE, FAKE, FAKE, FAKE, 0, None) == ra.RA_E_INVAL


def test_empty_step_enqueues_nothing():
    # Sq = 0: valid and a no-op, even with NULL pointers
    d = _desc(Sq=0, qspans=[(0, 0)])
    assert ra.lib.ra_step(ctypes.byref(d), None, None, None, None, None, 0, None) == ra.RA_OK


@pytest.mark.parametrize("fields,status", [
    (dict(S=100, P=8, order=1), ra.RA_E_INVAL),
    (dict(rank=8), ra.RA_E_INVAL),
    (dict(order=2), ra.RA_E_INVAL),
    (dict(Hq=5), ra.RA_E_INVAL),
    (dict(D=80), ra.RA_E_UNSUPPORTED),
])
@pytest.mark.parametrize("entry", ["ra_rank_forward", "ra_allgather_forward"])
def test_rank_forward_rejects_bad_descriptors(fields, status, entry):
    f = dict(dtype=1, B=1, Hq=8, Hkv=2, D=128, S=4096, P=8, rank=0, order=1, causal=1, scale=0.088)
    f.update(fields)
    d = ra.ra_rank_desc(*[f[k] for k in ("dtype", "B", "Hq", "Hkv", "D", "S", "P", "rank", "order",
                                         "causal", "scale")])
    assert getattr(ra.lib, entry)(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, None) == status
    assert ra.ra_last_error()
    assert getattr(ra.lib, entry)(None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ra.RA_E_INVAL


def test_merge_and_relayout_validation():
    assert ra.lib.ra_lse_merge(0, 128, None, None, None, None, None, None, None) == ra.RA_OK
    assert ra.lib.ra_lse_merge(-1, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ra.RA_E_INVAL
    assert ra.lib.ra_lse_merge(4, 0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ra.RA_E_INVAL
    assert ra.lib.ra_lse_merge(4, 8, None, FAKE, FAKE, FAKE, FAKE, FAKE, None) == ra.RA_E_INVAL
    rl = ra.lib.ra_ulysses_relayout
    assert rl(0, 2, 1, 16, 12, 8, 5, FAKE, ctypes.c_void_p(0x900000), None) == ra.RA_E_INVAL  # H % P_u
    assert rl(2, 2, 1, 16, 12, 8, 4, FAKE, ctypes.c_void_p(0x900000), None) == ra.RA_E_INVAL  # dir
    assert rl(0, 3, 1, 16, 12, 8, 4, FAKE, ctypes.c_void_p(0x900000), None) == ra.RA_E_INVAL  # elem
    assert rl(0, 2, 1, 16, 12, 8, 4, FAKE, ctypes.c_void_p(0x100010), None) == ra.RA_E_INVAL  # overlap
    assert rl(0, 2, 0, 16, 12, 8, 4, None, None, None) == ra.RA_OK                            # empty


def test_error_message_is_cleared_on_success():
    ra.lib.ra_lse_merge(-1, 128, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert ra.ra_last_error()
    assert ra.lib.ra_lse_merge(0, 128, None, None, None, None, None, None, None) == ra.RA_OK
    assert ra.ra_last_error() == ""


def test_one_hip_runtime_shared_with_torch():
    """libra.so binds to the HIP runtime torch loaded; a second runtime in the
    process would receive torch's streams and pointers and fail."""
    paths = ra.hip_runtime_path().split(";")
    assert len(paths) == 1, paths


def _mask(window=0, cu=None, dev=None):
    """An ra_mask (and the host array it points at, to keep alive)."""
    host = (ctypes.c_int64 * len(cu))(*cu) if cu is not None else None
    m = ra.ra_mask(window, len(cu) - 1 if cu is not None else 0,
                   ctypes.cast(host, ctypes.POINTER(ctypes.c_int64)) if host is not None else None,
                   FAKE if dev is None else dev)
    return m, host


@pytest.mark.parametrize("window,cu,dev,causal", [
    (-1, None, None, 1),                   # negative window
    (64, None, None, 0),                   # a window needs the causal mask
    (0, [1, 2048, 4096], None, 1),         # boundaries must start at 0
    (0, [0, 2048, 4000], None, 1),         # ... and end at S
    (0, [0, 3000, 2048, 4096], None, 1),   # ... and increase
    (0, [0, 2048, 4096], 4, 1),            # device copy not 8-byte aligned
])
@pytest.mark.parametrize("entry", ["forward", "backward"])
def test_masked_entries_reject_bad_masks(window, cu, dev, causal, entry):
    """Both masked entry points check the mask on the host before anything
    is enqueued."""
    d = ra.ra_rank_desc(1, 1, 8, 2, 128, 4096, 8, 0, 1, causal, 0.088)
    m, _keep = _mask(window, cu, dev)
    if entry == "forward":
        rc = ra.lib.ra_rank_forward_masked(ctypes.byref(d), ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, FAKE, None)
    else:
        rc = ra.lib.ra_rank_backward_masked(ctypes.byref(d), ctypes.byref(m), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, FAKE, FAKE, FAKE, None)
    assert rc == ra.RA_E_INVAL
    assert ra.ra_last_error()


def test_noalloc_backward_rejects_more_rows_than_its_scratch():
    """ra_rank_backward_noalloc refuses B * S/P * Hq above RA_NOALLOC_MAX_ROWS
    on the host, before it resolves its scratch or enqueues anything; the
    descriptor checks of ra_rank_backward come first."""
    d = ra.ra_rank_desc(1, 1, 16, 1, 128, 1 << 20, 2, 0, 1, 1, 0.088)   # 2^19 rows x 16 heads = 2^23
    rc = ra.lib.ra_rank_backward_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         None)
    assert rc == ra.RA_E_INVAL and "scratch" in ra.ra_last_error()
    assert (1 << 23) > ra.RA_NOALLOC_MAX_ROWS
    d = ra.ra_rank_desc(1, 1, 16, 1, 128, 4097, 2, 0, 1, 1, 0.088)      # S not divisible by 2P
    rc = ra.lib.ra_rank_backward_noalloc(ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                         None)
    assert rc == ra.RA_E_INVAL and "divisible" in ra.ra_last_error()
    m = re.search(r"#define RA_NOALLOC_MAX_ROWS (\d+)", open(HEADER).read())
    assert int(m.group(1)) == ra.RA_NOALLOC_MAX_ROWS
