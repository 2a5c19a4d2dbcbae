"""Python binding of libra.so: one rank's blockwise ring-attention step on
MI355X (gfx950).

The functions here carry the C ABI's names and only marshal arguments: they
check tensor devices, dtypes, shapes and contiguity, pass raw pointers and the
current HIP stream, and raise ``RaError`` on a non-zero status.  Every step of
the computation runs in the library's HIP kernels.  If libra.so is missing the
import fails; build it with ``python ring_attention_blockwise_amd/build.py``.

Layouts (see include/ra.h): q [B, Sq, Hq, D], k/v [B, Sk, Hkv, D] in float32
or bfloat16; o [B, Sq, Hq, D] float32; lse [B, Sq, Hq] float32 (natural log).
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# RA_LIBRARY names another build of the same library (the host-sanitizer build
# the CPU tests run against); by default the in-tree libra.so.
LIB_PATH = os.environ.get("RA_LIBRARY") or os.path.join(_HERE, "libra.so")

RA_OK, RA_E_INVAL, RA_E_UNSUPPORTED, RA_E_HIP = 0, -1, -2, -3
RA_DTYPE_F32, RA_DTYPE_BF16 = 0, 1
RA_ORDER_CONTIGUOUS, RA_ORDER_ZIGZAG = 0, 1
RA_STEP_INIT, RA_STEP_ACCUM = 0, 1
RA_SEQ2HEAD, RA_HEAD2SEQ = 0, 1
RA_GROUP_HEADS, RA_GROUP_SEQ = 0, 1
RA_CLASS_SKIP, RA_CLASS_FULL, RA_CLASS_DIAG = 0, 1, 2
CLASS_NAMES = {RA_CLASS_SKIP: "SKIP", RA_CLASS_FULL: "FULL", RA_CLASS_DIAG: "DIAG"}
ORDERS = {"contiguous": RA_ORDER_CONTIGUOUS, "zigzag": RA_ORDER_ZIGZAG}


class RaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class ra_span(ctypes.Structure):
    _fields_ = [("start", ctypes.c_int64), ("len", ctypes.c_int64)]


class ra_step_desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("Sq", ctypes.c_int64),
                ("Sk", ctypes.c_int64), ("causal", ctypes.c_int32), ("scale", ctypes.c_float),
                ("n_qspans", ctypes.c_int32), ("n_kspans", ctypes.c_int32),
                ("qspans", ra_span * 2), ("kspans", ra_span * 2)]


class ra_rank_desc(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int32), ("B", ctypes.c_int32), ("Hq", ctypes.c_int32),
                ("Hkv", ctypes.c_int32), ("D", ctypes.c_int32), ("S", ctypes.c_int64),
                ("P", ctypes.c_int32), ("rank", ctypes.c_int32), ("order", ctypes.c_int32),
                ("causal", ctypes.c_int32), ("scale", ctypes.c_float)]


class ra_mask(ctypes.Structure):
    _fields_ = [("window", ctypes.c_int64), ("n_seqs", ctypes.c_int32),
                ("cu_seqlens", ctypes.POINTER(ctypes.c_int64)), ("cu_seqlens_dev", ctypes.c_void_p)]


class ra_plan_out(ctypes.Structure):
    _fields_ = [("src", ctypes.c_int32), ("n_qspans", ctypes.c_int32), ("n_kspans", ctypes.c_int32),
                ("qspans", ra_span * 2), ("kspans", ra_span * 2),
                ("pair_class", (ctypes.c_int32 * 2) * 2),
                ("tiles_full", ctypes.c_int64), ("tiles_diag", ctypes.c_int64),
                ("tiles_skip", ctypes.c_int64)]


class ra_launch_info(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_int32), ("masked", ctypes.c_int32), ("items", ctypes.c_int32),
                ("grid", ctypes.c_int32), ("lpt", ctypes.c_int32), ("first_heavy", ctypes.c_int32)]


RA_KERNEL_NONE, RA_KERNEL_STEP_F32, RA_KERNEL_STEP_BF16, RA_KERNEL_STEP_BF16_KSPLIT = 0, 1, 2, 3
RA_KERNEL_BWD_FUSED, RA_KERNEL_BWD_SPLIT, RA_KERNEL_BWD_SIMT = 4, 5, 6
KERNEL_NAMES = {RA_KERNEL_NONE: "none", RA_KERNEL_STEP_F32: "step_f32", RA_KERNEL_STEP_BF16: "step_bf16",
                RA_KERNEL_STEP_BF16_KSPLIT: "step_bf16_ksplit",
                RA_KERNEL_BWD_FUSED: "bwd_fused", RA_KERNEL_BWD_SPLIT: "bwd_split", RA_KERNEL_BWD_SIMT: "bwd_simt"}


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python ring_attention_blockwise_amd/build.py`")
# The library must share PyTorch's HIP runtime: torch hands it device pointers
# and stream handles.  Both runtimes carry the soname libamdhip64.so.7, so
# loading torch first makes the dynamic loader bind libra.so to torch's copy
# instead of starting a second runtime from the system ROCm.
try:
    import torch as _torch_runtime  # noqa: F401
except ImportError:  # pragma: no cover - host-only use (ra_plan) without torch
    _torch_runtime = None
lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _u32, _fp = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p
lib.ra_step.argtypes = [ctypes.POINTER(ra_step_desc), _vp, _vp, _vp, _fp, _fp, _u32, _vp]
lib.ra_lse_merge.argtypes = [_i64, _i32, _fp, _fp, _fp, _fp, _fp, _fp, _vp]
lib.ra_rank_forward.argtypes = [ctypes.POINTER(ra_rank_desc), _vp, _vp, _vp, _fp, _fp, _vp]
lib.ra_allgather_forward.argtypes = [ctypes.POINTER(ra_rank_desc), _vp, _vp, _vp, _fp, _fp, _vp]
lib.ra_rank_forward_masked.argtypes = [ctypes.POINTER(ra_rank_desc), ctypes.POINTER(ra_mask), _vp, _vp, _vp,
                                       _fp, _fp, _vp]
lib.ra_rank_backward.argtypes = [ctypes.POINTER(ra_rank_desc), _vp, _vp, _vp, _fp, _fp, _vp, _fp, _fp, _fp,
                                 _fp, _vp]
lib.ra_rank_backward_masked.argtypes = [ctypes.POINTER(ra_rank_desc), ctypes.POINTER(ra_mask), _vp, _vp, _vp, _fp,
                                        _fp, _vp, _fp, _fp, _fp, _fp, _vp]
lib.ra_rank_backward_noalloc.argtypes = [ctypes.POINTER(ra_rank_desc), _vp, _vp, _vp, _fp, _fp, _vp, _fp, _fp, _fp,
                                         _vp]
lib.ra_ulysses_relayout.argtypes = [_i32, _i32, _i32, _i64, _i32, _i32, _i32, _vp, _vp, _vp]
lib.ra_ulysses_pieces.argtypes = [_i32, _i32, _i32, _i64, _i32, _i32, ctypes.POINTER(ctypes.c_void_p),
                                  ctypes.POINTER(ctypes.c_int64), _vp, _vp]
lib.ra_plan.argtypes = [_i32, _i64, _i32, _i32, _i32, _i32, _i32, _i32, ctypes.POINTER(ra_plan_out)]
lib.ra_rank_launches.argtypes = [ctypes.POINTER(ra_rank_desc), ctypes.POINTER(ra_mask), _i32, _i32,
                                 ctypes.POINTER(ra_launch_info)]
lib.ra_last_error.restype = ctypes.c_char_p
lib.ra_last_error.argtypes = []
lib.ra_abi_version.restype = ctypes.c_int
lib.ra_abi_version.argtypes = []
for _f in ("ra_step", "ra_lse_merge", "ra_rank_forward", "ra_rank_forward_masked", "ra_allgather_forward",
           "ra_rank_backward", "ra_rank_backward_masked", "ra_rank_backward_noalloc",
           "ra_ulysses_relayout", "ra_ulysses_pieces", "ra_plan", "ra_rank_launches"):
    getattr(lib, _f).restype = ctypes.c_int

EXPORTS = ("ra_step", "ra_lse_merge", "ra_rank_forward", "ra_rank_forward_masked", "ra_allgather_forward",
           "ra_rank_backward", "ra_rank_backward_masked", "ra_rank_backward_noalloc",
           "ra_ulysses_relayout", "ra_ulysses_pieces", "ra_plan", "ra_rank_launches",
           "ra_last_error", "ra_abi_version")


def hip_runtime_path() -> str:
    """Path of the libamdhip64 this process has loaded (one runtime expected)."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(line.split()[-1])
    return ";".join(sorted(paths))


def ra_last_error() -> str:
    return lib.ra_last_error().decode()


def ra_abi_version() -> int:
    return lib.ra_abi_version()


def _check(status: int) -> None:
    if status != RA_OK:
        raise RaError(status, ra_last_error())


# ---------------------------------------------------------------------------
# tensor marshalling

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return RA_DTYPE_F32
    if t.dtype == torch.bfloat16:
        return RA_DTYPE_BF16
    raise TypeError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _require(t, name, dtype=None, ndim=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def _spans(spans):
    arr = (ra_span * 2)()
    for i, (a, n) in enumerate(spans):
        arr[i] = ra_span(int(a), int(n))
    return arr


def ra_step(q, k, v, o, lse, qspans, kspans, *, causal: bool, scale: float | None = None,
            accum: bool = False, stream=None) -> None:
    """One ring step: (o, lse) := partial (INIT) or merge((o, lse), partial) (ACCUM).

    qspans/kspans: lists of (global start, length) of q's and k's rows, in
    local order (at most two each).
    """
    torch = _torch()
    _require(q, "q", ndim=4)
    _require(k, "k", dtype=q.dtype, ndim=4)
    _require(v, "v", dtype=q.dtype, ndim=4)
    _require(o, "o", dtype=torch.float32, ndim=4)
    _require(lse, "lse", dtype=torch.float32, ndim=3)
    B, Sq, Hq, D = q.shape
    Sk, Hkv = k.shape[1], k.shape[2]
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D:
        raise ValueError("k and v must be [B, Sk, Hkv, D] matching q")
    if tuple(o.shape) != (B, Sq, Hq, D) or tuple(lse.shape) != (B, Sq, Hq):
        raise ValueError("o must be [B, Sq, Hq, D] and lse [B, Sq, Hq]")
    d = ra_step_desc(_dtype_code(q), B, Hq, Hkv, D, Sq, Sk, 1 if causal else 0,
                     float(scale if scale is not None else D ** -0.5), len(qspans), len(kspans),
                     _spans(qspans), _spans(kspans))
    _check(lib.ra_step(ctypes.byref(d), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                       RA_STEP_ACCUM if accum else RA_STEP_INIT, _stream(stream)))


def ra_rank_forward(q_local, k_shards, v_shards, o, lse, *, S: int, P: int, rank: int, order: str,
                    causal: bool, scale: float | None = None, stream=None) -> None:
    """Rank ``rank``'s P ring steps.  q_local [B, S/P, Hq, D]; k_shards,
    v_shards [P, B, S/P, Hkv, D] (shard p in rank p's local order); o and lse
    are written."""
    torch = _torch()
    _require(q_local, "q_local", ndim=4)
    _require(k_shards, "k_shards", dtype=q_local.dtype, ndim=5)
    _require(v_shards, "v_shards", dtype=q_local.dtype, ndim=5)
    _require(o, "o", dtype=torch.float32, ndim=4)
    _require(lse, "lse", dtype=torch.float32, ndim=3)
    B, s_loc, Hq, D = q_local.shape
    Hkv = k_shards.shape[3]
    if P * s_loc != S:
        raise ValueError("q_local must hold S/P rows")
    if tuple(k_shards.shape) != (P, B, s_loc, Hkv, D) or k_shards.shape != v_shards.shape:
        raise ValueError("k_shards and v_shards must be [P, B, S/P, Hkv, D]")
    if tuple(o.shape) != (B, s_loc, Hq, D) or tuple(lse.shape) != (B, s_loc, Hq):
        raise ValueError("o must be [B, S/P, Hq, D] and lse [B, S/P, Hq]")
    d = ra_rank_desc(_dtype_code(q_local), B, Hq, Hkv, D, S, P, rank, ORDERS[order],
                     1 if causal else 0, float(scale if scale is not None else D ** -0.5))
    _check(lib.ra_rank_forward(ctypes.byref(d), _ptr(q_local), _ptr(k_shards), _ptr(v_shards),
                               _ptr(o), _ptr(lse), _stream(stream)))


def ra_rank_forward_masked(q_local, k_shards, v_shards, o, lse, *, S: int, P: int, rank: int, order: str,
                           causal: bool, scale: float | None = None, window: int = 0, cu_seqlens=None,
                           cu_seqlens_dev=None, stream=None) -> None:
    """ra_rank_forward with a sliding window (``window`` > 0, causal) and/or
    packed sequences (``cu_seqlens``: boundaries 0 = c_0 < ... < c_n = S, a
    sequence of ints; ``cu_seqlens_dev``, optional: the same boundaries in a
    caller-owned int64 GPU tensor, which lets the call be graph-captured).
    bf16 or float32 inputs."""
    torch = _torch()
    _require(q_local, "q_local", ndim=4)
    _require(k_shards, "k_shards", dtype=q_local.dtype, ndim=5)
    _require(v_shards, "v_shards", dtype=q_local.dtype, ndim=5)
    _require(o, "o", dtype=torch.float32, ndim=4)
    _require(lse, "lse", dtype=torch.float32, ndim=3)
    B, s_loc, Hq, D = q_local.shape
    Hkv = k_shards.shape[3]
    if P * s_loc != S:
        raise ValueError("q_local must hold S/P rows")
    if tuple(k_shards.shape) != (P, B, s_loc, Hkv, D) or k_shards.shape != v_shards.shape:
        raise ValueError("k_shards and v_shards must be [P, B, S/P, Hkv, D]")
    if tuple(o.shape) != (B, s_loc, Hq, D) or tuple(lse.shape) != (B, s_loc, Hq):
        raise ValueError("o must be [B, S/P, Hq, D] and lse [B, S/P, Hq]")
    d = ra_rank_desc(_dtype_code(q_local), B, Hq, Hkv, D, S, P, rank, ORDERS[order],
                     1 if causal else 0, float(scale if scale is not None else D ** -0.5))
    m, _keep = _mask(torch, window, cu_seqlens, stream, cu_seqlens_dev)
    _check(lib.ra_rank_forward_masked(ctypes.byref(d), ctypes.byref(m), _ptr(q_local), _ptr(k_shards),
                                      _ptr(v_shards), _ptr(o), _ptr(lse), _stream(stream)))


def _mask(torch, window, cu_seqlens, stream, cu_seqlens_dev=None):
    """An ra_mask and the buffers it points at (keep them alive across the
    call).  ``cu_seqlens_dev``: the caller's device copy of the boundaries
    (int64, contiguous, the same values); without it one is made here with a
    host-to-device copy, which a captured graph cannot hold."""
    host = dev = None
    n = 0
    if cu_seqlens is not None:
        cu = [int(c) for c in cu_seqlens]
        n = len(cu) - 1
        host = (ctypes.c_int64 * len(cu))(*cu)
        if cu_seqlens_dev is not None:
            _require(cu_seqlens_dev, "cu_seqlens_dev", dtype=torch.int64, ndim=1)
            if cu_seqlens_dev.numel() != len(cu):
                raise ValueError("cu_seqlens_dev must hold the same boundaries as cu_seqlens")
            dev = cu_seqlens_dev
        else:
            # allocated on the launch stream, so the stream-ordered allocator
            # keeps it for the kernels enqueued by the call
            with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
                dev = torch.tensor(cu, dtype=torch.int64, device="cuda")
    m = ra_mask(int(window), n, ctypes.cast(host, ctypes.POINTER(ctypes.c_int64)) if host is not None else None,
                dev.data_ptr() if dev is not None else None)
    return m, (host, dev)


def ra_allgather_forward(q_local, k_global, v_global, o, lse, *, S: int, P: int, rank: int, order: str,
                         causal: bool, scale: float | None = None, stream=None) -> None:
    """Rank ``rank``'s attention over the whole sequence in one launch.
    q_local [B, S/P, Hq, D]; k_global, v_global [B, S, Hkv, D] in global token
    order; o and lse are written."""
    torch = _torch()
    _require(q_local, "q_local", ndim=4)
    _require(k_global, "k_global", dtype=q_local.dtype, ndim=4)
    _require(v_global, "v_global", dtype=q_local.dtype, ndim=4)
    _require(o, "o", dtype=torch.float32, ndim=4)
    _require(lse, "lse", dtype=torch.float32, ndim=3)
    B, s_loc, Hq, D = q_local.shape
    Hkv = k_global.shape[2]
    if P * s_loc != S:
        raise ValueError("q_local must hold S/P rows")
    if tuple(k_global.shape) != (B, S, Hkv, D) or k_global.shape != v_global.shape:
        raise ValueError("k_global and v_global must be [B, S, Hkv, D]")
    if tuple(o.shape) != (B, s_loc, Hq, D) or tuple(lse.shape) != (B, s_loc, Hq):
        raise ValueError("o must be [B, S/P, Hq, D] and lse [B, S/P, Hq]")
    d = ra_rank_desc(_dtype_code(q_local), B, Hq, Hkv, D, S, P, rank, ORDERS[order],
                     1 if causal else 0, float(scale if scale is not None else D ** -0.5))
    _check(lib.ra_allgather_forward(ctypes.byref(d), _ptr(q_local), _ptr(k_global), _ptr(v_global),
                                    _ptr(o), _ptr(lse), _stream(stream)))


def ra_rank_backward(q_local, k_shards, v_shards, o, lse, dout, dq, dk_shards, dv_shards, delta, *,
                     S: int, P: int, rank: int, order: str, causal: bool, scale: float | None = None,
                     stream=None) -> None:
    """Backward of rank ``rank``'s ring attention.  q_local, dout
    [B, S/P, Hq, D]; k_shards, v_shards [P, B, S/P, Hkv, D] (one dtype); o,
    lse from ra_rank_forward.  dq [B, S/P, Hq, D] float32 is written;
    dk_shards, dv_shards [P, B, S/P, Hkv, D] float32 are added to; delta
    [B, S/P, Hq] float32 is workspace (written with rowsum(dout * o))."""
    d = _backward_desc(q_local, k_shards, v_shards, o, lse, dout, dq, dk_shards, dv_shards, delta,
                       S=S, P=P, rank=rank, order=order, causal=causal, scale=scale)
    _check(lib.ra_rank_backward(ctypes.byref(d), _ptr(q_local), _ptr(k_shards), _ptr(v_shards), _ptr(o),
                                _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk_shards), _ptr(dv_shards), _ptr(delta),
                                _stream(stream)))


def ra_rank_backward_masked(q_local, k_shards, v_shards, o, lse, dout, dq, dk_shards, dv_shards, delta, *,
                            S: int, P: int, rank: int, order: str, causal: bool, scale: float | None = None,
                            window: int = 0, cu_seqlens=None, cu_seqlens_dev=None, stream=None) -> None:
    """ra_rank_backward under the masks of ra_rank_forward_masked (o, lse
    from that call with the same ``window`` and ``cu_seqlens``)."""
    torch = _torch()
    d = _backward_desc(q_local, k_shards, v_shards, o, lse, dout, dq, dk_shards, dv_shards, delta,
                       S=S, P=P, rank=rank, order=order, causal=causal, scale=scale)
    m, _keep = _mask(torch, window, cu_seqlens, stream, cu_seqlens_dev)
    _check(lib.ra_rank_backward_masked(ctypes.byref(d), ctypes.byref(m), _ptr(q_local), _ptr(k_shards),
                                       _ptr(v_shards), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk_shards),
                                       _ptr(dv_shards), _ptr(delta), _stream(stream)))


RA_NOALLOC_MAX_ROWS = 4194304


def ra_rank_backward_noalloc(q_local, k_shards, v_shards, o, lse, dout, dq, dk_shards, dv_shards, *,
                             S: int, P: int, rank: int, order: str, causal: bool, scale: float | None = None,
                             stream=None) -> None:
    """ra_rank_backward without the delta workspace: the library keeps it in
    its own device scratch (at most RA_NOALLOC_MAX_ROWS = B * S/P * Hq rows),
    so the call allocates nothing.  Calls that overlap on one GPU share that
    scratch and must be ordered by the caller."""
    d = _backward_desc(q_local, k_shards, v_shards, o, lse, dout, dq, dk_shards, dv_shards, None,
                       S=S, P=P, rank=rank, order=order, causal=causal, scale=scale)
    _check(lib.ra_rank_backward_noalloc(ctypes.byref(d), _ptr(q_local), _ptr(k_shards), _ptr(v_shards), _ptr(o),
                                        _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk_shards), _ptr(dv_shards),
                                        _stream(stream)))


def _backward_desc(q_local, k_shards, v_shards, o, lse, dout, dq, dk_shards, dv_shards, delta, *,
                   S, P, rank, order, causal, scale):
    torch = _torch()
    _require(q_local, "q_local", ndim=4)
    for t, n in ((k_shards, "k_shards"), (v_shards, "v_shards")):
        _require(t, n, dtype=q_local.dtype, ndim=5)
    _require(dout, "dout", dtype=q_local.dtype, ndim=4)
    for t, n, nd in ((o, "o", 4), (lse, "lse", 3), (dq, "dq", 4), (dk_shards, "dk_shards", 5),
                     (dv_shards, "dv_shards", 5), (delta, "delta", 3)):
        if t is not None or n != "delta":
            _require(t, n, dtype=torch.float32, ndim=nd)
    B, s_loc, Hq, D = q_local.shape
    Hkv = k_shards.shape[3]
    if P * s_loc != S:
        raise ValueError("q_local must hold S/P rows")
    shard = (P, B, s_loc, Hkv, D)
    if any(tuple(t.shape) != shard for t in (k_shards, v_shards, dk_shards, dv_shards)):
        raise ValueError("k_shards, v_shards, dk_shards, dv_shards must be [P, B, S/P, Hkv, D]")
    if any(tuple(t.shape) != (B, s_loc, Hq, D) for t in (o, dout, dq)):
        raise ValueError("o, dout and dq must be [B, S/P, Hq, D]")
    if tuple(lse.shape) != (B, s_loc, Hq) or (delta is not None and tuple(delta.shape) != (B, s_loc, Hq)):
        raise ValueError("lse and delta must be [B, S/P, Hq]")
    return ra_rank_desc(_dtype_code(q_local), B, Hq, Hkv, D, S, P, rank, ORDERS[order],
                        1 if causal else 0, float(scale if scale is not None else D ** -0.5))


def ra_lse_merge(o_a, lse_a, o_b, lse_b, o_out, lse_out, *, stream=None) -> None:
    """Element-wise merge of two partials; o_* [..., D] and lse_* [...] float32.
    o_out may be o_a or o_b (in place)."""
    torch = _torch()
    for t, n in ((o_a, "o_a"), (o_b, "o_b"), (o_out, "o_out"), (lse_a, "lse_a"), (lse_b, "lse_b"),
                 (lse_out, "lse_out")):
        _require(t, n, dtype=torch.float32)
    D = o_a.shape[-1] if o_a.dim() else 0
    rows = o_a.numel() // D if D else 0
    if o_b.shape != o_a.shape or o_out.shape != o_a.shape:
        raise ValueError("o_a, o_b, o_out must have the same shape")
    for t in (lse_a, lse_b, lse_out):
        if t.numel() != rows:
            raise ValueError("lse tensors must hold one value per row of o")
    _check(lib.ra_lse_merge(rows, D, _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b),
                            _ptr(o_out), _ptr(lse_out), _stream(stream)))


def ra_ulysses_relayout(x, out, P_u: int, direction: int = RA_SEQ2HEAD, *, stream=None) -> None:
    """SEQ2HEAD: x [B, s_loc, H, D] -> out [P_u, B, s_loc, H/P_u, D];
    HEAD2SEQ: x [P_u, B, s_loc, H/P_u, D] -> out [B, s_loc, H, D]."""
    _require(x, "x")
    _require(out, "out", dtype=x.dtype)
    if direction == RA_SEQ2HEAD:
        if x.dim() != 4:
            raise ValueError("x must be [B, s_loc, H, D]")
        B, s_loc, H, D = x.shape
        want = (P_u, B, s_loc, H // P_u, D) if P_u > 0 and H % P_u == 0 else None
    elif direction == RA_HEAD2SEQ:
        if x.dim() != 5 or x.shape[0] != P_u:
            raise ValueError("x must be [P_u, B, s_loc, H/P_u, D]")
        _, B, s_loc, hp, D = x.shape
        H = hp * P_u
        want = (B, s_loc, H, D)
    else:
        raise ValueError("direction must be RA_SEQ2HEAD or RA_HEAD2SEQ")
    if want is not None and tuple(out.shape) != want:
        raise ValueError(f"out must have shape {want}")
    _check(lib.ra_ulysses_relayout(direction, x.element_size(), B, s_loc, H, D, P_u, _ptr(x),
                                   _ptr(out), _stream(stream)))


def ra_ulysses_pieces(tensors, pieces, P_u: int, *, to_pieces: bool, group: int, stream=None) -> None:
    """Messages of one Ulysses all-to-all for up to 4 tensors in one launch.

    group RA_GROUP_HEADS: tensors [B, s_loc, H_i, D_i] (any dtype); piece j
    section i is [B, s_loc, H_i/P_u, D_i] (head block j).  group RA_GROUP_SEQ:
    tensors [B, P_u*s_loc, Hp_i, D_i]; piece u section i is [B, s_loc, Hp_i,
    D_i] (token block u).  pieces: a contiguous buffer of P_u pieces (bytes
    in any dtype).  to_pieces selects the direction."""
    if not 1 <= len(tensors) <= 4:
        raise ValueError("1 to 4 tensors")
    t0 = tensors[0]
    B = t0.shape[0]
    runs = []
    for t in tensors:
        _require(t, "tensor", ndim=4)
        if t.shape[0] != B:
            raise ValueError("tensors must share the batch dimension")
        per_token = t.shape[2] * t.shape[3] * t.element_size()
        if group == RA_GROUP_HEADS:
            if t.shape[2] % P_u:
                raise ValueError("heads must be divisible by P_u")
            runs.append(per_token // P_u)
        else:
            runs.append(per_token)
    n_tok = t0.shape[1]
    if any(t.shape[1] != n_tok for t in tensors):
        raise ValueError("tensors must share the token dimension")
    if group == RA_GROUP_SEQ:
        if n_tok % P_u:
            raise ValueError("tokens must be divisible by P_u")
        s_loc = n_tok // P_u
    else:
        s_loc = n_tok
    need = P_u * B * s_loc * sum(runs)
    if not pieces.is_contiguous() or pieces.numel() * pieces.element_size() != need:
        raise ValueError(f"pieces must be a contiguous buffer of {need} bytes")
    ptrs = (ctypes.c_void_p * len(tensors))(*[t.data_ptr() for t in tensors])
    rb = (ctypes.c_int64 * len(tensors))(*runs)
    _check(lib.ra_ulysses_pieces(1 if to_pieces else 0, group, B, s_loc, P_u, len(tensors), ptrs, rb,
                                 _ptr(pieces), _stream(stream)))


def ra_plan(order: str, S: int, P: int, rank: int, step: int, causal: bool, tile_q: int,
            tile_k: int) -> dict:
    """Host plan of one ring step (no GPU work)."""
    out = ra_plan_out()
    _check(lib.ra_plan(ORDERS[order] if isinstance(order, str) else int(order), S, P, rank, step,
                       1 if causal else 0, tile_q, tile_k, ctypes.byref(out)))
    return {
        "src": out.src,
        "qspans": [(out.qspans[i].start, out.qspans[i].len) for i in range(out.n_qspans)],
        "kspans": [(out.kspans[i].start, out.kspans[i].len) for i in range(out.n_kspans)],
        "classes": [[CLASS_NAMES[out.pair_class[i][j]] for j in range(out.n_kspans)]
                    for i in range(out.n_qspans)],
        "tiles": {"FULL": out.tiles_full, "DIAG": out.tiles_diag, "SKIP": out.tiles_skip},
    }


def rank_spans(order: str, S: int, P: int, rank: int):
    """Global spans of ``rank``'s rows, from the library's plan."""
    return ra_plan(order, S, P, rank, 0, True, 1 << 30, 1 << 30)["qspans"]


def ra_rank_launches(*, dtype: str, B: int, Hq: int, Hkv: int, D: int, S: int, P: int, rank: int, order: str,
                     causal: bool, backward: bool = False, n_cus: int = 0, window: int = 0,
                     cu_seqlens=None) -> list:
    """Which kernel each ring step of ra_rank_forward (or ra_rank_backward)
    launches, as a list of P dicts in step order (host-only).  ``n_cus`` = 0
    asks the current device for its compute units; > 0 plans for that many.
    ``window`` / ``cu_seqlens`` as for the masked calls (only the host copy
    of the boundaries is read)."""
    d = ra_rank_desc(RA_DTYPE_BF16 if dtype == "bf16" else RA_DTYPE_F32, B, Hq, Hkv, D, S, P, rank,
                     ORDERS[order], 1 if causal else 0, float(D ** -0.5))
    host = None
    n = 0
    if cu_seqlens is not None:
        cu = [int(c) for c in cu_seqlens]
        n = len(cu) - 1
        host = (ctypes.c_int64 * len(cu))(*cu)
    # the device copy is not read by the plan; the host copy stands in for it
    # so that the mask passes the same checks as in a real call
    m = ra_mask(int(window), n, ctypes.cast(host, ctypes.POINTER(ctypes.c_int64)) if host is not None else None,
                ctypes.cast(host, ctypes.c_void_p).value if host is not None else None)
    out = (ra_launch_info * P)()
    _check(lib.ra_rank_launches(ctypes.byref(d), ctypes.byref(m) if (window or n) else None,
                                1 if backward else 0, int(n_cus), out))
    return [{"kernel": KERNEL_NAMES[o.kernel], "masked": bool(o.masked), "items": o.items, "grid": o.grid,
             "lpt": bool(o.lpt), "first_heavy": bool(o.first_heavy)} for o in out]
