"""Throughput of one rank's blockwise ring attention on one MI355X.

A step is one ra_rank_forward call: rank 0 of a 131,072-token causal zigzag
ring of 16 ranks (bf16, batch 1, 32 query heads over 8 K/V heads, head dim 128,
8,192 local query rows), all 16 ring steps with their fused log-sum-exp merges.
Inputs are seeded synthetic tensors already resident in HBM.  The value is
algorithmic TFLOP/s: 4*D FLOPs per visible (query, key) pair per head, divided
by the measured time (pairs hidden by the causal mask are not counted).

Also reported:
  ms_per_step_median / _min  of the timed steps (value uses their mean);
  roofline      the step kernel against the bf16 dense MFMA peak: the same
                ring's launches issued one by one (the ra_step calls
                ra_rank_forward makes) with HIP events around each launch on
                its stream, algorithmic FLOPs over the kernels' own time, and
                the same against the peak scaled to the GFX clock sampled
                under load;
  clock         the GFX clock (amd-smi) while the ring runs back to back;
  cpu_baseline  the CPU oracle (float64 numpy) timed on a sample of rows;
  configs       the other workloads' rings (32k, 64k non-causal, 524k);
  aux           the all-gather form, windowed ring, backward, HIP-graph
                replay, and HBM rates of the merge and the Ulysses kernels.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
METRIC = "attention TFLOPS per rank-share (1 GPU) and % of bf16 MFMA peak"
KERNEL_SOURCES = ["ring_attention_blockwise_amd/csrc/attn_step_bf16.hip",
                  "ring_attention_blockwise_amd/csrc/attn_common.h",
                  "ring_attention_blockwise_amd/csrc/ra_internal.h"]
KERNEL_NAME = "attn_step_bf16_kernel<128, false>"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_step_traffic.json")
# the other workloads of the method timed beside the headline (rank 0 each)
CONFIG_LEGS = ["bf16_gqa32x8_d128_s32k_ring8_zigzag_causal", "bf16_mha16_b2_d128_s64k_ring8_contiguous_full",
               "bf16_gqa32x8_d128_s512k_ring32_zigzag_causal_khalf"]


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(workload_name):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source for this workload."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_hash() or t.get("workload") != workload_name:
        return None
    return t.get("bytes_per_launch")


def to_device(x, dtype):
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda().view(torch.bfloat16)


def build_inputs(ra, w, rank):
    import torch
    import seeded_inputs as si
    s_loc = w.S // w.P
    q = to_device(si.tokens(w.seed_id, si.TENSOR_Q, w.B, w.S, w.Hq, w.D,
                            ra.rank_spans(w.order, w.S, w.P, rank), w.dtype), w.dtype)
    shards = []
    for tid, scale in ((si.TENSOR_K, w.k_scale), (si.TENSOR_V, 1.0)):
        out = torch.empty((w.P, w.B, s_loc, w.Hkv, w.D), dtype=q.dtype, device="cuda")
        for p in range(w.P):
            out[p] = to_device(si.tokens(w.seed_id, tid, w.B, w.S, w.Hkv, w.D,
                                         ra.rank_spans(w.order, w.S, w.P, p), w.dtype, scale=scale),
                               w.dtype)
        shards.append(out)
    o = torch.empty((w.B, s_loc, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, s_loc, w.Hq), dtype=torch.float32, device="cuda")
    return q, shards[0], shards[1], o, lse


def launches_per_step(ra, w, rank):
    """Steps of the ring that launch the kernel (a step whose whole block is
    masked is skipped by ra_rank_forward)."""
    n = 0
    for s in range(w.P):
        plan = ra.ra_plan(w.order, w.S, w.P, rank, s, w.causal, 1 << 30, 1 << 30)
        if s == 0 or any(c != "SKIP" for row in plan["classes"] for c in row):
            n += 1
    return n


def span_pairs(qa, qn, ka, kn, causal):
    """Visible (query, key) pairs between query positions [qa, qa+qn) and key
    positions [ka, ka+kn): all of them, or under the causal rule (key <= query)
    the sum over queries t of the keys of the span at or before t."""
    if qn <= 0 or kn <= 0:
        return 0
    if not causal:
        return qn * kn
    total = 0
    # queries before ka see nothing; from ka + kn - 1 on they see all kn keys
    t0, t1 = max(qa, ka), qa + qn - 1
    if t1 < t0:
        return 0
    full_from = max(t0, ka + kn - 1)
    if full_from <= t1:
        total += (t1 - full_from + 1) * kn
    lo, hi = t0, min(t1, ka + kn - 2)
    if hi >= lo:                       # query t sees t - ka + 1 keys
        n = hi - lo + 1
        total += n * (lo - ka + 1) + n * (n - 1) // 2
    return total


def step_flops(ra, w, rank, step):
    """Algorithmic FLOPs of one ring step: 4 D per visible pair per (batch,
    head), pairs of the rank's query spans against the held shard's key
    spans."""
    plan = ra.ra_plan(w.order, w.S, w.P, rank, step, w.causal, 1 << 30, 1 << 30)
    pairs = sum(span_pairs(a, n, b, m, w.causal) for a, n in plan["qspans"] for b, m in plan["kspans"])
    return 4.0 * w.D * w.B * w.Hq * pairs, plan


def algorithmic_flops(w, rank):
    """4*D per visible pair per (batch, head), pairs from the closed forms of
    the chunk maps (zigzag: c(S+1) per rank; contiguous: s^2 r + s(s+1)/2)."""
    s_loc = w.S // w.P
    if not w.causal:
        pairs = s_loc * w.S
    elif w.order == "zigzag":
        c = w.S // (2 * w.P)
        pairs = c * (w.S + 1)
    else:
        pairs = s_loc * s_loc * rank + s_loc * (s_loc + 1) // 2
    return 4.0 * w.D * w.B * w.Hq * pairs


def time_attention(ra, w, rank, steps, warmup):
    import torch
    q, ks, vs, o, lse = build_inputs(ra, w, rank)
    stream = torch.cuda.current_stream()

    def step():
        ra.ra_rank_forward(q, ks, vs, o, lse, S=w.S, P=w.P, rank=rank, order=w.order,
                           causal=w.causal, scale=w.scale, stream=stream)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in ev]   # ms, HIP events on the launch stream
    ok = bool(torch.isfinite(o).all().item() and torch.isfinite(lse).all().item())
    del q, ks, vs, o, lse
    torch.cuda.empty_cache()
    return wall, per, ok


def time_launches(ra, w, rank, steps):
    """Per-launch durations of the step kernel on the same ring: each ring
    step issued as the ra_step call that ra_rank_forward makes for it (INIT
    at step 0, ACCUM after; steps whose held block is hidden are not
    launched), with HIP events on the launch stream around every launch,
    ``steps`` times over.  Returns [(step, flops, [ms per repetition])]."""
    import torch
    q, ks, vs, o, lse = build_inputs(ra, w, rank)
    stream = torch.cuda.current_stream()
    launches = []
    for s in range(w.P):
        flops, plan = step_flops(ra, w, rank, s)
        if s > 0 and flops == 0:
            continue
        launches.append((s, flops, plan))
    ev = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in launches]
          for _ in range(steps + 1)]
    for rep in range(steps + 1):          # repetition 0 warms up
        for (s, _, plan), (a, b) in zip(launches, ev[rep]):
            src = plan["src"]
            a.record(stream)
            ra.ra_step(q, ks[src], vs[src], o, lse, plan["qspans"], plan["kspans"], causal=w.causal,
                       scale=w.scale, accum=s > 0, stream=stream)
            b.record(stream)
    torch.cuda.synchronize()
    out = [(s, flops, [ev[rep][i][0].elapsed_time(ev[rep][i][1]) for rep in range(1, steps + 1)])
           for i, (s, flops, _) in enumerate(launches)]
    del q, ks, vs, o, lse
    torch.cuda.empty_cache()
    return out


def sample_clock(ra, w, rank, seconds=1.5, settle=0.5):
    """GFX clocks (MHz) of the 8 XCDs, sampled with amd-smi while the same
    ring runs back to back for about ``seconds`` after ``settle`` seconds of
    the same load (the metrics lag: right after idle they still read the idle
    boost clock).  ``current_gfxclk`` is the first XCD's alone and the XCDs
    differ by up to ~7% under load, so each sample takes the mean and the
    minimum over ``current_gfxclks``; a launch ends with its slowest XCD.
    None where amd-smi is not available."""
    import threading
    import torch
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        h = amdsmi.amdsmi_get_processor_handles()[0]
    except Exception:          # noqa: BLE001 - the clock is a report, not a result
        return None
    q, ks, vs, o, lse = build_inputs(ra, w, rank)
    samples, stop, record = [], threading.Event(), threading.Event()

    def poll():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(h)
                cs = m.get("current_gfxclks")
                if not isinstance(cs, (list, tuple)):
                    cs = [m.get("current_gfxclk")]
                cs = [float(c) for c in cs if isinstance(c, (int, float)) and 0 < c < 10000]
                if cs and record.is_set():
                    samples.append((sum(cs) / len(cs), min(cs), len(cs)))
            except Exception:  # noqa: BLE001
                pass
            stop.wait(0.02)

    t = threading.Thread(target=poll)
    t0 = time.perf_counter()
    t.start()
    while time.perf_counter() - t0 < settle + seconds:
        if time.perf_counter() - t0 >= settle:
            record.set()
        for _ in range(20):
            ra.ra_rank_forward(q, ks, vs, o, lse, S=w.S, P=w.P, rank=rank, order=w.order, causal=w.causal,
                               scale=w.scale)
        torch.cuda.synchronize()
    stop.set()
    t.join()
    try:
        amdsmi.amdsmi_shut_down()
    except Exception:  # noqa: BLE001
        pass
    del q, ks, vs, o, lse
    torch.cuda.empty_cache()
    if not samples:
        return None
    means = sorted(x[0] for x in samples)
    mins = sorted(x[1] for x in samples)
    return {"gfxclk_mhz_median": round(means[len(means) // 2], 1), "gfxclk_mhz_min": round(means[0], 1),
            "gfxclk_mhz_max": round(means[-1], 1), "slowest_xcd_mhz_median": round(mins[len(mins) // 2], 1),
            "xcds": samples[0][2], "samples": len(samples),
            "source": "amdsmi current_gfxclks, mean over the XCDs per sample, after the load settled"}


def time_allgather(ra, w, rank, ring_ms, reps=5):
    """The all-gather form of the same rank's work: one launch over the whole
    resident sequence, no per-step merge.  Against the ring it shows what the
    per-step launches and fused merges cost."""
    import torch
    import seeded_inputs as si
    q = to_device(si.tokens(w.seed_id, si.TENSOR_Q, w.B, w.S, w.Hq, w.D,
                            ra.rank_spans(w.order, w.S, w.P, rank), w.dtype), w.dtype)
    kg = to_device(si.tokens(w.seed_id, si.TENSOR_K, w.B, w.S, w.Hkv, w.D, [(0, w.S)], w.dtype,
                             scale=w.k_scale), w.dtype)
    vg = to_device(si.tokens(w.seed_id, si.TENSOR_V, w.B, w.S, w.Hkv, w.D, [(0, w.S)], w.dtype), w.dtype)
    o = torch.empty((w.B, w.S // w.P, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.S // w.P, w.Hq), dtype=torch.float32, device="cuda")

    def run():
        ra.ra_allgather_forward(q, kg, vg, o, lse, S=w.S, P=w.P, rank=rank, order=w.order,
                                causal=w.causal, scale=w.scale)

    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = algorithmic_flops(w, rank)
    del q, kg, vg, o, lse
    torch.cuda.empty_cache()
    return {"kernel": "allgather_forward", "ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "frac_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "ring_ms": ring_ms,
            "ring_over_allgather": ring_ms / ms}


def time_backward(ra, w, rank, reps=3, window=0):
    """The backward pass of the same rank (reverse ring, dQ and dK/dV
    kernels per step), after one forward; with ``window`` > 0 both under a
    causal sliding window.  Algorithmic work: 2.5 times the forward's (five
    products per visible pair instead of two)."""
    import torch
    import seeded_inputs as si
    q, ks, vs, o, lse = build_inputs(ra, w, rank)
    do = to_device(si.tokens(w.seed_id, si.TENSOR_DO, w.B, w.S, w.Hq, w.D,
                             ra.rank_spans(w.order, w.S, w.P, rank), w.dtype), w.dtype)
    s_loc = w.S // w.P
    dq = torch.empty((w.B, s_loc, w.Hq, w.D), dtype=torch.float32, device="cuda")
    dk = torch.zeros((w.P, w.B, s_loc, w.Hkv, w.D), dtype=torch.float32, device="cuda")
    dv = torch.zeros_like(dk)
    delta = torch.empty((w.B, s_loc, w.Hq), dtype=torch.float32, device="cuda")
    kw = dict(S=w.S, P=w.P, rank=rank, order=w.order, causal=w.causal, scale=w.scale)
    if window:
        kw["window"] = window
        ra.ra_rank_forward_masked(q, ks, vs, o, lse, **kw)
    else:
        ra.ra_rank_forward(q, ks, vs, o, lse, **kw)

    def run():
        if window:
            ra.ra_rank_backward_masked(q, ks, vs, o, lse, do, dq, dk, dv, delta, **kw)
        else:
            ra.ra_rank_backward(q, ks, vs, o, lse, do, dq, dk, dv, delta, **kw)

    run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = 2.5 * (4.0 * w.D * w.B * w.Hq * masked_pairs(w, rank, window) if window else algorithmic_flops(w, rank))
    ok = bool(torch.isfinite(dq).all().item() and torch.isfinite(dk).all().item())
    del q, ks, vs, o, lse, do, dq, dk, dv, delta
    torch.cuda.empty_cache()
    return {"kernel": f"rank_backward_window{window}" if window else "rank_backward", "ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "frac_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, "finite": ok}


def masked_pairs(w, rank, window):
    """Visible (query, key) pairs per (batch, head) of one rank under a
    causal sliding window: query t sees min(t + 1, window) keys."""
    spans = []
    if w.order == "zigzag":
        c = w.S // (2 * w.P)
        spans = [(rank * c, c), ((2 * w.P - 1 - rank) * c, c)]
    else:
        c = w.S // w.P
        spans = [(rank * c, c)]
    t = np.concatenate([np.arange(a, a + n, dtype=np.int64) for a, n in spans])
    return int(np.minimum(t + 1, window).sum())


def time_window(ra, w, rank, window, reps=10, warmup=3):
    """The same rank's ring with a causal sliding window: masked tiles at both
    ends of each row's key range, hidden tiles and steps skipped."""
    import torch
    q, ks, vs, o, lse = build_inputs(ra, w, rank)
    kw = dict(S=w.S, P=w.P, rank=rank, order=w.order, causal=True, scale=w.scale, window=window)
    for _ in range(warmup):
        ra.ra_rank_forward_masked(q, ks, vs, o, lse, **kw)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        ra.ra_rank_forward_masked(q, ks, vs, o, lse, **kw)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    flops = 4.0 * w.D * w.B * w.Hq * masked_pairs(w, rank, window)
    del q, ks, vs, o, lse
    torch.cuda.empty_cache()
    return {"kernel": f"rank_forward_window{window}", "ms": ms, "TFLOP/s": flops / (ms * 1e-3) / 1e12,
            "frac_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def time_graph(ra, name, rank, reps=20):
    """A smaller ring, eager against HIP-graph replay: the 32k-token zigzag
    ring of 8 (about 0.1 ms of work per step) captured once as a graph of its
    launches (the library allocates nothing and records no memset)."""
    import torch
    from seeded_inputs import workload
    w = workload(name)
    q, ks, vs, o, lse = build_inputs(ra, w, rank)
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    kw = dict(S=w.S, P=w.P, rank=rank, order=w.order, causal=w.causal, scale=w.scale, stream=stream)

    def eager():
        ra.ra_rank_forward(q, ks, vs, o, lse, **kw)

    res = {}
    with torch.cuda.stream(stream):
        for _ in range(3):
            eager()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            eager()
        for mode, run in (("eager", eager), ("graph", g.replay)):
            run()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                run()
            b.record(stream)
            b.synchronize()
            res[mode] = a.elapsed_time(b) / reps
    torch.cuda.synchronize()
    flops = algorithmic_flops(w, rank)
    del q, ks, vs, o, lse, g
    torch.cuda.empty_cache()
    return {"kernel": "rank_forward_32k_graph", "workload": name, "ms": res["graph"], "eager_ms": res["eager"],
            "TFLOP/s": flops / (res["graph"] * 1e-3) / 1e12,
            "eager_TFLOP/s": flops / (res["eager"] * 1e-3) / 1e12,
            "frac_peak": flops / (res["graph"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}


def time_config(ra, name, rank, reps=10, warmup=3):
    """Another workload's ring: rank ``rank``'s forward (all steps, fused
    merges), eager, HIP events around each call after ``warmup`` untimed
    calls on the freshly allocated inputs; mean, median and min."""
    import torch
    from seeded_inputs import workload
    w = workload(name)
    q, ks, vs, o, lse = build_inputs(ra, w, rank)
    kw = dict(S=w.S, P=w.P, rank=rank, order=w.order, causal=w.causal, scale=w.scale)
    for _ in range(warmup):
        ra.ra_rank_forward(q, ks, vs, o, lse, **kw)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        ra.ra_rank_forward(q, ks, vs, o, lse, **kw)
        b.record()
    torch.cuda.synchronize()
    per = [a.elapsed_time(b) for a, b in ev]
    ms = float(np.mean(per))
    flops = algorithmic_flops(w, rank)
    kinds = sorted({s["kernel"] for s in ra.ra_rank_launches(dtype=w.dtype, B=w.B, Hq=w.Hq, Hkv=w.Hkv, D=w.D,
                                                               S=w.S, P=w.P, rank=rank, order=w.order,
                                                               causal=w.causal)} - {"none"})
    del q, ks, vs, o, lse
    torch.cuda.empty_cache()
    return {"kernel": f"rank_forward_{w.S // 1024}k_{'causal' if w.causal else 'noncausal'}", "workload": name,
            "rank": rank, "ms": ms, "ms_median": float(np.median(per)), "ms_min": float(min(per)),
            "TFLOP/s": flops / (ms * 1e-3) / 1e12, "frac_peak": flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "step_kernels": kinds}


def time_merge(ra, rows, D, reps=20):
    """Standalone merge, rotating buffer sets so the working set exceeds the
    256 MB Infinity Cache."""
    import torch
    per_call = rows * (12 * D + 12)
    nsets = max(2, int(np.ceil(1.2e9 / per_call)))
    sets = []
    g = torch.Generator(device="cuda").manual_seed(0)
    for _ in range(nsets):
        sets.append(tuple(torch.randn(rows, D, device="cuda", generator=g) for _ in range(3)) +
                    tuple(torch.randn(rows, device="cuda", generator=g) for _ in range(3)))
    for s in sets:
        ra.ra_lse_merge(s[0], s[3], s[1], s[4], s[2], s[5])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        s = sets[i % nsets]
        ra.ra_lse_merge(s[0], s[3], s[1], s[4], s[2], s[5])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    del sets
    torch.cuda.empty_cache()
    return {"kernel": "lse_merge", "rows": rows, "D": D, "bytes": per_call, "us": ms * 1e3,
            "GB/s": per_call / (ms * 1e-3) / 1e9, "frac_hbm": per_call / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def time_relayout(ra, B, s_loc, H, D, P_u, reps=20):
    import torch
    nbytes = B * s_loc * H * D * 2
    nsets = max(2, int(np.ceil(1.2e9 / (2 * nbytes))))
    xs = [torch.randn(B, s_loc, H, D, device="cuda").to(torch.bfloat16) for _ in range(nsets)]
    ys = [torch.empty(P_u, B, s_loc, H // P_u, D, device="cuda", dtype=torch.bfloat16) for _ in range(nsets)]
    for x, y in zip(xs, ys):
        ra.ra_ulysses_relayout(x, y, P_u, ra.RA_SEQ2HEAD)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(reps):
        ra.ra_ulysses_relayout(xs[i % nsets], ys[i % nsets], P_u, ra.RA_SEQ2HEAD)
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    moved = 2 * nbytes
    del xs, ys
    torch.cuda.empty_cache()
    return {"kernel": "ulysses_relayout_seq2head", "shape": [B, s_loc, H, D], "P_u": P_u, "bytes": moved,
            "us": ms * 1e3, "GB/s": moved / (ms * 1e-3) / 1e9,
            "frac_hbm": moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS}


def time_ulysses_pieces(ra, B, s_loc, H, D, P_u, reps=20):
    """Fused Q/K/V messages of the Ulysses all-to-all (one launch for three
    bf16 tensors): the sender's pack of [B, s_loc, H, D] shards into head
    blocks, and the receiver's regrouping of the pieces into all
    P_u * s_loc tokens of its H / P_u heads.  Buffer sets rotate past the
    Infinity Cache."""
    import torch
    nbytes = B * s_loc * H * D * 2
    nsets = max(2, int(np.ceil(1.2e9 / (6 * nbytes))))
    res = []
    for group, name, shape, to_pieces in (
            (ra.RA_GROUP_HEADS, "ulysses_pack_qkv", (B, s_loc, H, D), True),
            (ra.RA_GROUP_SEQ, "ulysses_regroup_qkv", (B, P_u * s_loc, H // P_u, D), False)):
        sets = [([torch.randn(shape, device="cuda").to(torch.bfloat16) for _ in range(3)],
                 torch.empty(3 * nbytes, dtype=torch.uint8, device="cuda")) for _ in range(nsets)]
        for xs, buf in sets:
            ra.ra_ulysses_pieces(xs, buf, P_u, to_pieces=to_pieces, group=group)
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            xs, buf = sets[i % nsets]
            ra.ra_ulysses_pieces(xs, buf, P_u, to_pieces=to_pieces, group=group)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        moved = 2 * 3 * nbytes
        res.append({"kernel": name, "shape": list(shape), "tensors": 3, "P_u": P_u, "bytes": moved,
                    "us": ms * 1e3, "GB/s": moved / (ms * 1e-3) / 1e9,
                    "frac_hbm": moved / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS})
        del sets
        torch.cuda.empty_cache()
    return res


def blas_threads():
    """Threads numpy's BLAS runs the oracle's products with (the host cores
    the oracle uses; its element-wise work is single-threaded numpy)."""
    try:
        import threadpoolctl
        n = [i["num_threads"] for i in threadpoolctl.threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:  # noqa: BLE001
        pass
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count()


def blas_vendor():
    """numpy's BLAS (name and version) as numpy reports it."""
    try:
        cfg = np.show_config(mode="dicts")
        b = cfg["Build Dependencies"]["blas"]
        return f"{b.get('name')} {b.get('version')}"
    except Exception:  # noqa: BLE001 - a report field only
        return None


def cpu_baseline(w, rank, target_s=15.0):
    """The CPU oracle, as it stands, on a bounded sample of rank ``rank``'s rows
    (all heads), scaled to TFLOP/s by the algorithmic FLOPs of those rows."""
    import seeded_inputs as si
    from oracle import attention as oa
    from oracle import index_maps as im
    pos = im.rank_positions(w.S, w.P, rank, w.order)
    rng = np.random.default_rng(1234)
    Kg = si.tokens(w.seed_id, si.TENSOR_K, w.B, w.S, w.Hkv, w.D, [(0, w.S)], w.dtype, scale=w.k_scale)
    Vg = si.tokens(w.seed_id, si.TENSOR_V, w.B, w.S, w.Hkv, w.D, [(0, w.S)], w.dtype)
    Kf, Vf = si.to_f64(Kg, w.dtype), si.to_f64(Vg, w.dtype)
    del Kg, Vg
    done_flops, done_s, rows_done = 0.0, 0.0, 0
    while done_s < target_s and rows_done < pos.size:
        rows = np.sort(rng.choice(pos.size, 16, replace=False))
        qsel = pos[rows]
        q = si.to_f64(si.tokens(w.seed_id, si.TENSOR_Q, w.B, w.S, w.Hq, w.D,
                                [(int(t), 1) for t in qsel], w.dtype), w.dtype)
        t0 = time.perf_counter()
        oa.attention_rows(q, qsel, Kf, Vf, np.arange(w.S), w.causal, w.scale)
        done_s += time.perf_counter() - t0
        vis = (qsel + 1).sum() if w.causal else qsel.size * w.S
        done_flops += 4.0 * w.D * w.B * w.Hq * float(vis)
        rows_done += rows.size
    return {"value": done_flops / done_s / 1e12, "unit": "TFLOP/s", "cores": blas_threads(), "kind": "oracle",
            "blas": blas_vendor(),
            "sample": f"{rows_done} random query rows of rank {rank} x {w.Hq} heads x all visible keys, "
                      f"float64 numpy, {done_s:.1f} s"}


def cpu_aux_baselines(w, rank):
    """The merge, relayout and backward oracles as they stand, timed on the
    host on the shapes the GPU legs use (bounded samples; float64 numpy)."""
    import seeded_inputs as si
    from oracle import attention as oa
    from oracle import attention_backward as ob
    from oracle import index_maps as im
    from oracle import relayout as rl
    out = []
    rng = np.random.default_rng(5)
    rows = w.B * (w.S // w.P) * w.Hq // 8        # an eighth of the merge's rows
    oa_, ob_ = rng.standard_normal((rows, w.D)), rng.standard_normal((rows, w.D))
    la, lb = rng.standard_normal(rows), rng.standard_normal(rows)
    t0 = time.perf_counter()
    oa.lse_merge(oa_, la, ob_, lb)
    dt = time.perf_counter() - t0
    nbytes = rows * (12 * w.D + 12)
    out.append({"kernel": "lse_merge", "kind": "oracle", "rows": rows, "GB/s": nbytes / dt / 1e9,
                "sample": f"{rows} rows x {w.D} (float64 inputs; bytes counted as the GPU's float32 ones)"})
    x = rng.standard_normal((2, 8192, 16, 128)).astype(np.float32).view(np.uint32).astype(np.uint16)
    t0 = time.perf_counter()
    rl.seq2head(x, 8)
    dt = time.perf_counter() - t0
    out.append({"kernel": "ulysses_relayout_seq2head", "kind": "oracle", "GB/s": 2 * x.nbytes / dt / 1e9,
                "sample": "[2, 8192, 16, 128] 2-byte elements, P_u = 8"})
    pos = im.rank_positions(w.S, w.P, rank, w.order)
    sel = np.sort(rng.choice(pos.size, 4, replace=False))
    qsel = pos[sel]
    kmax = int(qsel.max()) + 1
    q = si.to_f64(si.tokens(w.seed_id, si.TENSOR_Q, w.B, w.S, w.Hq, w.D, [(int(t), 1) for t in qsel], w.dtype), w.dtype)
    do = si.to_f64(si.tokens(w.seed_id, si.TENSOR_DO, w.B, w.S, w.Hq, w.D, [(int(t), 1) for t in qsel], w.dtype),
                   w.dtype)
    K = si.to_f64(si.tokens(w.seed_id, si.TENSOR_K, w.B, w.S, w.Hkv, w.D, [(0, kmax)], w.dtype, scale=w.k_scale),
                  w.dtype)
    V = si.to_f64(si.tokens(w.seed_id, si.TENSOR_V, w.B, w.S, w.Hkv, w.D, [(0, kmax)], w.dtype), w.dtype)
    t0 = time.perf_counter()
    ob.attention_grads(q, K, V, do, w.causal, w.scale, qpos=qsel, kpos=np.arange(kmax))
    dt = time.perf_counter() - t0
    vis = (qsel + 1).sum() if w.causal else qsel.size * w.S
    flops = 2.5 * 4.0 * w.D * w.B * w.Hq * float(vis)
    out.append({"kernel": "rank_backward", "kind": "oracle", "TFLOP/s": flops / dt / 1e12,
                "sample": f"{sel.size} random query rows of rank {rank} x {w.Hq} heads, all visible keys"})
    return out


# --------------------------------------------------------------------------
# Summaries of rocprofv3 output (host only: they read the CSV files a profiled
# run of this script wrote, and print or write the figures kept in profiles/).

def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True)):
        with open(f, newline="") as fh:
            rows.extend(dict(r, _file=f) for r in csv.DictReader(fh))
    return rows


def _short_kernel(name):
    """Kernel name without 'void ', namespaces and the parameter list."""
    n = name.strip()
    if n.startswith("void "):
        n = n[5:]
    if n.endswith(")"):         # the parameter list: the '(...)' that ends the name
        depth = 0
        for i in range(len(n) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(n[i], 0)
            if depth == 0:
                n = n[:i]
                break
    for ns in ("ra::(anonymous namespace)::", "ra::"):
        n = n.replace(ns, "")
    return n


def trace_summary(d, warmup, steps, kernel=KERNEL_NAME):
    """Markdown table of a --kernel-trace run of this script (``--no-aux``):
    every kernel's launches, and the step kernel's average over the timed
    dispatches only.  The script launches the step kernel per ring step in
    this order: ``warmup`` untimed steps, ``steps`` timed steps, then the
    per-launch leg's one untimed and ``steps`` timed repetitions."""
    rows = _csv_rows(d, "kernel_trace.csv")
    per = {}
    for r in rows:
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        per.setdefault(_short_kernel(r["Kernel_Name"]), []).append((int(r["Dispatch_Id"]), us))
    total = sum(u for v in per.values() for _, u in v)
    out = ["| kernel | calls | avg us | median us | min us | max us | share |", "|---|---|---|---|---|---|---|"]
    for k, v in sorted(per.items(), key=lambda kv: -sum(u for _, u in kv[1])):
        us = [u for _, u in v]
        name = k if len(k) <= 100 else k[:97] + "..."   # library template names run to kilobytes
        out.append(f"| `{name}` | {len(us)} | {np.mean(us):.1f} | {np.median(us):.1f} | {min(us):.1f} | "
                   f"{max(us):.1f} | {100 * sum(us) / total:.2f}% |")
    step = [u for _, u in sorted(per.get(kernel, []))]
    reps = warmup + 2 * steps + 1
    if step and len(step) % reps == 0:
        n = len(step) // reps
        ring = step[warmup * n:(warmup + steps) * n]
        leg = step[(warmup + steps + 1) * n:]
        out += ["", f"`{kernel}`: {n} launches per ring step; {len(step)} dispatches = ({warmup} untimed + "
                f"{steps} timed ring steps + 1 untimed + {steps} timed per-launch repetitions) x {n}.",
                f"- timed ring steps: {len(ring)} dispatches, mean {np.mean(ring):.1f} us, median "
                f"{np.median(ring):.1f} us, min {min(ring):.1f} us; {n} x mean = {n * np.mean(ring) / 1e3:.3f} ms "
                f"of kernel time per ring step",
                f"- timed per-launch repetitions: {len(leg)} dispatches, mean {np.mean(leg):.1f} us, median "
                f"{np.median(leg):.1f} us"]
    return "\n".join(out)


def counter_means(dirs, kernel=KERNEL_NAME):
    """Mean per dispatch of every counter of ``kernel`` in rocprofv3
    --pmc CSVs under ``dirs`` (a counter read per instance is summed over
    its instances first)."""
    vals = {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            if _short_kernel(r.get("Kernel_Name", "")) != kernel:
                continue
            key = (r["_file"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
            vals.setdefault(r["Counter_Name"], {}).setdefault(key, 0.0)
            vals[r["Counter_Name"]][key] += float(r["Counter_Value"])
    return {c: (float(np.mean(list(v.values()))), len(v)) for c, v in sorted(vals.items())}


def counter_summary(dirs, kernel=KERNEL_NAME):
    out = [f"`{kernel}`, mean per dispatch:", "", "| counter | per dispatch | dispatches |", "|---|---|---|"]
    for c, (m, n) in counter_means(dirs, kernel).items():
        out.append(f"| {c} | {m:.4e} | {n} |")
    return "\n".join(out)


def traffic_summary(fetch_dir, write_dir, cal_fetch_dir, cal_write_dir, workload_name, commands):
    """HBM bytes per launch of the step kernel from FETCH_SIZE and WRITE_SIZE
    (KiB per dispatch), each scaled by what the same counter reads for the
    plain 1 GiB device copy of ``--copy-calib``; the record carries the hash
    of the kernel's sources it was taken on."""
    def mean_of(d, counter, kernel):
        m = counter_means([d], kernel).get(counter)
        return m

    def copy_kib(d, counter):
        v = []
        for r in _csv_rows(d, "counter_collection.csv"):
            if r["Counter_Name"] == counter and "copy" in r.get("Kernel_Name", "").lower():
                v.append(float(r["Counter_Value"]))
        return float(np.median(v))

    f_raw, nf = mean_of(fetch_dir, "FETCH_SIZE", KERNEL_NAME)
    w_raw, nw = mean_of(write_dir, "WRITE_SIZE", KERNEL_NAME)
    cf, cw = copy_kib(cal_fetch_dir, "FETCH_SIZE"), copy_kib(cal_write_dir, "WRITE_SIZE")
    fs, ws = (1 << 30) / (cf * 1024), (1 << 30) / (cw * 1024)
    rec = {"workload": workload_name, "kernel": KERNEL_NAME, "kernel_hash": kernel_hash(), "commands": commands,
           "launches_sampled": min(nf, nw), "fetch_kib_per_launch_raw": round(f_raw, 1),
           "write_kib_per_launch_raw": round(w_raw, 1),
           "calibration": {"copy_bytes_read": 1 << 30, "copy_bytes_written": 1 << 30, "fetch_kib_raw": round(cf, 1),
                           "write_kib_raw": round(cw, 1), "fetch_scale": round(fs, 5), "write_scale": round(ws, 5)},
           "fetch_bytes_per_launch": int(f_raw * 1024 * fs), "write_bytes_per_launch": int(w_raw * 1024 * ws)}
    rec["bytes_per_launch"] = rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=None, help="workload name (default: the 131k zigzag ring)")
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-aux", action="store_true", help="skip the other workloads and the aux legs")
    ap.add_argument("--no-clock", action="store_true", help="skip sampling the GFX clock under load")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy (scale reference for HBM byte counters)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print the kernel table of a rocprofv3 --kernel-trace run of this script (--steps and "
                         "--warmup as that run's) and exit; no GPU")
    ap.add_argument("--counter-summary", metavar="DIR", nargs="+",
                    help="print the step kernel's mean counters from rocprofv3 --pmc runs and exit; no GPU")
    ap.add_argument("--kernel", default=KERNEL_NAME, help="kernel the summaries take (short name)")
    ap.add_argument("--traffic-summary", metavar="DIR", nargs=4,
                    help="FETCH_SIZE, WRITE_SIZE, copy FETCH_SIZE, copy WRITE_SIZE run directories: write the "
                         "HBM traffic record and exit; no GPU")
    ap.add_argument("--traffic-commands", nargs="*", default=[], help="the commands of the four runs, recorded")
    args = ap.parse_args()
    if args.trace_summary:
        print(trace_summary(args.trace_summary, args.warmup, args.steps, args.kernel))
        return
    if args.counter_summary:
        print(counter_summary(args.counter_summary, args.kernel))
        return
    if args.traffic_summary:
        from seeded_inputs.workloads import HEADLINE
        rec = traffic_summary(*args.traffic_summary, args.workload or HEADLINE, args.traffic_commands)
        with open(TRAFFIC_FILE, "w") as f:
            json.dump(rec, f, indent=1)
            f.write("\n")
        print(json.dumps(rec))
        return
    if args.gpus != 1:
        print(f"bench.py measures one rank's ring steps on one GPU; --gpus {args.gpus} is not "
              "supported (the ring's other ranks are simulated on this GPU, and no collective "
              "between GPUs is part of this library).", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calib:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calib_bytes_read": 1 << 30, "copy_calib_bytes_written": 1 << 30, "copies": 3}))
        return
    import ring_attention_blockwise_amd as ra
    from seeded_inputs import workload
    from seeded_inputs.workloads import HEADLINE

    name = args.workload or HEADLINE
    w = workload(name)
    rank = args.rank
    print(f"[bench] {name} rank {rank}: generating inputs", file=sys.stderr, flush=True)
    wall, per, ok = time_attention(ra, w, rank, args.steps, args.warmup)
    flops = algorithmic_flops(w, rank)
    ms = float(np.mean(per))
    value = flops / (ms * 1e-3) / 1e12
    print(f"[bench] attention: {ms:.3f} ms/step (median {np.median(per):.3f}, min {min(per):.3f}), "
          f"{value:.1f} TFLOP/s", file=sys.stderr, flush=True)
    # the roofline from the step kernel's own launches: per-launch HIP events
    lt = time_launches(ra, w, rank, args.steps)
    kern_ms = [float(np.mean(d)) for _, _, d in lt]
    kern_flops = sum(f for _, f, _ in lt)
    achieved = kern_flops / (sum(kern_ms) * 1e-3) / 1e12
    launch_us = float(np.mean(kern_ms)) * 1e3
    print(f"[bench] step kernel: {len(lt)} launches, mean {launch_us:.1f} us, {achieved:.1f} TFLOP/s over the "
          f"kernels' own time", file=sys.stderr, flush=True)
    clock = None if args.no_clock else sample_clock(ra, w, rank)
    if clock:
        print(f"[bench] gfx clock under load: {clock['gfxclk_mhz_median']:.0f} MHz", file=sys.stderr, flush=True)
    aux, configs = [], []
    if not args.no_aux:
        for other in CONFIG_LEGS:
            if other != name and w.dtype == "bf16":
                print(f"[bench] {other}", file=sys.stderr, flush=True)
                configs.append(time_config(ra, other, 0))
        aux.append(time_allgather(ra, w, rank, ms))
        if w.dtype == "bf16" and w.causal:
            aux.append(time_window(ra, w, rank, 4096))
        if w.dtype == "bf16" and w.D == 128:
            aux.append(time_backward(ra, w, rank))
            aux.append(time_backward(ra, w, rank, window=4096))
        if w.dtype == "bf16":
            aux.append(time_graph(ra, "bf16_gqa32x8_d128_s32k_ring8_zigzag_causal", 0))
        aux.append(time_merge(ra, w.B * (w.S // w.P) * w.Hq, w.D))
        aux.append(time_relayout(ra, 2, 8192, 16, 128, 8))
        aux.extend(time_ulysses_pieces(ra, 2, 8192, 16, 128, 8))
        for a in configs + aux:
            if "GB/s" in a:
                print(f"[bench] {a['kernel']}: {a['us']:.1f} us, {a['GB/s']:.0f} GB/s", file=sys.stderr, flush=True)
            else:
                print(f"[bench] {a['kernel']}: {a['ms']:.3f} ms, {a['TFLOP/s']:.1f} TFLOP/s", file=sys.stderr,
                      flush=True)
    cpu = None
    if not args.no_cpu:
        print("[bench] timing the CPU oracle on a sample", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, rank)
        cpu["aux"] = cpu_aux_baselines(w, rank)
    roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": measured_traffic(name),
            "kernel": KERNEL_NAME, "launches_per_step": len(lt), "avg_launch_us": round(launch_us, 2),
            "launch_us": [round(x * 1e3, 1) for x in kern_ms],
            "timing": "HIP events around each step-kernel launch on its stream (the ra_step calls "
                      "ra_rank_forward makes), mean over the timed repetitions"}
    if clock:
        peak_at_clk = PEAK_BF16_TFLOPS * clock["gfxclk_mhz_median"] / 2400.0
        roof["gfxclk_mhz"] = clock["gfxclk_mhz_median"]
        roof["peak_at_measured_clock"] = round(peak_at_clk, 1)
        roof["frac_at_measured_clock"] = round(achieved / peak_at_clk, 4)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(float(np.median(per)), 4),
        "ms_per_step_min": round(float(min(per)), 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) bf16, resident in HBM)",
        "config": {"workload": name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "S": w.S,
                   "ring": w.P, "rank": rank, "order": w.order, "causal": w.causal,
                   "local_query_rows": w.S // w.P},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "roofline": roof,
        "clock": clock,
        "cpu_baseline": cpu,
        "configs": configs,
        "aux": aux,
        "outputs_finite": ok,
        "wall_s_timed": round(wall, 3),
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
