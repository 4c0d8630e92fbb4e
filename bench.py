#!/usr/bin/env python3
"""Decode-attention benchmark on one MI355X.

A step is one full decode-attention call: the split-KV partial kernel plus
the LSE combine (or the single direct kernel when one piece suffices), over
one set of synthetic inputs already resident in HBM.  Inputs rotate over
enough distinct copies (>= 1 GiB in total) that no step can be served from
the 256 MB Infinity Cache.

Steps are captured in a HIP graph and timed with HIP events around its
replay (host launch cost stays outside, as in a graph-captured decode loop).
Prints ONE JSON line: value = achieved KV-read rate of the whole step
(algorithmic KV bytes / step time, TB/s), ms_per_step, the roofline of the
dominant kernel (its average duration from a graph of K launches of that
kernel alone, timed the same way on the stream it runs on), and the fp64 CPU
oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps 200] [--warmup 20] [--workload NAME]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from workloads import configs, synth  # noqa: E402

METRIC = "decode-attn µs/step + achieved KV-read HBM TB/s (fraction of MI355X peak)"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
ROTATION_BYTES = 1 << 30
COUNTERS_FILE = os.path.join(ROOT, "profiles", "hbm_counters.json")
WORKLOADS = {w.name: w for w in (configs.ALL_DECODE + configs.ALL_PAGED + configs.ALL_FP8 + configs.ALL_BIFURCATED +
                                  configs.ALL_PREFILL)}
DEFAULT_WORKLOAD = configs.CODELLAMA34B_SHARE.name


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------- inputs

def decode_inputs(w, copies, dev):
    import torch

    sets = []
    if w.ragged:
        lens = synth.device_lengths(w.batch, w.max_len // 2, w.max_len, w.seed + 7, dev)
    else:
        lens = torch.full((w.batch,), w.max_len, dtype=torch.int32, device=dev)
    for c in range(copies):
        s = w.seed + 1000 * c
        q = synth.device_normal((w.batch, w.q_heads, w.head_dim), s, w.dtype, dev)
        k = synth.device_normal((w.batch, w.kv_heads, w.max_len, w.head_dim), s + 1, w.dtype, dev)
        v = synth.device_normal((w.batch, w.kv_heads, w.max_len, w.head_dim), s + 2, w.dtype, dev)
        sets.append((q, k, v))
    return sets, lens


def paged_inputs(w, copies, dev):
    """Page pools (one per copy) sharing one shuffled block table."""
    import torch

    P = w.page_size
    per_seq = -(-w.max_len // P)
    n_pages = 1 + w.batch * per_seq
    table = torch.from_numpy(synth.shuffled_block_table(w.batch, per_seq, w.seed + 11)).to(dev)
    if w.ragged:
        lens = synth.device_lengths(w.batch, w.max_len // 2, w.max_len, w.seed + 7, dev)
    else:
        lens = torch.full((w.batch,), w.max_len, dtype=torch.int32, device=dev)
    sets = []
    for c in range(copies):
        s = w.seed + 1000 * c
        q = synth.device_normal((w.batch, w.q_heads, w.head_dim), s, w.dtype, dev)
        kp = synth.device_normal((n_pages, w.kv_heads, P, w.head_dim), s + 1, w.dtype, dev)
        vp = synth.device_normal((n_pages, w.kv_heads, P, w.head_dim), s + 2, w.dtype, dev)
        sets.append((q, kp, vp))
    return sets, table, lens


def bifurcated_inputs(w, copies, dev):
    sets = []
    dl = synth.device_lengths(w.samples, w.dec_lo, w.dec_max, w.seed + 7, dev)
    for c in range(copies):
        s = w.seed + 1000 * c
        sets.append({
            "q": synth.device_normal((w.samples, w.q_heads, w.head_dim), s, w.dtype, dev),
            "k_ctx": synth.device_normal((w.kv_heads, w.ctx_len, w.head_dim), s + 1, w.dtype, dev),
            "v_ctx": synth.device_normal((w.kv_heads, w.ctx_len, w.head_dim), s + 2, w.dtype, dev),
            "k_dec": synth.device_normal((w.samples, w.kv_heads, w.dec_max, w.head_dim), s + 3, w.dtype, dev),
            "v_dec": synth.device_normal((w.samples, w.kv_heads, w.dec_max, w.head_dim), s + 4, w.dtype, dev),
        })
    return sets, dl


# ------------------------------------------------------------- GPU timing

def timed_graph(fn, steps):
    """Capture fn(0..steps-1) into one HIP graph and time a replay with HIP
    events on the stream it runs on; returns ms per step.  Host launch cost
    is outside the timed region, as in a graph-captured decode loop."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for j in range(min(steps, 3)):
            fn(j)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for j in range(steps):
            fn(j)
    g.replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    t0.record(stream)
    g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    del g
    return ms


def timed_eager(fn, steps):
    """The same steps launched one by one from Python (includes host cost)."""
    import torch

    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for j in range(steps):
        fn(j)
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


ISOLATION_US = 300.0      # spin ahead of each isolated step: covers the host's launch of the step


def step_percentiles(fn, copies, samples):
    """Each step on its own: launched eagerly behind a spin kernel of about
    ISOLATION_US (calibrated here), so the host has queued the step's
    kernels before the GPU reaches them, and bracketed by two HIP events on
    its stream.  Copies rotate as in the timed loop, so every step reads
    cold inputs.  Returns the p10, median and p90 of the per-step times in
    ms, and the number of samples."""
    import numpy as np
    import torch

    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cal = 100000
    torch.cuda._sleep(cal)
    torch.cuda.synchronize()
    e0.record(stream)
    torch.cuda._sleep(cal)
    e1.record(stream)
    torch.cuda.synchronize()
    cycles = max(cal, int(cal * ISOLATION_US * 1e-3 / max(e0.elapsed_time(e1), 1e-6)))
    for j in range(min(copies, 2)):
        fn(j)
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(samples)]
    for i, (a, b) in enumerate(ev):
        torch.cuda._sleep(cycles)
        a.record(stream)
        fn(i % copies)
        b.record(stream)
    torch.cuda.synchronize()
    t = np.array([a.elapsed_time(b) for a, b in ev])
    p10, p50, p90 = np.percentile(t, [10, 50, 90])
    return {"p10_ms": float(p10), "median_ms": float(p50), "p90_ms": float(p90), "samples": int(samples)}


def time_decode(w, steps, warmup, force_splits=0, probe=True, percentiles=True, want_host=True):
    import torch

    import decode_attention_06_amd as fd

    dev = torch.device("cuda:0")
    sz = 2 if w.dtype == "bf16" else 4
    alloc_bytes = 2 * w.batch * w.kv_heads * w.max_len * w.head_dim * sz
    copies = max(2, math.ceil(ROTATION_BYTES / alloc_bytes))
    sets, lens = decode_inputs(w, copies, dev)
    kv_bytes = 2 * int(lens.sum().item()) * w.kv_heads * w.head_dim * sz   # algorithmic, per step
    dt = fd.FD_BF16 if w.dtype == "bf16" else fd.FD_F32
    ns = force_splits or (w.n_splits if w.n_splits > 0 else fd.plan_splits(
        w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_len, dt, fd.device_cu_count()))
    rows = w.batch * w.q_heads
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=sets[0][0].dtype, device=dev)
    o_part = torch.empty((rows, ns, w.head_dim), dtype=torch.float32, device=dev)
    lse_part = torch.empty((rows, ns), dtype=torch.float32, device=dev)

    ws_bytes = fd.decode_workspace_size(w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_len, dt, ns)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

    def step(j):
        q, k, v = sets[j % copies]
        fd.decode_attn(q, k, v, lens, n_splits=ns, out=out, workspace=ws)

    # The partial kernel alone, exactly as the step launches it (pieces
    # interleaved on the matrix-core kernel), for the roofline of the
    # dominant kernel.
    mfma = w.dtype == "bf16" and w.head_dim == 128 and w.q_heads // w.kv_heads >= 4
    layout = fd.FD_PIECES_INTERLEAVED if mfma else fd.FD_PIECES_CONTIGUOUS

    def partial_only(j):
        q, k, v = sets[j % copies]
        if ns == 1:
            fd.decode_attn(q, k, v, lens, n_splits=1, out=out, workspace=ws)
        else:
            fd.decode_attn_partials(q, k, v, ns, lens=lens, o_part=o_part, lse_part=lse_part, layout=layout)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    eager_ms = timed_eager(step, steps)
    step_ms = timed_graph(step, steps)
    kern_ms = timed_graph(partial_only, steps)
    pct = step_percentiles(step, copies, max(steps, 2 * copies)) if percentiles else None

    # Plain read of the same number of bytes in ONE launch per step, over
    # buffers rotated the same way: the single-launch read ceiling.
    probe_gbs = None
    if probe:
        probe_bytes = 2 * sets[0][1].numel() * sets[0][1].element_size()
        bufs = [torch.empty(probe_bytes, dtype=torch.uint8, device=dev) for _ in range(copies)]
        for b_ in bufs:
            b_.fill_(1)
        sink = torch.zeros(1, dtype=torch.int32, device=dev)

        def probe_step(j):
            fd.read_probe(bufs[j % copies], sink)

        probe_ms = timed_graph(probe_step, steps)
        probe_gbs = probe_bytes / (probe_ms * 1e-3) / 1e9
        del bufs

    info = {
        "n_splits": ns, "copies": copies, "kv_bytes": kv_bytes, "step_ms": step_ms, "kernel_ms": kern_ms,
        "eager_step_ms": eager_ms, "probe_gbs": probe_gbs, "percentiles": pct,
        "kernel": "partial_mfma_kernel" if mfma else "partial_valu_kernel",
        "flops": 4 * int(lens.sum().item()) * w.q_heads * w.head_dim,
    }
    if not want_host:
        return info, None
    host = [t.detach().float().cpu().numpy() for t in sets[0]]
    return info, (host, lens.cpu().numpy())


def fp8_inputs(w, copies, dev):
    """E4M3 caches (one per copy) with per-KV-head scales."""
    import torch

    if w.ragged:
        lens = synth.device_lengths(w.batch, w.max_len // 2, w.max_len, w.seed + 7, dev)
    else:
        lens = torch.full((w.batch,), w.max_len, dtype=torch.int32, device=dev)
    ks = synth.head_scales(w.kv_heads, w.seed + 3)
    vs = synth.head_scales(w.kv_heads, w.seed + 4)
    shape = (w.batch, w.kv_heads, w.max_len, w.head_dim)
    sets = []
    for c in range(copies):
        s = w.seed + 1000 * c
        q = synth.device_normal((w.batch, w.q_heads, w.head_dim), s, "bf16", dev)
        sets.append((q, synth.device_fp8(shape, s + 1, ks, dev), synth.device_fp8(shape, s + 2, vs, dev)))
    return sets, torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev), lens


def time_variant(w, steps, warmup, force_splits=0):
    """Decode over a paged or an E4M3 cache.  These entry points launch the
    partial kernel and the combine together, so the kernel figures here are
    those of the whole call (a lower bound on the partial kernel's rate);
    rocprofv3 gives the per-kernel split."""
    import torch

    import decode_attention_06_amd as fd

    dev = torch.device("cuda:0")
    sz = {"bf16": 2, "fp32": 4, "fp8": 1}[w.dtype]
    alloc_bytes = 2 * w.batch * w.kv_heads * w.max_len * w.head_dim * sz
    copies = max(2, math.ceil(ROTATION_BYTES / alloc_bytes))
    if w.dtype == "fp8":
        sets, ks, vs, lens = fp8_inputs(w, copies, dev)
        max_len, dt = w.max_len, fd.FD_FP8_E4M3
    else:
        sets, table, lens = paged_inputs(w, copies, dev)
        max_len = table.shape[1] * w.page_size
        dt = fd.FD_BF16 if w.dtype == "bf16" else fd.FD_F32
    kv_bytes = 2 * int(lens.sum().item()) * w.kv_heads * w.head_dim * sz
    ns = force_splits or (w.n_splits if w.n_splits > 0 else fd.plan_splits(
        w.batch, w.q_heads, w.kv_heads, w.head_dim, max_len, dt, fd.device_cu_count()))
    out = torch.empty((w.batch, w.q_heads, w.head_dim), dtype=sets[0][0].dtype, device=dev)
    ws = torch.empty(max(1, fd.decode_workspace_size(w.batch, w.q_heads, w.kv_heads, w.head_dim, max_len, dt, ns)),
                     dtype=torch.uint8, device=dev)

    def step(j):
        q, k, v = sets[j % copies]
        if w.dtype == "fp8":
            fd.decode_attn_fp8(q, k, v, ks, vs, lens, n_splits=ns, out=out, workspace=ws)
        else:
            fd.decode_attn_paged(q, k, v, table, lens, n_splits=ns, out=out, workspace=ws)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    eager_ms = timed_eager(step, steps)
    step_ms = timed_graph(step, steps)
    info = {
        "n_splits": ns, "copies": copies, "kv_bytes": kv_bytes, "step_ms": step_ms,
        "kernel_ms": step_ms, "eager_step_ms": eager_ms, "probe_gbs": None,
        "kernel": "partial_mfma_kernel" if (w.dtype in ("bf16", "fp8") and w.head_dim == 128 and
                                             w.q_heads // w.kv_heads >= 4) else "partial_valu_kernel",
        "kernel_timing": "whole call (partial kernel and combine)",
        "flops": 4 * int(lens.sum().item()) * w.q_heads * w.head_dim,
    }
    return info, None


def time_prefill(w, steps, warmup):
    """Causal prefill of whole sequences: the step is one fd_prefill_attn
    call; flops = 4 * D * Hq * sum over positions p of (p + 1)."""
    import torch

    import decode_attention_06_amd as fd

    dev = torch.device("cuda:0")
    per_copy = (w.batch * (w.q_heads + 2 * w.kv_heads) * w.max_len * w.head_dim) * 2
    copies = max(2, math.ceil(ROTATION_BYTES / per_copy))
    sets = []
    for c in range(copies):
        s = w.seed + 1000 * c
        sets.append(tuple(synth.device_normal((w.batch, h, w.max_len, w.head_dim), s + j, "bf16", dev)
                          for j, h in enumerate((w.q_heads, w.kv_heads, w.kv_heads))))
    out = torch.empty_like(sets[0][0])

    def step(j):
        q, k, v = sets[j % copies]
        fd.prefill_attn(q, k, v, None, out=out)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    eager_ms = timed_eager(step, steps)
    step_ms = timed_graph(step, steps)
    L = w.max_len
    flops = 4 * w.head_dim * w.q_heads * w.batch * (L * (L + 1) // 2)
    kv_bytes = 2 * w.batch * w.kv_heads * L * w.head_dim * 2
    info = {"n_splits": None, "copies": copies, "kv_bytes": kv_bytes, "step_ms": step_ms, "kernel_ms": step_ms,
            "eager_step_ms": eager_ms, "probe_gbs": None, "kernel": "prefill_kernel", "flops": flops}
    return info, None


def time_concatenated(w, sets, dl, steps):
    """Split-KV decode attention over [context ; own decode rows] per sample
    (the non-bifurcated way to get the same result): µs per step."""
    import torch

    import decode_attention_06_amd as fd

    t = sets[0]
    S, Hkv, Lc, Ld, D = w.samples, w.kv_heads, w.ctx_len, w.dec_max, w.head_dim
    kc = torch.empty((S, Hkv, Lc + Ld, D), dtype=t["k_ctx"].dtype, device=t["k_ctx"].device)
    vc = torch.empty_like(kc)
    kc[:, :, :Lc] = t["k_ctx"].unsqueeze(0)
    vc[:, :, :Lc] = t["v_ctx"].unsqueeze(0)
    kc[:, :, Lc:] = t["k_dec"]
    vc[:, :, Lc:] = t["v_dec"]
    lens = (dl + Lc).to(torch.int32)
    out = torch.empty((S, w.q_heads, D), dtype=t["q"].dtype, device=kc.device)
    ns = fd.plan_splits(S, w.q_heads, Hkv, D, Lc + Ld, fd.FD_BF16, fd.device_cu_count())
    ws = torch.empty(max(1, fd.decode_workspace_size(S, w.q_heads, Hkv, D, Lc + Ld, fd.FD_BF16, ns)),
                     dtype=torch.uint8, device=kc.device)

    def step(j):
        fd.decode_attn(t["q"], kc, vc, lens, n_splits=ns, out=out, workspace=ws)

    for j in range(3):
        step(j)
    ms = timed_graph(step, steps)
    del kc, vc
    torch.cuda.empty_cache()
    return ms, ns


def time_bifurcated(w, steps, warmup, compare_concat=False, percentiles=True):
    import torch

    import decode_attention_06_amd as fd

    dev = torch.device("cuda:0")
    sz = 2
    alloc = (2 * w.kv_heads * w.ctx_len + 2 * w.samples * w.kv_heads * w.dec_max) * w.head_dim * sz
    copies = max(2, math.ceil(ROTATION_BYTES / alloc))
    sets, dl = bifurcated_inputs(w, copies, dev)
    n_dec = int(dl.sum().item())
    kv_bytes = (2 * w.kv_heads * w.ctx_len + 2 * n_dec * w.kv_heads) * w.head_dim * sz
    flops = 4 * w.q_heads * w.head_dim * (w.samples * w.ctx_len + n_dec)
    out = torch.empty((w.samples, w.q_heads, w.head_dim), dtype=torch.bfloat16, device=dev)
    wsb = fd.bifurcated_workspace_size(w.samples, w.q_heads, w.kv_heads, w.head_dim, w.ctx_len, w.dec_max,
                                       fd.FD_BF16)
    ws = torch.empty(max(wsb, 1), dtype=torch.uint8, device=dev)

    def step(j):
        t = sets[j % copies]
        fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"], dl, out=out, workspace=ws)

    for j in range(warmup):
        step(j)
    torch.cuda.synchronize()
    eager_ms = timed_eager(step, steps)
    step_ms = timed_graph(step, steps)
    pct = step_percentiles(step, copies, max(steps, 2 * copies)) if percentiles else None
    info = {"n_splits": None, "copies": copies, "kv_bytes": kv_bytes, "step_ms": step_ms, "kernel_ms": step_ms,
            "eager_step_ms": eager_ms, "probe_gbs": None, "kernel": "bifurcated (whole call)", "flops": flops,
            "percentiles": pct}
    if compare_concat:
        info["concat_ms"], info["concat_splits"] = time_concatenated(w, sets, dl, max(5, steps // 4))
    return info, None


# ------------------------------------------------ every other workload

# The other workloads of the method, measured in the same run as the
# headline: the tiny fp32 case, MHA over 64K tokens at batch 1 and 16, and
# the two bifurcated workloads with split-KV over the concatenated cache
# (the non-bifurcated way to the same result) beside them.
EXTRA_DECODE = (configs.TINY,) + tuple(w for w in configs.MHA_SWEEP if w.max_len == 65536)
EXTRA_BIFURCATED = configs.ALL_BIFURCATED


def _pct_us(info):
    p = info.get("percentiles")
    if not p:
        return {}
    return {"p10_us": round(p["p10_ms"] * 1e3, 3), "median_us": round(p["median_ms"] * 1e3, 3),
            "p90_us": round(p["p90_ms"] * 1e3, 3), "isolated_samples": p["samples"]}


def run_extras(steps, warmup):
    """One record per workload: mean µs per step over a graph replay of
    `steps` steps, the p10 / median / p90 of steps timed one by one, the KV
    read rate as a fraction of 8 TB/s, and the kernel-level figures."""
    import torch

    recs = []
    for w in EXTRA_DECODE:
        log(f"[bench] extra workload {w.name}")
        info, _ = time_decode(w, steps, warmup, probe=False, want_host=False)
        step_s, kern_s = info["step_ms"] * 1e-3, info["kernel_ms"] * 1e-3
        rec = {"workload": w.name, "us_per_step": round(info["step_ms"] * 1e3, 3), **_pct_us(info),
               "kv_bytes": info["kv_bytes"], "tb_per_s": round(info["kv_bytes"] / step_s / 1e12, 4),
               "hbm_frac": round(info["kv_bytes"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
               "kernel": info["kernel"], "kernel_us": round(info["kernel_ms"] * 1e3, 3),
               "kernel_hbm_frac": round(info["kv_bytes"] / kern_s / 1e9 / HBM_PEAK_GBS, 4),
               "n_splits": info["n_splits"], "dtype": w.dtype}
        recs.append(rec)
        log(f"[bench]   {rec}")
        torch.cuda.empty_cache()
    for w in EXTRA_BIFURCATED:
        log(f"[bench] extra workload {w.name}")
        info, _ = time_bifurcated(w, steps, warmup, compare_concat=True)
        step_s = info["step_ms"] * 1e-3
        rec = {"workload": w.name, "us_per_step": round(info["step_ms"] * 1e3, 3), **_pct_us(info),
               "kv_bytes": info["kv_bytes"], "tb_per_s": round(info["kv_bytes"] / step_s / 1e12, 4),
               "hbm_frac": round(info["kv_bytes"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
               "flops": info["flops"], "tflops": round(info["flops"] / step_s / 1e12, 2),
               "mfma_frac": round(info["flops"] / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
               "concatenated_us_per_step": round(info["concat_ms"] * 1e3, 3),
               "concatenated_n_splits": info["concat_splits"],
               "speedup_vs_concatenated": round(info["concat_ms"] / info["step_ms"], 3), "dtype": w.dtype}
        recs.append(rec)
        log(f"[bench]   {rec}")
        torch.cuda.empty_cache()
    return recs


# --------------------------------------------------------- CPU baseline

def cpu_baseline(w, host_inputs, kv_bytes, budget_s):
    """Time the fp64 oracle on the host cores for one full step of w."""
    import numpy as np

    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    (q, k, v), lens = host_inputs
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    runs, total = 0, 0.0
    while runs < 1 or (total < budget_s and runs < 50):
        t = time.perf_counter()
        oracle.attention(q, k, v, lens)
        total += time.perf_counter() - t
        runs += 1
    per_step = total / runs
    return {
        "value": kv_bytes / per_step / 1e12, "unit": "TB/s", "cores": int(threads), "kind": "oracle",
        "sample": f"{runs} full step(s) of {w.name} (inputs already in host memory as float64), "
                  f"{per_step * 1e3:.1f} ms per step",
    }


def counters_for(kernel, workload, n_splits):
    """HBM traffic per launch from committed rocprofv3 counter runs, or None
    when the kernel's sources (or its split count) changed since then."""
    try:
        rec = json.load(open(COUNTERS_FILE))
    except (OSError, ValueError):
        return None
    entry = rec.get("entries", {}).get(f"{kernel}|{workload}")
    if not entry or entry.get("n_splits") != n_splits:
        return None
    h = hashlib.sha256()
    for rel in entry.get("sources", []):
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                h.update(f.read())
        except OSError:
            return None
    if h.hexdigest()[:16] != entry.get("source_hash"):
        return None
    return entry.get("traffic_bytes")


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=sorted(WORKLOADS))
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget for the oracle timing")
    ap.add_argument("--n-splits", type=int, default=0, help="force the split count (decode workloads; 0 = planner)")
    ap.add_argument("--compare-concat", action="store_true",
                    help="bifurcated workloads: also time split-KV decode over the concatenated cache")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads (the 'extra' object)")
    ap.add_argument("--extra-steps", type=int, default=20, help="timed steps per extra workload")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run 5 plain device copies of MIB MiB (HBM counter calibration)")
    args = ap.parse_args()

    if args.calibrate_copy:
        import torch

        src = torch.ones(args.calibrate_copy << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": args.calibrate_copy << 20, "copies": 5}))
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(a longer history would be split over GPUs with fd_decode_attn_partials and merged with "
              "fd_lse_combine after an all-gather); run with --gpus 1", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a visible GPU", file=sys.stderr)
        return 1
    import decode_attention_06_amd as fd

    fd.load()
    w = WORKLOADS[args.workload]
    bif = w.name in {b.name for b in configs.ALL_BIFURCATED}
    prefill = w.name in {x.name for x in configs.ALL_PREFILL}
    if prefill:
        info, host = time_prefill(w, args.steps, args.warmup)
        dtype = w.dtype
    elif bif:
        info, host = time_bifurcated(w, args.steps, args.warmup, args.compare_concat)
        dtype = w.dtype
    elif getattr(w, "page_size", 0) > 0 or w.dtype == "fp8":
        info, host = time_variant(w, args.steps, args.warmup, args.n_splits)
        dtype = "fp8_e4m3 cache, bf16 query" if w.dtype == "fp8" else w.dtype
    else:
        info, host = time_decode(w, args.steps, args.warmup, args.n_splits)
        dtype = w.dtype
    step_s = info["step_ms"] * 1e-3
    kern_s = info["kernel_ms"] * 1e-3
    achieved_gbs = info["kv_bytes"] / kern_s / 1e9
    value_tbs = info["kv_bytes"] / step_s / 1e12
    log(f"[bench] {w.name}: step {info['step_ms'] * 1e3:.2f} us in a graph (launched eagerly from Python: "
        f"{info['eager_step_ms'] * 1e3:.2f} us), dominant kernel {info['kernel_ms'] * 1e3:.2f} us, "
        f"n_splits={info['n_splits']}, plain read of the same bytes: {info['probe_gbs']} GB/s")

    cpu = None
    if not args.no_cpu_baseline and host is not None and int(os.environ.get("RANK", "0")) == 0:
        cpu = cpu_baseline(w, host, info["kv_bytes"], args.cpu_seconds)

    config = {"workload": w.name, "kv_bytes_per_step": info["kv_bytes"], "n_splits": info["n_splits"],
              "input_copies": info["copies"], "timing": "HIP events around a graph replay of the K steps; inputs rotated over >= 1 GiB",
              "eager_us_per_step": round(info["eager_step_ms"] * 1e3, 3)}
    if prefill:
        config.update(batch=w.batch, q_heads=w.q_heads, kv_heads=w.kv_heads, head_dim=w.head_dim,
                      seq_len=w.max_len, mask="causal")
    elif bif:
        config.update(samples=w.samples, q_heads=w.q_heads, kv_heads=w.kv_heads, head_dim=w.head_dim,
                      ctx_len=w.ctx_len, dec_len=f"{w.dec_lo}..{w.dec_max}")
    else:
        config.update(batch=w.batch, q_heads=w.q_heads, kv_heads=w.kv_heads, head_dim=w.head_dim,
                      kv_len=w.max_len, lens="uniform [L/2, L]" if w.ragged else "all L")
        if w.page_size:
            config.update(page_size=w.page_size, pages="shuffled pool, one block table")
    line = {
        "metric": METRIC,
        "value": round(value_tbs, 4),
        "unit": "TB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(info["step_ms"], 6),
        "us_per_step": round(info["step_ms"] * 1e3, 3),
        "frac_of_hbm_peak": round(value_tbs * 1000 / HBM_PEAK_GBS, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic N(0,1) inputs, seeded",
        "config": config,
        "roofline": {
            "bound": "hbm",
            "kernel": info["kernel"],
            "achieved": round(achieved_gbs, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved_gbs / HBM_PEAK_GBS, 4),
            "traffic": counters_for(info["kernel"], w.name, info["n_splits"]),
            "kernel_us": round(info["kernel_ms"] * 1e3, 3),
            "read_probe_gbs": None if info["probe_gbs"] is None else round(info["probe_gbs"], 1),
        },
        "cpu_baseline": cpu,
    }
    if prefill:
        tflops = info["flops"] / step_s / 1e12
        line.update(value=round(tflops, 2), unit="TFLOP/s", frac_of_hbm_peak=None)
        line["roofline"] = {"bound": "mfma", "kernel": info["kernel"], "achieved": round(tflops, 2),
                            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                            "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4), "traffic": None,
                            "kernel_us": round(info["kernel_ms"] * 1e3, 3), "flops": info["flops"]}
    if "kernel_timing" in info:
        line["roofline"]["kernel_timing"] = info["kernel_timing"]
    pct = _pct_us(info)
    if pct:
        line["step_percentiles"] = dict(pct, timing="each step alone, launched behind a spin kernel that covers "
                                                    "the host's launch, between two HIP events")
    if bif:
        line["roofline"]["mfma_tflops"] = round(info["flops"] / step_s / 1e12, 2)
        line["roofline"]["mfma_frac"] = round(info["flops"] / step_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
        if "concat_ms" in info:
            line["concatenated_us_per_step"] = round(info["concat_ms"] * 1e3, 3)
            line["speedup_vs_concatenated"] = round(info["concat_ms"] / info["step_ms"], 3)
            log(f"[bench] same result by split-KV over the concatenated cache: {info['concat_ms'] * 1e3:.2f} us "
                f"({info['concat_splits']} pieces); bifurcated speedup {info['concat_ms'] / info['step_ms']:.2f}x")
    if not args.no_extra and w.name == DEFAULT_WORKLOAD:
        del host
        torch.cuda.empty_cache()
        line["extra"] = {"timing": "as the headline: mean over a graph replay of the steps; p10 / median / p90 "
                                   "of steps timed one by one behind a spin kernel", "steps": args.extra_steps,
                         "workloads": run_extras(args.extra_steps, min(args.warmup, 5))}
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
