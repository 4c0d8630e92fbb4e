"""The five named workloads at full size, in the launch configuration the
bench times (planner-chosen split counts), against the fp64 oracle.

Inputs are drawn on the device (torch's seeded generator); the exact bits
of the sampled (sequence, KV head) units are copied back for the oracle,
which computes those units one by one.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import check_every_unit, dense_rows, max_abs, oracle_decode_rows, sampled_units, to_host
from workloads import configs, synth

pytestmark = pytest.mark.gpu


def make_decode(w, pad_nan=True):
    dev = "cuda"
    q = synth.device_normal((w.batch, w.q_heads, w.head_dim), w.seed, w.dtype, dev)
    k = synth.device_normal((w.batch, w.kv_heads, w.max_len, w.head_dim), w.seed + 1, w.dtype, dev)
    v = synth.device_normal((w.batch, w.kv_heads, w.max_len, w.head_dim), w.seed + 2, w.dtype, dev)
    if w.ragged:
        lens = synth.device_lengths(w.batch, w.max_len // 2, w.max_len, w.seed + 7, dev)
    else:
        lens = torch.full((w.batch,), w.max_len, dtype=torch.int32, device=dev)
    if pad_nan:
        for b, n in enumerate(lens.tolist()):
            k[b, :, n:] = float("nan")
            v[b, :, n:] = float("nan")
    return q, k, v, lens


@pytest.mark.parametrize("w", [configs.TINY, configs.CODELLAMA34B_SHARE] + list(configs.MHA_SWEEP),
                         ids=lambda w: w.name)
def test_decode_workload_full_size(fd, w):
    print(f"  workload {w.name}", flush=True)
    q, k, v, lens = make_decode(w)
    out, lse = fd.decode_attn(q, k, v, lens, n_splits=w.n_splits, return_lse=True)
    torch.cuda.synchronize()
    out_h, lse_h = to_host(out), to_host(lse)
    assert np.all(np.isfinite(out_h))
    G = w.q_heads // w.kv_heads
    units = sampled_units(w, 6, w.seed)
    ref = oracle_decode_rows(q, k, v, lens, units)
    worst = 0.0
    for (b, g), (ro, rl) in ref.items():
        rows = slice(g * G, (g + 1) * G)
        worst = max(worst, max_abs(out_h[b, rows], ro), max_abs(lse_h[b, rows], rl))
    print(f"  {len(units)} units, max-abs {worst:.3e} (tol {w.tol})", flush=True)
    assert worst <= w.tol
    lens_h = lens.cpu().numpy()
    rows = check_every_unit(q, dense_rows(k, v, lens_h), lens_h, out, lse, w.tol)
    print(f"  all {rows} output rows inside the value hull, lse inside its bounds", flush=True)
    del q, k, v
    torch.cuda.empty_cache()


def make_bifurcated(w):
    dev = "cuda"
    S, Hq, Hkv, D = w.samples, w.q_heads, w.kv_heads, w.head_dim
    t = {
        "q": synth.device_normal((S, Hq, D), w.seed, w.dtype, dev),
        "k_ctx": synth.device_normal((Hkv, w.ctx_len, D), w.seed + 1, w.dtype, dev),
        "v_ctx": synth.device_normal((Hkv, w.ctx_len, D), w.seed + 2, w.dtype, dev),
        "k_dec": synth.device_normal((S, Hkv, w.dec_max, D), w.seed + 3, w.dtype, dev),
        "v_dec": synth.device_normal((S, Hkv, w.dec_max, D), w.seed + 4, w.dtype, dev),
    }
    dl = synth.device_lengths(S, w.dec_lo, w.dec_max, w.seed + 7, dev)
    for s, n in enumerate(dl.tolist()):
        t["k_dec"][s, :, n:] = float("nan")
        t["v_dec"][s, :, n:] = float("nan")
    return t, dl


@pytest.mark.parametrize("w", configs.ALL_BIFURCATED, ids=lambda w: w.name)
def test_bifurcated_workload_full_size(fd, w):
    print(f"  workload {w.name}", flush=True)
    t, dl = make_bifurcated(w)
    out, lse = fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"], dl,
                                  return_lse=True)
    torch.cuda.synchronize()
    out_h, lse_h = to_host(out), to_host(lse)
    assert np.all(np.isfinite(out_h))
    kc, vc = to_host(t["k_ctx"]), to_host(t["v_ctx"])
    dl_h = dl.cpu().numpy()
    rng = np.random.Generator(np.random.PCG64(w.seed))
    samples = sorted({0, w.samples - 1, int(np.argmin(dl_h)), *rng.integers(w.samples, size=3).tolist()})
    worst = 0.0
    for s in samples:
        n = int(dl_h[s])
        ro, rl = oracle.bifurcated_attention(to_host(t["q"][s:s + 1]), kc, vc,
                                             to_host(t["k_dec"][s:s + 1, :, :max(n, 1)]),
                                             to_host(t["v_dec"][s:s + 1, :, :max(n, 1)]),
                                             np.array([n]))
        worst = max(worst, max_abs(out_h[s:s + 1], ro), max_abs(lse_h[s:s + 1], rl))
    print(f"  samples {samples}, max-abs {worst:.3e} (tol {w.tol})", flush=True)
    assert worst <= w.tol

    # every sample: its rows are [context ; own valid decode rows]
    def rows_of(s):
        n = int(dl_h[s])
        return (torch.cat([t["k_ctx"], t["k_dec"][s, :, :n]], dim=1).float(),
                torch.cat([t["v_ctx"], t["v_dec"][s, :, :n]], dim=1).float())

    n_rows = check_every_unit(t["q"], rows_of, dl_h + w.ctx_len, out, lse, w.tol)
    print(f"  all {n_rows} output rows inside the value hull, lse inside its bounds", flush=True)


@pytest.mark.parametrize("w", configs.ALL_BIFURCATED, ids=lambda w: w.name)
def test_concatenated_cache_full_size(fd, w):
    """The non-bifurcated way to the same result: split-KV decode attention
    (planner split count, as the bench times it) over the explicitly
    concatenated cache [context ; own decode rows] per sample, at full size.
    Sampled samples (first, last, shortest and longest decode part) against
    the oracle's plain attention over those rows ([BA] "Tiivistelmä": both
    ways compute the same attention)."""
    print(f"  workload {w.name} (concatenated cache)", flush=True)
    t, dl = make_bifurcated(w)
    S, Hkv, Lc, Ld, D = w.samples, w.kv_heads, w.ctx_len, w.dec_max, w.head_dim
    kc = torch.empty((S, Hkv, Lc + Ld, D), dtype=t["k_ctx"].dtype, device="cuda")
    vc = torch.empty_like(kc)
    kc[:, :, :Lc] = t["k_ctx"].unsqueeze(0)
    vc[:, :, :Lc] = t["v_ctx"].unsqueeze(0)
    kc[:, :, Lc:] = t["k_dec"]
    vc[:, :, Lc:] = t["v_dec"]
    lens = (dl + Lc).to(torch.int32)
    out, lse = fd.decode_attn(t["q"], kc, vc, lens, return_lse=True)
    torch.cuda.synchronize()
    out_h, lse_h = to_host(out), to_host(lse)
    assert np.all(np.isfinite(out_h))
    dl_h = dl.cpu().numpy()
    samples = sorted({0, S - 1, int(np.argmin(dl_h)), int(np.argmax(dl_h))})
    units = [(s, g) for s in samples for g in sorted({0, Hkv - 1})]
    ref = oracle_decode_rows(t["q"], kc, vc, lens, units)
    G = w.q_heads // Hkv
    worst = 0.0
    for (s, g), (ro, rl) in ref.items():
        rows = slice(g * G, (g + 1) * G)
        worst = max(worst, max_abs(out_h[s, rows], ro), max_abs(lse_h[s, rows], rl))
    print(f"  {len(units)} units, max-abs {worst:.3e} (tol {w.tol})", flush=True)
    assert worst <= w.tol
    del kc, vc
    torch.cuda.empty_cache()
