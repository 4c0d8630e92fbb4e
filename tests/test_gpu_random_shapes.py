"""Seeded random shapes for every entry point against the fp64 oracle.

Each case draws its own shape from its seed, within what the library
supports: head dims 64 and 128, groups of 1-32 query heads per KV head,
lengths from 1 row, any split count, page sizes 16-128 (decode caches and
the bifurcated decode part), empty decode parts.
Outputs are fp32, so the comparison measures the computation alone
(max-abs 1e-5 for fp32 inputs, 1e-2 for bf16 and E4M3 inputs); bf16
outputs are the same values rounded once (test_gpu_output_rounding.py).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import max_abs, to_dev, to_host
from workloads import synth

pytestmark = pytest.mark.gpu

N_CASES = 20
TOL = {"fp32": 1e-5, "bf16": 1e-2}


class Draw:
    def __init__(self, seed):
        self.rng = np.random.Generator(np.random.PCG64(seed))

    def pick(self, xs):
        return xs[int(self.rng.integers(len(xs)))]

    def int(self, lo, hi):          # inclusive
        return int(self.rng.integers(lo, hi + 1))

    def heads(self, groups=(1, 2, 3, 4, 5, 6, 8, 12, 16, 32)):
        hkv, g = self.pick([1, 2, 4, 8]), self.pick(list(groups))
        return g * hkv, hkv


def _lens(d, B, L):
    return [d.int(1, L) for _ in range(B)]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_decode(fd, i):
    d = Draw(70000 + i)
    dt, D = d.pick(["fp32", "bf16"]), d.pick([64, 128])
    (Hq, Hkv), B, L = d.heads(), d.int(1, 4), d.int(1, 2500)
    lens, ns = _lens(d, B, L), d.pick([0, 1, d.int(2, 80)])
    print(f"  decode {dt} B{B} Hq{Hq} Hkv{Hkv} D{D} L{L} lens{lens} n_splits {ns}", flush=True)
    c = synth.decode_case(B, Hq, Hkv, D, L, dt, seed=70000 + i, lens=lens)
    out, lse = fd.decode_attn(*(to_dev(c[x], dt) for x in ("q", "k", "v")), torch.from_numpy(c["lens"]).to("cuda"),
                              n_splits=ns, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention(c["q"], c["k"], c["v"], c["lens"])
    assert max(max_abs(to_host(out), ro), max_abs(to_host(lse), rl)) <= TOL[dt]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_paged(fd, i):
    d = Draw(71000 + i)
    dt, D = d.pick(["fp32", "bf16"]), d.pick([64, 128])
    (Hq, Hkv), B, L = d.heads(), d.int(1, 3), d.int(1, 2000)
    lens, ps, ns = _lens(d, B, L), d.pick([16, 32, 64, 128]), d.pick([0, 1, d.int(2, 40)])
    print(f"  paged {dt} B{B} Hq{Hq} Hkv{Hkv} D{D} L{L} lens{lens} page {ps} n_splits {ns}", flush=True)
    c = synth.decode_case(B, Hq, Hkv, D, L, dt, seed=71000 + i, lens=lens)
    kp, vp, table = synth.paginate(c["k"], c["v"], c["lens"], ps, seed=i)
    out, lse = fd.decode_attn_paged(to_dev(c["q"], dt), to_dev(kp, dt), to_dev(vp, dt),
                                    torch.from_numpy(table).to("cuda"), torch.from_numpy(c["lens"]).to("cuda"),
                                    n_splits=ns, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.paged_attention(c["q"], kp, vp, table, c["lens"])
    assert max(max_abs(to_host(out), ro), max_abs(to_host(lse), rl)) <= TOL[dt]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_fp8(fd, i):
    d = Draw(72000 + i)
    D, (Hq, Hkv), B, L = d.pick([64, 128]), d.heads(), d.int(1, 3), d.int(1, 2000)
    lens, ns = _lens(d, B, L), d.pick([0, 1, d.int(2, 40)])
    print(f"  fp8 B{B} Hq{Hq} Hkv{Hkv} D{D} L{L} lens{lens} n_splits {ns}", flush=True)
    c = synth.fp8_case(B, Hq, Hkv, D, L, seed=72000 + i, lens=lens)
    out, lse = fd.decode_attn_fp8(to_dev(c["q"], "bf16"), torch.from_numpy(c["k_bits"]).to("cuda"),
                                  torch.from_numpy(c["v_bits"]).to("cuda"), torch.from_numpy(c["k_scale"]).to("cuda"),
                                  torch.from_numpy(c["v_scale"]).to("cuda"), torch.from_numpy(c["lens"]).to("cuda"),
                                  n_splits=ns, out_dtype=torch.float32, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.attention_fp8kv(c["q"], c["k_bits"], c["v_bits"], c["k_scale"], c["v_scale"], c["lens"])
    assert max(max_abs(to_host(out), ro), max_abs(to_host(lse), rl)) <= 1e-2


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_bifurcated(fd, i):
    d = Draw(73000 + i)
    dt, D = d.pick(["fp32", "bf16"]), d.pick([64, 128])
    (Hq, Hkv), S = d.heads(), d.int(1, 10)
    Lc, Ld = d.int(1, 2000), d.int(1, 200)
    dl = [d.int(0, Ld) for _ in range(S)]
    print(f"  bifurcated {dt} S{S} Hq{Hq} Hkv{Hkv} D{D} Lc{Lc} Ld{Ld} dec{dl}", flush=True)
    c = synth.bifurcated_case(S, Hq, Hkv, D, Lc, Ld, dt, seed=73000 + i, dec_lens=dl)
    t = {x: to_dev(c[x], dt) for x in ("q", "k_ctx", "v_ctx", "k_dec", "v_dec")}
    out, lse = fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"],
                                  torch.from_numpy(c["dec_lens"]).to("cuda"), out_dtype=torch.float32,
                                  return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.bifurcated_attention(c["q"], c["k_ctx"], c["v_ctx"], c["k_dec"], c["v_dec"], c["dec_lens"])
    assert max(max_abs(to_host(out), ro), max_abs(to_host(lse), rl)) <= TOL[dt]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_bifurcated_paged(fd, i):
    d = Draw(75000 + i)
    dt, D = d.pick(["fp32", "bf16"]), d.pick([64, 128])
    (Hq, Hkv), S = d.heads(), d.int(1, 10)
    Lc, Ld, ps = d.int(1, 2000), d.int(1, 200), d.pick([16, 32, 64, 128])
    dl = [d.int(0, Ld) for _ in range(S)]
    print(f"  bifurcated paged {dt} S{S} Hq{Hq} Hkv{Hkv} D{D} Lc{Lc} Ld{Ld} page {ps} dec{dl}", flush=True)
    c = synth.bifurcated_case(S, Hq, Hkv, D, Lc, Ld, dt, seed=75000 + i, dec_lens=dl)
    kp, vp, table = synth.paginate(c["k_dec"], c["v_dec"], c["dec_lens"], ps, seed=i)
    t = {x: to_dev(c[x], dt) for x in ("q", "k_ctx", "v_ctx")}
    out, lse = fd.bifurcated_attn_paged(t["q"], t["k_ctx"], t["v_ctx"], to_dev(kp, dt), to_dev(vp, dt),
                                        torch.from_numpy(table).to("cuda"),
                                        torch.from_numpy(c["dec_lens"]).to("cuda"), out_dtype=torch.float32,
                                        return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.bifurcated_paged_attention(c["q"], c["k_ctx"], c["v_ctx"], kp, vp, table, c["dec_lens"])
    assert max(max_abs(to_host(out), ro), max_abs(to_host(lse), rl)) <= TOL[dt]


@pytest.mark.parametrize("i", range(N_CASES))
def test_random_prefill(fd, i):
    d = Draw(74000 + i)
    Hkv, G = d.pick([1, 2]), d.pick([1, 2, 3, 4, 8, 16, 32])
    Hq, B, L = G * Hkv, d.int(1, 2), d.int(1, 400)
    lens = np.asarray(_lens(d, B, L), dtype=np.int32)
    print(f"  prefill B{B} Hq{Hq} Hkv{Hkv} L{L} lens{lens.tolist()}", flush=True)
    q = synth.host_normal((B, Hq, L, 128), 74000 + i, "bf16")
    k = synth.host_normal((B, Hkv, L, 128), 74100 + i, "bf16")
    v = synth.host_normal((B, Hkv, L, 128), 74200 + i, "bf16")
    for b in range(B):           # rows past the length are NaN: never read
        q[b, :, lens[b]:] = np.nan
        k[b, :, lens[b]:] = np.nan
        v[b, :, lens[b]:] = np.nan
    out = torch.zeros((B, Hq, L, 128), dtype=torch.float32, device="cuda")
    out, lse = fd.prefill_attn(to_dev(q, "bf16"), to_dev(k, "bf16"), to_dev(v, "bf16"),
                               torch.from_numpy(lens).to("cuda"), out=out, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.prefill_attention(q, k, v, lens)
    oh, lh = to_host(out), to_host(lse)
    err = max(max(max_abs(oh[b, :, :n], ro[b, :, :n]), max_abs(lh[b, :, :n], rl[b, :, :n]))
              for b, n in enumerate(lens))
    assert err <= 1e-2
