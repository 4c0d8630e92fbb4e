"""Causal prefill attention (fd_prefill_attn) against the fp64 oracle.

Every valid position of every head is compared (max-abs 1e-2, bf16 inputs,
fp32 accumulation); positions past a sequence's length must stay untouched.
Full-size workloads are checked on sampled positions against decode
attention over rows [0, p], which is what position p computes.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import max_abs, to_dev, to_host
from workloads import configs, synth

pytestmark = pytest.mark.gpu

TOL = 1e-2

SHAPES = [
    # B, Hq, Hkv, L, lens
    (1, 16, 2, 300, [300]),             # G = 8: 16 positions per unit
    (2, 8, 8, 260, [260, 37]),          # MHA: 128 positions per unit
    (2, 8, 4, 500, [500, 129]),         # G = 2
    (1, 16, 4, 333, [333]),             # G = 4
    (2, 12, 4, 200, [200, 1]),          # G = 3: 42 positions, 126 rows per unit
    (1, 32, 2, 150, [150]),             # G = 16
    (1, 32, 1, 97, [97]),               # MQA, G = 32: 4 positions per unit
    (3, 4, 4, 33, [1, 32, 33]),         # short sequences, one tile
    (4, 8, 4, 150, [150, 3, 64, 129]),  # 16 (sequence, KV head) pairs: two per XCD, ragged
]


def run_prefill(fd, case, out_dtype=None):
    q = to_dev(case["q"], "bf16")
    k, v = to_dev(case["k"], "bf16"), to_dev(case["v"], "bf16")
    lens = torch.from_numpy(case["lens"]).to("cuda")
    sentinel = 123.0
    out = torch.full(q.shape, sentinel, dtype=out_dtype or torch.bfloat16, device="cuda")
    out, lse = fd.prefill_attn(q, k, v, lens, out=out, return_lse=True)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse), sentinel


def prefill_case(B, Hq, Hkv, L, lens, seed):
    q = synth.host_normal((B, Hq, L, 128), seed, "bf16")
    k = synth.host_normal((B, Hkv, L, 128), seed + 1, "bf16")
    v = synth.host_normal((B, Hkv, L, 128), seed + 2, "bf16")
    lens = np.asarray(lens, dtype=np.int32)
    for b in range(B):   # rows past the length are NaN: never read
        k[b, :, lens[b]:] = np.nan
        v[b, :, lens[b]:] = np.nan
        q[b, :, lens[b]:] = np.nan
    return {"q": q, "k": k, "v": v, "lens": lens}


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_hq{s[1]}_hkv{s[2]}_l{s[3]}")
def test_prefill_matches_oracle(fd, shape):
    B, Hq, Hkv, L, lens = shape
    case = prefill_case(B, Hq, Hkv, L, lens, seed=5000 + B * 7 + Hq + L)
    out, lse, sentinel = run_prefill(fd, case)
    ref_out, ref_lse = oracle.prefill_attention(case["q"], case["k"], case["v"], case["lens"])
    worst = 0.0
    for b in range(B):
        n = int(lens[b])
        worst = max(worst, max_abs(out[b, :, :n], ref_out[b, :, :n]), max_abs(lse[b, :, :n], ref_lse[b, :, :n]))
        assert np.all(out[b, :, n:] == sentinel), "positions past the length were written"
    print(f"  max-abs {worst:.3e}", flush=True)
    assert worst <= TOL


def test_prefill_fp32_output_and_scale(fd):
    case = prefill_case(1, 16, 2, 200, [200], seed=5100)
    q, k, v = (to_dev(case[x], "bf16") for x in ("q", "k", "v"))
    out, lse = fd.prefill_attn(q, k, v, None, out_dtype=torch.float32, scale=0.05, return_lse=True)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.prefill_attention(case["q"], case["k"], case["v"], None, 0.05)
    assert max_abs(to_host(out), ref_out) <= TOL and max_abs(to_host(lse), ref_lse) <= TOL


@pytest.mark.parametrize("w", configs.ALL_PREFILL, ids=lambda w: w.name)
def test_prefill_workload_full_size(fd, w):
    print(f"  workload {w.name}", flush=True)
    dev = "cuda"
    q = synth.device_normal((w.batch, w.q_heads, w.max_len, w.head_dim), w.seed, "bf16", dev)
    k = synth.device_normal((w.batch, w.kv_heads, w.max_len, w.head_dim), w.seed + 1, "bf16", dev)
    v = synth.device_normal((w.batch, w.kv_heads, w.max_len, w.head_dim), w.seed + 2, "bf16", dev)
    out, lse = fd.prefill_attn(q, k, v, None, return_lse=True)
    torch.cuda.synchronize()
    G = w.q_heads // w.kv_heads
    L = w.max_len
    rng = np.random.Generator(np.random.PCG64(w.seed))
    positions = sorted({0, 1, 15, 16, 127, 128, L // 2, L - 2, L - 1, *rng.integers(L, size=4).tolist()})
    worst = 0.0
    for b in range(w.batch):
        for g in sorted({0, w.kv_heads - 1}):
            kb, vb = to_host(k[b:b + 1, g:g + 1]), to_host(v[b:b + 1, g:g + 1])
            for p in positions:
                qp = to_host(q[b:b + 1, g * G:(g + 1) * G, p])
                ro, rl = oracle.attention(qp, kb, vb, np.array([p + 1]))
                worst = max(worst, max_abs(to_host(out[b, g * G:(g + 1) * G, p]), ro[0]),
                            max_abs(to_host(lse[b, g * G:(g + 1) * G, p]), rl[0]))
    print(f"  {len(positions)} positions x heads, max-abs {worst:.3e} (tol {w.tol})", flush=True)
    assert worst <= w.tol
