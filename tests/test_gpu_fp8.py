"""E4M3-cache decode attention (fd_decode_attn_fp8) against the fp64 oracle.

The oracle decodes the very codes the GPU reads (OCP E4M3 definition) and
multiplies by the per-KV-head scales, so the comparison carries no
quantisation error: the bound is the bf16 one, max-abs 1e-2 on every output
element and lse.  Rows past each sequence's length hold the NaN code.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import check_every_unit, max_abs, sampled_units, to_dev, to_host
from workloads import configs, synth

pytestmark = pytest.mark.gpu

TOL = 1e-2

SHAPES = [
    # B, Hq, Hkv, D, Lmax, lens
    (3, 16, 2, 128, 1000, [1, 777, 1000]),    # matrix-core kernel, G = 8
    (2, 32, 1, 128, 900, [900, 100]),         # MQA, 32-row blocks
    (2, 12, 4, 128, 400, [400, 129]),         # G = 3: vector-ALU kernel
    (2, 8, 8, 128, 700, [700, 300]),          # MHA: vector-ALU kernel
    (2, 16, 8, 128, 650, [650, 17]),          # G = 2
    (2, 8, 2, 64, 600, [600, 33]),            # D 64, G = 4 (vector-ALU, 4-row units)
    (2, 16, 2, 64, 500, [500, 250]),          # D 64, G = 8 (two 4-row units per KV head)
    (5, 6, 6, 64, 300, [1, 15, 16, 17, 300]),
]


def run_fp8(fd, case, n_splits=0, out_dtype=None, scales=True):
    q = to_dev(case["q"], "bf16")
    k = torch.from_numpy(case["k_bits"]).to("cuda")
    v = torch.from_numpy(case["v_bits"]).to("cuda")
    ks = torch.from_numpy(case["k_scale"]).to("cuda") if scales else None
    vs = torch.from_numpy(case["v_scale"]).to("cuda") if scales else None
    lens = torch.from_numpy(case["lens"]).to("cuda")
    out, lse = fd.decode_attn_fp8(q, k, v, ks, vs, lens, n_splits=n_splits, out_dtype=out_dtype, return_lse=True)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_hq{s[1]}_hkv{s[2]}_d{s[3]}_l{s[4]}")
@pytest.mark.parametrize("n_splits", [0, 1, 5, 33])
def test_fp8_matches_oracle(fd, shape, n_splits):
    B, Hq, Hkv, D, L, lens = shape
    case = synth.fp8_case(B, Hq, Hkv, D, L, seed=4000 + B * 7 + Hq, lens=lens)
    out, lse = run_fp8(fd, case, n_splits)
    ref_out, ref_lse = oracle.attention_fp8kv(case["q"], case["k_bits"], case["v_bits"], case["k_scale"],
                                              case["v_scale"], case["lens"])
    e_out, e_lse = max_abs(out, ref_out), max_abs(lse, ref_lse)
    print(f"  n_splits {n_splits}: max-abs out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= TOL and e_lse <= TOL


@pytest.mark.parametrize("kernel", ["mfma", "valu"])
def test_fp8_both_kernels_unit_scales_and_bf16_out(fd, kernel):
    """Scales left NULL (= 1) and a bf16 output, through each partial kernel
    (the test entry point picks the kernel where both support the shape)."""
    case = synth.fp8_case(2, 16, 2, 128, 800, seed=4100, lens=[800, 333])
    case["k_bits"] = synth.to_e4m3(synth.host_normal((2, 2, 800, 128), 4101, "fp32") * 0.2, np.ones(2))
    case["v_bits"] = synth.to_e4m3(synth.host_normal((2, 2, 800, 128), 4102, "fp32"), np.ones(2))
    q = to_dev(case["q"], "bf16")
    k = torch.from_numpy(case["k_bits"]).to("cuda")
    v = torch.from_numpy(case["v_bits"]).to("cuda")
    lens = torch.from_numpy(case["lens"]).to("cuda")
    for ns in (0, 4):
        o, l = fd.testing_decode_attn(q, k, v, kernel, lens=lens, n_splits=ns, out_dtype=torch.bfloat16,
                                      return_lse=True)
        torch.cuda.synchronize()
        out, lse = to_host(o), to_host(l)
        ref_out, ref_lse = oracle.attention_fp8kv(case["q"], case["k_bits"], case["v_bits"], None, None,
                                                  case["lens"])
        assert max_abs(out, ref_out) <= TOL and max_abs(lse, ref_lse) <= TOL


def test_fp8_extreme_codes(fd):
    """Largest codes (+-448), subnormals and zeros in the cache."""
    rng = np.random.Generator(np.random.PCG64(4200))
    case = synth.fp8_case(1, 8, 1, 128, 256, seed=4200, lens=[256])
    special = np.array([0x7E, 0xFE, 0x01, 0x81, 0x07, 0x00, 0x80, 0x08], dtype=np.uint8)
    pick = rng.integers(0, special.size, size=case["v_bits"].shape)
    mask = rng.random(case["v_bits"].shape) < 0.3
    case["v_bits"] = np.where(mask, special[pick], case["v_bits"]).astype(np.uint8)
    case["k_bits"] = np.where(rng.random(case["k_bits"].shape) < 0.1, 0x01, case["k_bits"]).astype(np.uint8)
    out, lse = run_fp8(fd, case, 0)
    ref_out, ref_lse = oracle.attention_fp8kv(case["q"], case["k_bits"], case["v_bits"], case["k_scale"],
                                              case["v_scale"], case["lens"])
    # V values reach 448 * scale (about 6).  The split-KV kernels pass each
    # softmax weight to the matrix cores as two bf16 parts (fp32-accurate),
    # so the flat bound holds whatever the spread of V.
    assert max_abs(out, ref_out) <= TOL and max_abs(lse, ref_lse) <= TOL


def make_fp8_workload(w):
    dev = "cuda"
    q = synth.device_normal((w.batch, w.q_heads, w.head_dim), w.seed, "bf16", dev)
    ks, vs = synth.head_scales(w.kv_heads, w.seed + 3), synth.head_scales(w.kv_heads, w.seed + 4)
    shape = (w.batch, w.kv_heads, w.max_len, w.head_dim)
    k = synth.device_fp8(shape, w.seed + 1, ks, dev)
    v = synth.device_fp8(shape, w.seed + 2, vs, dev)
    if w.ragged:
        lens = synth.device_lengths(w.batch, w.max_len // 2, w.max_len, w.seed + 7, dev)
    else:
        lens = torch.full((w.batch,), w.max_len, dtype=torch.int32, device=dev)
    for b, n in enumerate(lens.tolist()):
        k[b, :, n:] = 0x7F
        v[b, :, n:] = 0x7F
    return q, k, v, torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev), lens


@pytest.mark.parametrize("w", configs.ALL_FP8, ids=lambda w: w.name)
def test_fp8_workload_full_size(fd, w):
    print(f"  workload {w.name}", flush=True)
    q, k, v, ks, vs, lens = make_fp8_workload(w)
    out, lse = fd.decode_attn_fp8(q, k, v, ks, vs, lens, n_splits=w.n_splits, return_lse=True)
    torch.cuda.synchronize()
    out_h, lse_h = to_host(out), to_host(lse)
    assert np.all(np.isfinite(out_h))
    G = w.q_heads // w.kv_heads
    lens_h, ks_h, vs_h = lens.cpu().numpy(), ks.cpu().numpy(), vs.cpu().numpy()
    worst = 0.0
    units = sampled_units(w, 4, w.seed)
    for (b, g) in units:
        n = int(lens_h[b])
        kb = k[b:b + 1, g:g + 1, :n].cpu().numpy()
        vb = v[b:b + 1, g:g + 1, :n].cpu().numpy()
        ro, rl = oracle.attention_fp8kv(to_host(q[b:b + 1, g * G:(g + 1) * G]), kb, vb, ks_h[g:g + 1],
                                        vs_h[g:g + 1])
        worst = max(worst, max_abs(out_h[b, g * G:(g + 1) * G], ro[0]), max_abs(lse_h[b, g * G:(g + 1) * G], rl[0]))
    print(f"  {len(units)} units, max-abs {worst:.3e} (tol {w.tol})", flush=True)
    assert worst <= w.tol

    def rows_of(b):
        n = int(lens_h[b])
        deq = lambda c, sc: c[b, :, :n].view(torch.float8_e4m3fn).float() * sc[:, None, None]
        return deq(k, ks), deq(v, vs)

    rows = check_every_unit(q, rows_of, lens_h, out, lse, w.tol)
    print(f"  all {rows} output rows inside the value hull, lse inside its bounds", flush=True)
    del k, v
    torch.cuda.empty_cache()
