"""Tensors passed by descriptor with strides (fd_decode_attn_strided,
fd_bifurcated_attn_strided) against the fp64 oracle and against the dense
entry points, through the C ABI.

A token-major cache [B, L, Hkv, D] is the logical [B, Hkv, L, D] with
strides {L*Hkv*D, D, Hkv*D, 1}; q and out are slices of larger tensors.
The strided call must give the dense call's result bit for bit (same
kernels, same split count) and hold the oracle's bound: max-abs 1e-5 for
fp32 inputs, 1e-2 for bf16 and E4M3 caches.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import max_abs, to_dev, to_host
from workloads import synth

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 1e-2}


def token_major(x):
    """Device tensor [B, Hkv, L, D] -> same values stored [B, L, Hkv, D],
    returned as the logical [B, Hkv, L, D] view."""
    return x.permute(0, 2, 1, 3).contiguous().permute(0, 2, 1, 3)


def wide(x, extra):
    """Same values as x [A, H, D], stored with `extra` padding columns per row."""
    A, H, D = x.shape
    big = torch.full((A, H, D + extra), float("nan"), dtype=x.dtype, device=x.device)
    big[:, :, :D] = x
    return big[:, :, :D]


@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, D, Lmax, dtype, lens
    (3, 16, 2, 128, 1500, "bf16", [1500, 700, 1]),     # matrix-core kernel
    (2, 8, 8, 128, 900, "bf16", [900, 333]),           # vector-ALU kernel, MHA
    (2, 8, 2, 64, 700, "fp32", [700, 65]),             # vector-ALU kernel, fp32, D 64
    (1, 32, 1, 128, 600, "bf16", [600]),               # MQA: 32-row units
], ids=lambda s: f"B{s[0]}_hq{s[1]}_hkv{s[2]}_d{s[3]}_{s[5]}")
@pytest.mark.parametrize("n_splits", [1, 0, 6])
def test_token_major_cache_and_strided_io(fd, shape, n_splits):
    B, Hq, Hkv, D, L, dt, lens = shape
    case = synth.decode_case(B, Hq, Hkv, D, L, dt, seed=7100 + Hq, lens=lens)
    q, k, v = (to_dev(case[x], dt) for x in ("q", "k", "v"))
    lens_d = torch.from_numpy(case["lens"]).to("cuda")
    dense, dense_lse = fd.decode_attn(q, k, v, lens_d, n_splits=n_splits, return_lse=True)
    ks, vs = token_major(k), token_major(v)
    qs = wide(q, 8 if dt == "bf16" else 4)
    out_big = torch.full((B, Hq + 2, D), float("nan"), dtype=q.dtype, device="cuda")
    outs = out_big[:, 1:Hq + 1]
    got, got_lse = fd.decode_attn_strided(qs, ks, vs, lens_d, n_splits=n_splits, out=outs, return_lse=True)
    torch.cuda.synchronize()
    assert ks.stride()[2] == Hkv * D and ks.stride()[0] == L * Hkv * D
    assert np.array_equal(to_host(got), to_host(dense)) and np.array_equal(to_host(got_lse), to_host(dense_lse))
    assert torch.isnan(out_big[:, 0]).all() and torch.isnan(out_big[:, Hq + 1]).all(), "wrote outside out"
    ref_o, ref_l = oracle.attention(case["q"], case["k"], case["v"], case["lens"])
    e_o, e_l = max_abs(to_host(got), ref_o), max_abs(to_host(got_lse), ref_l)
    print(f"  strided n_splits={n_splits}: max-abs out {e_o:.3e} lse {e_l:.3e}", flush=True)
    assert e_o <= TOL[dt] and e_l <= TOL[dt]


def test_head_major_output_and_fp8_token_major(fd):
    """E4M3 codes in a token-major cache; the output written head-major
    ([Hq, B, D] storage seen as [B, Hq, D])."""
    B, Hq, Hkv, D, L = 2, 16, 2, 128, 800
    case = synth.fp8_case(B, Hq, Hkv, D, L, seed=7200, lens=[800, 97])
    q = to_dev(case["q"], "bf16")
    k = torch.from_numpy(case["k_bits"]).to("cuda")
    v = torch.from_numpy(case["v_bits"]).to("cuda")
    ksc = torch.from_numpy(case["k_scale"]).to("cuda")
    vsc = torch.from_numpy(case["v_scale"]).to("cuda")
    lens = torch.from_numpy(case["lens"]).to("cuda")
    dense = fd.decode_attn_fp8(q, k, v, ksc, vsc, lens, n_splits=5, out_dtype=torch.float32)
    out = torch.empty((Hq, B, D), dtype=torch.float32, device="cuda").permute(1, 0, 2)
    got = fd.decode_attn_strided(q, token_major(k), token_major(v), lens, n_splits=5, out=out, k_scale=ksc,
                                 v_scale=vsc)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(got), to_host(dense))
    ref_o, _ = oracle.attention_fp8kv(case["q"], case["k_bits"], case["v_bits"], case["k_scale"], case["v_scale"],
                                      case["lens"])
    assert max_abs(to_host(got), ref_o) <= 1e-2


@pytest.mark.parametrize("shape", [
    # S, Hq, Hkv, D, Lc, Ldmax, dec_lens, dtype
    (6, 32, 8, 128, 1000, 64, [64, 0, 1, 33, 17, 64], "bf16"),   # matrix-core context part
    (8, 32, 1, 128, 700, 40, (1, 40), "bf16"),                   # MQA
    (3, 4, 4, 64, 300, 16, [16, 0, 5], "fp32"),                  # split-KV context part
], ids=lambda s: f"S{s[0]}_hq{s[1]}_hkv{s[2]}_{s[7]}")
def test_bifurcated_token_major(fd, shape):
    S, Hq, Hkv, D, Lc, Ld, dl, dt = shape
    case = synth.bifurcated_case(S, Hq, Hkv, D, Lc, Ld, dt, seed=7300 + S, dec_lens=dl)
    t = {k: to_dev(case[k], dt) for k in ("q", "k_ctx", "v_ctx", "k_dec", "v_dec")}
    dlen = torch.from_numpy(case["dec_lens"]).cuda()
    dense, dense_lse = fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"], dlen,
                                          return_lse=True)
    # context stored token-major [Lc, Hkv, D]; decode rows [S, Ld, Hkv, D]
    kc = t["k_ctx"].permute(1, 0, 2).contiguous().permute(1, 0, 2)
    vc = t["v_ctx"].permute(1, 0, 2).contiguous().permute(1, 0, 2)
    out_big = torch.full((S, Hq + 1, D), float("nan"), dtype=t["q"].dtype, device="cuda")
    got, got_lse = fd.bifurcated_attn_strided(wide(t["q"], 8), kc, vc, token_major(t["k_dec"]),
                                              token_major(t["v_dec"]), dlen, out=out_big[:, 1:], return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(to_host(got), to_host(dense)) and np.array_equal(to_host(got_lse), to_host(dense_lse))
    ref_o, ref_l = oracle.bifurcated_attention(case["q"], case["k_ctx"], case["v_ctx"], case["k_dec"],
                                               case["v_dec"], case["dec_lens"])
    assert max_abs(to_host(got), ref_o) <= TOL[dt] and max_abs(to_host(got_lse), ref_l) <= TOL[dt]


def test_strided_rejects_bad_layouts(fd):
    B, Hq, Hkv, D, L = 1, 8, 2, 128, 64
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, L, D), dtype=torch.bfloat16, device="cuda")
    # K and V with different strides
    with pytest.raises(fd.FdError) as e:
        fd.decode_attn_strided(q, k, token_major(k.clone()), n_splits=2)
    assert e.value.status == fd.FD_ERR_UNSUPPORTED
    # overlapping output rows (head stride 0)
    out = torch.zeros((B, 1, D), dtype=torch.bfloat16, device="cuda").expand(B, Hq, D)
    with pytest.raises(fd.FdError) as e:
        fd.decode_attn_strided(q, k, k, n_splits=2, out=out)
    assert e.value.status == fd.FD_ERR_INVALID_ARG
    # a row stride that is not a multiple of 16 bytes
    kb = torch.zeros((B, Hkv, L, D + 4), dtype=torch.bfloat16, device="cuda")[..., :D]
    with pytest.raises(fd.FdError) as e:
        fd.decode_attn_strided(q, kb, kb, n_splits=2)
    assert e.value.status == fd.FD_ERR_INVALID_ARG
