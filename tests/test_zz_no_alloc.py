"""fd_decode_attn_noalloc (partials in the library's fixed per-GPU array)
against fd_decode_attn (partials in a caller workspace), through the C ABI.

Both run the same kernels with the same split count, so their outputs must
be equal bit for bit; each is also held to the oracle's bound (max-abs 1e-5
for fp32 inputs, 1e-2 for bf16).  Two calls in a row, the second on a
smaller input, so the second reuses an array the first left filled.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import max_abs, to_dev, to_host
from workloads import synth

pytestmark = pytest.mark.gpu

CASES = [
    # B, Hq, Hkv, D, Lmax, dtype, lens, n_splits (0 = planner)
    (3, 16, 2, 128, 4000, "bf16", [4000, 1777, 1], 0),     # matrix-core kernel, many pieces
    (1, 4, 4, 64, 512, "fp32", [512], 4),                  # smaller: vector-ALU kernel, 4 pieces
]


def _run_both(fd, case, dtype, n_splits):
    q, k, v = (to_dev(case[x], dtype) for x in ("q", "k", "v"))
    lens = torch.from_numpy(case["lens"]).to("cuda")
    ref, ref_lse = fd.decode_attn(q, k, v, lens, n_splits=n_splits, return_lse=True)
    got, got_lse = fd.decode_attn_noalloc(q, k, v, lens, n_splits=n_splits, return_lse=True)
    torch.cuda.synchronize()
    return to_host(ref), to_host(ref_lse), to_host(got), to_host(got_lse)


def test_noalloc_matches_workspace_call_twice_shrinking(fd):
    for i, (B, Hq, Hkv, D, L, dt, lens, ns) in enumerate(CASES):
        print(f"  call {i}: B{B} Hq{Hq} Hkv{Hkv} D{D} L{L} {dt} n_splits={ns}", flush=True)
        case = synth.decode_case(B, Hq, Hkv, D, L, dt, seed=5100 + i, lens=lens)
        ref, ref_lse, got, got_lse = _run_both(fd, case, dt, ns)
        assert np.array_equal(got, ref) and np.array_equal(got_lse, ref_lse)
        o, l = oracle.attention(case["q"], case["k"], case["v"], case["lens"])
        tol = 1e-5 if dt == "fp32" else 1e-2
        assert max_abs(got, o) <= tol and max_abs(got_lse, l) <= tol


def test_noalloc_rejects_partials_beyond_the_array(fd):
    # 1024 x 32 query rows x 256 pieces x (128 + 1) floats is far above 16 MiB
    B, Hq, Hkv, D, L = 1024, 32, 32, 128, 64
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, L, D), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(fd.FdError) as e:
        fd.decode_attn_noalloc(q, k, k, None, n_splits=256)
    assert e.value.status == fd.FD_ERR_WORKSPACE
    # a call that fits still works afterwards
    case = synth.decode_case(1, 8, 2, 128, 700, "bf16", seed=5200, lens=[700])
    ref, _, got, _ = _run_both(fd, case, "bf16", 3)
    assert np.array_equal(got, ref)
