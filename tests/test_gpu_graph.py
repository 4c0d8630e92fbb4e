"""Calls captured in a HIP graph give the eager call's bits on every replay.

Each entry point writes into preallocated outputs (and workspace) while
torch records a HIP graph; the graph is then replayed three times, with
eager kernels (a fill of the outputs with NaN, an unrelated decode call)
and synchronizations between the replays, and every replay must reproduce
the eager result bit for bit.  The library records no memset and allocates
nothing inside a call, and its kernels are deterministic.
"""

import numpy as np
import pytest
import torch

from tests.gpu_cases import to_dev
from workloads import synth

pytestmark = pytest.mark.gpu


def _other_work(fd):
    """An unrelated eager decode call, run between the replays."""
    c = synth.decode_case(1, 4, 4, 64, 300, "fp32", seed=91)
    q, k, v = (to_dev(c[x], "fp32") for x in ("q", "k", "v"))
    lens = torch.from_numpy(c["lens"]).to("cuda")
    return lambda: fd.decode_attn(q, k, v, lens, n_splits=3)


def _check_replays(fn, outs, other):
    fn()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    for r in range(3):
        for t in outs:
            t.fill_(float("nan"))
        other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, ref):
            assert torch.equal(t, e), f"replay {r} differs from the eager call"
    del g


def _decode_case(fd, B, Hq, Hkv, D, L, dtype, seed, lens, n_splits):
    c = synth.decode_case(B, Hq, Hkv, D, L, dtype, seed=seed, lens=lens)
    q, k, v = (to_dev(c[x], dtype) for x in ("q", "k", "v"))
    lens_d = torch.from_numpy(c["lens"]).to("cuda")
    dt = fd.FD_BF16 if dtype == "bf16" else fd.FD_F32
    ns = n_splits or fd.plan_splits(B, Hq, Hkv, D, L, dt, fd.device_cu_count())
    ws = torch.empty(max(1, fd.decode_workspace_size(B, Hq, Hkv, D, L, dt, ns)), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(q)
    return c, q, k, v, lens_d, ns, ws, out


@pytest.mark.parametrize("B,Hq,Hkv,D,L,dtype,lens,n_splits", [
    (2, 16, 2, 128, 4096, "bf16", [4096, 3000], 9),      # matrix-core partials + combine
    (1, 16, 2, 128, 8192, "bf16", [8192], 0),            # matrix-core, interleaved pieces (planner)
    (3, 8, 8, 128, 2000, "bf16", [2000, 1, 1234], 0),    # vector-ALU, ragged
    (1, 4, 4, 64, 512, "fp32", [512], 4),                # fp32
    (2, 8, 8, 128, 700, "bf16", [700, 333], 1),          # one piece: direct output
])
def test_decode_graph_replays(fd, B, Hq, Hkv, D, L, dtype, lens, n_splits):
    print(f"  decode B={B} Hq={Hq} Hkv={Hkv} D={D} L={L} {dtype} n_splits={n_splits}", flush=True)
    _, q, k, v, lens_d, ns, ws, out = _decode_case(fd, B, Hq, Hkv, D, L, dtype, 21, lens, n_splits)
    _check_replays(lambda: fd.decode_attn(q, k, v, lens_d, n_splits=ns, out=out, workspace=ws), [out],
                   _other_work(fd))


def test_paged_graph_replays(fd):
    print("  paged B=2 Hq=16 Hkv=2 D=128 L=1500 page 16", flush=True)
    c = synth.decode_case(2, 16, 2, 128, 1500, "bf16", seed=23, lens=[1500, 611])
    kp, vp, table = synth.paginate(c["k"], c["v"], c["lens"], 16, seed=23)
    q, kp, vp = to_dev(c["q"], "bf16"), to_dev(kp, "bf16"), to_dev(vp, "bf16")
    table = torch.from_numpy(table).to("cuda")
    lens = torch.from_numpy(c["lens"]).to("cuda")
    L = table.shape[1] * 16
    ns = fd.plan_splits(2, 16, 2, 128, L, fd.FD_BF16, fd.device_cu_count())
    ws = torch.empty(max(1, fd.decode_workspace_size(2, 16, 2, 128, L, fd.FD_BF16, ns)), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(q)
    _check_replays(lambda: fd.decode_attn_paged(q, kp, vp, table, lens, n_splits=ns, out=out, workspace=ws),
                   [out], _other_work(fd))


def test_bifurcated_graph_replays(fd):
    print("  bifurcated S=8 Hq=16 Hkv=2 D=128 Lc=1000 Ld=64", flush=True)
    S, Hq, Hkv, D, Lc, Ld = 8, 16, 2, 128, 1000, 64
    c = synth.bifurcated_case(S, Hq, Hkv, D, Lc, Ld, "bf16", seed=25, dec_lens=[64, 0, 7, 19, 64, 1, 33, 50])
    t = {x: to_dev(c[x], "bf16") for x in ("q", "k_ctx", "v_ctx", "k_dec", "v_dec")}
    dl = torch.from_numpy(c["dec_lens"]).to("cuda")
    ws = torch.empty(fd.bifurcated_workspace_size(S, Hq, Hkv, D, Lc, Ld, fd.FD_BF16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(t["q"])
    _check_replays(lambda: fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"], dl,
                                              out=out, workspace=ws), [out], _other_work(fd))


def test_prefill_graph_replays(fd):
    print("  prefill B=2 Hq=16 Hkv=2 D=128 L=700", flush=True)
    rng = np.random.Generator(np.random.PCG64(27))
    q = to_dev(rng.standard_normal((2, 16, 700, 128)), "bf16")
    k = to_dev(rng.standard_normal((2, 2, 700, 128)), "bf16")
    v = to_dev(rng.standard_normal((2, 2, 700, 128)), "bf16")
    lens = torch.tensor([700, 413], dtype=torch.int32, device="cuda")
    out = torch.zeros_like(q)
    _check_replays(lambda: fd.prefill_attn(q, k, v, lens, out=out), [out[0], out[1, :, :413]], _other_work(fd))
