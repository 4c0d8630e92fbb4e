"""Paged-KV decode attention (fd_decode_attn_paged) against the fp64 oracle,
and bit for bit against the dense entry point on the gathered cache.

The page pool is shuffled; page 0 is never used and holds NaN, table entries
past a sequence's pages hold -1 (which the library clamps to page 0), and rows
past a sequence's length inside its last page are NaN: reading anything that
is not a valid row poisons the result.
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import check_every_unit, dense_rows, max_abs, sampled_units, to_dev, to_host
from workloads import configs, synth

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 1e-2}

SHAPES = [
    # B, Hq, Hkv, D, Lmax, dtype, lens
    (3, 16, 2, 128, 1000, "bf16", [1, 777, 1000]),    # matrix-core kernel, G = 8
    (2, 8, 8, 128, 700, "bf16", [700, 300]),          # vector-ALU kernel, bf16 D 128
    (2, 8, 2, 64, 600, "bf16", [600, 33]),            # vector-ALU kernel, bf16 D 64
    (2, 4, 4, 128, 500, "fp32", [17, 500]),           # fp32 D 128 (8-row wave tiles)
    (3, 6, 6, 64, 300, "fp32", [1, 16, 300]),         # fp32 D 64
    (2, 32, 1, 128, 900, "bf16", [900, 100]),         # MQA, 32-row matrix-core blocks
    (2, 12, 4, 128, 400, "bf16", [400, 129]),         # G = 3
]


def run_paged(fd, case, dtype, page_size, n_splits, seed=0, out_dtype=None):
    kp, vp, table = synth.paginate(case["k"], case["v"], case["lens"], page_size, seed)
    q = to_dev(case["q"], dtype)
    kp_d, vp_d = to_dev(kp, dtype), to_dev(vp, dtype)
    table_d = torch.from_numpy(table).to("cuda")
    lens = torch.from_numpy(case["lens"]).to("cuda")
    out, lse = fd.decode_attn_paged(q, kp_d, vp_d, table_d, lens, n_splits=n_splits, out_dtype=out_dtype,
                                    return_lse=True)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse), (kp, vp, table)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_hq{s[1]}_hkv{s[2]}_d{s[3]}_l{s[4]}_{s[5]}")
@pytest.mark.parametrize("page_size", [16, 64])
@pytest.mark.parametrize("n_splits", [0, 1, 5])
def test_paged_matches_oracle(fd, shape, page_size, n_splits):
    B, Hq, Hkv, D, L, dt, lens = shape
    case = synth.decode_case(B, Hq, Hkv, D, L, dt, seed=2000 + B * 7 + Hq, lens=lens)
    out, lse, (kp, vp, table) = run_paged(fd, case, dt, page_size, n_splits, seed=page_size)
    ref_out, ref_lse = oracle.paged_attention(case["q"], kp, vp, table, case["lens"])
    e_out, e_lse = max_abs(out, ref_out), max_abs(lse, ref_lse)
    print(f"  page {page_size} n_splits {n_splits}: max-abs out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= TOL[dt] and e_lse <= TOL[dt]


@pytest.mark.parametrize("page_size", [16, 32, 128, 1024])
@pytest.mark.parametrize("shape", [(2, 16, 2, 128, 2500, "bf16", [2500, 1234]),
                                   (2, 4, 4, 128, 2100, "bf16", [2100, 17])],
                         ids=["mfma_g8", "valu_g1"])
def test_paged_bitwise_equals_dense(fd, shape, page_size):
    """Same rows, same pieces, same order: the paged call reproduces the
    dense call on the gathered cache exactly (for the same split count; the
    planner would see a different max_len, the table's width times the page
    size)."""
    B, Hq, Hkv, D, L, dt, lens = shape
    case = synth.decode_case(B, Hq, Hkv, D, L, dt, seed=3000 + page_size, lens=lens)
    for ns in (1, 3, 24):
        out_p, lse_p, _ = run_paged(fd, case, dt, page_size, ns, seed=page_size + 1)
        q, k, v = (to_dev(case[x], dt) for x in ("q", "k", "v"))
        lens_d = torch.from_numpy(case["lens"]).to("cuda")
        out_d, lse_d = fd.decode_attn(q, k, v, lens_d, n_splits=ns, return_lse=True)
        torch.cuda.synchronize()
        assert np.array_equal(out_p, to_host(out_d)), f"out differs (n_splits={ns})"
        assert np.array_equal(lse_p, to_host(lse_d)), f"lse differs (n_splits={ns})"


def test_paged_bf16_output_and_every_page_boundary(fd):
    # lengths on both sides of each page boundary, bf16 output
    lens = [15, 16, 17, 31, 32, 33, 63, 64]
    case = synth.decode_case(len(lens), 8, 1, 128, 64, "bf16", seed=3100, lens=lens)
    out, lse, (kp, vp, table) = run_paged(fd, case, "bf16", 16, 0, seed=5, out_dtype=torch.bfloat16)
    ref_out, ref_lse = oracle.paged_attention(case["q"], kp, vp, table, case["lens"])
    assert max_abs(out, ref_out) <= TOL["bf16"] and max_abs(lse, ref_lse) <= TOL["bf16"]


def make_paged_workload(w, pad_nan=True):
    """Full-size paged cache drawn on the device, pages in shuffled order."""
    dev = "cuda"
    P = w.page_size
    per_seq = -(-w.max_len // P)
    n_pages = 1 + w.batch * per_seq
    q = synth.device_normal((w.batch, w.q_heads, w.head_dim), w.seed, w.dtype, dev)
    kp = synth.device_normal((n_pages, w.kv_heads, P, w.head_dim), w.seed + 1, w.dtype, dev)
    vp = synth.device_normal((n_pages, w.kv_heads, P, w.head_dim), w.seed + 2, w.dtype, dev)
    table = torch.from_numpy(synth.shuffled_block_table(w.batch, per_seq, w.seed + 11)).to(dev)
    if w.ragged:
        lens = synth.device_lengths(w.batch, w.max_len // 2, w.max_len, w.seed + 7, dev)
    else:
        lens = torch.full((w.batch,), w.max_len, dtype=torch.int32, device=dev)
    if pad_nan:
        kp[0] = float("nan")
        vp[0] = float("nan")
        tab = table.cpu().numpy()
        for b, n in enumerate(lens.tolist()):
            last, used = tab[b, (n - 1) // P], (n - 1) % P + 1
            kp[int(last), :, used:] = float("nan")
            vp[int(last), :, used:] = float("nan")
    return q, kp, vp, table, lens


@pytest.mark.parametrize("w", configs.ALL_PAGED, ids=lambda w: w.name)
def test_paged_workload_full_size(fd, w):
    print(f"  workload {w.name}", flush=True)
    q, kp, vp, table, lens = make_paged_workload(w)
    out, lse = fd.decode_attn_paged(q, kp, vp, table, lens, n_splits=w.n_splits, return_lse=True)
    torch.cuda.synchronize()
    out_h, lse_h = to_host(out), to_host(lse)
    assert np.all(np.isfinite(out_h))
    G = w.q_heads // w.kv_heads
    P = w.page_size
    tab, lens_h = table.cpu().numpy(), lens.cpu().numpy()
    worst = 0.0
    units = sampled_units(w, 4, w.seed)
    for (b, g) in units:
        n = int(lens_h[b])
        used = tab[b, :-(-n // P)]
        # only this unit's pages, renumbered 0..m-1 (page ids are labels)
        kp_h = to_host(kp[torch.from_numpy(used.astype(np.int64)).to("cuda"), g:g + 1])
        vp_h = to_host(vp[torch.from_numpy(used.astype(np.int64)).to("cuda"), g:g + 1])
        ro, rl = oracle.paged_attention(to_host(q[b:b + 1, g * G:(g + 1) * G]), kp_h, vp_h,
                                        np.arange(len(used))[None], np.array([n]))
        worst = max(worst, max_abs(out_h[b, g * G:(g + 1) * G], ro[0]), max_abs(lse_h[b, g * G:(g + 1) * G], rl[0]))
    print(f"  {len(units)} units, max-abs {worst:.3e} (tol {w.tol})", flush=True)
    assert worst <= w.tol
    # bit for bit against the dense call on the gathered cache (same planner split)
    per_seq = table.shape[1]
    idx = table.long()
    k_dense = kp[idx].permute(0, 2, 1, 3, 4).reshape(w.batch, w.kv_heads, per_seq * P, w.head_dim).contiguous()
    v_dense = vp[idx].permute(0, 2, 1, 3, 4).reshape(w.batch, w.kv_heads, per_seq * P, w.head_dim).contiguous()
    out_d, lse_d = fd.decode_attn(q, k_dense, v_dense, lens, n_splits=w.n_splits, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out, out_d) and torch.equal(lse, lse_d)
    rows = check_every_unit(q, dense_rows(k_dense, v_dense, lens_h), lens_h, out, lse, w.tol)
    print(f"  all {rows} output rows inside the value hull, lse inside its bounds", flush=True)
    del kp, vp, k_dense, v_dense
    torch.cuda.empty_cache()
