"""fd_bifurcated_attn_paged: each sample's decode rows in a shuffled page
pool, against the fp64 oracle (bifurcated_paged_attention) and against
fd_bifurcated_attn on the gathered decode cache: bit for bit where both
decode roles use the same tile layout, else to 1e-5.

Page 0 and the rows past dec_lens[s] in a used page are NaN, and unused
table entries are -1, so any read outside the valid rows poisons the
result.  Bound: max-abs 1e-2 (bf16 inputs), 1e-5 (fp32 inputs).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import max_abs, to_dev, to_host
from workloads import configs, synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("shape", [
    # S, Hq, Hkv, D, Lc, Ldmax, page, dec_lens, dtype
    (5, 8, 2, 128, 700, 64, 16, [64, 0, 1, 33, 17], "bf16"),     # matrix-core context part, G 4
    (8, 32, 1, 128, 1024, 48, 16, (1, 48), "bf16"),               # MQA: two 16-row decode blocks
    (6, 32, 8, 128, 2000, 100, 32, (1, 100), "bf16"),             # GQA like the bifurcated GQA workload
    (3, 4, 4, 64, 300, 40, 16, [40, 0, 5], "fp32"),               # split-KV context and decode parts
], ids=lambda s: f"S{s[0]}_hq{s[1]}_hkv{s[2]}_p{s[6]}_{s[8]}")
def test_bifurcated_paged_matches_oracle_and_dense(fd, shape):
    S, Hq, Hkv, D, Lc, Ld, P, dl, dt = shape
    case = synth.bifurcated_case(S, Hq, Hkv, D, Lc, Ld, dt, seed=7500 + S, dec_lens=dl)
    kp, vp, table = synth.paginate(case["k_dec"], case["v_dec"], case["dec_lens"], P, seed=7600 + S)
    t = {k: to_dev(case[k], dt) for k in ("q", "k_ctx", "v_ctx", "k_dec", "v_dec")}
    dlen = torch.from_numpy(case["dec_lens"]).cuda()
    got, got_lse = fd.bifurcated_attn_paged(t["q"], t["k_ctx"], t["v_ctx"], to_dev(kp, dt), to_dev(vp, dt),
                                            torch.from_numpy(table).cuda(), dlen, return_lse=True)
    # dense call on the gathered cache (decode rows up to the table's reach)
    Lt = table.shape[1] * P
    kd = torch.zeros((S, Hkv, Lt, D), dtype=t["q"].dtype, device="cuda")
    vd = torch.zeros_like(kd)
    kd[:, :, :Ld] = t["k_dec"]
    vd[:, :, :Ld] = t["v_dec"]
    dense, dense_lse = fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], kd, vd, dlen, return_lse=True)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(to_host(got)))
    if dt == "bf16" and Hq // Hkv <= 8:
        # the dense decode role packs two heads' weights per matrix-core
        # tile and keeps its running sums there; the paged one does not, so
        # the two round the row sums in a different order
        assert max_abs(to_host(got), to_host(dense)) <= 1e-5
        assert max_abs(to_host(got_lse), to_host(dense_lse)) <= 1e-5
    else:
        assert np.array_equal(to_host(got), to_host(dense))
        assert np.array_equal(to_host(got_lse), to_host(dense_lse))
    ref_o, ref_l = oracle.bifurcated_paged_attention(case["q"], case["k_ctx"], case["v_ctx"], kp, vp, table,
                                                     case["dec_lens"])
    tol = 1e-5 if dt == "fp32" else 1e-2
    e_o, e_l = max_abs(to_host(got), ref_o), max_abs(to_host(got_lse), ref_l)
    print(f"  paged bifurcated: max-abs out {e_o:.3e} lse {e_l:.3e}", flush=True)
    assert e_o <= tol and e_l <= tol


def test_bifurcated_paged_gqa_workload_full_size(fd):
    """The bifurcated GQA workload (128 samples, 32768 context rows, decode
    rows uniform in [1, 512]) with its decode rows in 16-row pages: sampled
    samples (first, last, shortest decode part) against the oracle."""
    w = configs.BIFURCATED_GQA
    S, Hq, Hkv, D, Lc, Ld, P = w.samples, w.q_heads, w.kv_heads, w.head_dim, w.ctx_len, w.dec_max, 16
    dev = "cuda"
    q = synth.device_normal((S, Hq, D), w.seed, "bf16", dev)
    kc = synth.device_normal((Hkv, Lc, D), w.seed + 1, "bf16", dev)
    vc = synth.device_normal((Hkv, Lc, D), w.seed + 2, "bf16", dev)
    dl = synth.device_lengths(S, w.dec_lo, w.dec_max, w.seed + 7, dev)
    per = Ld // P
    table = torch.from_numpy(synth.shuffled_block_table(S, per, w.seed + 11)).to(dev)
    n_pages = 1 + S * per
    kp = synth.device_normal((n_pages, Hkv, P, D), w.seed + 3, "bf16", dev)
    vp = synth.device_normal((n_pages, Hkv, P, D), w.seed + 4, "bf16", dev)
    kp[0] = float("nan")
    vp[0] = float("nan")
    out, lse = fd.bifurcated_attn_paged(q, kc, vc, kp, vp, table, dl, return_lse=True)
    torch.cuda.synchronize()
    out_h, lse_h = to_host(out), to_host(lse)
    assert np.all(np.isfinite(out_h))
    dl_h, tab_h = dl.cpu().numpy(), table.cpu().numpy()
    samples = sorted({0, S - 1, int(np.argmin(dl_h)), int(np.argmax(dl_h))})
    kc_h, vc_h = to_host(kc), to_host(vc)
    worst = 0.0
    for s in samples:
        n = int(dl_h[s])
        pages = sorted({int(tab_h[s, j]) for j in range(-(-n // P))})
        # the sample's own pages, renumbered; the oracle reads them through its table row
        remap = {pg: i for i, pg in enumerate(pages)}
        kps = to_host(kp[pages]) if pages else np.zeros((0, Hkv, P, D))
        vps = to_host(vp[pages]) if pages else np.zeros((0, Hkv, P, D))
        trow = np.array([[remap.get(int(x), -1) for x in tab_h[s]]])
        ro, rl = oracle.bifurcated_paged_attention(to_host(q[s:s + 1]), kc_h, vc_h, kps, vps, trow, [n])
        worst = max(worst, max_abs(out_h[s:s + 1], ro), max_abs(lse_h[s:s + 1], rl))
    print(f"  samples {samples}: max-abs {worst:.3e}", flush=True)
    assert worst <= w.tol
    del kp, vp
    torch.cuda.empty_cache()
