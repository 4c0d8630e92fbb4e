"""HIP path against the fp64 oracle, through the C ABI (needs the GPU).

Tolerances: max-abs 1e-5 for fp32 inputs and 1e-2 for bf16 inputs with fp32
accumulation, on every output element (lse too, with the same bound).
"""

import numpy as np
import pytest
import torch

import oracle
from tests.gpu_cases import max_abs, oracle_decode_rows, to_dev, to_host
from workloads import configs, synth

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 1e-2}


def run_decode(fd, case, dtype, n_splits=0, out_dtype=None, scale=0.0):
    q, k, v = (to_dev(case[x], dtype) for x in ("q", "k", "v"))
    lens = torch.from_numpy(case["lens"]).to("cuda")
    out, lse = fd.decode_attn(q, k, v, lens, n_splits=n_splits, out_dtype=out_dtype, scale=scale,
                              return_lse=True)
    torch.cuda.synchronize()
    return to_host(out), to_host(lse)


def check_decode(fd, case, dtype, n_splits=0, out_dtype=None, scale=None, tol=None):
    out, lse = run_decode(fd, case, dtype, n_splits, out_dtype, scale or 0.0)
    ref_out, ref_lse = oracle.attention(case["q"], case["k"], case["v"], case["lens"], scale)
    tol = tol or TOL[dtype]
    e_out, e_lse = max_abs(out, ref_out), max_abs(lse, ref_lse)
    print(f"  n_splits={n_splits} max-abs out {e_out:.3e} lse {e_lse:.3e}", flush=True)
    assert e_out <= tol, f"out error {e_out} > {tol}"
    assert e_lse <= tol, f"lse error {e_lse} > {tol}"
    return out


# --------------------------------------------------------------------- tiny

@pytest.mark.parametrize("n_splits", [4, 1, 2, 3, 7, 16, 32, 64, 0])
def test_tiny_fp32_split_sweep(fd, n_splits):
    w = configs.TINY
    case = synth.decode_case(w.batch, w.q_heads, w.kv_heads, w.head_dim, w.max_len, w.dtype, w.seed)
    check_decode(fd, case, "fp32", n_splits=n_splits, tol=w.tol)


# ------------------------------------------------------ shapes and dtypes

SHAPES = [
    # B, Hq, Hkv, D, Lmax, dtype, lens
    (3, 16, 2, 128, 3000, "bf16", [1, 1777, 3000]),
    (4, 8, 8, 128, 2048, "bf16", (1024, 2048)),
    (2, 8, 2, 64, 1500, "bf16", [1500, 333]),
    (2, 4, 4, 128, 900, "fp32", [17, 900]),
    (2, 8, 4, 64, 777, "fp32", [777, 400]),
    (2, 32, 2, 128, 1200, "bf16", [1200, 650]),      # G = 16: two row blocks per KV head
    (1, 32, 1, 128, 2100, "bf16", [2100]),           # MQA, G = 32
    (2, 12, 4, 128, 640, "bf16", [640, 129]),        # G = 3
    (1, 24, 1, 128, 700, "bf16", [700]),             # G = 24: one 32-row matrix-core block
    (2, 48, 1, 128, 500, "bf16", [500, 77]),         # G = 48: two 32-row blocks
    (3, 64, 8, 128, 1100, "bf16", [1100, 64, 513]),  # G = 8
    (5, 6, 6, 64, 300, "fp32", [1, 15, 16, 17, 300]),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"B{s[0]}_hq{s[1]}_hkv{s[2]}_d{s[3]}_l{s[4]}_{s[5]}")
@pytest.mark.parametrize("n_splits", [0, 1, 5, 33])
def test_decode_shapes(fd, shape, n_splits):
    B, Hq, Hkv, D, L, dt, lens = shape
    case = synth.decode_case(B, Hq, Hkv, D, L, dt, seed=1000 + B * 7 + Hq, lens=lens)
    check_decode(fd, case, dt, n_splits=n_splits)


@pytest.mark.parametrize("lens_one", [1, 15, 16, 17, 255, 256, 257, 1023, 1024])
def test_boundary_lengths(fd, lens_one):
    case = synth.decode_case(2, 16, 2, 128, 1024, "bf16", seed=77, lens=[lens_one, 1024])
    for ns in (0, 4):
        check_decode(fd, case, "bf16", n_splits=ns)


@pytest.mark.parametrize("kernel", ["valu", "mfma"])
@pytest.mark.parametrize("G", [1, 2, 3, 4, 8, 16, 32])
def test_both_partial_kernels(fd, kernel, G):
    # the test entry point runs one of the two partial kernels (bf16, D 128)
    Hkv = 2
    case = synth.decode_case(2, G * Hkv, Hkv, 128, 1300, "bf16", seed=300 + G, lens=[1300, 555])
    q, k, v = (to_dev(case[x], "bf16") for x in ("q", "k", "v"))
    lens = torch.from_numpy(case["lens"]).to("cuda")
    ref_out, ref_lse = oracle.attention(case["q"], case["k"], case["v"], case["lens"])
    for ns in (1, 6):
        out, lse = fd.testing_decode_attn(q, k, v, kernel, lens=lens, n_splits=ns, return_lse=True)
        torch.cuda.synchronize()
        e_out, e_lse = max_abs(to_host(out), ref_out), max_abs(to_host(lse), ref_lse)
        print(f"  {kernel} n_splits={ns} max-abs out {e_out:.3e} lse {e_lse:.3e}", flush=True)
        assert e_out <= TOL["bf16"] and e_lse <= TOL["bf16"]


def test_bf16_output_and_explicit_scale(fd):
    case = synth.decode_case(2, 8, 2, 128, 1000, "bf16", seed=91, lens=[1000, 501])
    check_decode(fd, case, "bf16", n_splits=3, out_dtype=torch.float32, scale=0.05)
    check_decode(fd, case, "bf16", n_splits=3, out_dtype=torch.bfloat16)


def test_padding_rows_are_never_read(fd):
    # NaN in every row at or beyond lens must leave the output finite and equal
    case = synth.decode_case(2, 16, 2, 128, 2048, "bf16", seed=5, lens=[700, 1301], pad_nan=True)
    clean = dict(case)
    for key in ("k", "v"):
        clean[key] = np.where(np.isnan(case[key]), 0.0, case[key]).astype(np.float32)
    a, _ = run_decode(fd, case, "bf16", n_splits=7)
    b, _ = run_decode(fd, clean, "bf16", n_splits=7)
    assert np.all(np.isfinite(a))
    assert np.array_equal(a, b)


def test_bitwise_repeatable(fd):
    case = synth.decode_case(2, 16, 2, 128, 4096, "bf16", seed=6, lens=[4096, 3000])
    outs = [run_decode(fd, case, "bf16", n_splits=9)[0] for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


# ------------------------------------------------------------ combine op

@pytest.mark.parametrize("rows,P,D", [(37, 19, 128), (5, 64, 128), (9, 65, 128), (4, 300, 128), (7, 3, 64),
                                      (6, 40, 100), (3, 70, 100), (2, 1, 128), (3, 17, 512),
                                      (1100, 40, 128), (1024, 64, 64), (1030, 17, 512), (1024, 33, 256),
                                      (1025, 1, 128), (1024, 13, 128), (1027, 24, 128), (1024, 9, 64),
                                      (1026, 20, 64), (1024, 7, 256)])
def test_lse_combine_matches_oracle(fd, rows, P, D):
    # >= 1024 rows with <= 64 pieces: one wave per row (batches of 8, 16, 24
    # or 32 pieces, the smallest that covers the pieces within the head
    # dim's limit, so 33..64 pieces take a second batch); otherwise the
    # column-slice kernels
    rng = np.random.Generator(np.random.PCG64(12 + P))
    o = rng.standard_normal((rows, P, D)).astype(np.float32)
    lse = (rng.standard_normal((rows, P)) * 5).astype(np.float32)
    empty = rng.random((rows, P)) < 0.3
    empty[:, P // 2] = False               # every row keeps one finite piece
    lse[empty] = -np.inf
    o[np.isneginf(lse)] = 0.0
    out, l = fd.lse_combine(torch.from_numpy(o).cuda(), torch.from_numpy(lse).cuda(), return_lse=True)
    ref_o, ref_l = oracle.lse_combine(np.moveaxis(o, 1, 0), lse.T)
    assert max_abs(to_host(out), ref_o) <= 1e-5
    assert max_abs(to_host(l), ref_l) <= 1e-5


# ------------------------------------------------------- partial stage

def piece_rows(layout, n, n_splits, i, tile):
    """Cache rows of piece i as include/fd.h defines the two layouts."""
    if layout == 0:
        c = -(-n // n_splits)
        c = -(-c // 16) * 16
        return np.arange(min(i * c, n), min((i + 1) * c, n))
    tiles = range(i, -(-n // tile), n_splits)
    return np.concatenate([np.arange(j * tile, min((j + 1) * tile, n)) for j in tiles] or [np.arange(0)])


@pytest.mark.parametrize("layout", [0, 1], ids=["contiguous", "interleaved"])
@pytest.mark.parametrize("shape,n_splits", [
    # (B, Hq, Hkv, D, Lmax, dtype, lens), pieces
    ((2, 16, 2, 128, 3000, "bf16", [3000, 1111]), 7),   # matrix-core kernel, G = 8
    ((2, 64, 2, 128, 2000, "bf16", [2000, 5]), 4),      # G = 32: 32-row units; pieces past a short sequence
    ((2, 8, 8, 128, 1500, "bf16", [1500, 700]), 5),     # vector-ALU kernel (MHA)
    ((2, 8, 2, 64, 1800, "bf16", [1800, 333]), 3),      # vector-ALU, D 64, 4-row units
    ((1, 4, 4, 64, 512, "fp32", None), 4),              # fp32, D 64
], ids=lambda s: str(s))
def test_partials_pieces_match_oracle(fd, shape, n_splits, layout):
    """fd_decode_attn_partials on its own: each piece's output and lse
    against the oracle's attention over exactly the rows the layout assigns
    it (-inf and 0 for an empty piece)."""
    B, Hq, Hkv, D, L, dtype, lens = shape
    case = synth.decode_case(B, Hq, Hkv, D, L, dtype, seed=70 + Hq, lens=lens)
    q, k, v = (to_dev(case[x], dtype) for x in ("q", "k", "v"))
    lens_d = torch.from_numpy(case["lens"]).to("cuda")
    o_part, lse_part = fd.decode_attn_partials(q, k, v, n_splits, lens=lens_d, layout=layout)
    torch.cuda.synchronize()
    o_h = to_host(o_part).reshape(B, Hq, n_splits, D)
    l_h = to_host(lse_part).reshape(B, Hq, n_splits)
    G = Hq // Hkv
    tile = fd.piece_tile_rows(Hq, Hkv, D, fd.FD_BF16 if dtype == "bf16" else fd.FD_F32)
    assert tile > 0
    worst = 0.0
    for b in range(B):
        n = int(case["lens"][b])
        for i in range(n_splits):
            sel = piece_rows(layout, n, n_splits, i, tile)
            for g in range(Hkv):
                rows = slice(g * G, (g + 1) * G)
                if sel.size == 0:
                    assert np.all(np.isneginf(l_h[b, rows, i])) and np.all(o_h[b, rows, i] == 0.0)
                    continue
                ro, rl = oracle.split_partials(case["q"][b, rows], case["k"][b, g, sel], case["v"][b, g, sel],
                                               [0, sel.size])
                worst = max(worst, max_abs(o_h[b, rows, i], ro[0]), max_abs(l_h[b, rows, i], rl[0]))
    print(f"  tile {tile}, worst max-abs {worst:.3e}", flush=True)
    assert worst <= TOL[dtype]


# ------------------------------------------------------------ bifurcated

@pytest.mark.parametrize("shape", [
    # S, Hq, Hkv, D, Lc, Ldmax, dec_lens
    (5, 8, 2, 128, 700, 64, [64, 0, 1, 33, 17]),
    (8, 32, 1, 128, 1024, 40, (1, 40)),
    (6, 32, 8, 128, 2000, 100, (1, 100)),
    (3, 4, 4, 64, 300, 16, [16, 0, 5]),
], ids=lambda s: f"S{s[0]}_hq{s[1]}_hkv{s[2]}_lc{s[4]}_ld{s[5]}")
def test_bifurcated_small(fd, shape):
    S, Hq, Hkv, D, Lc, Ld, dl = shape
    case = synth.bifurcated_case(S, Hq, Hkv, D, Lc, Ld, "bf16", seed=2000 + S, dec_lens=dl)
    t = {k: to_dev(case[k], "bf16") for k in ("q", "k_ctx", "v_ctx", "k_dec", "v_dec")}
    dlen = torch.from_numpy(case["dec_lens"]).cuda()
    out, lse = fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"], dlen,
                                  return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.bifurcated_attention(case["q"], case["k_ctx"], case["v_ctx"], case["k_dec"],
                                               case["v_dec"], case["dec_lens"])
    e_o, e_l = max_abs(to_host(out), ref_o), max_abs(to_host(lse), ref_l)
    print(f"  bifurcated max-abs out {e_o:.3e} lse {e_l:.3e}", flush=True)
    assert e_o <= 1e-2 and e_l <= 1e-2


def test_concatenated_cache_matches_oracle(fd):
    """Split-KV decode attention over the explicitly concatenated cache
    [context ; own decode rows] -- the non-bifurcated way to the bifurcated
    result -- at a reduced bifurcated-GQA shape (16 samples, 4096 context
    rows, decode rows uniform in [1, 512], 32 query / 8 KV heads), element by
    element against the oracle, both as plain attention over the
    concatenated rows and as bifurcated attention ([BA] "Tiivistelmä")."""
    S, Hq, Hkv, D, Lc, Ld = 16, 32, 8, 128, 4096, 512
    case = synth.bifurcated_case(S, Hq, Hkv, D, Lc, Ld, "bf16", seed=8100, dec_lens=(1, 512))
    kcat = np.concatenate([np.broadcast_to(case["k_ctx"][None], (S, Hkv, Lc, D)), case["k_dec"]], axis=2)
    vcat = np.concatenate([np.broadcast_to(case["v_ctx"][None], (S, Hkv, Lc, D)), case["v_dec"]], axis=2)
    lens = (case["dec_lens"] + Lc).astype(np.int32)
    q = to_dev(case["q"], "bf16")
    out, lse = fd.decode_attn(q, to_dev(kcat, "bf16"), to_dev(vcat, "bf16"), torch.from_numpy(lens).cuda(),
                              return_lse=True)
    t = {k: to_dev(case[k], "bf16") for k in ("k_ctx", "v_ctx", "k_dec", "v_dec")}
    bif, bif_lse = fd.bifurcated_attn(q, t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"],
                                      torch.from_numpy(case["dec_lens"]).cuda(), return_lse=True)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.attention(case["q"], kcat, vcat, lens)
    ref_bo, ref_bl = oracle.bifurcated_attention(case["q"], case["k_ctx"], case["v_ctx"], case["k_dec"],
                                                 case["v_dec"], case["dec_lens"])
    assert max_abs(ref_o, ref_bo) <= 1e-12 and max_abs(ref_l, ref_bl) <= 1e-12
    e = [max_abs(to_host(out), ref_o), max_abs(to_host(lse), ref_l),
         max_abs(to_host(bif), ref_o), max_abs(to_host(bif_lse), ref_l)]
    print(f"  concatenated out {e[0]:.3e} lse {e[1]:.3e}; bifurcated out {e[2]:.3e} lse {e[3]:.3e}", flush=True)
    assert max(e) <= 1e-2


def test_bifurcated_equals_decode_on_concatenated_cache(fd):
    S, Hq, Hkv, D, Lc, Ld = 4, 16, 2, 128, 1500, 80
    case = synth.bifurcated_case(S, Hq, Hkv, D, Lc, Ld, "bf16", seed=31, dec_lens=[80, 3, 0, 41])
    t = {k: to_dev(case[k], "bf16") for k in ("q", "k_ctx", "v_ctx", "k_dec", "v_dec")}
    dlen = torch.from_numpy(case["dec_lens"]).cuda()
    bif = fd.bifurcated_attn(t["q"], t["k_ctx"], t["v_ctx"], t["k_dec"], t["v_dec"], dlen)
    kc = torch.cat([t["k_ctx"].unsqueeze(0).expand(S, -1, -1, -1), t["k_dec"]], dim=2).contiguous()
    vc = torch.cat([t["v_ctx"].unsqueeze(0).expand(S, -1, -1, -1), t["v_dec"]], dim=2).contiguous()
    cat = fd.decode_attn(t["q"], kc, vc, (dlen + Lc).to(torch.int32))
    torch.cuda.synchronize()
    assert max_abs(to_host(bif), to_host(cat)) <= 2e-3


# ------------------------------------------------------- large |V| values

@pytest.mark.parametrize("shape", [
    # B, Hq, Hkv, Lmax, lens
    (2, 16, 2, 1500, [1500, 3]),      # matrix-core kernel, G = 8
    (1, 32, 1, 900, [900]),           # matrix-core kernel, MQA: 32-row units
    (2, 8, 8, 700, [700, 40]),        # vector-ALU kernel (MHA)
    (2, 12, 4, 600, [600, 17]),       # vector-ALU kernel, G = 3
], ids=lambda s: f"B{s[0]}_hq{s[1]}_hkv{s[2]}")
@pytest.mark.parametrize("v_scale", [8.0, 64.0])
def test_large_values_hold_the_flat_bound(fd, shape, v_scale):
    """V entries of N(0, v_scale^2) (|v| up to about 4.5 v_scale, bf16) and
    K scaled by 3 (sharp softmax, a few rows of similar weight): the
    split-KV kernels keep max-abs 1e-2 on fp32 outputs, independent of the
    spread of V."""
    B, Hq, Hkv, L, lens = shape
    case = synth.decode_case(B, Hq, Hkv, 128, L, "bf16", seed=610 + Hq, lens=lens)
    case["v"] = synth.round_to_bf16(case["v"] * np.float32(v_scale))
    case["k"] = synth.round_to_bf16(case["k"] * np.float32(3.0))
    for ns in (0, 1, 5):
        check_decode(fd, case, "bf16", n_splits=ns, out_dtype=torch.float32)
    # the other partial kernel on the same shape, where it supports it
    q, k, v = (to_dev(case[x], "bf16") for x in ("q", "k", "v"))
    lens_d = torch.from_numpy(case["lens"]).to("cuda")
    ref_out, ref_lse = oracle.attention(case["q"], case["k"], case["v"], case["lens"])
    for kernel in ("valu", "mfma"):
        out, lse = fd.testing_decode_attn(q, k, v, kernel, lens=lens_d, n_splits=3, out_dtype=torch.float32,
                                          return_lse=True)
        torch.cuda.synchronize()
        assert max_abs(to_host(out), ref_out) <= TOL["bf16"] and max_abs(to_host(lse), ref_lse) <= TOL["bf16"]
