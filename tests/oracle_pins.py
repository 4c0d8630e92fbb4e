"""Checks that pin the fp64 oracle to facts other than its own formula.

Each ``pin_*`` function takes an oracle namespace (the real ``oracle`` package,
or a deliberately broken copy in the mutation tests) and raises
AssertionError when the oracle disagrees with:

* hand-worked closed-form examples (tests/golden/hand_examples.json);
* 60-digit decimal arithmetic on tiny inputs (a different arithmetic route:
  no max subtraction, no numpy);
* torch's CPU float64 scaled_dot_product_attention with K/V repeated per
  query-head group (a library routine);
* closed forms: one row, equal keys, two rows, a dominant score;
* invariants the pages' exactness claims imply: independence of the split,
  bifurcated = split into context and decode pieces, GQA = MHA with repeated
  KV, row permutation, shift and linearity in V, convex hull, lse value;
* paged = dense attention on a cache scattered into a shuffled, poisoned
  page pool by an independently written inverse of the page layout, and
  likewise bifurcated attention with paged decode rows = dense bifurcated;
* E4M3 code values against torch's float8_e4m3fn decoder and hand-worked
  landmarks; fp8-cache attention = dense attention on the values that
  decoder gives, times the per-head scales;
* prefill: position 0 in closed form, every position against 60-digit
  brute force, and the whole result against torch's causal
  scaled_dot_product_attention.
"""

import decimal
import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def _rand(shape, seed, scale=1.0):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape) * scale


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    err = np.max(np.abs(a - b)) if a.size else 0.0
    assert np.isfinite(err) and err <= tol, f"{what}: max-abs error {err} > {tol}"


# --------------------------------------------------------------------------
# hand-worked examples


def pin_golden(orc):
    ex = json.load(open(GOLDEN))
    for e in ex["examples"]:
        out, lse = orc.attention(np.array(e["q"]), np.array(e["k"]), np.array(e["v"]),
                                 np.array(e["lens"]), e["scale"])
        _close(out, e["out"], 1e-12, e["name"] + " out")
        _close(lse, e["lse"], 1e-12, e["name"] + " lse")
    for e in ex["combine_examples"]:
        lp = np.array([[(-np.inf if x is None else x) for x in row] for row in e["lse_part"]])
        out, lse = orc.lse_combine(np.array(e["o_part"]), lp)
        _close(out, e["out"], 1e-12, e["name"] + " out")
        _close(lse, e["lse"], 1e-12, e["name"] + " lse")
    for e in ex["paged_examples"]:
        out, lse = orc.paged_attention(np.array(e["q"]), np.array(e["k_pages"]), np.array(e["v_pages"]),
                                       np.array(e["block_table"]), np.array(e["lens"]), e["scale"])
        _close(out, e["out"], 1e-12, e["name"] + " out")
        _close(lse, e["lse"], 1e-12, e["name"] + " lse")
    for e in ex["fp8kv_examples"]:
        out, lse = orc.attention_fp8kv(np.array(e["q"]), np.array(e["k_bits"]), np.array(e["v_bits"]),
                                       np.array(e["k_scale"]), np.array(e["v_scale"]), np.array(e["lens"]),
                                       e["scale"])
        _close(out, e["out"], 1e-12, e["name"] + " out")
        _close(lse, e["lse"], 1e-12, e["name"] + " lse")
    for e in ex["bifurcated_examples"]:
        out, lse = orc.bifurcated_attention(np.array(e["q"]), np.array(e["k_ctx"]),
                                            np.array(e["v_ctx"]), np.array(e["k_dec"]),
                                            np.array(e["v_dec"]), np.array(e["dec_lens"]),
                                            e["scale"])
        _close(out, e["out"], 1e-12, e["name"] + " out")
        _close(lse, e["lse"], 1e-12, e["name"] + " lse")


# --------------------------------------------------------------------------
# high-precision brute force


def _decimal_attention(q, k, v, lens, scale):
    """Attention in 60-digit decimal arithmetic, straight from exp(s)/sum exp(s)."""
    ctx = decimal.Context(prec=60)
    Dec = decimal.Decimal
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    sc = Dec(repr(float(scale)))
    out = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    for b in range(B):
        for h in range(Hq):
            g = h // G
            num = [Dec(0)] * D
            den = Dec(0)
            for j in range(int(lens[b])):
                s = Dec(0)
                for d in range(D):
                    s = ctx.add(s, ctx.multiply(Dec(repr(float(q[b, h, d]))),
                                                Dec(repr(float(k[b, g, j, d])))))
                w = ctx.exp(ctx.multiply(sc, s))
                den = ctx.add(den, w)
                for d in range(D):
                    num[d] = ctx.add(num[d], ctx.multiply(w, Dec(repr(float(v[b, g, j, d])))))
            for d in range(D):
                out[b, h, d] = float(ctx.divide(num[d], den))
            lse[b, h] = float(ctx.ln(den))
    return out, lse


def pin_decimal_bruteforce(orc):
    for seed, (B, Hq, Hkv, D, L) in enumerate([(1, 1, 1, 3, 5), (2, 4, 2, 4, 7), (2, 6, 3, 2, 9),
                                               (1, 4, 1, 8, 6)]):
        q = _rand((B, Hq, D), 10 + seed, 1.5)
        k = _rand((B, Hkv, L, D), 20 + seed, 1.5)
        v = _rand((B, Hkv, L, D), 30 + seed)
        lens = np.array([L - (b % 3) for b in range(B)])
        scale = 0.37 + 0.1 * seed
        ref_out, ref_lse = _decimal_attention(q, k, v, lens, scale)
        out, lse = orc.attention(q, k, v, lens, scale)
        _close(out, ref_out, 1e-13, f"decimal brute force case {seed} out")
        _close(lse, ref_lse, 1e-13, f"decimal brute force case {seed} lse")


# --------------------------------------------------------------------------
# library routine


def pin_torch_sdpa(orc):
    import torch
    import torch.nn.functional as F

    for seed, (B, Hq, Hkv, D, L) in enumerate([(2, 8, 2, 16, 33), (3, 4, 4, 64, 70),
                                               (1, 32, 1, 128, 40)]):
        q = _rand((B, Hq, D), 40 + seed)
        k = _rand((B, Hkv, L, D), 50 + seed)
        v = _rand((B, Hkv, L, D), 60 + seed)
        lens = np.array([L - 5 * b for b in range(B)])
        out, lse = orc.attention(q, k, v, lens)
        G = Hq // Hkv
        for b in range(B):
            n = int(lens[b])
            Q = torch.from_numpy(q[b]).reshape(1, Hq, 1, D)
            K = torch.from_numpy(k[b, :, :n]).repeat_interleave(G, dim=0).reshape(1, Hq, n, D)
            V = torch.from_numpy(v[b, :, :n]).repeat_interleave(G, dim=0).reshape(1, Hq, n, D)
            ref = F.scaled_dot_product_attention(Q, K, V).reshape(Hq, D).numpy()
            _close(out[b], ref, 1e-12, f"torch sdpa case {seed} batch {b}")
            s = torch.einsum("hd,hnd->hn", Q.reshape(Hq, D), K.reshape(Hq, n, D)) / math.sqrt(D)
            _close(lse[b], torch.logsumexp(s, dim=1).numpy(), 1e-12, f"torch logsumexp {seed}")


# --------------------------------------------------------------------------
# closed forms


def pin_closed_forms(orc):
    D = 6
    # one valid row: the output is that value row; lse is its score
    q = _rand((1, 2, D), 70)
    k = _rand((1, 1, 4, D), 71)
    v = _rand((1, 1, 4, D), 72)
    out, lse = orc.attention(q, k, v, np.array([1]), 0.5)
    _close(out[0], np.repeat(v[0, 0, :1], 2, axis=0), 0.0, "single row")
    _close(lse[0], 0.5 * (q[0] @ k[0, 0, 0]), 1e-15, "single row lse")
    # all keys equal: uniform weights, output is the mean of the valid V rows
    k = np.repeat(_rand((1, 1, 1, D), 73), 9, axis=2)
    v = _rand((1, 1, 9, D), 74)
    out, lse = orc.attention(q, k, v, np.array([7]), 0.8)
    _close(out[0], np.repeat(v[0, 0, :7].mean(axis=0, keepdims=True), 2, axis=0), 1e-14,
           "equal keys")
    _close(lse[0], 0.8 * (q[0] @ k[0, 0, 0]) + math.log(7.0), 1e-13, "equal keys lse")
    # two rows: logistic weights
    k = _rand((1, 1, 2, D), 75)
    v = _rand((1, 1, 2, D), 76)
    out, _ = orc.attention(q, k, v, None, 0.3)
    for h in range(2):
        s0, s1 = 0.3 * (q[0, h] @ k[0, 0, 0]), 0.3 * (q[0, h] @ k[0, 0, 1])
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        _close(out[0, h], w0 * v[0, 0, 0] + (1.0 - w0) * v[0, 0, 1], 1e-14, "two rows")
    # dominant score: k_j* = c q with a score margin above 200 returns v_j*
    q1 = _rand((1, 1, D), 77)
    k = _rand((1, 1, 12, D), 78) * 0.01
    c = 400.0 / float(q1[0, 0] @ q1[0, 0])
    k[0, 0, 5] = c * q1[0, 0]
    v = _rand((1, 1, 12, D), 79)
    out, _ = orc.attention(q1, k, v, None, 1.0)
    _close(out[0, 0], v[0, 0, 5], 1e-14, "dominant score")


# --------------------------------------------------------------------------
# invariants implied by the exactness claims


def pin_split_independence(orc):
    rng = np.random.Generator(np.random.PCG64(80))
    R, D, n = 4, 16, 50
    q = _rand((R, D), 81)
    k = _rand((n, D), 82)
    v = _rand((n, D), 83)
    full_out, full_lse = orc.attention(q[None], k[None, None], v[None, None], None, 0.25)
    for trial in range(6):
        cuts = sorted(rng.integers(0, n + 1, size=trial + 1).tolist())
        bounds = [0] + cuts + [n]          # may repeat cut points: empty pieces
        O, L = orc.split_partials(q, k, v, bounds, 0.25)
        out, lse = orc.lse_combine(O, L)
        _close(out, full_out[0], 1e-12, f"split {bounds}")
        _close(lse, full_lse[0], 1e-12, f"split {bounds} lse")
    # one piece: combine is the identity
    O, L = orc.split_partials(q, k, v, [0, n], 0.25)
    out, lse = orc.lse_combine(O, L)
    _close(out, O[0], 1e-15, "single piece")
    _close(lse, L[0], 0.0, "single piece lse")


def pin_bifurcated_split(orc):
    S, Hq, Hkv, D, Lc, Ld = 3, 4, 2, 8, 11, 6
    q = _rand((S, Hq, D), 90)
    kc, vc = _rand((Hkv, Lc, D), 91), _rand((Hkv, Lc, D), 92)
    kd, vd = _rand((S, Hkv, Ld, D), 93), _rand((S, Hkv, Ld, D), 94)
    dl = np.array([6, 0, 3])
    out, lse = orc.bifurcated_attention(q, kc, vc, kd, vd, dl, 0.4)
    G = Hq // Hkv
    for s in range(S):
        for g in range(Hkv):
            rows = slice(g * G, (g + 1) * G)
            Oc, Lc_ = orc.split_partials(q[s, rows], kc[g], vc[g], [0, Lc], 0.4)
            n = int(dl[s])
            Od, Ld_ = orc.split_partials(q[s, rows], kd[s, g, :n], vd[s, g, :n], [0, n], 0.4)
            o, l = orc.lse_combine(np.concatenate([Oc, Od]), np.concatenate([Lc_, Ld_]))
            _close(out[s, rows], o, 1e-12, f"bifurcated sample {s} head {g}")
            _close(lse[s, rows], l, 1e-12, f"bifurcated lse sample {s} head {g}")
    # ... and equal to plain attention over an explicitly built concatenated cache
    kcat = np.full((S, Hkv, Lc + Ld, D), np.nan)
    vcat = np.full((S, Hkv, Lc + Ld, D), np.nan)
    for s in range(S):
        kcat[s, :, :Lc], vcat[s, :, :Lc] = kc, vc
        kcat[s, :, Lc:Lc + dl[s]], vcat[s, :, Lc:Lc + dl[s]] = kd[s, :, :dl[s]], vd[s, :, :dl[s]]
    o2, l2 = orc.attention(q, kcat, vcat, Lc + dl, 0.4)
    _close(out, o2, 1e-12, "bifurcated vs concatenated")
    _close(lse, l2, 1e-12, "bifurcated vs concatenated lse")


def pin_gqa_is_repeated_mha(orc):
    B, Hq, Hkv, D, L = 2, 12, 3, 8, 10
    q, k, v = _rand((B, Hq, D), 100), _rand((B, Hkv, L, D), 101), _rand((B, Hkv, L, D), 102)
    lens = np.array([10, 4])
    o1, l1 = orc.attention(q, k, v, lens)
    o2, l2 = orc.attention(q, np.repeat(k, Hq // Hkv, axis=1), np.repeat(v, Hq // Hkv, axis=1), lens)
    _close(o1, o2, 1e-15, "gqa vs repeated mha")
    _close(l1, l2, 1e-15, "gqa vs repeated mha lse")


def pin_row_and_value_invariants(orc):
    B, Hq, Hkv, D, L = 2, 4, 2, 8, 13
    q, k, v = _rand((B, Hq, D), 110, 2.0), _rand((B, Hkv, L, D), 111), _rand((B, Hkv, L, D), 112)
    lens = np.array([13, 9])
    out, lse = orc.attention(q, k, v, lens)
    # permuting the valid rows (K and V together) changes nothing
    perm = np.random.Generator(np.random.PCG64(113)).permutation(9)
    k2, v2 = k.copy(), v.copy()
    k2[1, :, :9], v2[1, :, :9] = k[1][:, perm], v[1][:, perm]
    o2, l2 = orc.attention(q, k2, v2, lens)
    _close(o2, out, 1e-14, "row permutation")
    _close(l2, lse, 1e-13, "row permutation lse")
    # shifting V by a constant vector shifts the output by it
    c = _rand((D,), 114)
    o3, l3 = orc.attention(q, k, v + c, lens)
    _close(o3, out + c, 1e-13, "value shift")
    _close(l3, lse, 0.0, "value shift lse")
    # linear in V
    w = _rand((B, Hkv, L, D), 115)
    o4, _ = orc.attention(q, k, w, lens)
    o5, _ = orc.attention(q, k, 2.0 * v - 3.0 * w, lens)
    _close(o5, 2.0 * out - 3.0 * o4, 1e-13, "value linearity")
    # each coordinate lies in the hull of the valid V rows
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            rows = v[b, h // G, :lens[b]]
            assert np.all(out[b, h] >= rows.min(axis=0) - 1e-15)
            assert np.all(out[b, h] <= rows.max(axis=0) + 1e-15)
    # scaling q by c equals scaling the temperature by c
    o6, l6 = orc.attention(1.7 * q, k, v, lens, 0.2)
    o7, l7 = orc.attention(q, k, v, lens, 0.34)
    _close(o6, o7, 1e-13, "q scale vs temperature")
    _close(l6, l7, 1e-13, "q scale vs temperature lse")


def scatter_to_pages(k, v, lens, page_size, extra_pages, seed):
    """Place a dense cache [B, Hkv, L, D] into a shuffled page pool.

    The inverse of the paged layout, written independently of the oracle:
    sequence b's j-th block of page_size rows goes to a randomly chosen page.
    Rows past lens[b] inside a used page, every unused page and every unused
    table entry are poisoned (NaN rows, page id -1), so any read outside the
    valid rows shows up.  Returns (k_pages, v_pages, block_table).
    """
    B, Hkv, L, D = k.shape
    per_seq = -(-L // page_size)
    n_pages = B * per_seq + extra_pages
    order = np.random.Generator(np.random.PCG64(seed)).permutation(n_pages)
    kp = np.full((n_pages, Hkv, page_size, D), np.nan)
    vp = np.full((n_pages, Hkv, page_size, D), np.nan)
    table = np.full((B, per_seq + 1), -1, dtype=np.int64)
    used = 0
    for b in range(B):
        n = int(lens[b])
        for j in range(-(-n // page_size)):
            page = int(order[used])
            used += 1
            table[b, j] = page
            r0, r1 = j * page_size, min((j + 1) * page_size, n)
            kp[page, :, :r1 - r0] = k[b, :, r0:r1]
            vp[page, :, :r1 - r0] = v[b, :, r0:r1]
    return kp, vp, table


def pin_paged_is_dense_attention(orc):
    # [MW] PagedAttention: the table only relocates rows; the result is the
    # dense result on the same rows, and no poisoned row or entry is read.
    for seed, (B, Hq, Hkv, D, L, P) in enumerate([(3, 4, 2, 8, 37, 4), (2, 3, 1, 5, 16, 16),
                                                  (2, 2, 2, 4, 9, 1), (4, 8, 4, 6, 50, 3)]):
        q = _rand((B, Hq, D), 120 + seed)
        k, v = _rand((B, Hkv, L, D), 130 + seed), _rand((B, Hkv, L, D), 140 + seed)
        lens = np.array([L - 7 * b if L - 7 * b > 0 else 1 for b in range(B)])
        kp, vp, table = scatter_to_pages(k, v, lens, P, extra_pages=3, seed=150 + seed)
        out, lse = orc.paged_attention(q, kp, vp, table, lens, 0.3)
        ref_out, ref_lse = orc.attention(q, k, v, lens, 0.3)
        _close(out, ref_out, 0.0, f"paged case {seed} out")
        _close(lse, ref_lse, 0.0, f"paged case {seed} lse")


def pin_bifurcated_paged_is_dense_bifurcated(orc):
    # [BA] "Tiivistelmä" with [MW] PagedAttention: paging every sample's
    # decode rows only relocates them; the result is the dense bifurcated
    # result on the same rows (empty decode parts included), and no poisoned
    # row, page or table entry is read.
    for seed, (S, Hq, Hkv, D, Lc, Ld, P) in enumerate([(4, 4, 2, 8, 13, 21, 4), (3, 2, 1, 5, 3, 16, 16),
                                                       (5, 6, 3, 4, 7, 9, 1)]):
        q = _rand((S, Hq, D), 190 + seed)
        kc, vc = _rand((Hkv, Lc, D), 191 + seed), _rand((Hkv, Lc, D), 192 + seed)
        kd, vd = _rand((S, Hkv, Ld, D), 193 + seed), _rand((S, Hkv, Ld, D), 194 + seed)
        dl = np.array([Ld, 0, 1, Ld - 3, 5][:S])
        kp, vp, table = scatter_to_pages(kd, vd, dl, P, extra_pages=2, seed=195 + seed)
        out, lse = orc.bifurcated_paged_attention(q, kc, vc, kp, vp, table, dl, 0.4)
        ref_out, ref_lse = orc.bifurcated_attention(q, kc, vc, kd, vd, dl, 0.4)
        _close(out, ref_out, 0.0, f"bifurcated paged case {seed} out")
        _close(lse, ref_lse, 0.0, f"bifurcated paged case {seed} lse")


def pin_fp8_codes(orc):
    # every E4M3 code against torch's float8_e4m3fn (a library decoder) ...
    import torch

    codes = np.arange(256)
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = orc.fp8_e4m3_value(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), "fp8 NaN codes"
    fin = ~np.isnan(ref)
    assert np.array_equal(got[fin], ref[fin]), "fp8 code values"
    assert np.array_equal(np.signbit(got[fin]), np.signbit(ref[fin])), "fp8 signed zeros"
    # ... and against the format's landmarks, worked by hand
    for code, val in ((0x38, 1.0), (0x7E, 448.0), (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9),
                      (0x08, 2.0 ** -6), (0x40, 2.0), (0xC0, -2.0), (0x3C, 1.5)):
        assert orc.fp8_e4m3_value(np.array([code]))[0] == val, f"fp8 code {code:#x}"


def pin_fp8_attention_is_dense_attention(orc):
    # dequantising with torch's decoder and per-head scales, then plain attention
    import torch

    B, Hq, Hkv, D, L = 2, 8, 2, 16, 40
    rng = np.random.Generator(np.random.PCG64(160))
    kb = rng.integers(0, 256, size=(B, Hkv, L, D))
    vb = rng.integers(0, 256, size=(B, Hkv, L, D))
    kb[(kb & 0x7F) == 0x7F] = 0x38          # no NaN codes
    vb[(vb & 0x7F) == 0x7F] = 0x30
    q = _rand((B, Hq, D), 161, 0.05)
    ks, vs = np.array([0.02, 0.005]), np.array([1.5, 0.25])
    lens = np.array([40, 23])
    dec = lambda c: torch.from_numpy(c.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    k = dec(kb) * ks[None, :, None, None]
    v = dec(vb) * vs[None, :, None, None]
    out, lse = orc.attention_fp8kv(q, kb, vb, ks, vs, lens, 0.3)
    ref_out, ref_lse = orc.attention(q, k, v, lens, 0.3)
    _close(out, ref_out, 0.0, "fp8 kv out")
    _close(lse, ref_lse, 0.0, "fp8 kv lse")


def pin_prefill(orc):
    # position 0 sees only row 0: its value row and its score
    q, k, v = _rand((1, 4, 9, 8), 170), _rand((1, 2, 9, 8), 171), _rand((1, 2, 9, 8), 172)
    out, lse = orc.prefill_attention(q, k, v, None, 0.6)
    _close(out[0, :, 0], np.repeat(v[0, :, 0], 2, axis=0), 0.0, "prefill position 0")
    _close(lse[0, :, 0], 0.6 * np.einsum("hd,hd->h", q[0, :, 0], np.repeat(k[0, :, 0], 2, axis=0)), 1e-15,
           "prefill position 0 lse")
    # 60-digit brute force per position (decode attention with lens = p + 1)
    B, Hq, Hkv, D, L = 2, 4, 2, 3, 6
    q, k, v = _rand((B, Hq, L, D), 173, 1.5), _rand((B, Hkv, L, D), 174, 1.5), _rand((B, Hkv, L, D), 175)
    lens = np.array([6, 4])
    out, lse = orc.prefill_attention(q, k, v, lens, 0.45)
    for b in range(B):
        for p in range(int(lens[b])):
            ro, rl = _decimal_attention(q[b:b + 1, :, p], k[b:b + 1], v[b:b + 1], np.array([p + 1]), 0.45)
            _close(out[b, :, p], ro[0], 1e-13, f"prefill decimal b{b} p{p}")
            _close(lse[b, :, p], rl[0], 1e-13, f"prefill decimal lse b{b} p{p}")
        assert np.all(np.isnan(out[b, :, int(lens[b]):])), "positions past lens must stay empty"
    # torch's causal scaled_dot_product_attention (a library routine), KV
    # repeated per query-head group
    import torch
    import torch.nn.functional as F

    B, Hq, Hkv, D, L = 2, 8, 2, 16, 37
    q, k, v = _rand((B, Hq, L, D), 176), _rand((B, Hkv, L, D), 177), _rand((B, Hkv, L, D), 178)
    out, _ = orc.prefill_attention(q, k, v)
    G = Hq // Hkv
    ref = F.scaled_dot_product_attention(torch.from_numpy(q), torch.from_numpy(k).repeat_interleave(G, dim=1),
                                         torch.from_numpy(v).repeat_interleave(G, dim=1), is_causal=True)
    _close(out, ref.numpy(), 1e-12, "prefill vs torch causal sdpa")


ALL_PINS = [pin_golden, pin_decimal_bruteforce, pin_torch_sdpa, pin_closed_forms,
            pin_split_independence, pin_bifurcated_split, pin_gqa_is_repeated_mha,
            pin_row_and_value_invariants, pin_paged_is_dense_attention, pin_bifurcated_paged_is_dense_bifurcated,
            pin_fp8_codes,
            pin_fp8_attention_is_dense_attention, pin_prefill]
