"""The fp64 oracle against its pins (CPU only), plus planted-mistake checks.

The mutation tests plant one plausible mistake at a time in a copy of the
oracle (on the CPU) and require that at least one pin catches it.
"""

import types

import numpy as np
import pytest

import oracle
from oracle import fp64 as oa
from tests import oracle_pins as pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin(oracle)


def _mutant(**overrides):
    """A namespace like the oracle package with some functions replaced."""
    ns = types.SimpleNamespace(
        attention=oa.attention, bifurcated_attention=oa.bifurcated_attention,
        split_partials=oa.split_partials, lse_combine=oa.lse_combine,
        default_scale=oa.default_scale, paged_attention=oa.paged_attention,
        fp8_e4m3_value=oa.fp8_e4m3_value, attention_fp8kv=oa.attention_fp8kv,
        prefill_attention=oa.prefill_attention, bifurcated_paged_attention=oa.bifurcated_paged_attention)
    for name, fn in overrides.items():
        setattr(ns, name, fn)
    return ns


def _with_rows(rows_fn):
    """Rebuild attention/bifurcated/split_partials over a broken row kernel."""
    saved = oa._attend_rows

    def wrap(fn):
        def inner(*a, **kw):
            oa._attend_rows = rows_fn
            try:
                return fn(*a, **kw)
            finally:
                oa._attend_rows = saved
        return inner

    return _mutant(attention=wrap(oa.attention), bifurcated_attention=wrap(oa.bifurcated_attention),
                   split_partials=wrap(oa.split_partials), paged_attention=wrap(oa.paged_attention),
                   prefill_attention=wrap(oa.prefill_attention))


def _rows_no_scale(q, k, v, scale):
    return oa.__dict__["_attend_rows_ref"](q, k, v, 1.0)


def _rows_log2_lse(q, k, v, scale):
    o, l = oa._attend_rows_ref(q, k, v, scale)
    return o, l / np.log(2.0)


def _rows_no_normalise(q, k, v, scale):
    if k.shape[0] == 0:
        return oa._attend_rows_ref(q, k, v, scale)
    s = scale * (q @ k.T)
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    return e @ v, m[:, 0] + np.log(e.sum(axis=1))


def _rows_keys_for_values(q, k, v, scale):
    return oa._attend_rows_ref(q, k, k, scale)


def _rows_drop_last(q, k, v, scale):
    return oa._attend_rows_ref(q, k[:-1] if k.shape[0] > 1 else k, v[:-1] if v.shape[0] > 1 else v, scale)


def _rows_wrong_sign(q, k, v, scale):
    return oa._attend_rows_ref(q, k, v, -scale)


def _attention_interleaved_gqa(q, k, v, lens=None, scale=None):
    # query head h reads KV head h % Hkv instead of h // G
    q = np.asarray(q, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    perm = np.array([(h % Hkv) * G + h // Hkv for h in range(Hq)])
    out, lse = oa.attention(q[:, np.argsort(perm)], k, v, lens, scale)
    return out[:, perm], lse[:, perm]


def _combine_wrong_sign(o_part, lse_part):
    o_part = np.asarray(o_part, dtype=np.float64)
    lse_part = np.asarray(lse_part, dtype=np.float64)
    M = lse_part.max(axis=0)
    w = np.where(np.isneginf(lse_part), 0.0, np.exp(M - lse_part))
    z = w.sum(axis=0)
    return (w[..., None] * o_part).sum(axis=0) / z[..., None], M + np.log(z)


def _combine_plain_mean(o_part, lse_part):
    lse_part = np.asarray(lse_part, dtype=np.float64)
    live = ~np.isneginf(lse_part)
    o = (np.asarray(o_part) * live[..., None]).sum(axis=0) / live.sum(axis=0)[..., None]
    return o, lse_part.max(axis=0)


def _paged_gather(mapping):
    """paged_attention with the row -> (page, slot) mapping replaced."""
    def paged(q, k_pages, v_pages, block_table, lens=None, scale=None):
        k_pages, v_pages = np.asarray(k_pages, np.float64), np.asarray(v_pages, np.float64)
        table = np.asarray(block_table)
        B = table.shape[0]
        P = k_pages.shape[2]
        Lmax = table.shape[1] * P
        lens = np.full(B, Lmax) if lens is None else np.asarray(lens)
        D = k_pages.shape[3]
        k = np.full((B, k_pages.shape[1], Lmax, D), np.nan)
        v = np.full_like(k, np.nan)
        for b in range(B):
            for t in range(int(lens[b])):
                page, slot, head_axis_swapped = mapping(table, b, t, P)
                if head_axis_swapped:
                    # pages read as [P, Hkv, D] instead of [Hkv, P, D]
                    Hkv = k.shape[1]
                    k[b, :, t] = k_pages[page].reshape(-1, D)[slot * Hkv: (slot + 1) * Hkv]
                    v[b, :, t] = v_pages[page].reshape(-1, D)[slot * Hkv: (slot + 1) * Hkv]
                else:
                    k[b, :, t] = k_pages[page, :, slot]
                    v[b, :, t] = v_pages[page, :, slot]
        return oa.attention(q, k, v, lens, scale)
    return paged


def _bif_paged_gather(mapping, keep_context=True):
    """bifurcated_paged_attention with the decode row -> (page, slot) mapping
    replaced (or the context left out)."""
    def bif(q, k_ctx, v_ctx, k_pages, v_pages, block_table, dec_lens, scale=None):
        k_pages, v_pages = np.asarray(k_pages, np.float64), np.asarray(v_pages, np.float64)
        table = np.asarray(block_table)
        S, P, D = table.shape[0], k_pages.shape[2], k_pages.shape[3]
        Ld = table.shape[1] * P
        kd = np.full((S, k_pages.shape[1], Ld, D), np.nan)
        vd = np.full_like(kd, np.nan)
        for s_ in range(S):
            for t in range(int(dec_lens[s_])):
                page, slot, _ = mapping(table, s_, t, P)
                kd[s_, :, t] = k_pages[page, :, slot]
                vd[s_, :, t] = v_pages[page, :, slot]
        if not keep_context:
            k_ctx, v_ctx = np.asarray(k_ctx)[:, :1] * 0.0, np.asarray(v_ctx)[:, :1] * 0.0
        return oa.bifurcated_attention(q, k_ctx, v_ctx, kd, vd, dec_lens, scale)
    return bif


def _map_identity(table, b, t, P):
    return table[b, t // P], t % P, False


def _map_page_slot_swapped(table, b, t, P):
    return table[b, t % P], t // P, False


def _map_table_transposed(table, b, t, P):
    return table.T.reshape(table.shape)[b, t // P], t % P, False


def _map_head_axis_swapped(table, b, t, P):
    return table[b, t // P], t % P, True


def _map_whole_last_page(table, b, t, P):
    # reads the page of row t but always from slot P - 1 of the last page
    return table[b, t // P], (t % P if t + P < table.shape[1] * P else P - 1), False


def _fp8_bias8(bits):
    # exponent bias 8 (the FNUZ variant's) instead of 7
    return oa.fp8_e4m3_value(bits) / 2.0


def _fp8_no_subnormals(bits):
    b = np.asarray(bits).astype(np.int64) & 0xFF
    v = oa.fp8_e4m3_value(bits)
    return np.where((b & 0x78) == 0, np.where(b >> 7, -1.0, 1.0) * (1 + (b & 7) / 8.0) * 2.0 ** -7, v)


def _fp8_with(value_fn):
    def attn(q, k_bits, v_bits, k_scale=None, v_scale=None, lens=None, scale=None):
        Hkv = np.asarray(k_bits).shape[1]
        ks = np.ones(Hkv) if k_scale is None else np.asarray(k_scale, np.float64)
        vs = np.ones(Hkv) if v_scale is None else np.asarray(v_scale, np.float64)
        k = value_fn(k_bits) * ks[None, :, None, None]
        v = value_fn(v_bits) * vs[None, :, None, None]
        return oa.attention(q, k, v, lens, scale)
    return attn


def _fp8_scales_swapped(q, k_bits, v_bits, k_scale=None, v_scale=None, lens=None, scale=None):
    return oa.attention_fp8kv(q, k_bits, v_bits, v_scale, k_scale, lens, scale)


def _prefill_window(first, last):
    """prefill_attention where position p sees rows [first(p), last(p))."""
    def prefill(q, k, v, lens=None, scale=None):
        q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
        B, Hq, L, D = q.shape
        Hkv = k.shape[1]
        G = Hq // Hkv
        lens = np.full(B, L) if lens is None else np.asarray(lens)
        scale = oa.default_scale(D) if scale is None else scale
        out = np.full(q.shape, np.nan)
        lse = np.full((B, Hq, L), np.nan)
        for b in range(B):
            n = int(lens[b])
            for g in range(Hkv):
                for p in range(n):
                    lo, hi = first(p, n), max(first(p, n) + 1, min(last(p, n), n))
                    rows = slice(g * G, (g + 1) * G)
                    out[b, rows, p], lse[b, rows, p] = oa._attend_rows_ref(q[b, rows, p], k[b, g, lo:hi],
                                                                           v[b, g, lo:hi], scale)
        return out, lse
    return prefill


MUTANTS = {
    "dropped_scale": lambda: _with_rows(_rows_no_scale),
    "lse_in_log2": lambda: _with_rows(_rows_log2_lse),
    "missing_normalisation": lambda: _with_rows(_rows_no_normalise),
    "keys_used_as_values": lambda: _with_rows(_rows_keys_for_values),
    "off_by_one_rows": lambda: _with_rows(_rows_drop_last),
    "wrong_score_sign": lambda: _with_rows(_rows_wrong_sign),
    "interleaved_gqa": lambda: _mutant(attention=_attention_interleaved_gqa),
    "combine_wrong_sign": lambda: _mutant(lse_combine=_combine_wrong_sign),
    "combine_unweighted": lambda: _mutant(lse_combine=_combine_plain_mean),
    "paged_page_slot_swapped": lambda: _mutant(paged_attention=_paged_gather(_map_page_slot_swapped)),
    "paged_table_transposed": lambda: _mutant(paged_attention=_paged_gather(_map_table_transposed)),
    "paged_head_axis_swapped": lambda: _mutant(paged_attention=_paged_gather(_map_head_axis_swapped)),
    "paged_wrong_slot_in_tail": lambda: _mutant(paged_attention=_paged_gather(_map_whole_last_page)),
    "bifurcated_paged_page_slot_swapped": lambda: _mutant(
        bifurcated_paged_attention=_bif_paged_gather(_map_page_slot_swapped)),
    "bifurcated_paged_table_transposed": lambda: _mutant(
        bifurcated_paged_attention=_bif_paged_gather(_map_table_transposed)),
    "bifurcated_paged_context_dropped": lambda: _mutant(
        bifurcated_paged_attention=_bif_paged_gather(_map_identity, keep_context=False)),
    "fp8_exponent_bias_8": lambda: _mutant(fp8_e4m3_value=_fp8_bias8, attention_fp8kv=_fp8_with(_fp8_bias8)),
    "fp8_subnormals_as_normals": lambda: _mutant(fp8_e4m3_value=_fp8_no_subnormals,
                                                 attention_fp8kv=_fp8_with(_fp8_no_subnormals)),
    "fp8_scales_swapped": lambda: _mutant(attention_fp8kv=_fp8_scales_swapped),
    "prefill_excludes_own_row": lambda: _mutant(prefill_attention=_prefill_window(lambda p, n: 0, lambda p, n: p)),
    "prefill_one_row_too_many": lambda: _mutant(prefill_attention=_prefill_window(lambda p, n: 0,
                                                                                 lambda p, n: p + 2)),
    "prefill_anti_causal": lambda: _mutant(prefill_attention=_prefill_window(lambda p, n: p, lambda p, n: n)),
    "prefill_not_causal": lambda: _mutant(prefill_attention=_prefill_window(lambda p, n: 0, lambda p, n: n)),
}


@pytest.fixture(autouse=True, scope="module")
def _keep_reference_rows():
    oa._attend_rows_ref = oa._attend_rows
    yield
    del oa._attend_rows_ref


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name):
    orc = MUTANTS[name]()
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name}"
