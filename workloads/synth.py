"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module draws numbers and nothing else: it holds none of the attention
arithmetic, and neither the oracle nor the HIP binding imports it.

Distribution (the same for every workload): q, K and V entries are i.i.d.
N(0, 1) drawn in float32; bf16 workloads round each draw to the nearest bf16
value (ties to even).  Ragged lengths are integers drawn uniformly from an
inclusive range.  Cache rows beyond a sequence's length are padding; parity
runs fill them with NaN so that any read of them poisons the result.
"""

import numpy as np

__all__ = [
    "round_to_bf16",
    "host_normal",
    "host_lengths",
    "decode_case",
    "bifurcated_case",
    "device_normal",
    "device_lengths",
    "paginate",
    "shuffled_block_table",
    "head_scales",
    "to_e4m3",
    "fp8_case",
    "device_fp8",
]


def round_to_bf16(x):
    """float32 array -> float32 array holding the nearest bf16 values (RNE).

    bf16 keeps the top 16 bits of an IEEE float32; rounding to nearest-even
    adds 0x7FFF plus the lowest kept bit before truncating.  NaN stays NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)) << np.uint64(16)
    r = r.astype(np.uint32)
    out = r.view(np.float32).copy()
    nan = np.isnan(x)
    out[nan] = np.float32(np.nan)
    return out


def host_normal(shape, seed, dtype="bf16"):
    """N(0,1) float32 draws from PCG64(seed), bf16-rounded for dtype 'bf16'."""
    g = np.random.Generator(np.random.PCG64(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        x = round_to_bf16(x)
    elif dtype != "fp32":
        raise ValueError(dtype)
    return x


def host_lengths(count, lo, hi, seed):
    """`count` integers uniform in [lo, hi] (both ends included)."""
    g = np.random.Generator(np.random.PCG64(seed))
    return g.integers(lo, hi + 1, size=count, dtype=np.int64)


def decode_case(B, Hq, Hkv, D, Lmax, dtype, seed, lens=None, pad_nan=True):
    """Host inputs for one decode-attention call.

    Returns dict(q [B,Hq,D], k, v [B,Hkv,Lmax,D] float32 arrays holding the
    exact input values, lens [B] int32).  lens=None means every sequence is
    Lmax long; a (lo, hi) tuple draws ragged lengths from seed + 7.
    """
    q = host_normal((B, Hq, D), seed, dtype)
    k = host_normal((B, Hkv, Lmax, D), seed + 1, dtype)
    v = host_normal((B, Hkv, Lmax, D), seed + 2, dtype)
    if lens is None:
        lens = np.full(B, Lmax, dtype=np.int64)
    elif isinstance(lens, tuple):
        lens = host_lengths(B, lens[0], lens[1], seed + 7)
    lens = np.asarray(lens, dtype=np.int64)
    if pad_nan:
        for b in range(B):
            k[b, :, lens[b]:, :] = np.nan
            v[b, :, lens[b]:, :] = np.nan
    return {"q": q, "k": k, "v": v, "lens": lens.astype(np.int32)}


def bifurcated_case(S, Hq, Hkv, D, Lc, Ldmax, dtype, seed, dec_lens=None, pad_nan=True):
    """Host inputs for one bifurcated call.

    Returns dict(q [S,Hq,D], k_ctx, v_ctx [Hkv,Lc,D], k_dec, v_dec
    [S,Hkv,Ldmax,D], dec_lens [S] int32).  dec_lens: None = all Ldmax, a
    (lo, hi) tuple = uniform draw from seed + 7, or an explicit sequence.
    """
    q = host_normal((S, Hq, D), seed, dtype)
    kc = host_normal((Hkv, Lc, D), seed + 1, dtype)
    vc = host_normal((Hkv, Lc, D), seed + 2, dtype)
    kd = host_normal((S, Hkv, Ldmax, D), seed + 3, dtype)
    vd = host_normal((S, Hkv, Ldmax, D), seed + 4, dtype)
    if dec_lens is None:
        dec_lens = np.full(S, Ldmax, dtype=np.int64)
    elif isinstance(dec_lens, tuple):
        dec_lens = host_lengths(S, dec_lens[0], dec_lens[1], seed + 7)
    dec_lens = np.asarray(dec_lens, dtype=np.int64)
    if pad_nan:
        for s in range(S):
            kd[s, :, dec_lens[s]:, :] = np.nan
            vd[s, :, dec_lens[s]:, :] = np.nan
    return {"q": q, "k_ctx": kc, "v_ctx": vc, "k_dec": kd, "v_dec": vd,
            "dec_lens": dec_lens.astype(np.int32)}


def device_normal(shape, seed, dtype, device):
    """N(0,1) draws made on the device by torch's seeded generator.

    Used where the host cannot draw the data in reasonable time (the
    multi-GiB caches); the exact bits are copied back wherever the oracle
    needs them.  dtype is 'bf16' or 'fp32'.
    """
    import torch

    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(0.0, 1.0, generator=g)
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    return x


def device_lengths(count, lo, hi, seed, device):
    """host_lengths() moved to the device as int32."""
    import torch

    return torch.tensor(host_lengths(count, lo, hi, seed), dtype=torch.int32, device=device)


def shuffled_block_table(batch, pages_per_seq, seed, first_page=1):
    """Page ids for a paged cache: sequence b's j-th page is entry [b, j].

    The batch * pages_per_seq pages first_page, first_page + 1, ... are
    handed out in an order shuffled by PCG64(seed), as a pool allocator that
    has served many sequences would.  Returns int32 [batch, pages_per_seq].
    """
    g = np.random.Generator(np.random.PCG64(seed))
    ids = first_page + g.permutation(batch * pages_per_seq)
    return ids.reshape(batch, pages_per_seq).astype(np.int32)


def paginate(k, v, lens, page_size, seed):
    """A dense host cache [B, Hkv, L, D] laid out as a shuffled page pool.

    Returns (k_pages, v_pages [n_pages, Hkv, page_size, D], block_table
    [B, ceil(L / page_size) + 1] int32).  Page 0 is never handed out and is
    filled with NaN; table entries past a sequence's last page hold -1; rows
    past lens[b] inside a used page keep the dense cache's padding.  Only
    data movement: rows are copied, never combined.
    """
    B, Hkv, L, D = k.shape
    per_seq = -(-L // page_size)
    ids = shuffled_block_table(B, per_seq, seed)
    n_pages = 1 + B * per_seq
    kp = np.full((n_pages, Hkv, page_size, D), np.nan, dtype=np.float32)
    vp = np.full((n_pages, Hkv, page_size, D), np.nan, dtype=np.float32)
    table = np.full((B, per_seq + 1), -1, dtype=np.int32)
    for b in range(B):
        used = -(-int(lens[b]) // page_size)
        for j in range(used):
            page = int(ids[b, j])
            table[b, j] = page
            r0, r1 = j * page_size, min((j + 1) * page_size, L)
            kp[page, :, :r1 - r0] = k[b, :, r0:r1]
            vp[page, :, :r1 - r0] = v[b, :, r0:r1]
    return kp, vp, table


def head_scales(kv_heads, seed):
    """Per-KV-head cache scales for an E4M3 cache of N(0, 1) data: about
    5 / 448 (a 5-sigma value lands near the largest code), varied per head
    by up to +-25% so that a scale applied to the wrong head shows."""
    g = np.random.Generator(np.random.PCG64(seed))
    return (5.0 / 448.0 * g.uniform(0.75, 1.25, size=kv_heads)).astype(np.float32)


def to_e4m3(x, scales):
    """Codes of x / scale (scale per KV head, axis 1 of x), rounded to the
    nearest E4M3 value (ties to even) after clamping to +-448, via torch's
    float8_e4m3fn conversion on the host.  Returns uint8 codes."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    sc = torch.from_numpy(np.asarray(scales, dtype=np.float32)).view(1, -1, *([1] * (t.dim() - 2)))
    y = (t / sc).clamp(-448.0, 448.0)
    return y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def fp8_case(B, Hq, Hkv, D, Lmax, seed, lens=None, pad_nan=True):
    """Host inputs for one E4M3-cache call: q bf16-rounded N(0,1); K, V drawn
    N(0,1) and stored as E4M3 codes with per-head scales.  Rows past lens[b]
    hold the NaN code 0x7F when pad_nan.  Returns dict(q, k_bits, v_bits
    [B, Hkv, Lmax, D] uint8, k_scale, v_scale [Hkv] float32, lens int32)."""
    q = host_normal((B, Hq, D), seed, "bf16")
    k = host_normal((B, Hkv, Lmax, D), seed + 1, "fp32")
    v = host_normal((B, Hkv, Lmax, D), seed + 2, "fp32")
    ks, vs = head_scales(Hkv, seed + 3), head_scales(Hkv, seed + 4)
    kb, vb = to_e4m3(k, ks), to_e4m3(v, vs)
    if lens is None:
        lens = np.full(B, Lmax, dtype=np.int64)
    elif isinstance(lens, tuple):
        lens = host_lengths(B, lens[0], lens[1], seed + 7)
    lens = np.asarray(lens, dtype=np.int64)
    if pad_nan:
        for b in range(B):
            kb[b, :, lens[b]:, :] = 0x7F
            vb[b, :, lens[b]:, :] = 0x7F
    return {"q": q, "k_bits": kb, "v_bits": vb, "k_scale": ks, "v_scale": vs, "lens": lens.astype(np.int32)}


def device_fp8(shape, seed, scales, device):
    """E4M3 codes (uint8) of N(0,1) draws made on the device, divided by the
    per-KV-head scales (axis 1) and clamped to +-448 before rounding."""
    import torch

    x = device_normal(shape, seed, "fp32", device)
    sc = torch.as_tensor(np.asarray(scales, dtype=np.float32), device=device).view(1, -1, *([1] * (len(shape) - 2)))
    return (x / sc).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
