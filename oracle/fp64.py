"""Plain fp64 CPU oracle for exact single-query (decode-step) attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the GPU path imports this module; only
the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of the bench
may call it.  It shares no code, constant or helper with the HIP library.

Sources (the pages this follows; cited by title and section):

* [FD]  "¿Qué es Flash-Decoding y cuándo acelera los LLMs?" (slavadubrov.com),
  section "Por qué la decodificación necesita otra planificación": during
  decoding every active sequence contributes one new query position that has
  to read its whole cached history; the history can be cut into pieces, each
  piece yields a partial attention result together with its log-sum-exp, and a
  reduction merges the pieces into exactly the attention over the full history.
* [FA]  "In che modo Flash Attention riduce il traffico di memoria durante
  l'inferenza locale?" (shop.zimaspace.com), sections "L'attenzione standard
  sposta grandi tensori intermedi attraverso la HBM" (attention = scores from
  query and keys, normalised, then combined with the values) and "La softmax
  online evita di memorizzare l'intera matrice dei punteggi".
* [MW]  gyaansetu.com article on the memory wall of LLM decoding (Kannada),
  section "ಮೆಮೊರಿ ವಾಲ್ (Memory Wall) ವಿರುದ್ಧ ಹೋರಾಟ", paragraph on
  PagedAttention: KV cache entries are kept in fixed-size blocks, allocated
  non-contiguously and found through an indirection table.
* [BA]  "Effiziente Verarbeitung und Analyse von Inhalten durch bifurkierte
  Aufmerksamkeit für Single-Context-Batch-Sampling" (linnk.ai), section
  "Tiivistelmä": incremental-decode attention is split into a part over the
  shared prefill (context) KV and a part over the per-sample decode KV; the
  result is exact and the FLOPs are unchanged.  Section "Tilastot": KV-cache
  IO is b*g*m*k for multi-query versus b*h*m*k for multi-head attention.

Readings taken where the pages are silent:

* scale defaults to 1/sqrt(D);
* query head h reads KV head h // (Hq // Hkv) (contiguous GQA groups);
* the valid cache rows of sequence b are rows [0, lens[b]); nothing else is
  masked, and rows at or beyond lens[b] are never read;
* lse is the natural-log log-sum-exp of the scaled scores;
* an empty piece has lse = -inf and output 0 and carries zero weight in the
  reduction.

Everything is computed naively in float64 from the exact input values (bf16
inputs are passed in already widened, which is exact).  A matrix-vector
product (numpy ``@``) is the only library primitive used.
"""

import math

import numpy as np

__all__ = [
    "default_scale",
    "attention",
    "bifurcated_attention",
    "bifurcated_paged_attention",
    "split_partials",
    "lse_combine",
    "paged_attention",
    "fp8_e4m3_value",
    "attention_fp8kv",
    "prefill_attention",
]


def default_scale(head_dim):
    """Softmax temperature 1/sqrt(D) (reading: the pages name none)."""
    return 1.0 / math.sqrt(float(head_dim))


def _as_f64(x):
    return np.asarray(x, dtype=np.float64)


def _attend_rows(qrows, keys, values, scale):
    """Attention of a few query rows over one KV slice.

    qrows [R, D], keys/values [n, D] with n >= 0.  Returns (out [R, D],
    lse [R]).  Follows [FA] "L'attenzione standard ...": scores
    s_j = scale * <q, k_j>, weights softmax(s), output sum_j p_j v_j.  The
    softmax is evaluated with the row maximum subtracted before exp, which is
    the same number in exact arithmetic.  With n == 0 (an empty piece, a
    reading) the output is 0 and lse is -inf.
    """
    R, D = qrows.shape
    n = keys.shape[0]
    if n == 0:
        return np.zeros((R, D)), np.full(R, -np.inf)
    s = scale * (qrows @ keys.T)                 # [R, n]
    m = s.max(axis=1, keepdims=True)             # [R, 1]
    e = np.exp(s - m)                            # [R, n]
    z = e.sum(axis=1)                            # [R]
    out = (e @ values) / z[:, None]              # [R, D]
    lse = m[:, 0] + np.log(z)
    return out, lse


def attention(q, k, v, lens=None, scale=None):
    """Exact decode attention, one query position per sequence.

    q     [B, Hq, D]
    k, v  [B, Hkv, Lmax, D]
    lens  [B] integers in [1, Lmax] (None: every sequence is Lmax long)
    Returns out [B, Hq, D] float64 and lse [B, Hq] float64 (natural log).

    [FD] "Por qué la decodificación necesita otra planificación": each
    sequence's single new query attends over its whole cached history.
    [BA] "Tilastot": K/V are stored per KV head; query heads share them in
    groups of G = Hq / Hkv.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, D = q.shape
    Bk, Hkv, Lmax, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape:
        raise ValueError("shape mismatch between q, k and v")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if lens is None:
        lens = np.full(B, Lmax, dtype=np.int64)
    lens = np.asarray(lens, dtype=np.int64)
    if scale is None:
        scale = default_scale(D)
    out = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    for b in range(B):
        n = int(lens[b])
        if not 1 <= n <= Lmax:
            raise ValueError(f"lens[{b}]={n} outside [1, {Lmax}]")
        for g in range(Hkv):
            rows = slice(g * G, (g + 1) * G)
            o, l = _attend_rows(q[b, rows], k[b, g, :n], v[b, g, :n], scale)
            out[b, rows] = o
            lse[b, rows] = l
    return out, lse


def paged_attention(q, k_pages, v_pages, block_table, lens=None, scale=None):
    """Exact decode attention over a paged KV cache.

    q                 [B, Hq, D]
    k_pages, v_pages  [n_pages, Hkv, P, D]  pages of P rows for each KV head
    block_table       [B, max_pages] integer page ids
    lens              [B] integers in [1, max_pages * P] (None: all of them)
    Returns out [B, Hq, D] and lse [B, Hq], as ``attention``.

    [MW] "ಮೆಮೊರಿ ವಾಲ್ (Memory Wall) ವಿರುದ್ಧ ಹೋರಾಟ", PagedAttention: the cache
    rows sit in fixed-size blocks reached through an indirection table; the
    attention itself does not change.  Logical row t of sequence b is row
    t mod P of page block_table[b, t div P].  Those rows, in order, are the
    sequence's cache; only the table entries that cover rows below lens[b]
    are read, and each of them must name a page of the pool.
    """
    q, k_pages, v_pages = _as_f64(q), _as_f64(k_pages), _as_f64(v_pages)
    B, Hq, D = q.shape
    n_pages, Hkv, P, Dk = k_pages.shape
    table = np.asarray(block_table, dtype=np.int64)
    if Dk != D or v_pages.shape != k_pages.shape or table.ndim != 2 or table.shape[0] != B:
        raise ValueError("shape mismatch between q, the pages and the block table")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    Lmax = table.shape[1] * P
    if lens is None:
        lens = np.full(B, Lmax, dtype=np.int64)
    lens = np.asarray(lens, dtype=np.int64)
    if scale is None:
        scale = default_scale(D)
    out = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    for b in range(B):
        n = int(lens[b])
        if not 1 <= n <= Lmax:
            raise ValueError(f"lens[{b}]={n} outside [1, {Lmax}]")
        t = np.arange(n)
        page = table[b, t // P]
        slot = t % P
        if page.min() < 0 or page.max() >= n_pages:
            raise ValueError(f"sequence {b} names a page outside [0, {n_pages})")
        for g in range(Hkv):
            rows = slice(g * G, (g + 1) * G)
            o, l = _attend_rows(q[b, rows], k_pages[page, g, slot], v_pages[page, g, slot], scale)
            out[b, rows] = o
            lse[b, rows] = l
    return out, lse


def prefill_attention(q, k, v, lens=None, scale=None):
    """Causal many-query (prefill) attention: every position of a sequence
    attends to the cache rows up to and including its own.

    q     [B, Hq, Lmax, D]   one query per position
    k, v  [B, Hkv, Lmax, D]
    lens  [B] integers in [1, Lmax] (None: every sequence is Lmax long)
    Returns out [B, Hq, Lmax, D] and lse [B, Hq, Lmax]; positions at or
    beyond lens[b] hold NaN (no query there).

    [FD] "Por qué la decodificación necesita otra planificación": during
    prefill many query positions are processed in parallel.  [MW] the
    section on why prompts are fast and generation slow: prefill is
    matrix-matrix work.  Reading: position p of sequence b sees rows
    [0, p], i.e. decode attention with lens = p + 1 for each position.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, Hq, Lq, D = q.shape
    Bk, Hkv, Lmax, Dk = k.shape
    if Bk != B or Dk != D or v.shape != k.shape or Lq != Lmax:
        raise ValueError("shape mismatch between q, k and v")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    if lens is None:
        lens = np.full(B, Lmax, dtype=np.int64)
    lens = np.asarray(lens, dtype=np.int64)
    if scale is None:
        scale = default_scale(D)
    out = np.full((B, Hq, Lmax, D), np.nan)
    lse = np.full((B, Hq, Lmax), np.nan)
    for b in range(B):
        n = int(lens[b])
        if not 1 <= n <= Lmax:
            raise ValueError(f"lens[{b}]={n} outside [1, {Lmax}]")
        for g in range(Hkv):
            for p in range(n):
                rows = slice(g * G, (g + 1) * G)
                o, l = _attend_rows(q[b, rows, p], k[b, g, :p + 1], v[b, g, :p + 1], scale)
                out[b, rows, p] = o
                lse[b, rows, p] = l
    return out, lse


def fp8_e4m3_value(bits):
    """Values of OCP 8-bit floating-point E4M3 codes (the "fn" variant).

    Bit layout s eeee mmm, exponent bias 7.  Exponent field 0 holds the
    subnormals m/8 * 2^-6 (and +-0); otherwise the value is
    (1 + m/8) * 2^(e - 7).  The codes with every exponent and mantissa bit
    set (0x7F, 0xFF) are NaN; there are no infinities, so the largest finite
    magnitude is 1.75 * 2^8 = 448.
    """
    b = np.asarray(bits).astype(np.int64) & 0xFF
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((b & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def attention_fp8kv(q, k_bits, v_bits, k_scale=None, v_scale=None, lens=None, scale=None):
    """Decode attention over an 8-bit E4M3 KV cache with per-KV-head scales.

    q               [B, Hq, D] values
    k_bits, v_bits  [B, Hkv, Lmax, D] E4M3 codes
    k_scale, v_scale  [Hkv] (None: 1); cache row value = code value * scale
    [MW] "ಮೆಮೊರಿ ವಾಲ್ (Memory Wall) ವಿರುದ್ಧ ಹೋರಾಟ", quantisation paragraph:
    fewer bits per stored value move fewer bytes over the memory bus.  The
    codes follow the OCP 8-bit floating-point specification (E4M3, see
    fp8_e4m3_value); the attention is the plain attention over the
    dequantised cache.
    """
    k_bits = np.asarray(k_bits)
    Hkv = k_bits.shape[1]
    ks = np.ones(Hkv) if k_scale is None else _as_f64(k_scale)
    vs = np.ones(Hkv) if v_scale is None else _as_f64(v_scale)
    k = fp8_e4m3_value(k_bits) * ks[None, :, None, None]
    v = fp8_e4m3_value(v_bits) * vs[None, :, None, None]
    return attention(q, k, v, lens, scale)


def bifurcated_attention(q, k_ctx, v_ctx, k_dec, v_dec, dec_lens=None, scale=None):
    """Bifurcated single-context batch-sampling attention, by its definition.

    q             [S, Hq, D]      one query position per sample
    k_ctx, v_ctx  [Hkv, Lc, D]    context (prefill) KV shared by all samples
    k_dec, v_dec  [S, Hkv, Ldmax, D]  each sample's own decode KV
    dec_lens      [S] integers in [0, Ldmax] (None: all Ldmax)

    [BA] "Tiivistelmä": the split into a context part and a decode part is
    exact, so the result is standard attention of sample s over the rows
    [context rows ; its own decode rows].  That concatenation is what is
    computed here.
    """
    q = _as_f64(q)
    k_ctx, v_ctx, k_dec, v_dec = map(_as_f64, (k_ctx, v_ctx, k_dec, v_dec))
    S, Hq, D = q.shape
    Hkv, Lc, _ = k_ctx.shape
    Ldmax = k_dec.shape[2]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    if Lc < 1:
        raise ValueError("the context must hold at least one row")
    G = Hq // Hkv
    if dec_lens is None:
        dec_lens = np.full(S, Ldmax, dtype=np.int64)
    dec_lens = np.asarray(dec_lens, dtype=np.int64)
    if scale is None:
        scale = default_scale(D)
    out = np.empty((S, Hq, D))
    lse = np.empty((S, Hq))
    for s in range(S):
        n = int(dec_lens[s])
        if not 0 <= n <= Ldmax:
            raise ValueError(f"dec_lens[{s}]={n} outside [0, {Ldmax}]")
        for g in range(Hkv):
            rows = slice(g * G, (g + 1) * G)
            keys = np.concatenate([k_ctx[g], k_dec[s, g, :n]], axis=0)
            vals = np.concatenate([v_ctx[g], v_dec[s, g, :n]], axis=0)
            o, l = _attend_rows(q[s, rows], keys, vals, scale)
            out[s, rows] = o
            lse[s, rows] = l
    return out, lse


def bifurcated_paged_attention(q, k_ctx, v_ctx, k_pages, v_pages, block_table, dec_lens, scale=None):
    """Bifurcated attention with each sample's decode rows in a paged pool.

    q                 [S, Hq, D]
    k_ctx, v_ctx      [Hkv, Lc, D]          shared context, dense
    k_pages, v_pages  [n_pages, Hkv, P, D]  pages of P rows for each KV head
    block_table       [S, max_pages] integer page ids
    dec_lens          [S] integers in [0, max_pages * P]

    [BA] "Tiivistelmä": sample s attends over [context rows ; its own decode
    rows].  [MW] "ಮೆಮೊರಿ ವಾಲ್ (Memory Wall) ವಿರುದ್ಧ ಹೋರಾಟ", PagedAttention:
    decode row t of sample s is row t mod P of page block_table[s, t div P];
    only the entries covering rows below dec_lens[s] are read.
    """
    q = _as_f64(q)
    k_ctx, v_ctx, k_pages, v_pages = map(_as_f64, (k_ctx, v_ctx, k_pages, v_pages))
    S, Hq, D = q.shape
    Hkv, Lc, _ = k_ctx.shape
    n_pages, Hkp, P, _ = k_pages.shape
    table = np.asarray(block_table, dtype=np.int64)
    if Hkp != Hkv or v_pages.shape != k_pages.shape or table.shape[0] != S:
        raise ValueError("shape mismatch between q, the context, the pages and the block table")
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    dec_lens = np.asarray(dec_lens, dtype=np.int64)
    if scale is None:
        scale = default_scale(D)
    out = np.empty((S, Hq, D))
    lse = np.empty((S, Hq))
    for s in range(S):
        n = int(dec_lens[s])
        if not 0 <= n <= table.shape[1] * P:
            raise ValueError(f"dec_lens[{s}]={n} outside [0, {table.shape[1] * P}]")
        pages = [int(table[s, t // P]) for t in range(n)]
        if any(pg < 0 or pg >= n_pages for pg in pages):
            raise ValueError(f"sample {s} names a page outside [0, {n_pages})")
        for g in range(Hkv):
            rows = slice(g * G, (g + 1) * G)
            dk = np.array([k_pages[pages[t], g, t % P] for t in range(n)]).reshape(n, D)
            dv = np.array([v_pages[pages[t], g, t % P] for t in range(n)]).reshape(n, D)
            o, l = _attend_rows(q[s, rows], np.concatenate([k_ctx[g], dk]), np.concatenate([v_ctx[g], dv]), scale)
            out[s, rows] = o
            lse[s, rows] = l
    return out, lse


def split_partials(q, k, v, bounds, scale=None):
    """Per-piece partial results of [FD]'s split of the history.

    q [R, D] query rows that share one KV slice k, v [n, D].
    bounds: increasing row indices 0 = t_0 <= t_1 <= ... <= t_P = n; piece i
    covers rows [t_i, t_{i+1}) and may be empty.
    Returns O [P, R, D] (each piece's own normalised attention output) and
    lse [P, R] (natural-log log-sum-exp of that piece's scaled scores;
    -inf for an empty piece).

    [FD] "Por qué la decodificación necesita otra planificación": each unit
    computes a partial result and a log-sum-exp normalisation value.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    if scale is None:
        scale = default_scale(q.shape[1])
    bounds = [int(t) for t in bounds]
    if bounds[0] != 0 or bounds[-1] != k.shape[0] or any(
        b1 < b0 for b0, b1 in zip(bounds, bounds[1:])
    ):
        raise ValueError("bounds must rise from 0 to n")
    P = len(bounds) - 1
    R, D = q.shape
    O = np.empty((P, R, D))
    L = np.empty((P, R))
    for i in range(P):
        t0, t1 = bounds[i], bounds[i + 1]
        O[i], L[i] = _attend_rows(q, k[t0:t1], v[t0:t1], scale)
    return O, L


def lse_combine(o_part, lse_part):
    """[FD]'s reduction: merge per-piece (output, lse) into the full result.

    o_part [P, ..., D] normalised partial outputs, lse_part [P, ...] their
    natural-log log-sum-exps (-inf marks an empty piece).  Piece i carries
    weight w_i = exp(lse_i - M) with M = max_i lse_i, so that
    out = sum_i w_i O_i / sum_i w_i and lse = M + ln(sum_i w_i).  This is the
    exact renormalisation: piece i's own softmax denominator is exp(lse_i),
    and the full denominator is the sum of them.  At least one piece must be
    non-empty.
    """
    o_part = _as_f64(o_part)
    lse_part = _as_f64(lse_part)
    M = lse_part.max(axis=0)
    if not np.all(np.isfinite(M)):
        raise ValueError("every row needs at least one non-empty piece")
    w = np.where(np.isneginf(lse_part), 0.0, np.exp(lse_part - M))
    z = w.sum(axis=0)
    out = (w[..., None] * o_part).sum(axis=0) / z[..., None]
    return out, M + np.log(z)
