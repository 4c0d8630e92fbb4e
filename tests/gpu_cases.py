"""Helpers shared by the GPU parity tests: host<->device moves and error stats."""

import numpy as np
import torch

import oracle


def to_dev(x, dtype):
    """Host float32 array holding exact input values -> device tensor of dtype."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to("cuda").to(torch.bfloat16 if dtype == "bf16" else torch.float32).contiguous()


def to_host(t):
    """Device tensor -> float64 numpy with the exact stored values."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def max_abs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    if not np.all(np.isfinite(a)):
        return float("inf")
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def oracle_decode_rows(q, k, v, lens, rows, scale=None):
    """Oracle for selected (b, kv-head) units: q, k, v are device tensors.

    Copies only the valid rows of the selected units to the host.  Returns
    {(b, g): (out [G, D], lse [G])}.
    """
    B, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    lens_h = lens.cpu().numpy() if lens is not None else np.full(B, k.shape[2])
    res = {}
    for (b, g) in rows:
        n = int(lens_h[b])
        qb = to_host(q[b:b + 1, g * G:(g + 1) * G])
        kb = to_host(k[b:b + 1, g:g + 1, :n])
        vb = to_host(v[b:b + 1, g:g + 1, :n])
        o, l = oracle.attention(qb, kb, vb, None, scale)
        res[(b, g)] = (o[0], l[0])
    return res


def sampled_units(w, count, seed):
    """(sequence, KV head) units of a full-size workload to check one by one:
    the first, the last, and seeded random ones."""
    rng = np.random.Generator(np.random.PCG64(seed))
    units = {(0, 0), (w.batch - 1, w.kv_heads - 1)}
    while len(units) < min(count, w.batch * w.kv_heads):
        units.add((int(rng.integers(w.batch)), int(rng.integers(w.kv_heads))))
    return sorted(units)


def check_every_unit(q, fetch_kv, lens_h, out, lse, tol, scale=None):
    """Properties of exact attention checked on every output row of a
    full-size call (the oracle covers sampled units one by one):

    * every output element lies in the convex hull of its KV head's valid
      value rows: min_j V[j, d] - tol <= out[d] <= max_j V[j, d] + tol;
    * the lse lies between the largest scaled score and that plus ln(n):
      max_j s_j - tol <= lse <= max_j s_j + ln(n) + tol.

    q [B, Hq, D] and out [B, Hq, D], lse [B, Hq] are device tensors;
    fetch_kv(b) returns sequence b's valid rows as fp32 device tensors
    k, v [Hkv, n, D] (n = lens_h[b]).  The scores are formed in fp32 on the
    device, one sequence at a time; they only bound the lse.  Returns the
    number of rows checked.
    """
    B, Hq, D = q.shape
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    for b in range(B):
        n = int(lens_h[b])
        kb, vb = fetch_kv(b)
        Hkv = kb.shape[0]
        G = Hq // Hkv
        assert kb.shape == (Hkv, n, D) and vb.shape == (Hkv, n, D)
        qb = q[b].float().reshape(Hkv, G, D).transpose(1, 2).contiguous()   # [Hkv, D, G]
        s = torch.matmul(kb.contiguous(), qb) * scale             # [Hkv, n, G]
        smax = s.amax(dim=1).reshape(Hq)                          # [Hq]
        lo = vb.amin(dim=1).repeat_interleave(G, dim=0)           # [Hq, D]
        hi = vb.amax(dim=1).repeat_interleave(G, dim=0)
        ob = out[b].float()
        assert torch.isfinite(ob).all(), f"non-finite output in sequence {b}"
        assert bool((ob >= lo - tol).all() and (ob <= hi + tol).all()), f"output outside the value hull, seq {b}"
        lb = lse[b].float()
        assert bool((lb >= smax - tol).all() and (lb <= smax + float(np.log(n)) + tol).all()), \
            f"lse outside [max score, max score + ln n], seq {b}"
        del kb, vb, s
    return B * Hq


def dense_rows(k, v, lens_h):
    """fetch_kv for a dense cache [B, Hkv, L, D]."""
    return lambda b: (k[b, :, :int(lens_h[b])].float(), v[b, :, :int(lens_h[b])].float())
