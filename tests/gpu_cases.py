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
