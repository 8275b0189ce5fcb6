"""Materialised standard attention in NumPy fp64 -- TEST INFRASTRUCTURE.

This is the three-kernel computation the pages use as the baseline
("FlashAttention" explainer, Step 2 "Standard Attention"; "13% more FLOPs,
5.7x faster", section "The hierarchy attention keeps ignoring"):
S = scale * Q K^T is formed in full, P = softmax(S) in full, then O = P V.
Its backward keeps P and forms the chain-rule gradients with whole matrices.
Meant for tiny inputs only (memory is N x N per head).  It shares no code
with the C oracle, so agreement between the two is a cross-check of both.
"""
import numpy as np


def _mask(N, causal):
    if not causal:
        return np.ones((N, N), dtype=bool)
    return np.tril(np.ones((N, N), dtype=bool))


def fwd(q, k, v, scale, causal=False):
    """q, k, v: [..., N, d] fp64.  Returns (o, lse, p)."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    N = q.shape[-2]
    s = scale * (q @ np.swapaxes(k, -1, -2))
    keep = _mask(N, causal)
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    e = np.exp(s - m)
    l = e.sum(axis=-1, keepdims=True)
    p = e / l
    o = p @ v
    lse = (m + np.log(l))[..., 0]
    return o, lse, p


def bwd(q, k, v, dO, scale, causal=False):
    """Returns (o, lse, dq, dk, dv) for L = sum(O * dO)."""
    q, k, v, dO = (np.asarray(t, np.float64) for t in (q, k, v, dO))
    o, lse, p = fwd(q, k, v, scale, causal)
    dv = np.swapaxes(p, -1, -2) @ dO
    dp = dO @ np.swapaxes(v, -1, -2)
    D = (p * dp).sum(axis=-1, keepdims=True)
    ds = p * (dp - D)
    dq = scale * (ds @ k)
    dk = scale * (np.swapaxes(ds, -1, -2) @ q)
    return o, lse, dq, dk, dv
