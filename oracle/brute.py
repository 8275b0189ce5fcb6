"""Materialised standard attention in NumPy fp64 -- TEST INFRASTRUCTURE.

This is the three-kernel computation the pages use as the baseline
("FlashAttention" explainer, Step 2 "Standard Attention"; "13% more FLOPs,
5.7x faster", section "The hierarchy attention keeps ignoring"):
S = scale * Q K^T is formed in full, P = softmax(S) in full, then O = P V.
Its backward keeps P and forms the chain-rule gradients with whole matrices.
Meant for tiny inputs only (memory is N x N per head).  It shares no code
with the C oracle, so agreement between the two is a cross-check of both.
:func:`split_merge` states the split-K/V forward (softmax per chunk of the
keys, then the merge rule) on the same materialised scores.
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


def split_merge(q, k, v, scale, causal, bounds):
    """Forward computed over chunks of the keys and merged.  Chunk c holds
    keys bounds[c] .. bounds[c+1]-1 (bounds ascending, bounds[0] = 0 and
    bounds[-1] = N; empty chunks allowed).  Per chunk and row, the softmax
    over the chunk's visible keys gives a partial output O_c normalised by
    its own sum and lse_c = m_c + log(l_c) (O_c = 0, lse_c = -inf when the
    row sees no key of the chunk).  The partials are merged by the rescale
    rule of the online softmax ("13% more FLOPs, 5.7x faster", section
    "FlashAttention's move: rescale the output, too"; explainer "Common
    questions", Flash-Decoding) in logsumexp form:
        lse = log sum_c exp(lse_c),   O = sum_c exp(lse_c - lse) O_c.
    Returns (o, lse)."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    N = q.shape[-2]
    s = scale * (q @ np.swapaxes(k, -1, -2))
    keep = _mask(N, causal)
    keys = np.arange(N)
    outs, lses = [], []
    for c in range(len(bounds) - 1):
        inside = keep & (keys >= bounds[c]) & (keys < bounds[c + 1])
        sc = np.where(inside, s, -np.inf)
        m = sc.max(axis=-1, keepdims=True)
        seen = np.isfinite(m)
        e = np.where(seen, np.exp(sc - np.where(seen, m, 0.0)), 0.0)
        l = e.sum(axis=-1, keepdims=True)
        o_c = np.where(seen, (e @ v) / np.where(seen, l, 1.0), 0.0)
        lse_c = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)[..., 0]
        outs.append(o_c)
        lses.append(lse_c)
    lses = np.stack(lses)                       # [C, ..., N]
    top = lses.max(axis=0)
    w = np.exp(lses - top)                      # exp(-inf) = 0 for chunks a row does not see
    total = w.sum(axis=0)
    lse = top + np.log(total)
    o = sum(w[c][..., None] * outs[c] for c in range(len(outs))) / total[..., None]
    return o, lse
