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
:func:`fwd_dropout` / :func:`bwd_dropout` apply dropout to the materialised
probabilities, with the keep mask built here from a vectorised Philox4x32-10
written separately from the C oracle's (same published definition, same
element-to-byte mapping; see :func:`dropout_keep`).
"""
import numpy as np


def _mask(N, causal):
    if not causal:
        return np.ones((N, N), dtype=bool)
    return np.tril(np.ones((N, N), dtype=bool))


def scores(q, k, scale):
    """The full score matrix S = scale * Q K^T, [..., N, N] fp64 (no mask)."""
    q, k = (np.asarray(t, np.float64) for t in (q, k))
    return scale * (q @ np.swapaxes(k, -1, -2))


def fwd(q, k, v, scale, causal=False):
    """q, k, v: [..., N, d] fp64.  Returns (o, lse, p)."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    N = q.shape[-2]
    s = scores(q, k, scale)
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


_M0, _M1 = np.uint64(0xD2511F53), np.uint64(0xCD9E8D57)
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_LO = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC 2011) over arrays.

    ctr: uint32 array [..., 4]; key: two integers.  Each of the ten rounds
    forms the 64-bit products M0 c0 and M1 c2 and maps the counter to
    (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
    then advances by the Weyl constants.  Returns uint32 [..., 4]."""
    c = [np.asarray(ctr, dtype=np.uint64)[..., n] for n in range(4)]
    k0, k1 = int(key[0]) & 0xFFFFFFFF, int(key[1]) & 0xFFFFFFFF
    for _ in range(10):
        p0 = _M0 * c[0]
        p1 = _M1 * c[2]
        c = [(p1 >> np.uint64(32)) ^ c[1] ^ np.uint64(k0), p1 & _LO,
             (p0 >> np.uint64(32)) ^ c[3] ^ np.uint64(k1), p0 & _LO]
        k0, k1 = (k0 + _W0) & 0xFFFFFFFF, (k1 + _W1) & 0xFFFFFFFF
    return np.stack(c, axis=-1).astype(np.uint32)


def dropout_threshold(p):
    """t = floor(256 p + 1/2): an element is kept when its byte is >= t."""
    t = int(np.floor(256.0 * float(p) + 0.5))
    if not (0.0 <= p < 1.0) or t > 255:
        raise ValueError("dropout probability out of range")
    return t


def dropout_keep(p, seed, offset, BH, N):
    """Keep mask [BH, N, N] (bool) before any causal mask.  Element (bh, i, j)
    takes byte j mod 4 of word (j mod 32) // 8 of Philox4x32-10 with key
    (seed mod 2^32, seed // 2^32) and counter
    (i, 2 (j // 32) + (j // 4) mod 2, bh, offset)."""
    t = dropout_threshold(p)
    bh, i, j = np.meshgrid(np.arange(BH), np.arange(N), np.arange(N), indexing="ij")
    ctr = np.stack([i, 2 * (j // 32) + (j // 4) % 2, bh, np.full_like(i, int(offset) & 0xFFFFFFFF)],
                   axis=-1).astype(np.uint32)
    seed = int(seed) & (2**64 - 1)
    words = philox4x32_10(ctr, (seed & 0xFFFFFFFF, seed >> 32))
    word = np.take_along_axis(words, ((j % 32) // 8)[..., None], axis=-1)[..., 0]
    byte = (word >> (8 * (j % 4)).astype(np.uint32)) & np.uint32(0xFF)
    return byte >= t


def fwd_dropout(q, k, v, scale, causal, p, seed, offset):
    """Materialised forward with dropout: O = (keep * r * P) V with
    r = 256 / (256 - t); lse of the undropped softmax.  q, k, v: [BH, N, d].
    Returns (o, lse, w) with w the dropped, rescaled weights."""
    q, k, v = (np.asarray(x, np.float64) for x in (q, k, v))
    BH, N = q.shape[0], q.shape[1]
    _, lse, prob = fwd(q, k, v, scale, causal)
    t = dropout_threshold(p)
    w = np.where(dropout_keep(p, seed, offset, BH, N), prob * (256.0 / (256.0 - t)), 0.0)
    return w @ v, lse, w


def bwd_dropout(q, k, v, dO, scale, causal, p, seed, offset):
    """Gradients of sum(O * dO) through the dropped weights w = keep r P:
    dV = w^T dO, dP = keep r (dO V^T), D = rowsum(P dP), dS = P (dP - D).
    Returns (o, lse, dq, dk, dv)."""
    q, k, v, dO = (np.asarray(x, np.float64) for x in (q, k, v, dO))
    BH, N = q.shape[0], q.shape[1]
    _, lse, prob = fwd(q, k, v, scale, causal)
    t = dropout_threshold(p)
    kr = dropout_keep(p, seed, offset, BH, N) * (256.0 / (256.0 - t))
    w = kr * prob
    o = w @ v
    dv = np.swapaxes(w, -1, -2) @ dO
    dp = kr * (dO @ np.swapaxes(v, -1, -2))
    D = (prob * dp).sum(axis=-1, keepdims=True)
    ds = prob * (dp - D)
    dq = scale * (ds @ k)
    dk = scale * (np.swapaxes(ds, -1, -2) @ q)
    return o, lse, dq, dk, dv


def fwd_rect(q, k, v, scale, causal=False):
    """Materialised forward of Nq queries against Nk keys ([BH, Nq, d] and
    [BH, Nk, d]); under the causal mask query i sees keys j <= i + Nk - Nq.
    Rows with no visible key get o = 0 and lse = -inf.  Returns (o, lse)."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    Nq, Nk = q.shape[-2], k.shape[-2]
    s = scale * (q @ np.swapaxes(k, -1, -2))
    if causal:
        keep = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
    else:
        keep = np.ones((Nq, Nk), dtype=bool)
    s = np.where(keep, s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    seen = np.isfinite(m)
    e = np.where(seen, np.exp(s - np.where(seen, m, 0.0)), 0.0)
    l = e.sum(axis=-1, keepdims=True)
    o = np.where(seen, (e @ v) / np.where(seen, l, 1.0), 0.0)
    lse = np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf)[..., 0]
    return o, lse
