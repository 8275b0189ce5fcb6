"""FP8 (E4M3) forward: input decoding, the definition, the error bound -- TEST
INFRASTRUCTURE.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this module; it imports nothing from the product path.

The pages name the low-precision forward of FlashAttention-3 as later work
("FlashAttention" explainer, "Common questions" and its reference list) and
fix nothing about it.  The reading taken here:

* Q, K and V arrive as 8-bit E4M3 codes (the OCP 8-bit floating-point
  format: 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent field 0 encodes subnormals m/8 * 2^-6; the codes S.1111.111 are
  NaN; there is no infinity), each tensor with one fp32 descale factor, so
  that element x stands for decode(x) * descale.
* The result is the same exact attention as the 16-bit path, on those
  values: the oracle is :func:`oracle.fwd` on the decoded, descaled inputs
  (every product decode(x) * descale is exact in fp64).
* The method's one approximation beyond fp32 rounding is that the
  probabilities P enter the P.V product rounded to E4M3 (round to nearest
  even); the row sums and lse use P in fp32.  :func:`error_bound` states
  what that rounding can change.
"""
import numpy as np

from . import fwd as _fwd
from . import fwd_rect as _fwd_rect

E4M3_MAX = 448.0


def decode_e4m3(codes):
    """E4M3 codes (uint8, any shape) -> their values in fp64 (NaN for the two
    NaN codes), from the format's definition."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, (m / 8.0) * 2.0**-6, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((e == 15) & (c & 0x7 == 7), np.nan, mag)
    return sign * mag


def dequantize(codes, descale):
    """decode(codes) * descale in fp64 (exact: 4 significant bits times 24)."""
    return decode_e4m3(codes) * float(np.float32(descale))


def fwd_fp8(q8, k8, v8, scale, descale, causal=False, rows=None, threads=None):
    """Exact attention of the dequantised inputs.  q8, k8, v8: uint8 codes
    [..., N, d]; descale: (q, k, v) factors.  Returns (o, lse) as
    :func:`oracle.fwd` does (all rows, or the flattened `rows`)."""
    q = dequantize(q8, descale[0])
    k = dequantize(k8, descale[1])
    v = dequantize(v8, descale[2])
    return _fwd(q, k, v, scale, causal, rows=rows, threads=threads)


def fwd_fp8_rect(q8, k8, v8, scale, descale, causal=False, rows=None, threads=None):
    """:func:`oracle.fwd_rect` (Nq queries against Nk keys, causal query i
    seeing keys 0 .. i + Nk - Nq) of the dequantised inputs."""
    q = dequantize(q8, descale[0])
    k = dequantize(k8, descale[1])
    v = dequantize(v8, descale[2])
    return _fwd_rect(q, k, v, scale, causal, rows=rows, threads=threads)


def error_bound(q8, k8, v8, scale, descale, causal=False, rows=None, out_rel=0.0):
    """:func:`error_bound_values` of the dequantised inputs."""
    q = dequantize(q8, descale[0])
    k = dequantize(k8, descale[1])
    v = dequantize(v8, descale[2])
    return error_bound_values(q, k, v, scale, causal, rows, out_rel)


def error_bound_values(q, k, v, scale, causal=False, rows=None, out_rel=0.0):
    """Element-wise bound on |O_fp8 - O| for the method read as above, for
    fp64 inputs q [..., Nq, d] and k, v [..., Nk, d] (the values the codes
    stand for; under the causal mask query i sees keys 0 .. i + Nk - Nq).

    The reading of the method's scaling (FlashAttention-3's low-precision
    forward scales P into the format's range; the pages fix no more): each
    probability is rounded at some scale -- P_j = sigma_j w_j, one scale per
    key or shared by many -- under which no P exceeds 2^8 (below E4M3's
    largest value, 448) and the row's largest weight (among the keys summed
    with it) maps to at least 2^4.  With w_j the exact softmax weights of a
    row and v_j its visible V rows: rounding P_j to nearest in E4M3 changes
    it by at most 2^-4 P_j while P_j is in E4M3's normal range, and by at
    most 2^-10 (half the subnormal spacing 2^-9) below it, which in units of
    the normalised output is at most 2^-14 times the largest weight.  Hence,
    per output element c,
        |dO_c| <= 2^-4 sum_j w_j |v_jc| + 2^-14 max_j w_j sum_j |v_jc|
                  + 2^-10 sum_j w_j |v_jc| + out_rel |O_c| + 1e-6,
    the third term a generous allowance for fp32 accumulation over up to
    N keys and the fourth the rounding of the output (2^-8 for bf16, 0 for
    fp32).  The same bound holds when the keys are processed in chunks whose
    normalised partial outputs are merged with exact weights: each chunk's
    error is bounded by its own terms, and the merge weights turn the chunk
    weights back into w.  A row that sees no key has O = 0 and bound 1e-6.
    Returns the bound in the layout of :func:`fwd_fp8`'s o."""
    q, k, v = (np.asarray(t, np.float64) for t in (q, k, v))
    lead, N, d = q.shape[:-2], q.shape[-2], q.shape[-1]
    Nk = k.shape[-2]
    BH = int(np.prod(lead)) if lead else 1
    q, k, v = q.reshape(BH, N, d), k.reshape(BH, Nk, d), v.reshape(BH, Nk, d)
    all_rows = rows is None
    if all_rows:
        rows = np.arange(BH * N, dtype=np.int64)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.size, d), np.float64)
    for bh in np.unique(rows // N):
        sel = np.nonzero(rows // N == bh)[0]
        i = rows[sel] % N
        s = float(scale) * (q[bh, i] @ k[bh].T)
        if causal:
            vis = np.arange(Nk)[None, :] <= i[:, None] + (Nk - N)
        else:
            vis = np.ones((i.size, Nk), bool)
        s = np.where(vis, s, -np.inf)
        top = s.max(axis=1, keepdims=True)
        seen = np.isfinite(top)
        w = np.where(seen, np.exp(s - np.where(seen, top, 0.0)), 0.0)
        w /= np.where(seen, w.sum(axis=1, keepdims=True), 1.0)
        av = np.abs(v[bh])
        o = w @ v[bh]
        t1 = w @ av
        t2 = w.max(axis=1, keepdims=True) * (vis.astype(np.float64) @ av)
        out[sel] = (2.0**-4 + 2.0**-10) * t1 + 2.0**-14 * t2 + out_rel * np.abs(o) + 1e-6
    if all_rows:
        return out.reshape(*lead, N, d) if lead else out.reshape(N, d)
    return out
