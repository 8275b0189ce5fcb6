"""Pins of the FP8 (E4M3) oracle, on the CPU.

* The decoder against torch's float8_e4m3fn conversion (a library routine)
  for all 256 codes, and against values the format's definition fixes.
* The definition (decode, descale, exact attention in the C oracle) against
  the materialised NumPy attention on the same decoded values.
* The error bound, from the reading alone (no tiling of the kernel's): the
  oracle's exact softmax weights w_j (the materialised NumPy attention) are
  scaled and rounded to nearest even E4M3 by torch at every scale the
  reading admits -- each key j at a scale sigma_j with the row's largest
  weight mapped to at least 2^4 and sigma_j w_j at most 2^8 -- one scale for
  the whole row at offsets across [2^4, 2^8], and independent per-key
  scales drawn over the whole admissible range (which covers any order in
  which a reference can move).  The output those rounded weights give stays
  within the bound everywhere and comes within a factor of ten of it
  somewhere; planted mistakes (V paired with the neighbouring key, a
  missed rescale, equal merge weights for split chunks) break it.
"""
import math

import numpy as np
import pytest
import torch

from exact_io_aware_40_amd.inputs import WORKLOADS, make_fp8_inputs, quantize_e4m3
from oracle import brute
from oracle import fp8 as ofp8


def test_decode_matches_torch_for_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = ofp8.decode_e4m3(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    # signed zeros decode with their sign
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


@pytest.mark.parametrize("code,value", [
    (0x00, 0.0), (0x38, 1.0), (0xB8, -1.0), (0x7E, 448.0), (0xFE, -448.0),
    (0x01, 2.0**-9), (0x07, 7 * 2.0**-9), (0x08, 2.0**-6), (0x3C, 1.5), (0x40, 2.0),
    (0x30, 0.5), (0x77, 240.0), (0x78, 256.0),
])
def test_decode_fixed_values(code, value):
    assert ofp8.decode_e4m3(np.array([code], np.uint8))[0] == value


def test_decode_nan_codes():
    d = ofp8.decode_e4m3(np.array([0x7F, 0xFF], np.uint8))
    assert np.isnan(d).all()


def test_quantize_roundtrip_within_half_ulp():
    x = torch.randn(4096) * 3
    codes, ds = quantize_e4m3(x)
    back = ofp8.decode_e4m3(codes.numpy()) * ds
    xs = x.double().numpy()
    # normal range: |error| <= 2^-4 |x| (plus the scale's fp32 rounding)
    big = np.abs(xs) * (448.0 / np.abs(xs).max()) >= 2.0**-6
    assert np.all(np.abs(back - xs)[big] <= 2.0**-4 * np.abs(xs[big]) * (1 + 1e-6) + 1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_equals_materialised(causal):
    w = WORKLOADS["llama7b_layer_fwd"]
    x, ds = make_fp8_inputs(w, seed=11, shape=(1, 2, 70, 128))
    scale = 1 / math.sqrt(128)
    o, lse = ofp8.fwd_fp8(x["q"], x["k"], x["v"], scale, ds, causal)
    q, k, v = (ofp8.dequantize(x[n].numpy(), d) for n, d in zip("qkv", ds))
    o2, lse2, _ = brute.fwd(q, k, v, scale, causal)
    assert np.abs(o - o2).max() <= 1e-12 * max(1.0, np.abs(o2).max())
    assert np.abs(lse - lse2).max() <= 1e-12 * max(1.0, np.abs(lse2).max())


def _e4m3_round(x):
    return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(torch.float8_e4m3fn).double().numpy()


def _rounded_weights(w, mode, rng):
    """Weights of one softmax (w: [rows, keys], each row summing to one,
    masked keys 0) as the reading uses them: w_j scaled by sigma_j, rounded
    to E4M3, scaled back.  mode: a number a -- one scale per row, mapping the
    row's largest weight to 2^a (4 <= a <= 8); "random" -- each key its own
    scale, log2 sigma_j uniform over [4 - log2 max w, 8 - log2 w_j]; "low" /
    "high" -- each key at the lower / upper end of that range."""
    wmax = w.max(axis=1, keepdims=True)
    pos = w > 0
    lw = np.log2(np.where(pos, w, 1.0))
    lo = 4.0 - np.log2(wmax) + np.zeros_like(w)
    hi = 8.0 - lw
    if mode == "random":
        e = lo + rng.random(w.shape) * (hi - lo)
    elif mode == "low":
        e = lo
    elif mode == "high":
        e = hi
    else:
        e = float(mode) - np.log2(wmax) + np.zeros_like(w)
    sig = np.exp2(e)
    assert np.all(sig * w <= 256.0 * (1 + 1e-12))
    return np.where(pos, _e4m3_round(sig * w) / sig, 0.0)


MODES = [4.0, 5.5, 6.3, 7.0, 8.0, "low", "high", "random", "random"]


def _weights_and_values(x, ds, causal):
    scale = 1 / math.sqrt(128)
    q, k, v = (ofp8.dequantize(x[n].numpy(), d) for n, d in zip("qkv", ds))
    o, _, w = brute.fwd(q, k, v, scale, causal)
    return w, v, o


@pytest.mark.parametrize("outliers", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_bound_covers_every_admissible_rounding(outliers, causal):
    name = "llama7b_layer_fwd" if outliers else "long_context_fwd"
    x, ds = make_fp8_inputs(WORKLOADS[name], seed=12, shape=(1, 2, 200, 128))
    scale = 1 / math.sqrt(128)
    w, v, o = _weights_and_values(x, ds, causal)
    bound = ofp8.error_bound(x["q"], x["k"], x["v"], scale, ds, causal)
    rng = np.random.default_rng(5)
    worst = 0.0
    for mode in MODES:
        wh = np.stack([_rounded_weights(w[0, h], mode, rng) for h in range(2)])[None]
        err = np.abs(wh @ v - o)
        assert np.all(err <= bound), (mode, float((err / bound).max()))
        worst = max(worst, float((err / bound).max()))
    # the bound is not vacuous: some rounding comes within a factor of ten of it
    assert worst > 0.1


def test_bound_needs_the_lower_scale_limit():
    """Outside the reading -- the row's largest weight mapped far below 2^4,
    so that most weights fall into E4M3's subnormals -- the rounding breaks
    the bound: its subnormal term relies on the lower limit."""
    x, ds = make_fp8_inputs(WORKLOADS["long_context_fwd"], seed=12, shape=(1, 1, 200, 128))
    scale = 1 / math.sqrt(128)
    w, v, o = _weights_and_values(x, ds, False)
    bound = ofp8.error_bound(x["q"], x["k"], x["v"], scale, ds, False)
    wmax = w[0, 0].max(axis=1, keepdims=True)
    sig = 2.0**-4 / wmax
    wh = _e4m3_round(sig * w[0, 0]) / sig
    assert np.any(np.abs(wh @ v[0, 0] - o[0, 0]) > bound[0, 0])


@pytest.mark.parametrize("mistake", ["shift_v", "no_rescale"])
def test_bound_catches_mistakes(mistake):
    x, ds = make_fp8_inputs(WORKLOADS["llama7b_layer_fwd"], seed=13, shape=(1, 1, 200, 128))
    scale = 1 / math.sqrt(128)
    w, v, o = _weights_and_values(x, ds, True)
    w, v, o = w[0, 0], v[0, 0], o[0, 0]
    bound = ofp8.error_bound(x["q"], x["k"], x["v"], scale, ds, True)[0, 0]
    rng = np.random.default_rng(6)
    wh = _rounded_weights(w, "random", rng)
    assert np.all(np.abs(wh @ v - o) <= bound)
    if mistake == "shift_v":
        # each weight applied to the next key's V row
        bad = wh @ np.concatenate([v[1:], v[-1:]])
    else:
        # the first half of the keys keeps the weight of a reference that
        # later moved up by 4 binades: the accumulated output and sum both
        # miss the factor 2^-4
        f = np.where(np.arange(w.shape[1]) < w.shape[1] // 2, 16.0, 1.0)
        bad = ((wh * f) @ v) / (w * f).sum(axis=1, keepdims=True)
    assert np.any(np.abs(bad - o) > bound)


@pytest.mark.parametrize("causal", [False, True])
def test_fwd_fp8_rect_equals_materialised(causal):
    w = WORKLOADS["long_context_fwd"]
    xq, ds = make_fp8_inputs(w, seed=14, shape=(1, 2, 5, 128))
    xk, dk = make_fp8_inputs(w, seed=15, shape=(1, 2, 90, 128))
    desc = (ds[0], dk[1], dk[2])
    scale = 1 / math.sqrt(128)
    o, lse = ofp8.fwd_fp8_rect(xq["q"], xk["k"], xk["v"], scale, desc, causal)
    q = ofp8.dequantize(xq["q"].numpy(), desc[0])
    k = ofp8.dequantize(xk["k"].numpy(), desc[1])
    v = ofp8.dequantize(xk["v"].numpy(), desc[2])
    o2, lse2 = brute.fwd_rect(q, k, v, scale, causal)
    assert np.abs(o - o2).max() <= 1e-12
    assert np.abs(lse - lse2).max() <= 1e-12


def _chunked_rounded(q, k, v, scale, causal, bounds, rng, mistake=None):
    """Nq queries against Nk keys, the keys cut at `bounds`: per chunk and
    row the exact softmax over the chunk's visible keys, its weights rounded
    as in _rounded_weights (mode "random", the chunk's own largest weight
    mapped to at least 2^4), the chunk's partial output; then the exact
    logsumexp merge of the chunks.  Rows that see no key get 0."""
    Nq, Nk = q.shape[-2], k.shape[-2]
    s = scale * (q @ k.T)
    vis = (np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)) if causal else np.ones((Nq, Nk), bool)
    out = np.zeros((Nq, q.shape[-1]))
    parts_o, parts_l = [], []
    for c0, c1 in zip(bounds[:-1], bounds[1:]):
        inside = vis.copy()
        inside[:, :c0] = False
        inside[:, c1:] = False
        sc = np.where(inside, s, -np.inf)
        m = sc.max(axis=1, keepdims=True)
        seen = np.isfinite(m)
        e = np.where(inside, np.exp(sc - np.where(seen, m, 0.0)), 0.0)
        l = e.sum(axis=1, keepdims=True)
        w = e / np.where(seen, l, 1.0)
        wh = np.zeros_like(w)
        if seen.any():
            rws = seen[:, 0]
            wh[rws] = _rounded_weights(w[rws], "random", rng)
        parts_o.append(wh @ v)
        parts_l.append(np.where(seen, m + np.log(np.where(seen, l, 1.0)), -np.inf))
    L = np.concatenate(parts_l, axis=1)
    top = L.max(axis=1, keepdims=True)
    seen = np.isfinite(top)
    wts = np.where(np.isfinite(L), np.exp(L - np.where(seen, top, 0.0)), 0.0)
    if mistake == "equal_weights":
        wts = np.where(np.isfinite(L), 1.0, 0.0)
    wts = wts / np.where(seen, wts.sum(axis=1, keepdims=True), 1.0)
    for c, oc in enumerate(parts_o):
        out += wts[:, c:c + 1] * oc
    return out


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,cuts", [(1, 700, [0, 128, 256, 640, 700]), (4, 300, [0, 64, 300]),
                                        (16, 16, [0, 16]), (40, 20, [0, 8, 20]),
                                        (130, 500, [0, 192, 384, 500])])
def test_bound_holds_for_chunks(Nq, Nk, cuts, causal):
    w = WORKLOADS["llama7b_layer_fwd"]
    xq, ds = make_fp8_inputs(w, seed=16, shape=(1, 1, Nq, 128))
    xk, dk = make_fp8_inputs(w, seed=17, shape=(1, 1, Nk, 128))
    desc = (ds[0], dk[1], dk[2])
    scale = 1 / math.sqrt(128)
    q = ofp8.dequantize(xq["q"].numpy(), desc[0]).reshape(Nq, 128)
    k = ofp8.dequantize(xk["k"].numpy(), desc[1]).reshape(Nk, 128)
    v = ofp8.dequantize(xk["v"].numpy(), desc[2]).reshape(Nk, 128)
    o_ref, _ = ofp8.fwd_fp8_rect(xq["q"], xk["k"], xk["v"], scale, desc, causal)
    bound = ofp8.error_bound(xq["q"], xk["k"], xk["v"], scale, desc, causal).reshape(Nq, 128)
    rng = np.random.default_rng(7)
    for _ in range(3):
        o_c = _chunked_rounded(q, k, v, scale, causal, cuts, rng)
        assert np.all(np.abs(o_c - o_ref.reshape(Nq, 128)) <= bound)


def test_bound_catches_wrong_merge():
    w = WORKLOADS["llama7b_layer_fwd"]
    xq, ds = make_fp8_inputs(w, seed=18, shape=(1, 1, 2, 128))
    xk, dk = make_fp8_inputs(w, seed=19, shape=(1, 1, 640, 128))
    desc = (ds[0], dk[1], dk[2])
    scale = 1 / math.sqrt(128)
    q = ofp8.dequantize(xq["q"].numpy(), desc[0]).reshape(2, 128)
    k = ofp8.dequantize(xk["k"].numpy(), desc[1]).reshape(640, 128)
    v = ofp8.dequantize(xk["v"].numpy(), desc[2]).reshape(640, 128)
    o_ref, _ = ofp8.fwd_fp8_rect(xq["q"], xk["k"], xk["v"], scale, desc, False)
    bound = ofp8.error_bound(xq["q"], xk["k"], xk["v"], scale, desc, False).reshape(2, 128)
    rng = np.random.default_rng(8)
    cuts = [0, 128, 640]
    assert np.all(np.abs(_chunked_rounded(q, k, v, scale, False, cuts, rng) - o_ref.reshape(2, 128)) <= bound)
    o_bad = _chunked_rounded(q, k, v, scale, False, cuts, rng, mistake="equal_weights")
    assert np.any(np.abs(o_bad - o_ref.reshape(2, 128)) > bound)
