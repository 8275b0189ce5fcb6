"""Pins of the FP8 (E4M3) oracle, on the CPU.

* The decoder against torch's float8_e4m3fn conversion (a library routine)
  for all 256 codes, and against values the format's definition fixes.
* The definition (decode, descale, exact attention in the C oracle) against
  the materialised NumPy attention on the same decoded values.
* The error bound: an emulation written here of the method as the oracle's
  reading states it (64-key tiles, a reference point kept within the stated
  range, P rounded to nearest even E4M3 by torch, P.V and sums in fp64) stays
  within the bound on random and outlier inputs, and plausible mistakes (V
  paired with the neighbouring key, a missed rescale) break it.
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


def _emulate(q, k, v, scale, causal, mistake=None):
    """The method as read: 64-key tiles per row; reference r (binades) moved
    to (tile max - 4) when the tile max exceeds r + 8; P = 2^(s log2e - r)
    rounded to E4M3 for P.V; l and lse from unrounded P."""
    BH, N, d = q.shape
    o = np.zeros((BH, N, d))
    for bh in range(BH):
        s = scale * (q[bh] @ k[bh].T) * math.log2(math.e)
        for i in range(N):
            kend = i + 1 if causal else N
            ref, l, acc = -np.inf, 0.0, np.zeros(d)
            for j0 in range(0, kend, 64):
                x = s[i, j0:min(kend, j0 + 64)]
                tmax = x.max()
                if tmax > ref + 8:
                    alpha = 0.0 if ref == -np.inf else 2.0 ** (ref - (tmax - 4))
                    if mistake != "no_rescale":
                        acc *= alpha
                        l *= alpha
                    ref = tmax - 4
                p = np.exp2(x - ref)
                assert p.max() <= 256.0
                pr = _e4m3_round(p)
                vv = v[bh, j0:j0 + x.size]
                if mistake == "shift_v":
                    vv = v[bh, np.minimum(np.arange(j0, j0 + x.size) + 1, N - 1)]
                acc += pr @ vv
                l += p.sum()
            o[bh, i] = acc / l
    return o


@pytest.mark.parametrize("outliers", [False, True])
@pytest.mark.parametrize("causal", [False, True])
def test_bound_holds_for_emulated_method(outliers, causal):
    name = "llama7b_layer_fwd" if outliers else "long_context_fwd"
    w = WORKLOADS[name]
    x, ds = make_fp8_inputs(w, seed=12, shape=(1, 2, 200, 128))
    scale = 1 / math.sqrt(128)
    q, k, v = (ofp8.dequantize(x[n].numpy(), d).reshape(2, 200, 128) for n, d in zip("qkv", ds))
    o_ref, _ = ofp8.fwd_fp8(x["q"], x["k"], x["v"], scale, ds, causal)
    bound = ofp8.error_bound(x["q"], x["k"], x["v"], scale, ds, causal)
    o_emu = _emulate(q, k, v, scale, causal)
    err = np.abs(o_emu - o_ref.reshape(2, 200, 128))
    assert np.all(err <= bound.reshape(2, 200, 128))
    # the bound is not vacuous: somewhere the rounding comes within a
    # factor of ten of it
    assert (err / bound.reshape(2, 200, 128)).max() > 0.1


@pytest.mark.parametrize("mistake", ["shift_v", "no_rescale"])
def test_bound_catches_mistakes(mistake):
    w = WORKLOADS["llama7b_layer_fwd"]
    x, ds = make_fp8_inputs(w, seed=13, shape=(1, 1, 200, 128))
    scale = 1 / math.sqrt(128)
    q, k, v = (ofp8.dequantize(x[n].numpy(), d).reshape(1, 200, 128) for n, d in zip("qkv", ds))
    if mistake == "no_rescale":
        # key 150 scores far above every earlier key for each row that sees
        # it, so the reference moves in the row's third tile
        u = np.full(128, 0.5)
        q = q + u
        k[0, 150] = 10 * u
    o_ref = brute.fwd(q, k, v, scale, True)[0]
    bound = ofp8.error_bound_values(q, k, v, scale, True)
    o_ok = _emulate(q, k, v, scale, True)
    assert np.all(np.abs(o_ok - o_ref) <= bound)
    o_bad = _emulate(q, k, v, scale, True, mistake=mistake)
    assert np.any(np.abs(o_bad - o_ref) > bound)


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


def _emulate_split(q, k, v, scale, causal, tiles_per_chunk, mistake=None):
    """Nq queries against Nk keys in chunks of whole 64-key tiles: per chunk
    and row the method as in _emulate (own reference, P rounded to E4M3,
    normalised by the chunk's fp32 sum), then the exact logsumexp merge.
    Rows that see no key get 0."""
    BH, Nq, d = q.shape
    Nk = k.shape[1]
    o = np.zeros((BH, Nq, d))
    for bh in range(BH):
        s = scale * (q[bh] @ k[bh].T) * math.log2(math.e)
        for i in range(Nq):
            kend = min(Nk, i + 1 + Nk - Nq) if causal else Nk
            parts = []
            for c0 in range(0, max(kend, 0), 64 * tiles_per_chunk):
                ref, l, acc = -np.inf, 0.0, np.zeros(d)
                for j0 in range(c0, min(kend, c0 + 64 * tiles_per_chunk), 64):
                    x = s[i, j0:min(kend, j0 + 64)]
                    tmax = x.max()
                    if tmax > ref + 8:
                        alpha = 0.0 if ref == -np.inf else 2.0 ** (ref - (tmax - 4))
                        acc *= alpha
                        l *= alpha
                        ref = tmax - 4
                    p = np.exp2(x - ref)
                    acc += _e4m3_round(p) @ v[bh, j0:j0 + x.size]
                    l += p.sum()
                parts.append((acc / l, (ref + math.log2(l)) * math.log(2)))
            if not parts:
                continue
            lses = np.array([lc for _, lc in parts])
            wts = np.exp(lses - lses.max())
            if mistake == "equal_weights":
                wts = np.ones_like(wts)
            o[bh, i] = sum(wc * oc for wc, (oc, _) in zip(wts, parts)) / wts.sum()
    return o


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,tpc", [(1, 700, 2), (4, 300, 1), (16, 16, 1), (40, 20, 1), (130, 500, 3)])
def test_bound_holds_for_chunked_rect(Nq, Nk, tpc, causal):
    w = WORKLOADS["llama7b_layer_fwd"]
    xq, ds = make_fp8_inputs(w, seed=16, shape=(1, 1, Nq, 128))
    xk, dk = make_fp8_inputs(w, seed=17, shape=(1, 1, Nk, 128))
    desc = (ds[0], dk[1], dk[2])
    scale = 1 / math.sqrt(128)
    q = ofp8.dequantize(xq["q"].numpy(), desc[0]).reshape(1, Nq, 128)
    k = ofp8.dequantize(xk["k"].numpy(), desc[1]).reshape(1, Nk, 128)
    v = ofp8.dequantize(xk["v"].numpy(), desc[2]).reshape(1, Nk, 128)
    o_ref, _ = ofp8.fwd_fp8_rect(xq["q"], xk["k"], xk["v"], scale, desc, causal)
    bound = ofp8.error_bound(xq["q"], xk["k"], xk["v"], scale, desc, causal).reshape(1, Nq, 128)
    o_emu = _emulate_split(q, k, v, scale, causal, tpc)
    assert np.all(np.abs(o_emu - o_ref.reshape(1, Nq, 128)) <= bound)


def test_bound_catches_wrong_merge():
    w = WORKLOADS["llama7b_layer_fwd"]
    xq, ds = make_fp8_inputs(w, seed=18, shape=(1, 1, 2, 128))
    xk, dk = make_fp8_inputs(w, seed=19, shape=(1, 1, 640, 128))
    desc = (ds[0], dk[1], dk[2])
    scale = 1 / math.sqrt(128)
    q = ofp8.dequantize(xq["q"].numpy(), desc[0]).reshape(1, 2, 128)
    k = ofp8.dequantize(xk["k"].numpy(), desc[1]).reshape(1, 640, 128)
    v = ofp8.dequantize(xk["v"].numpy(), desc[2]).reshape(1, 640, 128)
    o_ref, _ = ofp8.fwd_fp8_rect(xq["q"], xk["k"], xk["v"], scale, desc, False)
    bound = ofp8.error_bound(xq["q"], xk["k"], xk["v"], scale, desc, False).reshape(1, 2, 128)
    o_bad = _emulate_split(q, k, v, scale, False, 2, mistake="equal_weights")
    assert np.any(np.abs(o_bad - o_ref.reshape(1, 2, 128)) > bound)
