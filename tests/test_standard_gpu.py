"""The materialised standard attention (attn_std_*) on the GPU against the
fp64 oracle.

The unfused baseline of the explainer's Step 2 ("Standard Attention"):
S = scale Q K^T is written to device memory in full, P = softmax(S) is
written in full, and O = P V reads P back.  Its outputs are checked like
the fused kernel's (O within the stated tolerance with fp32 output, the
16-bit output equal to the rounded fp32 one bit for bit, lse within 1e-3),
and the materialised S and P themselves against the NumPy brute force:
S within the rounding of an fp32 dot product, P within half an ulp of its
16-bit type plus the fp32 softmax's own rounding.  Every expected value
comes from the oracle; no GPU output is passed to it.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_40_amd as attn
import oracle
from exact_io_aware_40_amd import inputs
from oracle import brute
from tests._util import LSE_TOL, TOL, announce, f64, half_ulp, randn, report

pytestmark = pytest.mark.gpu
DEV = "cuda"


def s32(x):
    return float(np.float32(x))


def check_sp(q, k, scale, causal, s_gpu, p_gpu, dtype, tag):
    """Materialised S and P of the given heads ([n, N, d] fp64 inputs,
    [n, N, N] GPU results as fp64) against the brute force."""
    sc = s32(scale)
    s_ref = brute.scores(q, k, sc)
    d = q.shape[-1]
    # fp32 dot product of exactly representable products: at most d roundings
    # of the running sum, then one for the scale
    qk_abs = np.matmul(np.abs(q), np.swapaxes(np.abs(k), -1, -2))   # sum_c |q_ic k_jc|
    bound_s = abs(sc) * d * 2.0 ** -24 * qk_abs + 2.0 ** -23 * np.abs(s_ref) + 1e-30
    err_s = np.abs(s_gpu - s_ref)
    i = np.unravel_index(np.argmax(err_s - bound_s), err_s.shape)
    assert np.all(err_s <= bound_s), f"{tag} S: {err_s[i]:.3e} > {bound_s[i]:.3e} at {i}"
    v0 = np.zeros_like(q)
    _, _, p_ref = brute.fwd(q, k, v0, sc, causal)
    # half an ulp of the 16-bit type plus the fp32 softmax's rounding (well
    # below 1e-4 relative); masked entries must be exactly zero
    bound_p = half_ulp(p_ref, dtype) + 1e-4 * p_ref
    err_p = np.abs(p_gpu - p_ref)
    i = np.unravel_index(np.argmax(err_p - bound_p), err_p.shape)
    assert np.all(err_p <= bound_p), (f"{tag} P: {err_p[i]:.3e} > {bound_p[i]:.3e} at {i} "
                                      f"(gpu {p_gpu[i]:.6g}, oracle {p_ref[i]:.6g})")
    announce(f"{tag}: max|dS| {err_s.max():.2e}, max|dP| {err_p.max():.2e}")


def compare(q, k, v, causal, scale, tag, sp_heads=None):
    announce(f"std {tag} shape={tuple(q.shape)} {q.dtype} causal={causal} scale={scale}")
    B, H, N, d = q.shape
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    o32, lse, s, p = attn.forward_standard(qd, kd, vd, causal=causal, scale=scale,
                                           out_dtype=torch.float32, return_sp=True)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), s32(scale), causal)
    report(f"{tag} O(fp32 out)", f64(o32), o_ref, TOL[q.dtype])
    report(f"{tag} lse", f64(lse), lse_ref, LSE_TOL)
    heads = range(B * H) if sp_heads is None else sp_heads
    hs = list(heads)
    sel = lambda x, n: f64(x.reshape(B * H, N, n)[hs])  # noqa: E731
    check_sp(sel(q, d), sel(k, d), scale, causal, sel(s, N), sel(p, N), q.dtype, tag)
    o16, lse16 = attn.forward_standard(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o16, o32.to(q.dtype)), f"{tag}: 16-bit O is not the rounded fp32 O"
    assert torch.equal(lse16, lse)


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 100, 129, 256, 300])
def test_small_shapes(dtype, d, causal, N):
    seed = 4000 + N + d + (7 if causal else 0)
    q, k, v = (randn((2, 2, N, d), dtype, seed + i) for i in range(3))
    compare(q, k, v, causal, 1 / math.sqrt(d), f"small N={N}")


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_zero_and_negative_scale(scale):
    q, k, v = (randn((1, 2, 150, 64), torch.float16, 4100 + i) for i in range(3))
    for causal in (False, True):
        compare(q, k, v, causal, scale, f"scale={scale}")


@pytest.mark.parametrize("N", [4099, 4100])
def test_rows_streamed_twice(N):
    """Rows longer than 4096 scores go through the softmax that streams S
    twice (online maximum and sum, then P); N = 4099 also takes the
    element-wise loads and stores."""
    q, k, v = (randn((1, 1, N, 64), torch.bfloat16, 4200 + N + i) for i in range(3))
    for causal in (False, True):
        compare(q, k, v, causal, 0.125, f"long rows N={N}")


def test_outlier_scores():
    """Keys scaled by 8 (the 7B-layer workload's outliers): large scores in
    S, rows dominated by a few keys in P."""
    q, k, v = (randn((1, 2, 256, 128), torch.bfloat16, 4300 + i) for i in range(3))
    k[:, :, ::37] *= 8
    compare(q, k, v, True, 1 / math.sqrt(128), "outliers")


def test_matches_fused_forward():
    """Same inputs through the fused kernel and the materialised passes:
    both within the tolerance of each other (each is within it of the
    oracle, checked above)."""
    q, k, v = (randn((2, 3, 333, 128), torch.bfloat16, 4400 + i).to(DEV) for i in range(3))
    announce("std vs fused")
    for causal in (False, True):
        o_f, l_f = attn.forward(q, k, v, causal=causal, out_dtype=torch.float32)
        o_s, l_s = attn.forward_standard(q, k, v, causal=causal, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert float((o_f - o_s).abs().max()) <= TOL[q.dtype]
        assert float((l_f - l_s).abs().max()) <= LSE_TOL


def test_workload_full_size():
    """The GPT-2-medium-shaped workload (the shape of the pages' standard
    attention measurement) at full size: sampled O rows against the oracle,
    whole heads' S and P against the brute force."""
    w = inputs.WORKLOADS["gpt2_medium_fwd"]
    t = inputs.make_inputs(w)
    scale = 1 / math.sqrt(w.d)
    announce(f"std workload {w.describe()}")
    qd, kd, vd = (t[n].to(DEV) for n in ("q", "k", "v"))
    o32, lse, s, p = attn.forward_standard(qd, kd, vd, causal=w.causal, scale=scale,
                                           out_dtype=torch.float32, return_sp=True)
    torch.cuda.synchronize()
    BH, N, d = w.B * w.H, w.N, w.d
    rows = np.random.default_rng(9).choice(BH * N, 400, replace=False)
    rows = np.concatenate([rows, [0, N - 1, BH * N - 1]])
    o_ref, lse_ref = oracle.fwd(f64(t["q"]), f64(t["k"]), f64(t["v"]), s32(scale), w.causal,
                                rows=rows)
    report("full O(fp32 out)", f64(o32).reshape(BH * N, d)[rows], o_ref, TOL[w.torch_dtype])
    report("full lse", f64(lse).reshape(BH * N)[rows], lse_ref, LSE_TOL)
    hs = [0, 517, BH - 1]
    sel = lambda x, n: f64(x.reshape(BH, N, n)[hs])  # noqa: E731
    check_sp(sel(t["q"], d), sel(t["k"], d), scale, w.causal, sel(s, N), sel(p, N),
             w.torch_dtype, "full")
