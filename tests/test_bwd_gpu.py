"""GPU parity of the backward kernels against the fp64 oracle.

Every expected value comes from the oracle alone; no GPU output is ever
passed to it.  Three checks per case:
  * the pipeline with fp32 outputs (GPU forward, then GPU backward from its
    o and lse) against the plain definition, within the stated tolerance;
  * the backward's contract with 16-bit outputs: the GPU backward is given
    the oracle's own o rounded to the input type and its lse in fp32, and
    the oracle forms D from that same o;
  * the whole 16-bit pipeline (GPU forward, then GPU backward) against the
    plain definition, with an allowance for the rounded o derived from
    oracle quantities only.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_40_amd as attn
import oracle
from exact_io_aware_40_amd import inputs
from tests._util import (TOL, announce, f64, randn, report, report_rounded, rounded,
                         stored_o_allowance)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def s32(x):
    return float(np.float32(x))


def gpu_fwd_bwd(q, k, v, dO, causal, scale, out_dtype=None):
    """The pipeline as a user runs it: forward, then backward from its o and lse."""
    qd, kd, vd, gd = (t.to(DEV) for t in (q, k, v, dO))
    o, lse = attn.forward(qd, kd, vd, causal=causal, scale=scale, out_dtype=out_dtype)
    dq, dk, dv = attn.backward(qd, kd, vd, o, lse, gd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return dq, dk, dv


def gpu_bwd_from(q, k, v, dO, o, lse, causal, scale):
    """The GPU backward alone, from a given stored o and lse (CPU tensors)."""
    qd, kd, vd, gd, od, ld = (t.to(DEV) for t in (q, k, v, dO, o, lse))
    g = attn.backward(qd, kd, vd, od, ld, gd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return g


def check_16bit(q, k, v, dO, causal, scale, tag, heads=None):
    """The 16-bit checks on the heads `heads` (flattened b*H + h; None for
    all); the oracle runs on those heads only.  Returns the oracle's fp64
    gradients of those heads, [n_heads, N, d] (or q's shape for all)."""
    tol, dt = TOL[q.dtype], q.dtype
    B, H, N, d = q.shape
    if heads is None:
        part = lambda x: x  # noqa: E731
    else:
        part = lambda x: x.reshape(B * H, N, d)[heads].reshape(1, len(heads), N, d)  # noqa: E731
    Q, K, V, G = (f64(part(x)) for x in (q, k, v, dO))
    o_ref, lse_ref, rq, rk, rv = oracle.bwd(Q, K, V, G, s32(scale), causal)
    # the contract: a stored o (the oracle's, rounded to the input type) and
    # its lse, given to both sides; D_i = dO_i . o_i on both
    o_st = rounded(o_ref, dt)
    lse_st = torch.from_numpy(lse_ref).float()
    hq, hk, hv = gpu_bwd_from(part(q), part(k), part(v), part(dO), o_st, lse_st, causal, scale)
    _, _, sq, sk, sv = oracle.bwd(Q, K, V, G, s32(scale), causal, o_in=f64(o_st))
    report_rounded(f"{tag} dq(stored o)", f64(hq), sq, tol, dt)
    report_rounded(f"{tag} dk(stored o)", f64(hk), sk, tol, dt)
    report_rounded(f"{tag} dv(stored o)", f64(hv), sv, tol, dt)
    del hq, hk, hv
    # the whole 16-bit pipeline, at the full launch, against the plain definition
    hq, hk, hv = gpu_fwd_bwd(q, k, v, dO, causal, scale)
    aq, ak = stored_o_allowance(Q, K, G, o_ref, lse_ref, s32(scale), causal, dt)
    report_rounded(f"{tag} dq(pipeline)", f64(part(hq)), rq, tol, dt, extra=aq)
    report_rounded(f"{tag} dk(pipeline)", f64(part(hk)), rk, tol, dt, extra=ak)
    report_rounded(f"{tag} dv(pipeline)", f64(part(hv)), rv, tol, dt)
    return rq, rk, rv


def compare(q, k, v, dO, causal, scale, tag):
    """fp32 outputs meet the stated tolerance element by element against the
    plain definition; then the 16-bit checks (module docstring)."""
    announce(f"bwd {tag} shape={tuple(q.shape)} {q.dtype} causal={causal} scale={scale}")
    tol = TOL[q.dtype]
    rq, rk, rv = check_16bit(q, k, v, dO, causal, scale, tag)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, dO, causal, scale, out_dtype=torch.float32)
    report(f"{tag} dq(fp32 out)", f64(dq), rq, tol)
    report(f"{tag} dk(fp32 out)", f64(dk), rk, tol)
    report(f"{tag} dv(fp32 out)", f64(dv), rv, tol)
    return dq, dk, dv


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 129, 200, 256])
def test_small_shapes(dtype, d, causal, N):
    seed = 2000 + N + d + (7 if causal else 0)
    q, k, v, dO = (randn((2, 2, N, d), dtype, seed + i) for i in range(4))
    compare(q, k, v, dO, causal, 1 / math.sqrt(d), f"small N={N}")


@pytest.mark.parametrize("causal", [False, True])
def test_several_blocks(causal):
    q, k, v, dO = (randn((1, 2, 555, 128), torch.bfloat16, 300 + i) for i in range(4))
    compare(q, k, v, dO, causal, 1 / math.sqrt(128), "multi-block")


@pytest.mark.parametrize("scale", [0.0, -0.3])
def test_zero_and_negative_scale(scale):
    q, k, v, dO = (randn((1, 2, 150, 64), torch.float16, 310 + i) for i in range(4))
    for causal in (False, True):
        compare(q, k, v, dO, causal, scale, f"scale={scale}")


def test_single_key_closed_form():
    """N = 1: P = 1, so dq = dk = 0 and dv = dO.  dv is exact; dq and dk are
    scale * (dO.v - D) k with D = dO.o, two fp32 dot products of the same
    vectors summed in different orders, so they vanish up to fp32 rounding."""
    q, k, v, dO = (randn((3, 2, 1, 128), torch.bfloat16, 320 + i) for i in range(4))
    announce("bwd N=1")
    for od in (None, torch.float32):
        dq, dk, dv = gpu_fwd_bwd(q, k, v, dO, True, 0.1, out_dtype=od)
        assert float(dq.abs().max()) <= 1e-5 and float(dk.abs().max()) <= 1e-5
        assert torch.equal(dv.cpu().to(torch.bfloat16), dO)


def test_gradient_invariants():
    """Key gradients sum to ~0 per head; value gradients sum to sum(dO)."""
    q, k, v, dO = (randn((2, 2, 640, 128), torch.bfloat16, 330 + i) for i in range(4))
    announce("bwd invariants")
    dq, dk, dv = gpu_fwd_bwd(q, k, v, dO, True, 1 / math.sqrt(128))
    sk = dk.double().sum(dim=2).abs().max().item()
    sv = (dv.double().sum(dim=2) - dO.to(DEV).double().sum(dim=2)).abs().max().item()
    # bounded by 1% of the summed magnitudes (the sums cancel; rounding does not)
    bk = 1e-2 * dk.double().abs().sum(dim=2).max().item()
    bv = 1e-2 * dv.double().abs().sum(dim=2).max().item()
    assert sk <= bk and sv <= bv, (sk, bk, sv, bv)


@pytest.mark.parametrize("causal", [False, True])
def test_split_calls_match_attn_bwd(causal):
    """attn_bwd_dq then attn_bwd_dkdv give exactly what attn_bwd gives."""
    dt = torch.bfloat16
    q, k, v, dO = (randn((1, 3, 300, 128), dt, 350 + i).to(DEV) for i in range(4))
    announce(f"split backward causal={causal}")
    o, lse = attn.forward(q, k, v, causal=causal)
    dq, dk, dv = attn.backward(q, k, v, o, lse, dO, causal=causal)
    B, H, N, d = q.shape
    code = attn.ATTN_BF16
    nbytes = attn.attn_bwd_workspace_size(B, H, N, d, code)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    dq2, dk2, dv2 = (torch.full_like(q, float("nan")) for _ in range(3))
    sp = torch.cuda.current_stream().cuda_stream
    sc = 1 / math.sqrt(d)
    assert attn.attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dO.data_ptr(),
                            lse.data_ptr(), dq2.data_ptr(), ws.data_ptr(), nbytes, B, H, N, d, sc,
                            int(causal), code, code, sp) == 0
    assert attn.attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dO.data_ptr(),
                              dk2.data_ptr(), dv2.data_ptr(), ws.data_ptr(), nbytes, B, H, N, d,
                              sc, int(causal), code, code, sp) == 0
    torch.cuda.synchronize()
    assert torch.equal(dq, dq2) and torch.equal(dk, dk2) and torch.equal(dv, dv2)


def test_repeatable_bitwise():
    q, k, v, dO = (randn((1, 4, 700, 128), torch.bfloat16, 340 + i) for i in range(4))
    announce("bwd repeatability")
    a = gpu_fwd_bwd(q, k, v, dO, True, 0.1)
    b = gpu_fwd_bwd(q, k, v, dO, True, 0.1)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_workload_full_size():
    """The backward workload at full size; the oracle checks whole heads."""
    w = inputs.WORKLOADS["recompute_bwd"]
    t = inputs.make_inputs(w)
    scale = 1 / math.sqrt(w.d)
    announce(f"bwd workload {w.describe()}")
    BH = w.B * w.H
    heads = [0, 19, 37, 64, 90, 101, 117, BH - 1]
    sel = lambda x: f64(x.reshape(BH, w.N, w.d)[heads]).reshape(1, len(heads), w.N, w.d)  # noqa: E731
    tol = TOL[w.torch_dtype]
    rq, rk, rv = check_16bit(t["q"], t["k"], t["v"], t["dO"], w.causal, scale, "full", heads=heads)
    dq, dk, dv = gpu_fwd_bwd(t["q"], t["k"], t["v"], t["dO"], w.causal, scale,
                             out_dtype=torch.float32)
    for g in (dq, dk, dv):
        assert bool(torch.isfinite(g).all())
    report("full dq(fp32 out)", sel(dq), rq, tol)
    report("full dk(fp32 out)", sel(dk), rk, tol)
    report("full dv(fp32 out)", sel(dv), rv, tol)


@pytest.mark.parametrize("B,H,N,d,dtype", [
    (8, 16, 1153, 64, torch.bfloat16),     # 128 heads: groups of 4, 10 query blocks each
    (2, 12, 2200, 128, torch.float16),     # 24 heads: groups of 3, ragged tail
    (1, 16, 3000, 64, torch.bfloat16),     # 16 heads: groups of 2
    (1, 8, 2500, 128, torch.bfloat16),     # 8 heads: one head per XCD
    (1, 13, 1500, 64, torch.float16),      # 13 heads: pairs of query blocks
])
def test_many_blocks_causal(B, H, N, d, dtype):
    """Causal grids of several rounds of workgroups over the dq kernel's two
    mappings (head counts that are and are not multiples of 8): whole heads
    spread over the grid against the oracle, every gradient finite."""
    tag = f"many blocks B={B} H={H} N={N} d={d}"
    announce(f"bwd {tag} {dtype} causal")
    q, k, v, dO = (randn((B, H, N, d), dtype, 700 + N + d + i) for i in range(4))
    scale = 1 / math.sqrt(d)
    BH = B * H
    heads = sorted({0, 1, BH // 3, BH // 2, (2 * BH) // 3, BH - 1})
    sel = lambda x: f64(x.reshape(BH, N, d)[heads]).reshape(1, len(heads), N, d)  # noqa: E731
    tol = TOL[dtype]
    rq, rk, rv = check_16bit(q, k, v, dO, True, scale, tag, heads=heads)
    dq, dk, dv = gpu_fwd_bwd(q, k, v, dO, True, scale, out_dtype=torch.float32)
    for g in (dq, dk, dv):
        assert bool(torch.isfinite(g).all())
    report(f"{tag} dq(fp32 out)", sel(dq), rq, tol)
    report(f"{tag} dk(fp32 out)", sel(dk), rk, tol)
    report(f"{tag} dv(fp32 out)", sel(dv), rv, tol)


@pytest.mark.parametrize("B,H,N,d", [(8, 16, 1153, 64), (2, 12, 2200, 128), (1, 16, 3000, 64),
                                     (1, 8, 2500, 128), (1, 13, 1500, 64)])
@pytest.mark.parametrize("out_f32", [False, True])
def test_every_output_written(B, H, N, d, out_f32):
    """Causal grids over the forward's and dq's head groups (1 to 4 heads)
    and pairs: o, lse, dq, dk and dv start as NaN and come out finite in
    every element, so every (head, block) of every grid was computed."""
    announce(f"every output written B={B} H={H} N={N} d={d} fp32 out={out_f32}")
    dt = torch.bfloat16
    q, k, v, dO = (randn((B, H, N, d), dt, 900 + N + i).to(DEV) for i in range(4))
    code = attn.ATTN_BF16
    oc = attn.ATTN_F32 if out_f32 else code
    odt = torch.float32 if out_f32 else dt
    o, dq, dk, dv = (torch.full((B, H, N, d), float("nan"), dtype=odt, device=DEV) for _ in range(4))
    lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device=DEV)
    sp = torch.cuda.current_stream().cuda_stream
    sc = 1 / math.sqrt(d)
    assert attn.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         B, H, N, d, sc, 1, code, oc, sp) == 0
    nbytes = attn.attn_bwd_workspace_size(B, H, N, d, code)
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device=DEV)
    assert attn.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dO.data_ptr(),
                         lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), ws.data_ptr(),
                         nbytes, B, H, N, d, sc, 1, code, oc, sp) == 0
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        bad = (~torch.isfinite(t)).sum().item()
        assert bad == 0, (name, bad)


def test_many_heads():
    """4,097 (batch, head) pairs of 70 rows (a prime-ish count of workgroups
    for both kernels): every gradient element against the oracle."""
    q, k, v, dO = (randn((17, 241, 70, 64), torch.bfloat16, 360 + i) for i in range(4))
    for causal in (False, True):
        compare(q, k, v, dO, causal, 0.125, "many heads")
