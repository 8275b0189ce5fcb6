"""FP8 (E4M3) forward and decode step on the GPU (attn_fwd_fp8,
attn_fwd_decode_fp8) against the CPU oracle.

The oracle is exact attention on the decoded, descaled inputs; the kernel
rounds P to E4M3 for the P.V product, so each fp32 output element must lie
within the oracle's element-wise bound for that rounding (oracle.fp8), lse
within LSE_TOL, and a 16-bit output must be exactly the fp32 output rounded
to nearest even.  Cases: ragged tails and a single row, both masks, inputs
with outlier keys, every output type, both tensor types that carry the
codes, a negative scale, and sampled rows of the seven-billion-parameter
layer's full shape in the launch the benchmark times.  The decode step
(Nq queries against an Nk-key cache, keys split in chunks and merged) is
held to the same bound, including rows that see no key (O = 0, lse = -inf),
and at the benchmark's 16 x 32 x 16384-key cache.
"""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_40_amd as attn
from exact_io_aware_40_amd.inputs import WORKLOADS, make_fp8_inputs
from oracle import fp8 as ofp8
from tests._util import LSE_TOL, _emit, announce, f64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def s32(x):
    return float(np.float32(x))


def check_bound(name, got, ref, bound):
    err = np.abs(got - ref)
    ratio = err / bound
    i = np.unravel_index(np.argmax(ratio), ratio.shape)
    _emit(f"[err] {name}: max|gpu-oracle| = {err.max():.3e}, max err/bound = {ratio.max():.3f}")
    assert ratio.max() <= 1.0, (f"{name}: |gpu-oracle| = {err[i]:.3e} > bound {bound[i]:.3e} at {i} "
                                f"(gpu {got[i]:.6f}, oracle {ref[i]:.6f})")


def run_fp8(x, ds, causal, scale, tag, out_dtype=torch.bfloat16, rows=None, heads=None,
            as_float8=False):
    """x: uint8 code tensors [B, H, N, d] on the CPU.  rows: flattened row ids
    (b H + h) N + i to check (all rows when None); heads: the (b H + h) ids
    those rows lie in, so that the oracle decodes only those heads."""
    announce(f"fp8 {tag} shape={tuple(x['q'].shape)} causal={causal} out={out_dtype}")
    dev = {n: x[n].to(DEV) for n in "qkv"}
    if as_float8:
        dev = {n: t.view(torch.float8_e4m3fn) for n, t in dev.items()}
    o32, lse32 = attn.forward_fp8(dev["q"], dev["k"], dev["v"], descale=ds, causal=causal,
                                  scale=scale, out_dtype=torch.float32)
    if out_dtype != torch.float32:
        o, lse = attn.forward_fp8(dev["q"], dev["k"], dev["v"], descale=ds, causal=causal,
                                  scale=scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    if out_dtype != torch.float32:
        assert torch.equal(o, o32.to(out_dtype)), f"{tag}: 16-bit O is not RNE(fp32 O)"
        assert torch.equal(lse, lse32)
    B, H, N, d = x["q"].shape
    codes = {n: x[n].numpy().reshape(B * H, N, d) for n in "qkv"}
    go, gl = o32.view(B * H * N, d), lse32.view(B * H * N)
    if rows is None:
        sel_rows = None
        got_o, got_l = f64(go), f64(gl)
    else:
        # oracle over the listed heads only; rows renumbered within them
        heads = np.asarray(heads)
        codes = {n: c[heads] for n, c in codes.items()}
        pos = {h: j for j, h in enumerate(heads.tolist())}
        sel_rows = np.array([pos[r // N] * N + r % N for r in rows.tolist()], dtype=np.int64)
        idx = torch.from_numpy(np.asarray(rows, dtype=np.int64)).to(DEV)
        got_o, got_l = f64(go[idx]), f64(gl[idx])
    sc = s32(scale)
    o_ref, lse_ref = ofp8.fwd_fp8(codes["q"], codes["k"], codes["v"], sc, ds, causal, rows=sel_rows)
    bound = ofp8.error_bound(codes["q"], codes["k"], codes["v"], sc, ds, causal, rows=sel_rows)
    o_ref, bound = o_ref.reshape(-1, d), bound.reshape(-1, d)
    check_bound(f"{tag} O(fp32 out)", got_o, o_ref, bound)
    err_l = np.abs(got_l - lse_ref.reshape(-1)).max()
    _emit(f"[err] {tag} lse: max|gpu-oracle| = {err_l:.3e} (tol {LSE_TOL:.1e})")
    assert err_l <= LSE_TOL


@pytest.mark.parametrize("outliers", [False, True])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 64, 200, 777])
def test_fp8_small(N, causal, outliers):
    w = WORKLOADS["llama7b_layer_fwd" if outliers else "long_context_fwd"]
    x, ds = make_fp8_inputs(w, seed=300 + N, shape=(1, 2, N, 128))
    run_fp8(x, ds, causal, 1 / math.sqrt(128), f"N={N} outliers={outliers}")


@pytest.mark.parametrize("out_dtype", [torch.float16, torch.float32])
def test_fp8_output_types(out_dtype):
    x, ds = make_fp8_inputs(WORKLOADS["llama7b_layer_fwd"], seed=310, shape=(2, 2, 300, 128))
    run_fp8(x, ds, True, 1 / math.sqrt(128), f"out={out_dtype}", out_dtype=out_dtype)


def test_fp8_float8_tensors_same_as_bytes():
    x, ds = make_fp8_inputs(WORKLOADS["long_context_fwd"], seed=320, shape=(1, 2, 333, 128))
    run_fp8(x, ds, True, 1 / math.sqrt(128), "float8 tensors", as_float8=True)
    dev = {n: x[n].to(DEV) for n in "qkv"}
    a = attn.forward_fp8(dev["q"], dev["k"], dev["v"], descale=ds, causal=True)
    b = attn.forward_fp8(*(dev[n].view(torch.float8_e4m3fn) for n in "qkv"), descale=ds, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("scale", [-0.05, 0.3])
def test_fp8_scale_cases(scale):
    x, ds = make_fp8_inputs(WORKLOADS["long_context_fwd"], seed=330, shape=(1, 2, 260, 128))
    run_fp8(x, ds, False, scale, f"scale={scale}")


def test_fp8_descales_fold_into_scores_and_output():
    """Halving q's descale while doubling scale, and scaling v's descale,
    changes nothing but O's scale."""
    x, ds = make_fp8_inputs(WORKLOADS["long_context_fwd"], seed=340, shape=(1, 2, 200, 128))
    dev = {n: x[n].to(DEV) for n in "qkv"}
    o1, l1 = attn.forward_fp8(dev["q"], dev["k"], dev["v"], descale=ds, causal=True, scale=0.1,
                              out_dtype=torch.float32)
    ds2 = (ds[0] / 2, ds[1], ds[2] * 4)
    o2, l2 = attn.forward_fp8(dev["q"], dev["k"], dev["v"], descale=ds2, causal=True, scale=0.2,
                              out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(l1, l2)
    assert torch.equal(o1 * 4, o2)


def test_fp8_llama7b_layer_sampled():
    """The seven-billion-parameter layer's full shape (B=4 H=32 N=4096
    d=128, causal, 1% outlier K rows), one launch; sampled rows of six
    heads, including the first and last row of every query block, checked."""
    w = WORKLOADS["llama7b_layer_fwd"]
    x, ds = make_fp8_inputs(w)
    B, H, N = w.B, w.H, w.N
    rng = np.random.default_rng(9)
    heads = np.sort(rng.choice(B * H, size=6, replace=False))
    rows = []
    for hd in heads.tolist():
        rr = {0, 1, 127, 128, 2047, 2048, N - 2, N - 1}
        rr |= set(rng.choice(N, size=24, replace=False).tolist())
        rows += [hd * N + r for r in sorted(rr)]
    run_fp8(x, ds, True, 1 / math.sqrt(w.d), "llama7b layer", rows=np.array(rows), heads=heads)


def run_decode_fp8(x, ds, causal, nsplit, tag, out_dtype=torch.bfloat16, heads=None):
    """x: uint8 codes q [B, H, Nq, d], k, v [B, H, Nk, d] on the CPU.  heads:
    the (b H + h) ids whose rows are checked (all when None)."""
    B, H, Nq, d = x["q"].shape
    Nk = x["k"].shape[2]
    announce(f"fp8 decode {tag} B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} nsplit={nsplit} out={out_dtype}")
    q, k, v = (x[n].to(DEV) for n in "qkv")
    o32, lse32 = attn.forward_decode_fp8(q, k, v, descale=ds, causal=causal, nsplit=nsplit,
                                         out_dtype=torch.float32)
    if out_dtype != torch.float32:
        o, lse = attn.forward_decode_fp8(q, k, v, descale=ds, causal=causal, nsplit=nsplit,
                                         out_dtype=out_dtype)
    torch.cuda.synchronize()
    if out_dtype != torch.float32:
        assert torch.equal(o, o32.to(out_dtype)), f"{tag}: 16-bit O is not RNE(fp32 O)"
        assert torch.equal(lse, lse32)
    hs = np.arange(B * H) if heads is None else np.asarray(heads)
    cq = x["q"].numpy().reshape(B * H, Nq, d)[hs]
    ck = x["k"].numpy().reshape(B * H, Nk, d)[hs]
    cv = x["v"].numpy().reshape(B * H, Nk, d)[hs]
    idx = torch.from_numpy(hs.astype(np.int64)).to(DEV)
    got_o = f64(o32.view(B * H, Nq, d)[idx])
    got_l = f64(lse32.view(B * H, Nq)[idx])
    sc = s32(1 / math.sqrt(d))
    o_ref, lse_ref = ofp8.fwd_fp8_rect(cq, ck, cv, sc, ds, causal)
    bound = ofp8.error_bound(cq, ck, cv, sc, ds, causal)
    check_bound(f"{tag} O(fp32 out)", got_o.reshape(-1, d), o_ref.reshape(-1, d), bound.reshape(-1, d))
    lr, lg = lse_ref.reshape(-1), got_l.reshape(-1)
    assert np.array_equal(np.isfinite(lr), np.isfinite(lg)), f"{tag}: rows without keys differ"
    fin = np.isfinite(lr)
    assert np.all(lg[~fin] == -np.inf) and np.all(got_o.reshape(-1, d)[~fin] == 0)
    err_l = float(np.abs(lg[fin] - lr[fin]).max()) if fin.any() else 0.0
    _emit(f"[err] {tag} lse: max|gpu-oracle| = {err_l:.3e} (tol {LSE_TOL:.1e})")
    assert err_l <= LSE_TOL


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk,nsplit", [(1, 1, 1), (1, 700, 8), (4, 300, 3), (16, 2000, 16),
                                          (130, 500, 2), (40, 20, 2), (3, 64, 64)])
def test_fp8_decode_small(Nq, Nk, nsplit, causal):
    from exact_io_aware_40_amd.inputs import make_decode_fp8_inputs
    x, ds = make_decode_fp8_inputs(2, 2, Nq, Nk, 128, seed=400 + Nq + Nk)
    run_decode_fp8(x, ds, causal, nsplit, f"Nq={Nq} Nk={Nk}")


def test_fp8_decode_output_types():
    from exact_io_aware_40_amd.inputs import make_decode_fp8_inputs
    x, ds = make_decode_fp8_inputs(1, 3, 5, 900, 128, seed=420)
    for od in (torch.float16, torch.float32):
        run_decode_fp8(x, ds, True, 4, f"out={od}", out_dtype=od)


def test_fp8_decode_equals_square_when_nq_is_nk():
    """Nq = Nk with one chunk: the split kernel's partial is the whole
    softmax, so the merged result equals attn_fwd_fp8's within the merge's
    fp32 rounding."""
    x, ds = make_fp8_inputs(WORKLOADS["long_context_fwd"], seed=430, shape=(1, 2, 300, 128))
    q, k, v = (x[n].to(DEV) for n in "qkv")
    o1, l1 = attn.forward_fp8(q, k, v, descale=ds, causal=True, out_dtype=torch.float32)
    o2, l2 = attn.forward_decode_fp8(q, k, v, descale=ds, causal=True, nsplit=1, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() <= 1e-5
    assert (l1 - l2).abs().max().item() <= 1e-5


def test_fp8_decode_cache_16k_sampled():
    """The decode step the benchmark times (B=16 H=32, one query against a
    16384-key cache, 8 chunks), with six heads checked against the oracle."""
    from exact_io_aware_40_amd.inputs import make_decode_fp8_inputs
    B, H, Nq, Nk = 16, 32, 1, 16384
    x, ds = make_decode_fp8_inputs(B, H, Nq, Nk, 128, seed=12)
    heads = np.sort(np.random.default_rng(3).choice(B * H, size=6, replace=False))
    run_decode_fp8(x, ds, True, 8, "16k cache", heads=heads)
