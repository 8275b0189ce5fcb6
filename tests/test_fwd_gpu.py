"""GPU parity of the forward kernel against the fp64 oracle.

Every case runs the HIP kernel through the C ABI (via the Python binding)
and compares with the oracle on the same rounded inputs: element by element
at sizes the oracle finishes quickly, on sampled rows (plus whole-tensor
properties) at the full workload sizes.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import exact_io_aware_40_amd as attn
from exact_io_aware_40_amd import inputs
from tests._util import LSE_TOL, TOL, announce, f64, oracle_fwd, randn, report

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEV = "cuda"


def s32(x):
    """The fp32 value the kernel receives."""
    return float(np.float32(x))


def run_and_compare(q, k, v, causal, scale, tag):
    """fp32 outputs meet the stated tolerance element by element; outputs
    in the input type are exactly those fp32 results rounded to nearest even."""
    announce(f"fwd {tag} shape={tuple(q.shape)} {q.dtype} causal={causal} scale={scale}")
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o32, lse32 = attn.forward(qd, kd, vd, causal=causal, scale=scale, out_dtype=torch.float32)
    o, lse = attn.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle_fwd(q, k, v, s32(scale), causal)
    tol = TOL[q.dtype]
    report(f"{tag} O(fp32 out)", f64(o32), o_ref, tol)
    report(f"{tag} lse", f64(lse32), lse_ref, LSE_TOL)
    assert torch.equal(o, o32.to(q.dtype)), f"{tag}: 16-bit O is not RNE(fp32 O)"
    assert torch.equal(lse, lse32)
    return o, lse


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 17, 64, 129, 255, 256, 300])
def test_small_shapes(dtype, d, causal, N):
    B, H = 2, 3
    seed = 1000 + N + d + (7 if causal else 0)
    q, k, v = (randn((B, H, N, d), dtype, seed + i) for i in range(3))
    run_and_compare(q, k, v, causal, 1 / math.sqrt(d), f"small N={N}")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("causal", [False, True])
def test_several_tiles_and_blocks(dtype, causal):
    """Several query blocks and K/V tiles per head, ragged tail."""
    q, k, v = (randn((1, 2, 777, 128), dtype, 50 + i) for i in range(3))
    run_and_compare(q, k, v, causal, 1 / math.sqrt(128), "multi-block")


@pytest.mark.parametrize("N", [640, 641, 1024])
def test_causal_block_pairs(N):
    """Causal workgroups take a heavy and a light query block of one head:
    an odd number of blocks leaves the middle one alone (640, 641), an even
    number pairs them all (1024); several heads and batches check the mapping
    from workgroup to (batch, head, pair)."""
    q, k, v = (randn((2, 3, N, 64), torch.bfloat16, 130 + i) for i in range(3))
    run_and_compare(q, k, v, True, 1 / math.sqrt(64), f"pairs N={N}")


@pytest.mark.parametrize("B,H,N", [(2, 4, 300), (2, 8, 257), (4, 8, 129), (1, 24, 200), (3, 16, 385)])
def test_causal_head_groups(B, H, N):
    """With B*H a multiple of 8 the causal grid runs one query block per
    workgroup in each XCD's heaviest-first order over groups of heads
    (groups of 1, 2, 4, 3 and 3 heads here, ragged tails): every (batch,
    head, block) is computed exactly once, and the result equals the paired
    grid's (the same per-block computation) bit for bit."""
    q, k, v = (randn((B, H, N, 64), torch.bfloat16, 140 + N + i) for i in range(3))
    o, lse = run_and_compare(q, k, v, True, 1 / math.sqrt(64), f"head groups B={B} H={H}")
    # the same heads plus one more (B*H + 1, not a multiple of 8) take the paired grid
    q2, k2, v2 = (torch.cat([x.reshape(B * H, N, 64), x.reshape(B * H, N, 64)[:1]]).reshape(1, B * H + 1, N, 64)
                  for x in (q, k, v))
    o2, lse2 = attn.forward(q2.to(DEV), k2.to(DEV), v2.to(DEV), causal=True, scale=1 / math.sqrt(64))
    torch.cuda.synchronize()
    assert torch.equal(o2[0, :B * H].reshape(o.shape), o)
    assert torch.equal(lse2[0, :B * H].reshape(lse.shape), lse)


@pytest.mark.parametrize("scale", [0.0, -0.2, 0.9])
def test_zero_negative_and_large_scale(scale):
    q, k, v = (randn((1, 2, 200, 64), torch.float16, 60 + i) for i in range(3))
    for causal in (False, True):
        run_and_compare(q, k, v, causal, scale, f"scale={scale}")


def test_outlier_scores():
    """Scores scaled far apart stress the running-max rescale."""
    dt = torch.bfloat16
    q, k, v = (randn((1, 4, 512, 128), dt, 70 + i) for i in range(3))
    kf = k.view(-1, 128)
    rows = torch.randperm(kf.shape[0], generator=torch.Generator().manual_seed(5))[:40]
    kf[rows] *= 8
    for causal in (False, True):
        run_and_compare(q, k, v, causal, 1 / math.sqrt(128), "outliers")


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_reference_moves_and_bound(dtype, d, causal):
    """Scores placed in binades around the exponent reference's bound (2^32
    for bf16 operands, 2^15 for fp16; one K/V tile is 8 KiB of keys):
    tile 0 all zero (the first tile moves the reference to 0); in tile 2
    the keys held by one lane half sit one binade below the bound, so those
    lanes' sums of P exceed it while no score asks the reference to move;
    tile 4 has one key one binade past the bound (it must move); tile 6 a
    whole tile a further 27 binades up (under the bf16 bound, whose lane
    sums stay below 2^32; past the fp16 one, a second move).  The other
    keys are N(0,1) / 4.  q = e_0 and scale = 1 make the score of key j its
    k_j[0]."""
    tau = 32.0 if dtype == torch.bfloat16 else 15.0
    bc = 8192 // (2 * d)                     # keys per tile
    N = 8 * bc
    log2e = 1.0 / math.log(2.0)
    B, H = 1, 2
    k = randn((B, H, N, d), torch.float32, 4100 + d, scale=0.25)
    q = torch.zeros((B, H, N, d))
    q[..., 0] = 1.0
    k[..., 0:bc, 0] = 0.0
    j = torch.arange(2 * bc, 3 * bc)
    k[..., j[(j % 8) < 4], 0] = (tau - 1.0) / log2e    # lane half 0 of every 32-key block
    k[..., 4 * bc + 5, 0] = (tau + 1.0) / log2e
    k[..., 6 * bc:7 * bc, 0] = (tau + 1.0 + 27.0) / log2e
    v = randn((B, H, N, d), torch.float32, 4200 + d)
    q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    run_and_compare(q, k, v, causal, 1.0, f"reference bound d={d}")


def test_page_example_probe():
    """Explainer Step 4's eight scores through the kernel: q = e0,
    k_j = x_j e0, one-hot v_j = e_j, scale 1 -> each row of O is the
    softmax of the scores, shown on the page to two decimals."""
    with open(os.path.join(GOLDEN, "online_softmax_8.json")) as f:
        g = json.load(f)
    N, d = 8, 64
    q = torch.zeros((1, 1, N, d), dtype=torch.float16)
    q[..., 0] = 1
    k = torch.zeros((1, 1, N, d), dtype=torch.float16)
    k[0, 0, :, 0] = torch.tensor(g["scores"], dtype=torch.float16)
    v = torch.zeros((1, 1, N, d), dtype=torch.float16)
    v[0, 0, :, :N] = torch.eye(N, dtype=torch.float16)
    o, lse = run_and_compare(q, k, v, False, 1.0, "page probe")
    row = f64(o)[0, 0, 0, :N]
    np.testing.assert_array_equal(np.round(row, 2), np.array(g["full_softmax_2dp"]))


@pytest.mark.parametrize("dtype", [torch.float16, torch.bfloat16])
@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(dtype, causal):
    q, k = (randn((2, 2, 333, 128), dtype, 80 + i, scale=2.0) for i in range(2))
    v = randn((2, 2, 333, 128), dtype, 82)
    v[..., 0] = 1
    announce(f"ones column {dtype} causal={causal}")
    o, _ = attn.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=causal)
    err = (o[..., 0].float() - 1).abs().max().item()
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("causal", [False, True])
def test_equal_scores_mean_v(causal):
    dt = torch.bfloat16
    q = torch.zeros((1, 2, 300, 64), dtype=dt)
    k, v = (randn((1, 2, 300, 64), dt, 90 + i) for i in range(2))
    o, lse = run_and_compare(q, k, v, causal, 0.125, "Q=0")
    n = np.arange(1, 301) if causal else np.full(300, 300)
    assert np.abs(f64(lse) - np.log(n)).max() <= 1e-5


def test_causal_row_zero_is_v0_bitwise():
    for dt in (torch.float16, torch.bfloat16):
        q, k, v = (randn((2, 2, 130, 128), dt, 95 + i) for i in range(3))
        announce(f"causal row 0 {dt}")
        o, _ = attn.forward(q.to(DEV), k.to(DEV), v.to(DEV), causal=True)
        assert torch.equal(o[:, :, 0].cpu(), v[:, :, 0])


def test_repeatable_bitwise():
    q, k, v = (randn((2, 4, 1000, 128), torch.bfloat16, 100 + i).to(DEV) for i in range(3))
    announce("repeatability")
    o1, l1 = attn.forward(q, k, v, causal=True)
    o2, l2 = attn.forward(q, k, v, causal=True)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_no_writes_outside_outputs():
    """Canary words around o and lse stay untouched."""
    B, H, N, d = 1, 2, 131, 64
    q, k, v = (randn((B, H, N, d), torch.float16, 110 + i).to(DEV) for i in range(3))
    pad = 4096
    obuf = torch.full((pad + B * H * N * d + pad,), 1234.0, dtype=torch.float16, device=DEV)
    lbuf = torch.full((pad + B * H * N + pad,), -77.0, dtype=torch.float32, device=DEV)
    o = obuf[pad:pad + B * H * N * d].view(B, H, N, d)
    lse = lbuf[pad:pad + B * H * N].view(B, H, N)
    announce("canary")
    for causal in (False, True):
        attn.forward(q, k, v, causal=causal, out=(o, lse))
        torch.cuda.synchronize()
        assert bool((obuf[:pad] == 1234).all()) and bool((obuf[-pad:] == 1234).all())
        assert bool((lbuf[:pad] == -77).all()) and bool((lbuf[-pad:] == -77).all())


def test_stream_ordering():
    """Work goes to torch's current stream."""
    q, k, v = (randn((1, 2, 512, 128), torch.bfloat16, 120 + i).to(DEV) for i in range(3))
    announce("side stream")
    ref, _ = attn.forward(q, k, v)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        o, _ = attn.forward(q, k, v)
    s.synchronize()
    assert torch.equal(o, ref)


# ---------------------------------------------------------------------------
# The workloads at their full sizes, as the bench launches them
# ---------------------------------------------------------------------------

FWD_WORKLOADS = ["tiny_fwd", "gpt2_medium_fwd", "llama7b_layer_fwd", "long_context_fwd"]


def sample_rows(B, H, N, n_heads, per_head, seed):
    """Flattened row ids: first/last heads and random ones; rows 0, N-1,
    block edges and random rows."""
    rng = np.random.default_rng(seed)
    BH = B * H
    heads = sorted(set([0, BH - 1] + list(rng.choice(BH, size=min(BH, n_heads), replace=False))))
    fixed = [0, 1, 127, 128, N // 2, N - 2, N - 1]
    rows = []
    for hd in heads:
        rr = set(r for r in fixed if 0 <= r < N) | set(rng.choice(N, size=min(N, per_head), replace=False))
        rows += [hd * N + r for r in sorted(rr)]
    return np.array(rows, dtype=np.int64)


@pytest.mark.parametrize("name", FWD_WORKLOADS)
def test_workload_full_size(name):
    w = inputs.WORKLOADS[name]
    t = inputs.make_inputs(w)
    scale = 1 / math.sqrt(w.d)
    announce(f"workload {name} {w.describe()}")
    qd, kd, vd = (t[x].to(DEV) for x in ("q", "k", "v"))
    o32, lse = attn.forward(qd, kd, vd, causal=w.causal, scale=scale, out_dtype=torch.float32)
    o, lse16 = attn.forward(qd, kd, vd, causal=w.causal, scale=scale)
    torch.cuda.synchronize()
    # the production output is the fp32 result rounded once
    assert torch.equal(o, o32.to(w.torch_dtype)) and torch.equal(lse, lse16)
    B, H, N, d = w.B, w.H, w.N, w.d
    if B * H * N <= 1024:
        rows = np.arange(B * H * N)
    else:
        # about 32,768 rows from up to 64 heads (the first and last rows of
        # each among them), element by element against the oracle
        nh = min(B * H, 64)
        rows = sample_rows(B, H, N, n_heads=nh, per_head=max(48, 32768 // nh), seed=w.seed)
    o_ref, lse_ref = oracle_fwd(t["q"], t["k"], t["v"], s32(scale), w.causal, rows=rows)
    of = o32.view(-1, d)[torch.from_numpy(rows).to(DEV)]
    lf = lse.view(-1)[torch.from_numpy(rows).to(DEV)]
    report(f"{name} O(fp32 out)", f64(of), o_ref, TOL[w.torch_dtype])
    report(f"{name} lse", f64(lf), lse_ref, LSE_TOL)
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    # at any size: a column of ones in V comes out as ones
    vd[..., 0] = 1
    o1, _ = attn.forward(qd, kd, vd, causal=w.causal, scale=scale)
    err = (o1[..., 0].float() - 1).abs().max().item()
    assert err <= TOL[w.torch_dtype], err


@pytest.mark.parametrize("B,H,N,d,dtype,causal", [
    (1, 64, 2048, 128, torch.bfloat16, True),      # head groups of 4, 16 blocks per head
    (2, 64, 1024, 64, torch.float16, False),       # 1024 blocks, two rounds of workgroups
    (1, 13, 4096, 128, torch.bfloat16, True),      # 13 heads: causal pairs
    (3, 7, 2560, 64, torch.bfloat16, True),        # 21 heads, pairs
    (4, 64, 777, 128, torch.float16, False),       # 1792 blocks, ragged tail
    (8, 16, 1153, 64, torch.bfloat16, True),       # odd block count (10), head groups
    (1, 24, 1000, 128, torch.bfloat16, True),      # head groups of 3, ragged tail
    (2, 8, 1500, 64, torch.float16, True),         # head groups of 2
    (1, 8, 2000, 128, torch.bfloat16, True),       # one head per XCD
])
def test_many_blocks(B, H, N, d, dtype, causal):
    """Grids of several rounds of workgroups over many heads and blocks:
    head counts that are and are not multiples of 8 (head groups or causal
    pairs), odd block counts, ragged tails: sampled rows of fp32 O and lse
    against the oracle, the 16-bit O equal to RNE(fp32 O) everywhere, and a
    column of ones in V reproduced in every row."""
    tag = f"many blocks B={B} H={H} N={N} d={d}"
    announce(f"fwd {tag} {dtype} causal={causal}")
    q, k, v = (randn((B, H, N, d), dtype, 300 + N + d + i) for i in range(3))
    scale = 1 / math.sqrt(d)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o32, lse32 = attn.forward(qd, kd, vd, causal=causal, scale=scale, out_dtype=torch.float32)
    o, lse = attn.forward(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    assert torch.equal(o, o32.to(dtype)) and torch.equal(lse, lse32)
    rows = sample_rows(B, H, N, n_heads=min(B * H, 24), per_head=160, seed=N + d)
    o_ref, lse_ref = oracle_fwd(q, k, v, s32(scale), causal, rows=rows)
    idx = torch.from_numpy(rows).to(DEV)
    report(f"{tag} O(fp32 out)", f64(o32.view(-1, d)[idx]), o_ref, TOL[dtype])
    report(f"{tag} lse", f64(lse32.view(-1)[idx]), lse_ref, LSE_TOL)
    vd[..., 0] = 1
    o1, _ = attn.forward(qd, kd, vd, causal=causal, scale=scale, out_dtype=torch.float32)
    err = (o1[..., 0] - 1).abs().max().item()
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("causal", [False, True])
def test_many_heads(causal):
    """16,384 (batch, head) pairs of 40 rows: a grid far larger than the chip,
    with a total not a multiple of the XCD count, checks the mapping from
    workgroup to (batch, head, block) at scale (every row against the
    oracle)."""
    q, k, v = (randn((64, 256, 40, 64), torch.bfloat16, 150 + i) for i in range(3))
    run_and_compare(q, k, v, causal, 0.125, "many heads")
