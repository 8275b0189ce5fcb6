"""attn_bwd_noalloc (the backward with its workspace in a fixed per-GPU
array, for callers that cannot allocate) against attn_bwd with a caller
workspace: the same kernels, so the same gradients bit for bit, on two calls
in a row, the second with a smaller input; the smaller call's fp32
gradients also against the oracle within the stated tolerance."""
import math

import numpy as np
import pytest
import torch

import exact_io_aware_40_amd as attn
import oracle
from tests._util import TOL, announce, f64, randn, report

pytestmark = pytest.mark.gpu
DEV = "cuda"


def run_both(B, H, N, d, dtype, causal, out_dtype, seed):
    """attn_bwd (caller workspace) and attn_bwd_noalloc on the same inputs,
    both through the C ABI; returns (gradients of each, inputs)."""
    q, k, v, dO = (randn((B, H, N, d), dtype, seed + i).to(DEV) for i in range(4))
    o, lse = attn.forward(q, k, v, causal=causal, out_dtype=out_dtype)
    code = attn.ATTN_BF16 if dtype == torch.bfloat16 else attn.ATTN_F16
    ocode = attn.ATTN_F32 if out_dtype == torch.float32 else code
    od = o.dtype
    scale = 1.0 / math.sqrt(d)
    sp = torch.cuda.current_stream().cuda_stream
    nbytes = attn.attn_bwd_workspace_size(B, H, N, d, code)
    assert nbytes <= 16 << 20
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    ref = [torch.full((B, H, N, d), float("nan"), dtype=od, device=DEV) for _ in range(3)]
    got = [torch.full((B, H, N, d), float("nan"), dtype=od, device=DEV) for _ in range(3)]
    st = attn.attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dO.data_ptr(),
                       lse.data_ptr(), *(g.data_ptr() for g in ref), ws.data_ptr(), nbytes,
                       B, H, N, d, scale, int(causal), code, ocode, sp)
    assert st == 0, attn.attn_status_str(st)
    st = attn.attn_bwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dO.data_ptr(),
                               lse.data_ptr(), *(g.data_ptr() for g in got), B, H, N, d, scale,
                               int(causal), code, ocode, sp)
    assert st == 0, attn.attn_status_str(st)
    torch.cuda.synchronize()
    return ref, got, (q, k, v, dO, scale)


def test_noalloc_matches_attn_bwd_twice():
    announce("bwd noalloc: large call, then a smaller one")
    # first call: 8 x 700 rows of d = 128, bf16, causal, 16-bit gradients
    ref, got, _ = run_both(2, 4, 700, 128, torch.bfloat16, True, None, 900)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
    # second call, smaller, on the same scratch: 2 x 129 rows of d = 64, fp16,
    # no mask, fp32 gradients; also against the oracle
    ref, got, (q, k, v, dO, scale) = run_both(1, 2, 129, 64, torch.float16, False, torch.float32, 910)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
    _, _, rq, rk, rv = oracle.bwd(f64(q), f64(k), f64(v), f64(dO), float(np.float32(scale)), False)
    for name, g, r in zip(("dq", "dk", "dv"), got, (rq, rk, rv)):
        report(f"noalloc {name}(fp32 out)", f64(g), r, TOL[torch.float16])


def test_noalloc_at_the_bench_shape():
    """The 7B-layer shape (4 MiB of workspace rows), after the calls above."""
    announce("bwd noalloc: 4 x 32 x 4096 x 128")
    ref, got, _ = run_both(4, 32, 4096, 128, torch.bfloat16, True, None, 920)
    for r, g in zip(ref, got):
        assert torch.equal(r, g)
