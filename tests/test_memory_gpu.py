"""The library allocates no device memory: every entry point works in
caller-owned buffers (outputs and, where needed, a workspace), as the header
states.  After one warm-up call of each (which lets the runtime load the code
objects), further calls through the C ABI leave the device's free memory
unchanged."""
import math

import pytest
import torch

import exact_io_aware_40_amd as attn
from tests._util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_entry_points_allocate_nothing():
    announce("device memory across calls")
    B, H, N, d = 2, 4, 1000, 128
    g = torch.Generator(device="cpu").manual_seed(3)
    q, k, v, dO = (torch.randn((B, H, N, d), generator=g).to(torch.bfloat16).to(DEV) for _ in range(4))
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    code = attn.ATTN_BF16
    wsb = attn.attn_bwd_workspace_size(B, H, N, d, code)
    ws = torch.empty(wsb, dtype=torch.uint8, device=DEV)
    ns = 4
    swsb = attn.attn_fwd_split_workspace_size(B, H, N, d, ns)
    sws = torch.empty(swsb, dtype=torch.uint8, device=DEV)
    qd = q[:, :, :3].contiguous()
    od = torch.empty_like(qd)
    lsed = torch.empty((B, H, 3), dtype=torch.float32, device=DEV)
    dwsb = attn.attn_fwd_split_workspace_size(B, H, 3, d, ns)
    dws = torch.empty(dwsb, dtype=torch.uint8, device=DEV)
    sp = torch.cuda.current_stream().cuda_stream
    scale = 1 / math.sqrt(d)
    P = lambda t: t.data_ptr()  # noqa: E731

    def calls():
        st = [
            attn.attn_fwd(P(q), P(k), P(v), P(o), P(lse), B, H, N, d, scale, 1, code, code, sp),
            attn.attn_bwd(P(q), P(k), P(v), P(o), P(dO), P(lse), P(dq), P(dk), P(dv), P(ws), wsb,
                          B, H, N, d, scale, 1, code, code, sp),
            attn.attn_fwd_split(P(q), P(k), P(v), P(o), P(lse), P(sws), swsb, B, H, N, d, scale, 1,
                                code, code, ns, sp),
            attn.attn_fwd_decode(P(qd), P(k), P(v), P(od), P(lsed), P(dws), dwsb, B, H, 3, N, d,
                                 scale, 1, code, code, ns, sp),
            attn.attn_fwd_dropout(P(q), P(k), P(v), P(o), P(lse), B, H, N, d, scale, 1, 0.1, 5, 6,
                                  code, code, sp),
            attn.attn_bwd_dropout(P(q), P(k), P(v), P(o), P(dO), P(lse), P(dq), P(dk), P(dv),
                                  P(ws), wsb, B, H, N, d, scale, 1, 0.1, 5, 6, code, code, sp),
        ]
        assert st == [0] * len(st), st

    calls()
    torch.cuda.synchronize()
    free0, _ = torch.cuda.mem_get_info()
    for _ in range(3):
        calls()
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0, f"device free memory changed by {free0 - free1} bytes across calls"
