"""Exact fused attention for AMD Instinct MI355X (gfx950).

Thin Python binding over the C ABI of ``libattn.so`` (declared in
``include/attn.h``).  It only marshals arguments: every step of the
computation runs in the library's HIP kernels.  torch supplies device
memory and the current stream.

Low level (same names and argument order as the C ABI, raw integers and
device pointers):  :func:`attn_fwd`, :func:`attn_fwd_split`,
:func:`attn_fwd_split_workspace_size`, :func:`attn_bwd`, :func:`attn_bwd_noalloc`,
:func:`attn_bwd_dq`,
:func:`attn_bwd_dkdv`, :func:`attn_bwd_workspace_size`, :func:`attn_fwd_fp8`,
:func:`attn_fwd_decode_fp8`, :func:`attn_std_fwd`, :func:`attn_std_scores`,
:func:`attn_std_softmax`, :func:`attn_std_pv`, :func:`attn_std_workspace_size`,
:func:`attn_status_str`.

Tensor level:  :func:`forward`, :func:`forward_split`, :func:`forward_decode`,
:func:`forward_fp8`, :func:`forward_decode_fp8` and :func:`backward`;
:func:`forward_standard` is the materialised (unfused) baseline.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = [
    "attn_fwd", "attn_fwd_split", "attn_fwd_split_workspace_size",
    "attn_bwd", "attn_bwd_noalloc", "attn_bwd_dq", "attn_bwd_dkdv", "attn_bwd_workspace_size",
    "attn_fwd_fp8", "attn_fwd_decode_fp8", "attn_status_str",
    "attn_std_fwd", "attn_std_scores", "attn_std_softmax", "attn_std_pv", "attn_std_workspace_size",
    "forward_standard",
    "forward", "forward_split", "forward_decode", "forward_fp8", "forward_decode_fp8", "backward", "AttnError", "ATTN_F16", "ATTN_BF16", "ATTN_F32", "library_path",
]

ATTN_F16 = 0
ATTN_BF16 = 1
ATTN_F32 = 2
_DTYPE_CODE = {torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16}
_OUT_CODE = {torch.float16: ATTN_F16, torch.bfloat16: ATTN_BF16, torch.float32: ATTN_F32}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libattn.so")
_lib = None


class AttnError(RuntimeError):
    """A non-zero status returned by the attention library."""

    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {attn_status_str(status)} (status {status})")


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(
            f"{_LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'` "
            "(or python exact_io_aware_40_amd/csrc/build.py) first")
    lib = ctypes.CDLL(_LIB_PATH)
    vp, i64, f32, i32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int,
                             ctypes.c_size_t)
    lib.attn_fwd.restype = i32
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.attn_fwd_split_workspace_size.restype = sz
    lib.attn_fwd_split_workspace_size.argtypes = [i64, i64, i64, i64, i32]
    lib.attn_fwd_split.restype = i32
    lib.attn_fwd_split.argtypes = [vp] * 6 + [sz, i64, i64, i64, i64, f32, i32, i32, i32, i32, vp]
    lib.attn_fwd_decode.restype = i32
    lib.attn_fwd_decode.argtypes = [vp] * 6 + [sz, i64, i64, i64, i64, i64, f32, i32, i32, i32, i32, vp]
    lib.attn_bwd_workspace_size.restype = sz
    lib.attn_bwd_workspace_size.argtypes = [i64, i64, i64, i64, i32]
    lib.attn_bwd.restype = i32
    lib.attn_bwd.argtypes = [vp] * 10 + [sz, i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.attn_bwd_noalloc.restype = i32
    lib.attn_bwd_noalloc.argtypes = [vp] * 9 + [i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.attn_bwd_dq.restype = i32
    lib.attn_bwd_dq.argtypes = [vp] * 8 + [sz, i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.attn_bwd_dkdv.restype = i32
    lib.attn_bwd_dkdv.argtypes = [vp] * 7 + [sz, i64, i64, i64, i64, f32, i32, i32, i32, vp]
    u64, u32 = ctypes.c_uint64, ctypes.c_uint32
    lib.attn_fwd_dropout.restype = i32
    lib.attn_fwd_dropout.argtypes = [vp] * 5 + [i64, i64, i64, i64, f32, i32, f32, u64, u32, i32, i32, vp]
    lib.attn_bwd_dropout.restype = i32
    lib.attn_bwd_dropout.argtypes = [vp] * 10 + [sz, i64, i64, i64, i64, f32, i32, f32, u64, u32, i32,
                                                 i32, vp]
    lib.attn_fwd_fp8.restype = i32
    lib.attn_fwd_fp8.argtypes = [vp] * 5 + [i64, i64, i64, i64, f32, f32, f32, f32, i32, i32, vp]
    lib.attn_fwd_decode_fp8.restype = i32
    lib.attn_fwd_decode_fp8.argtypes = [vp] * 6 + [sz, i64, i64, i64, i64, i64, f32, f32, f32, f32,
                                                   i32, i32, i32, vp]
    lib.attn_std_workspace_size.restype = sz
    lib.attn_std_workspace_size.argtypes = [i64, i64, i64, i64, i32]
    lib.attn_std_fwd.restype = i32
    lib.attn_std_fwd.argtypes = [vp] * 6 + [sz, i64, i64, i64, i64, f32, i32, i32, i32, vp]
    lib.attn_std_scores.restype = i32
    lib.attn_std_scores.argtypes = [vp] * 3 + [i64, i64, i64, i64, f32, i32, vp]
    lib.attn_std_softmax.restype = i32
    lib.attn_std_softmax.argtypes = [vp] * 3 + [i64, i64, i64, i32, i32, vp]
    lib.attn_std_pv.restype = i32
    lib.attn_std_pv.argtypes = [vp] * 3 + [i64, i64, i64, i64, i32, i32, vp]
    lib.attn_probe_mfma.restype = i32
    lib.attn_probe_mfma.argtypes = [vp, i64, i64, vp]
    lib.attn_probe_hbm.restype = i32
    lib.attn_probe_hbm.argtypes = [vp, i64, vp, i64, vp]
    lib.attn_status_str.restype = ctypes.c_char_p
    lib.attn_status_str.argtypes = [i32]
    _lib = lib
    return lib


# ---------------------------------------------------------------------------
# C ABI, one to one
# ---------------------------------------------------------------------------

def attn_fwd(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int,
             scale: float, causal: int, dtype: int, out_dtype: int, stream: int) -> int:
    return _load().attn_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, out_dtype, stream)


def attn_fwd_split_workspace_size(B: int, H: int, N: int, d: int, nsplit: int) -> int:
    return _load().attn_fwd_split_workspace_size(B, H, N, d, nsplit)


def attn_fwd_split(q: int, k: int, v: int, o: int, lse: int, workspace: int, workspace_bytes: int,
                   B: int, H: int, N: int, d: int, scale: float, causal: int, dtype: int,
                   out_dtype: int, nsplit: int, stream: int) -> int:
    return _load().attn_fwd_split(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale,
                                  causal, dtype, out_dtype, nsplit, stream)


def attn_fwd_decode(q: int, k: int, v: int, o: int, lse: int, workspace: int, workspace_bytes: int,
                    B: int, H: int, Nq: int, Nk: int, d: int, scale: float, causal: int, dtype: int,
                    out_dtype: int, nsplit: int, stream: int) -> int:
    return _load().attn_fwd_decode(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d,
                                   scale, causal, dtype, out_dtype, nsplit, stream)


def attn_bwd_workspace_size(B: int, H: int, N: int, d: int, dtype: int) -> int:
    return _load().attn_bwd_workspace_size(B, H, N, d, dtype)


def attn_bwd(q: int, k: int, v: int, o: int, dO: int, lse: int, dq: int, dk: int, dv: int,
             workspace: int, workspace_bytes: int, B: int, H: int, N: int, d: int,
             scale: float, causal: int, dtype: int, out_dtype: int, stream: int) -> int:
    return _load().attn_bwd(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes,
                            B, H, N, d, scale, causal, dtype, out_dtype, stream)


def attn_bwd_noalloc(q: int, k: int, v: int, o: int, dO: int, lse: int, dq: int, dk: int, dv: int,
                     B: int, H: int, N: int, d: int, scale: float, causal: int, dtype: int,
                     out_dtype: int, stream: int) -> int:
    return _load().attn_bwd_noalloc(q, k, v, o, dO, lse, dq, dk, dv, B, H, N, d, scale, causal,
                                    dtype, out_dtype, stream)


def attn_bwd_dq(q: int, k: int, v: int, o: int, dO: int, lse: int, dq: int, workspace: int,
                workspace_bytes: int, B: int, H: int, N: int, d: int, scale: float, causal: int,
                dtype: int, out_dtype: int, stream: int) -> int:
    return _load().attn_bwd_dq(q, k, v, o, dO, lse, dq, workspace, workspace_bytes, B, H, N, d,
                               scale, causal, dtype, out_dtype, stream)


def attn_bwd_dkdv(q: int, k: int, v: int, dO: int, dk: int, dv: int, workspace: int,
                  workspace_bytes: int, B: int, H: int, N: int, d: int, scale: float,
                  causal: int, dtype: int, out_dtype: int, stream: int) -> int:
    return _load().attn_bwd_dkdv(q, k, v, dO, dk, dv, workspace, workspace_bytes, B, H, N, d,
                                 scale, causal, dtype, out_dtype, stream)


def attn_fwd_dropout(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int,
                     scale: float, causal: int, dropout_p: float, seed: int, offset: int, dtype: int,
                     out_dtype: int, stream: int) -> int:
    return _load().attn_fwd_dropout(q, k, v, o, lse, B, H, N, d, scale, causal, dropout_p, seed,
                                    offset, dtype, out_dtype, stream)


def attn_bwd_dropout(q: int, k: int, v: int, o: int, dO: int, lse: int, dq: int, dk: int, dv: int,
                     workspace: int, workspace_bytes: int, B: int, H: int, N: int, d: int,
                     scale: float, causal: int, dropout_p: float, seed: int, offset: int,
                     dtype: int, out_dtype: int, stream: int) -> int:
    return _load().attn_bwd_dropout(q, k, v, o, dO, lse, dq, dk, dv, workspace, workspace_bytes,
                                    B, H, N, d, scale, causal, dropout_p, seed, offset, dtype,
                                    out_dtype, stream)


def attn_fwd_fp8(q: int, k: int, v: int, o: int, lse: int, B: int, H: int, N: int, d: int,
                 scale: float, q_descale: float, k_descale: float, v_descale: float, causal: int,
                 out_dtype: int, stream: int) -> int:
    return _load().attn_fwd_fp8(q, k, v, o, lse, B, H, N, d, scale, q_descale, k_descale, v_descale,
                                causal, out_dtype, stream)


def attn_fwd_decode_fp8(q: int, k: int, v: int, o: int, lse: int, workspace: int,
                        workspace_bytes: int, B: int, H: int, Nq: int, Nk: int, d: int, scale: float,
                        q_descale: float, k_descale: float, v_descale: float, causal: int,
                        out_dtype: int, nsplit: int, stream: int) -> int:
    return _load().attn_fwd_decode_fp8(q, k, v, o, lse, workspace, workspace_bytes, B, H, Nq, Nk, d,
                                       scale, q_descale, k_descale, v_descale, causal, out_dtype,
                                       nsplit, stream)


def attn_std_workspace_size(B: int, H: int, N: int, d: int, dtype: int) -> int:
    return _load().attn_std_workspace_size(B, H, N, d, dtype)


def attn_std_fwd(q: int, k: int, v: int, o: int, lse: int, workspace: int, workspace_bytes: int,
                 B: int, H: int, N: int, d: int, scale: float, causal: int, dtype: int,
                 out_dtype: int, stream: int) -> int:
    return _load().attn_std_fwd(q, k, v, o, lse, workspace, workspace_bytes, B, H, N, d, scale,
                                causal, dtype, out_dtype, stream)


def attn_std_scores(q: int, k: int, s: int, B: int, H: int, N: int, d: int, scale: float,
                    dtype: int, stream: int) -> int:
    return _load().attn_std_scores(q, k, s, B, H, N, d, scale, dtype, stream)


def attn_std_softmax(s: int, p: int, lse: int, B: int, H: int, N: int, causal: int, dtype: int,
                     stream: int) -> int:
    return _load().attn_std_softmax(s, p, lse, B, H, N, causal, dtype, stream)


def attn_std_pv(p: int, v: int, o: int, B: int, H: int, N: int, d: int, dtype: int,
                out_dtype: int, stream: int) -> int:
    return _load().attn_std_pv(p, v, o, B, H, N, d, dtype, out_dtype, stream)


def attn_probe_mfma(out: int, workgroups: int, rounds: int, stream: int) -> int:
    return _load().attn_probe_mfma(out, workgroups, rounds, stream)


def attn_probe_hbm(buf: int, nbytes: int, out: int, workgroups: int, stream: int) -> int:
    return _load().attn_probe_hbm(buf, nbytes, out, workgroups, stream)


def attn_status_str(status: int) -> str:
    return _load().attn_status_str(status).decode()


# ---------------------------------------------------------------------------
# Tensor level
# ---------------------------------------------------------------------------

def _check(t: torch.Tensor, name: str, like: Optional[torch.Tensor] = None, dtype=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")
    if like is not None:
        want = like.dtype if dtype is None else dtype
        if t.shape != like.shape or t.dtype != want or t.device != like.device:
            raise ValueError(f"{name} must be {want} and match q in shape and device")


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _out_dtype(q: torch.Tensor, out_dtype) -> torch.dtype:
    od = q.dtype if out_dtype is None else out_dtype
    if od not in (q.dtype, torch.float32):
        raise ValueError(f"out_dtype must be {q.dtype} or torch.float32, got {od}")
    return od


def forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
            scale: Optional[float] = None, out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None,
            out_dtype: Optional[torch.dtype] = None,
            dropout: Optional[Tuple[float, int, int]] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact attention forward.  q, k, v: [B, H, N, d] fp16/bf16 on the GPU.

    Returns (o [B, H, N, d], lse [B, H, N] float32); o has q's dtype unless
    out_dtype=torch.float32.  scale defaults to 1/sqrt(d).  dropout, if
    given, is (p, seed, offset) for attn_fwd_dropout.  The work is enqueued
    on torch's current stream.
    """
    _check(q, "q")
    _check(k, "k", q)
    _check(v, "v", q)
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"dtype must be float16 or bfloat16, got {q.dtype}")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    od = _out_dtype(q, out_dtype if out is None else out[0].dtype)
    if out is None:
        o = torch.empty(q.shape, dtype=od, device=q.device)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _check(o, "o", q, od)
        if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be contiguous float32 [B, H, N]")
    if dropout is None:
        st = attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, H, N, d, float(scale), int(bool(causal)), _DTYPE_CODE[q.dtype],
                      _OUT_CODE[od], _stream(q))
    else:
        p, seed, offset = dropout
        st = attn_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              lse.data_ptr(), B, H, N, d, float(scale), int(bool(causal)), float(p),
                              int(seed) & (2**64 - 1), int(offset) & (2**32 - 1),
                              _DTYPE_CODE[q.dtype], _OUT_CODE[od], _stream(q))
    if st != 0:
        raise AttnError(st, "attn_fwd" if dropout is None else "attn_fwd_dropout")
    return o, lse


_FP8_TYPES = (torch.uint8, torch.float8_e4m3fn)


def forward_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                descale: Tuple[float, float, float] = (1.0, 1.0, 1.0), causal: bool = False,
                scale: Optional[float] = None, out_dtype: torch.dtype = torch.bfloat16,
                out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Forward with E4M3 inputs (attn_fwd_fp8).  q, k, v: [B, H, N, 128] GPU
    tensors of E4M3 codes (torch.float8_e4m3fn, or their bytes as uint8),
    standing for code * descale[i].  Returns (o [B, H, N, 128] of out_dtype
    (float16, bfloat16 or float32), lse [B, H, N] float32); scale defaults
    to 1/sqrt(d).  The work is enqueued on torch's current stream."""
    _check(q, "q")
    _check(k, "k", q)
    _check(v, "v", q)
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.dtype not in _FP8_TYPES:
        raise ValueError(f"q, k, v must hold E4M3 codes (float8_e4m3fn or uint8), got {q.dtype}")
    if out_dtype not in _OUT_CODE:
        raise ValueError(f"out_dtype must be float16, bfloat16 or float32, got {out_dtype}")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    od = out_dtype if out is None else out[0].dtype
    if od not in _OUT_CODE:
        raise ValueError(f"o must be float16, bfloat16 or float32, got {od}")
    if out is None:
        o = torch.empty(q.shape, dtype=od, device=q.device)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    else:
        o, lse = out
        _check(o, "o", q, od)
        if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
            raise ValueError("lse must be contiguous float32 [B, H, N]")
    qd, kd, vd = (float(x) for x in descale)
    st = attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      B, H, N, d, float(scale), qd, kd, vd, int(bool(causal)), _OUT_CODE[od], _stream(q))
    if st != 0:
        raise AttnError(st, "attn_fwd_fp8")
    return o, lse


def forward_decode_fp8(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                       descale: Tuple[float, float, float] = (1.0, 1.0, 1.0), causal: bool = False,
                       scale: Optional[float] = None, nsplit: int = 8,
                       out_dtype: torch.dtype = torch.bfloat16,
                       workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """attn_fwd_decode_fp8: E4M3 q [B, H, Nq, 128] against E4M3 k, v
    [B, H, Nk, 128] (codes as float8_e4m3fn or uint8), keys split in nsplit
    chunks and merged.  Returns (o [B, H, Nq, 128] of out_dtype, lse
    [B, H, Nq] float32).  A workspace (uint8, at least
    attn_fwd_split_workspace_size(B, H, Nq, 128, nsplit) bytes) is allocated
    when none is given."""
    _check(q, "q")
    _check(k, "k")
    _check(v, "v", k)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.dtype not in _FP8_TYPES or k.dtype not in _FP8_TYPES:
        raise ValueError("q, k, v must hold E4M3 codes (float8_e4m3fn or uint8)")
    if out_dtype not in _OUT_CODE:
        raise ValueError(f"out_dtype must be float16, bfloat16 or float32, got {out_dtype}")
    B, H, Nq, d = q.shape
    if k.shape[:2] != (B, H) or k.shape[3] != d or k.device != q.device:
        raise ValueError("k, v must be [B, H, Nk, d] on q's device")
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, Nq, d), dtype=out_dtype, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    need = attn_fwd_split_workspace_size(B, H, Nq, d, nsplit)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    qd, kd, vd = (float(x) for x in descale)
    st = attn_fwd_decode_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                             workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                             B, H, Nq, Nk, d, float(scale), qd, kd, vd, int(bool(causal)),
                             _OUT_CODE[out_dtype], int(nsplit), _stream(q))
    if st != 0:
        raise AttnError(st, "attn_fwd_decode_fp8")
    return o, lse


def forward_split(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                  scale: Optional[float] = None, nsplit: int = 2,
                  out_dtype: Optional[torch.dtype] = None,
                  workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Exact attention forward with each query block's K/V split into nsplit
    chunks and the partial results merged (attn_fwd_split).  Arguments and
    results as for :func:`forward`; workspace, if given, is a uint8 CUDA
    tensor of at least attn_fwd_split_workspace_size(...) bytes."""
    _check(q, "q")
    _check(k, "k", q)
    _check(v, "v", q)
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"dtype must be float16 or bfloat16, got {q.dtype}")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    od = _out_dtype(q, out_dtype)
    o = torch.empty(q.shape, dtype=od, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    need = attn_fwd_split_workspace_size(B, H, N, d, int(nsplit))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                        B, H, N, d, float(scale), int(bool(causal)), _DTYPE_CODE[q.dtype],
                        _OUT_CODE[od], int(nsplit), _stream(q))
    if st != 0:
        raise AttnError(st, "attn_fwd_split")
    return o, lse


def forward_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                   scale: Optional[float] = None, nsplit: int = 8,
                   out_dtype: Optional[torch.dtype] = None,
                   workspace: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Split K/V forward of q [B, H, Nq, d] against k, v [B, H, Nk, d]
    (attn_fwd_decode); under the causal mask the queries are the last Nq
    positions.  Returns (o [B, H, Nq, d], lse [B, H, Nq] float32)."""
    _check(q, "q")
    _check(k, "k")
    _check(v, "v", k)
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-d")
    if q.dtype not in _DTYPE_CODE or k.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype, float16 or bfloat16")
    B, H, Nq, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d:
        raise ValueError("k, v must be [B, H, Nk, d] with q's B, H and d")
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    od = _out_dtype(q, out_dtype)
    o = torch.empty(q.shape, dtype=od, device=q.device)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    need = attn_fwd_split_workspace_size(B, H, Nq, d, int(nsplit))
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = attn_fwd_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                         workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                         B, H, Nq, Nk, d, float(scale), int(bool(causal)), _DTYPE_CODE[q.dtype],
                         _OUT_CODE[od], int(nsplit), _stream(q))
    if st != 0:
        raise AttnError(st, "attn_fwd_decode")
    return o, lse


def backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
             lse: torch.Tensor, dO: torch.Tensor, causal: bool = False,
             scale: Optional[float] = None, workspace: Optional[torch.Tensor] = None,
             dropout: Optional[Tuple[float, int, int]] = None
             ) -> Tuple[torch.Tensor, torch.Tensor, torch.Tensor]:
    """Gradients (dq, dk, dv) of sum(o * dO) from the forward's o and lse.

    The backward recomputes S and P from q, k and lse.  The gradients have
    o's dtype (q's dtype, or float32 when the forward wrote float32).
    `workspace` (a uint8 device tensor of at least attn_bwd_workspace_size
    bytes) may be passed to avoid an allocation per call.  dropout, if
    given, is the forward's (p, seed, offset) for attn_bwd_dropout.
    """
    _check(q, "q")
    od = _out_dtype(q, o.dtype)
    for t, n in ((k, "k"), (v, "v"), (dO, "dO")):
        _check(t, n, q)
    _check(o, "o", q, od)
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"dtype must be float16 or bfloat16, got {q.dtype}")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    code = _DTYPE_CODE[q.dtype]
    need = attn_bwd_workspace_size(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    dq, dk, dv = (torch.empty(q.shape, dtype=od, device=q.device) for _ in range(3))
    ptrs = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dO.data_ptr(), lse.data_ptr(),
            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), workspace.data_ptr(),
            workspace.numel() * workspace.element_size())
    if dropout is None:
        st = attn_bwd(*ptrs, B, H, N, d, float(scale), int(bool(causal)), code, _OUT_CODE[od],
                      _stream(q))
    else:
        p, seed, offset = dropout
        st = attn_bwd_dropout(*ptrs, B, H, N, d, float(scale), int(bool(causal)), float(p),
                              int(seed) & (2**64 - 1), int(offset) & (2**32 - 1), code,
                              _OUT_CODE[od], _stream(q))
    if st != 0:
        raise AttnError(st, "attn_bwd" if dropout is None else "attn_bwd_dropout")
    return dq, dk, dv


def forward_standard(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = False,
                     scale: Optional[float] = None, out_dtype: Optional[torch.dtype] = None,
                     workspace: Optional[torch.Tensor] = None, return_sp: bool = False):
    """The materialised standard attention (attn_std_fwd): S = scale Q K^T
    written to device memory in full (fp32), P = softmax(S) written in full
    (q's dtype), then O = P V.  Same result as :func:`forward` up to
    rounding, at N x N traffic per head; it exists as the baseline the fused
    path is measured against.  Returns (o, lse), and with return_sp also
    (s [B, H, N, N] float32, p [B, H, N, N] q.dtype), views of the workspace
    (a uint8 device tensor of at least attn_std_workspace_size bytes,
    allocated when not given)."""
    _check(q, "q")
    _check(k, "k", q)
    _check(v, "v", q)
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, d]")
    if q.dtype not in _DTYPE_CODE:
        raise ValueError(f"dtype must be float16 or bfloat16, got {q.dtype}")
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    od = _out_dtype(q, out_dtype)
    code = _DTYPE_CODE[q.dtype]
    o = torch.empty(q.shape, dtype=od, device=q.device)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    need = attn_std_workspace_size(B, H, N, d, code)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    st = attn_std_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                      workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                      B, H, N, d, float(scale), int(bool(causal)), code, _OUT_CODE[od], _stream(q))
    if st != 0:
        raise AttnError(st, "attn_std_fwd")
    if not return_sp:
        return o, lse
    nel = B * H * N * N
    sbytes = (nel * 4 + 255) // 256 * 256
    raw = workspace.view(torch.uint8).reshape(-1)
    s = raw[:nel * 4].view(torch.float32).reshape(B, H, N, N)
    p = raw[sbytes:sbytes + nel * 2].view(q.dtype).reshape(B, H, N, N)
    return o, lse, s, p
