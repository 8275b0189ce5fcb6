"""Seeded synthetic inputs for the attention workloads.

This module only draws numbers and lays them out; it holds none of the
attention arithmetic, so both the HIP path's tests and the fp64 oracle's
tests can take their inputs from here.

Every tensor is drawn as float32 iid N(0, 1) from NumPy's PCG64 seeded with
(seed, tensor id) -- ids: q=0, k=1, v=2, dO=3, outlier-row choice=4 -- and
rounded to fp16 or bf16 (round to nearest even) by torch.  The seven-billion-
parameter-layer workload then multiplies 1% of the rows of K (flattened over
batch, head and position; chosen by the seed without replacement) by 8, an
exact operation in bf16, to create large score outliers.
"""
from __future__ import annotations

import dataclasses
import hashlib
from typing import Dict, Optional

import numpy as np
import torch

TENSOR_IDS = {"q": 0, "k": 1, "v": 2, "dO": 3, "outlier_rows": 4}
DTYPES = {"f16": torch.float16, "bf16": torch.bfloat16}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f16" or "bf16"
    causal: bool
    kind: str           # "fwd" or "bwd"
    seed: int
    outlier_frac: float = 0.0
    outlier_scale: float = 1.0

    @property
    def torch_dtype(self) -> torch.dtype:
        return DTYPES[self.dtype]

    def flops(self) -> float:
        """Credited FLOPs: 4*B*H*N^2*d forward, halved under the causal mask;
        the backward is credited 2.5x the forward (five N^2*d contractions
        counting the recomputation of Q K^T)."""
        f = 4.0 * self.B * self.H * self.N * self.N * self.d
        if self.causal:
            f *= 0.5
        return f * (2.5 if self.kind == "bwd" else 1.0)

    def describe(self) -> str:
        mask = "causal" if self.causal else "non-causal"
        s = f"B={self.B} H={self.H} N={self.N} d={self.d} {self.dtype} {mask} {self.kind}"
        if self.outlier_frac:
            s += f", {self.outlier_frac:.0%} of K rows x{self.outlier_scale:g}"
        return s


WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_fwd", 1, 2, 256, 64, "f16", False, "fwd", seed=1),
        Workload("gpt2_medium_fwd", 64, 16, 1024, 64, "f16", False, "fwd", seed=2),
        Workload("llama7b_layer_fwd", 4, 32, 4096, 128, "bf16", True, "fwd", seed=3,
                 outlier_frac=0.01, outlier_scale=8.0),
        Workload("long_context_fwd", 1, 16, 16384, 128, "bf16", True, "fwd", seed=4),
        Workload("recompute_bwd", 8, 16, 2048, 128, "bf16", True, "bwd", seed=5),
    ]
}


def normal(shape, seed: int, tensor_id: int, dtype: torch.dtype) -> torch.Tensor:
    """iid N(0,1) float32 from PCG64([seed, tensor_id]), rounded to `dtype`."""
    rng = np.random.Generator(np.random.PCG64([seed, tensor_id]))
    x = rng.standard_normal(size=int(np.prod(shape)), dtype=np.float32).reshape(shape)
    return torch.from_numpy(x).to(dtype)


def outlier_rows(n_rows: int, frac: float, seed: int) -> np.ndarray:
    """floor(frac * n_rows) distinct row ids, drawn without replacement."""
    count = int(np.floor(frac * n_rows))
    rng = np.random.Generator(np.random.PCG64([seed, TENSOR_IDS["outlier_rows"]]))
    return np.sort(rng.choice(n_rows, size=count, replace=False)).astype(np.int64)


def make_inputs(w: Workload, seed: Optional[int] = None, shape=None) -> Dict[str, torch.Tensor]:
    """CPU tensors q, k, v (and dO for backward workloads) in [B, H, N, d].

    `shape` = (B, H, N, d) overrides the workload's sizes (same recipe),
    which the tests use for reduced-size cases of a workload.
    """
    seed = w.seed if seed is None else seed
    B, H, N, d = shape if shape is not None else (w.B, w.H, w.N, w.d)
    dt = w.torch_dtype
    out = {name: normal((B, H, N, d), seed, TENSOR_IDS[name], dt) for name in ("q", "k", "v")}
    if w.outlier_frac:
        rows = outlier_rows(B * H * N, w.outlier_frac, seed)
        kf = out["k"].view(B * H * N, d)
        kf[torch.from_numpy(rows)] *= w.outlier_scale
    if w.kind == "bwd":
        out["dO"] = normal((B, H, N, d), seed, TENSOR_IDS["dO"], dt)
    return out


def quantize_e4m3(x: torch.Tensor):
    """Per-tensor scaled E4M3 codes of a CPU tensor: with a = max |x| (in
    fp32), the codes are x * (448 / a) rounded to nearest even E4M3 by torch
    (the product clamped to +-448 first), and descale = a / 448 in fp32, so
    that decode(code) * descale approximates x.  Returns (codes as a uint8
    tensor of x's shape, descale as a Python float)."""
    xf = x.float()
    amax = float(xf.abs().max())
    amax = amax if amax > 0 else 1.0
    s = np.float32(448.0) / np.float32(amax)
    codes = (xf * float(s)).clamp(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    return codes, float(np.float32(1.0) / s)


def make_fp8_inputs(w: Workload, seed: Optional[int] = None, shape=None):
    """The workload's q, k, v (make_inputs) quantised per tensor to E4M3:
    returns ({"q", "k", "v"}: uint8 code tensors, (q, k, v) descales)."""
    src = make_inputs(w, seed, shape)
    out, desc = {}, []
    for name in ("q", "k", "v"):
        out[name], ds = quantize_e4m3(src[name])
        desc.append(ds)
    return out, tuple(desc)


def make_decode_fp8_inputs(B: int, H: int, Nq: int, Nk: int, d: int, seed: int):
    """A decode step's E4M3 inputs: q [B, H, Nq, d] and a key/value cache k, v
    [B, H, Nk, d], each drawn as normal() with its tensor id (bf16) and
    quantised per tensor by quantize_e4m3.  Returns ({"q", "k", "v"}: uint8
    code tensors, (q, k, v) descales)."""
    shapes = {"q": (B, H, Nq, d), "k": (B, H, Nk, d), "v": (B, H, Nk, d)}
    out, desc = {}, []
    for name in ("q", "k", "v"):
        out[name], ds = quantize_e4m3(normal(shapes[name], seed, TENSOR_IDS[name], torch.bfloat16))
        desc.append(ds)
    return out, tuple(desc)


def checksum(t: torch.Tensor) -> str:
    """sha256 of the tensor's raw bytes (first 16 hex digits)."""
    raw = t.contiguous().view(torch.uint8).numpy().tobytes()
    return hashlib.sha256(raw).hexdigest()[:16]
