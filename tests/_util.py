"""Helpers shared by the GPU parity tests."""
import math
import sys

import numpy as np
import torch

import oracle

# max-abs tolerances against the fp64 oracle, per input element type
TOL = {torch.float16: 2e-3, torch.bfloat16: 1.5e-2}
LSE_TOL = 1e-3


PYTEST_CONFIG = None   # set by conftest.pytest_configure


def _emit(line: str):
    """Write past pytest's output capture, flushed, so the line survives
    even if the process dies in the next GPU call."""
    capman = PYTEST_CONFIG.pluginmanager.getplugin("capturemanager") if PYTEST_CONFIG else None
    if capman is not None:
        with capman.global_and_fixture_disabled():
            print(line, file=sys.stderr, flush=True)
    else:
        print(line, file=sys.stderr, flush=True)


def announce(msg: str):
    """Name the case on the real stderr before any GPU work."""
    _emit(f"[case] {msg}")


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 copy of a (CPU or GPU) fp16/bf16/fp32 tensor."""
    return t.detach().cpu().double().numpy()


def randn(shape, dtype, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(shape, generator=g, dtype=torch.float32) * scale).to(dtype)


def report(name, got, ref, tol):
    err = np.abs(got - ref)
    i = np.unravel_index(np.argmax(err), err.shape) if err.size else ()
    m = float(err.max()) if err.size else 0.0
    _emit(f"[err] {name}: max|gpu-oracle| = {m:.3e} (tol {tol:.1e})")
    assert m <= tol, (f"{name}: max|gpu-oracle| = {m:.3e} > {tol:.1e} at {i} "
                      f"(gpu {got[i]:.6f}, oracle {ref[i]:.6f})")
    return m


def half_ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """Half the spacing of `dtype` at |x|: the error of rounding x to it."""
    mant = {torch.bfloat16: 7, torch.float16: 10}[dtype]
    ax = np.abs(x)
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    if dtype == torch.float16:
        e = np.maximum(e, -14)          # subnormal spacing
    else:
        e = np.maximum(e, -126)
    return np.where(ax > 0, 2.0 ** (e - mant) / 2, 0.0)


def report_rounded(name, got, ref, tol, dtype):
    """16-bit outputs: the stated tolerance plus half an ulp of the output
    format at the exact value (the error of rounding the exact result)."""
    allow = tol + half_ulp(ref, dtype)
    excess = np.abs(got - ref) - allow
    if excess.size:
        _emit(f"[err] {name}: max|gpu-oracle| = {np.abs(got - ref).max():.3e}, "
              f"{int((np.abs(got - ref) > tol).sum())} elements beyond tol, "
              f"max excess over tol+half-ulp {excess.max():.2e}")
    i = np.unravel_index(np.argmax(excess), excess.shape) if excess.size else ()
    assert excess.size == 0 or excess.max() <= 0, (
        f"{name}: |gpu-oracle| = {abs(got[i] - ref[i]):.3e} > tol + half-ulp = {allow[i]:.3e} "
        f"at {i} (gpu {got[i]:.6f}, oracle {ref[i]:.6f})")
    return float(np.abs(got - ref).max()) if excess.size else 0.0


def default_scale(d):
    return 1.0 / math.sqrt(d)


def oracle_fwd(q, k, v, scale, causal, rows=None):
    return oracle.fwd(f64(q), f64(k), f64(v), scale, causal, rows=rows)
