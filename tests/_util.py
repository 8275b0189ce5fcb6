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


def ulp(x: np.ndarray, dtype: torch.dtype) -> np.ndarray:
    """The spacing of `dtype` at |x| (zero maps to the smallest spacing)."""
    mant = {torch.bfloat16: 7, torch.float16: 10}[dtype]
    emin = {torch.bfloat16: -126, torch.float16: -14}[dtype]
    ax = np.abs(x)
    e = np.maximum(np.floor(np.log2(np.where(ax > 0, ax, 2.0 ** emin))), emin)
    return 2.0 ** (e - mant)


def rounding_misses(ref: np.ndarray, tol: float, dtype: torch.dtype) -> int:
    """How many exact values are farther than tol from their own rounding
    to `dtype`: elements no output of that type can bring within tol."""
    r = torch.from_numpy(np.ascontiguousarray(ref)).to(dtype).double().numpy()
    return int((np.abs(r - ref) > tol).sum())


def report_rounded(name, got, ref, tol, dtype, extra=None):
    """16-bit outputs: the stated tolerance plus half an ulp of the output
    format at the exact value (the error of rounding the exact result), plus
    `extra` (an element-wise allowance derived from oracle quantities, e.g.
    the effect of a rounded stored o on the gradients).  Reports how many
    elements lie beyond the literal tolerance and how many exact values
    their own rounding already puts beyond it."""
    allow = tol + half_ulp(ref, dtype)
    if extra is not None:
        allow = allow + extra
    err = np.abs(got - ref)
    excess = err - allow
    if excess.size:
        _emit(f"[err] {name}: max|gpu-oracle| = {err.max():.3e}, "
              f"{int((err > tol).sum())} elements beyond tol "
              f"({rounding_misses(ref, tol, dtype)} exact values beyond it by their own rounding), "
              f"max excess over the allowance {excess.max():.2e}")
    i = np.unravel_index(np.argmax(excess), excess.shape) if excess.size else ()
    assert excess.size == 0 or excess.max() <= 0, (
        f"{name}: |gpu-oracle| = {abs(got[i] - ref[i]):.3e} > allowance {allow[i]:.3e} "
        f"at {i} (gpu {got[i]:.6f}, oracle {ref[i]:.6f})")
    return float(err.max()) if excess.size else 0.0


def rounded(x: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    """A CPU tensor of `dtype` holding the fp64 values x rounded by torch."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(dtype)


def stored_o_allowance(q, k, dO, o_ref, lse_ref, scale, causal, dtype):
    """Element-wise bound on how far dq and dk move when the backward forms
    D_i = dO_i . o_i from an o rounded to `dtype` instead of the exact o.

    Every input is an fp64 array from the inputs or the oracle ([..., N, d];
    lse [..., N]).  D enters the gradients only through dS_ij = P_ij (dP_ij -
    D_i), so an error e_i in D_i changes dq_i by -scale e_i sum_j P_ij k_j and
    dk_j by -scale sum_i P_ij e_i q_i.  With |o16 - o| <= ulp(o) (the kernel's
    fp32 o rounded once to dtype, its own error covered by the tolerance):
    |e_i| <= sum_c |dO_ic| ulp(o_ic).  Returns (allow_dq, allow_dk)."""
    lead, N, d = q.shape[:-2], q.shape[-2], q.shape[-1]
    BH = int(np.prod(lead)) if lead else 1
    q, k, dO, o_ref = (np.asarray(x, np.float64).reshape(BH, N, d) for x in (q, k, dO, o_ref))
    lse = np.asarray(lse_ref, np.float64).reshape(BH, N)
    e = (np.abs(dO) * ulp(o_ref, dtype)).sum(-1)              # [BH, N]
    aq = np.empty_like(q)
    ak = np.empty_like(k)
    vis = np.tril(np.ones((N, N), bool)) if causal else np.ones((N, N), bool)
    step = max(1, (1 << 24) // max(1, N * N))                 # heads per batch of work
    for h0 in range(0, BH, step):
        hs = slice(h0, min(BH, h0 + step))
        s = scale * np.matmul(q[hs], np.swapaxes(k[hs], -1, -2))
        p = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse[hs, :, None]), 0.0)
        aq[hs] = abs(scale) * e[hs, :, None] * np.matmul(p, np.abs(k[hs]))
        ak[hs] = abs(scale) * np.matmul(np.swapaxes(p, -1, -2), e[hs, :, None] * np.abs(q[hs]))
    return aq.reshape(*lead, N, d), ak.reshape(*lead, N, d)


def default_scale(d):
    return 1.0 / math.sqrt(d)


def oracle_fwd(q, k, v, scale, causal, rows=None):
    return oracle.fwd(f64(q), f64(k), f64(v), scale, causal, rows=rows)
