"""The C-ABI library without a GPU: it loads, exports every declared entry
point, and rejects bad arguments before touching the HIP runtime.

Only calls that fail validation (or have nothing to do) are made here; the
fake device addresses below are never dereferenced or handed to a kernel.
"""
import ctypes
import os
import re

import pytest

import exact_io_aware_40_amd as attn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")

# status codes as declared in the header
OK, E_NULL, E_SHAPE, E_HD, E_DT, E_ALIGN, E_WS, E_LAUNCH, E_SCALE, E_CAUSAL, E_ALIAS, E_SPLIT = (
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11)

# fake, 16-byte aligned, far-apart addresses (validation only)
P = [0x10000000 * (i + 1) for i in range(12)]


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[\w\s\*]*?\b(attn_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    assert declared_functions() == ["attn_bwd", "attn_bwd_dkdv", "attn_bwd_dq", "attn_bwd_dropout",
                                    "attn_bwd_noalloc",
                                    "attn_bwd_workspace_size", "attn_fwd", "attn_fwd_decode", "attn_fwd_decode_fp8",
                                    "attn_fwd_dropout", "attn_fwd_fp8", "attn_fwd_split",
                                    "attn_fwd_split_workspace_size", "attn_probe_hbm", "attn_probe_mfma", "attn_status_str",
                                    "attn_std_fwd",
                                    "attn_std_pv", "attn_std_scores", "attn_std_softmax",
                                    "attn_std_workspace_size"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(attn.library_path())
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings():
    for code in (OK, E_NULL, E_SHAPE, E_HD, E_DT, E_ALIGN, E_WS, E_LAUNCH, E_SCALE, E_CAUSAL,
                 E_ALIAS, E_SPLIT, E_DROP):
        s = attn.attn_status_str(code)
        assert s.startswith("ATTN_")
    assert "unknown" in attn.attn_status_str(12345)


def fwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=3, N=100, d=128, scale=0.1,
             causal=0, dtype=1, out_dtype=None, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    return attn.attn_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                         a["d"], a["scale"], a["causal"], a["dtype"], od, a["stream"])


def fwd_split(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], ws=P[5], wsb=None, B=2, H=3, N=100,
             d=128, scale=0.1, causal=0, dtype=1, out_dtype=None, nsplit=4, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    wsb = a["wsb"]
    if wsb is None:
        wsb = attn.attn_fwd_split_workspace_size(a["B"], a["H"], a["N"], a["d"], a["nsplit"])
    return attn.attn_fwd_split(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], wsb, a["B"],
                               a["H"], a["N"], a["d"], a["scale"], a["causal"], a["dtype"], od,
                               a["nsplit"], a["stream"])


def bwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], dO=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8],
             ws=P[9], wsb=1 << 20, B=2, H=3, N=100, d=128, scale=0.1, causal=1, dtype=1,
             out_dtype=None, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    return attn.attn_bwd(a["q"], a["k"], a["v"], a["o"], a["dO"], a["lse"], a["dq"], a["dk"],
                         a["dv"], a["ws"], a["wsb"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                         a["causal"], a["dtype"], od, a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), E_NULL), (dict(k=0), E_NULL), (dict(v=0), E_NULL), (dict(o=0), E_NULL),
    (dict(lse=0), E_NULL),
    (dict(B=-1), E_SHAPE), (dict(H=-2), E_SHAPE), (dict(N=-5), E_SHAPE),
    (dict(N=1 << 23), E_SHAPE),
    (dict(d=96), E_HD), (dict(d=0), E_HD), (dict(d=256), E_HD),
    (dict(dtype=2), E_DT), (dict(dtype=-1), E_DT), (dict(dtype=1, out_dtype=0), E_DT),
    (dict(dtype=0, out_dtype=1), E_DT), (dict(out_dtype=3), E_DT),
    (dict(out_dtype=2, o=P[4] - 200000), E_ALIAS),   # fp32 o reaches lse
    (dict(q=P[0] + 8), E_ALIGN), (dict(o=P[3] + 2), E_ALIGN), (dict(lse=P[4] + 4), E_ALIGN),
    (dict(scale=float("nan")), E_SCALE), (dict(scale=float("inf")), E_SCALE),
    (dict(causal=2), E_CAUSAL), (dict(causal=-1), E_CAUSAL),
    (dict(o=P[0]), E_ALIAS), (dict(lse=P[1] + 64), E_ALIAS), (dict(lse=P[3] + 128), E_ALIAS),
])
def test_fwd_rejects(kw, code):
    assert fwd(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(N=0, q=0, o=0)])
def test_fwd_empty_is_noop(kw):
    assert fwd(**kw) == OK


def test_workspace_size():
    # two fp32 values per row (D and lse * log2 e), rows padded to 64 per head
    assert attn.attn_bwd_workspace_size(2, 3, 100, 128, 1) == 2 * 6 * 128 * 4
    assert attn.attn_bwd_workspace_size(8, 16, 2048, 128, 1) == 2 * 8 * 16 * 2048 * 4
    assert attn.attn_bwd_workspace_size(0, 3, 100, 128, 1) == 0
    assert attn.attn_bwd_workspace_size(1, 1, 100, 96, 1) == 0
    assert attn.attn_bwd_workspace_size(1, 1, 100, 64, 7) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(dO=0), E_NULL), (dict(lse=0), E_NULL), (dict(dq=0), E_NULL), (dict(dv=0), E_NULL),
    (dict(ws=0), E_WS), (dict(wsb=6143), E_WS),
    (dict(d=32), E_HD), (dict(dtype=5), E_DT), (dict(N=-1), E_SHAPE),
    (dict(ws=P[9] + 4), E_ALIGN), (dict(dk=P[7] + 8), E_ALIGN),
    (dict(scale=float("-inf")), E_SCALE), (dict(causal=3), E_CAUSAL),
    (dict(dq=P[0]), E_ALIAS), (dict(dk=P[6] + 4096), E_ALIAS), (dict(ws=P[8] + 1024), E_ALIAS),
    (dict(dv=P[5]), E_ALIAS), (dict(out_dtype=0), E_DT), (dict(dtype=2, out_dtype=2), E_DT),
    (dict(out_dtype=2, dq=P[7] - 200000), E_ALIAS),   # fp32 dq reaches dk
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def test_bwd_empty_is_noop():
    assert bwd(B=0, ws=0, wsb=0) == OK


def bwd_dq(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], dO=P[4], lse=P[5], dq=P[6], ws=P[9], wsb=1 << 20,
             B=2, H=3, N=100, d=128, scale=0.1, causal=1, dtype=1, out_dtype=None, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    return attn.attn_bwd_dq(a["q"], a["k"], a["v"], a["o"], a["dO"], a["lse"], a["dq"], a["ws"],
                            a["wsb"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                            a["dtype"], od, a["stream"])


def bwd_dkdv(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], dO=P[4], dk=P[7], dv=P[8], ws=P[9], wsb=1 << 20,
             B=2, H=3, N=100, d=128, scale=0.1, causal=1, dtype=1, out_dtype=None, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    return attn.attn_bwd_dkdv(a["q"], a["k"], a["v"], a["dO"], a["dk"], a["dv"], a["ws"],
                              a["wsb"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                              a["dtype"], od, a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(o=0), E_NULL), (dict(lse=0), E_NULL), (dict(dq=0), E_NULL), (dict(q=0), E_NULL),
    (dict(ws=0), E_WS), (dict(wsb=6143), E_WS), (dict(d=80), E_HD), (dict(dtype=3), E_DT),
    (dict(dq=P[9] + 4096), E_ALIAS),           # dq over the workspace it also writes
    (dict(ws=P[3]), E_ALIAS), (dict(dq=P[5]), E_ALIAS), (dict(causal=5), E_CAUSAL),
])
def test_bwd_dq_rejects(kw, code):
    assert bwd_dq(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(dk=0), E_NULL), (dict(dv=0), E_NULL), (dict(dO=0), E_NULL),
    (dict(ws=0), E_WS), (dict(wsb=100), E_WS), (dict(dk=P[7] + 2), E_ALIGN),
    (dict(dk=P[9]), E_ALIAS),                  # dk over the workspace it reads
    (dict(dv=P[7] + 64), E_ALIAS), (dict(dv=P[1]), E_ALIAS), (dict(scale=float("nan")), E_SCALE),
])
def test_bwd_dkdv_rejects(kw, code):
    assert bwd_dkdv(**kw) == code


def test_split_backward_ignores_unused_pointers():
    """Each half validates only what it uses: o, lse may be NULL for the
    dk/dv half, and an empty problem does nothing."""
    assert bwd_dkdv(B=0) == OK and bwd_dq(N=0) == OK
    assert bwd_dkdv(d=96) == E_HD      # still validated before anything else


def test_split_workspace_size():
    # nsplit partial outputs and lse, fp32: nsplit * B*H*N * (d + 1) * 4 bytes
    assert attn.attn_fwd_split_workspace_size(2, 3, 100, 128, 4) == 4 * 6 * 100 * 129 * 4
    assert attn.attn_fwd_split_workspace_size(1, 1, 1, 64, 1) == 65 * 4
    assert attn.attn_fwd_split_workspace_size(0, 3, 100, 128, 4) == 0
    assert attn.attn_fwd_split_workspace_size(2, 3, 100, 96, 4) == 0
    assert attn.attn_fwd_split_workspace_size(2, 3, 100, 128, 0) == 0
    assert attn.attn_fwd_split_workspace_size(2, 3, 100, 128, 65) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(nsplit=0), E_SPLIT), (dict(nsplit=65), E_SPLIT), (dict(nsplit=-3), E_SPLIT),
    (dict(ws=0), E_WS), (dict(wsb=100), E_WS), (dict(ws=P[5] + 8), E_ALIGN),
    (dict(ws=P[0]), E_ALIAS), (dict(ws=P[3]), E_ALIAS), (dict(lse=P[5]), E_ALIAS),
    (dict(o=0), E_NULL), (dict(d=80), E_HD), (dict(causal=2), E_CAUSAL),
    (dict(scale=float("nan")), E_SCALE), (dict(dtype=7), E_DT), (dict(q=P[0] + 2), E_ALIGN),
])
def test_fwd_split_rejects(kw, code):
    assert fwd_split(**kw) == code


def test_fwd_split_empty_is_noop():
    assert fwd_split(B=0) == OK
    assert fwd_split(N=0, ws=0, wsb=0) == OK


E_DROP = -12


def fwd_drop(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=3, N=100, d=128, scale=0.1,
             causal=0, p=0.1, seed=7, offset=3, dtype=1, out_dtype=None, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    return attn.attn_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                                 a["d"], a["scale"], a["causal"], a["p"], a["seed"], a["offset"],
                                 a["dtype"], od, a["stream"])


def bwd_drop(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], dO=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8],
             ws=P[9], wsb=1 << 20, B=2, H=3, N=100, d=128, scale=0.1, causal=1, p=0.1, seed=7,
             offset=3, dtype=1, out_dtype=None, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    return attn.attn_bwd_dropout(a["q"], a["k"], a["v"], a["o"], a["dO"], a["lse"], a["dq"],
                                 a["dk"], a["dv"], a["ws"], a["wsb"], a["B"], a["H"], a["N"],
                                 a["d"], a["scale"], a["causal"], a["p"], a["seed"], a["offset"],
                                 a["dtype"], od, a["stream"])


@pytest.mark.parametrize("p", [-0.1, 1.0, 0.999, float("nan"), float("inf"), 255.5 / 256])
def test_dropout_rejects_probability(p):
    """p must be finite, >= 0, and round to a threshold floor(256 p + 1/2) of
    at most 255; it is checked before anything else, also for empty calls."""
    assert fwd_drop(p=p) == E_DROP
    assert bwd_drop(p=p) == E_DROP
    assert fwd_drop(p=p, B=0) == E_DROP


@pytest.mark.parametrize("p", [0.0, 0.5, 254.49 / 256])
def test_dropout_accepts_probability(p):
    """A valid probability passes on to the shared checks (here: NULL o)."""
    assert fwd_drop(p=p, o=0) == E_NULL
    assert bwd_drop(p=p, dq=0) == E_NULL
    assert fwd_drop(p=p, B=0) == OK


@pytest.mark.parametrize("kw,code", [
    (dict(d=80), E_HD), (dict(causal=2), E_CAUSAL), (dict(scale=float("nan")), E_SCALE),
    (dict(dtype=7), E_DT), (dict(q=P[0] + 2), E_ALIGN), (dict(o=P[0]), E_ALIAS),
])
def test_dropout_shared_validation(kw, code):
    assert fwd_drop(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(ws=0), E_WS), (dict(wsb=100), E_WS), (dict(dq=P[0]), E_ALIAS), (dict(d=96), E_HD),
])
def test_dropout_backward_validation(kw, code):
    assert bwd_drop(**kw) == code


def fwd_decode(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], ws=P[5], wsb=None, B=2, H=3, Nq=4, Nk=1000,
             d=128, scale=0.1, causal=1, dtype=1, out_dtype=None, nsplit=8, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    wsb = a["wsb"]
    if wsb is None:
        wsb = attn.attn_fwd_split_workspace_size(a["B"], a["H"], max(a["Nq"], 1), a["d"], a["nsplit"])
    return attn.attn_fwd_decode(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], wsb, a["B"],
                                a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"],
                                a["dtype"], od, a["nsplit"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Nq=-1), E_SHAPE), (dict(Nk=-5), E_SHAPE), (dict(Nk=2**23), E_SHAPE),
    (dict(nsplit=0), E_SPLIT), (dict(nsplit=65), E_SPLIT), (dict(ws=0), E_WS), (dict(wsb=64), E_WS),
    (dict(k=0), E_NULL), (dict(o=P[1]), E_ALIAS), (dict(ws=P[2]), E_ALIAS), (dict(d=32), E_HD),
    (dict(causal=3), E_CAUSAL), (dict(v=P[2] + 4), E_ALIGN),
])
def test_fwd_decode_rejects(kw, code):
    assert fwd_decode(**kw) == code


def test_fwd_decode_empty_is_noop():
    """No query rows (or no heads) means nothing to do; no keys still has
    rows to write (o = 0, lse = -inf), so the pointers are checked."""
    assert fwd_decode(Nq=0, ws=0, wsb=0) == OK
    assert fwd_decode(B=0) == OK
    assert fwd_decode(Nk=0, o=0) == E_NULL


def fwd_fp8(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], B=2, H=3, N=100, d=128, scale=0.1,
             qd=0.01, kd=0.02, vd=0.03, causal=1, out_dtype=1, stream=0)
    a.update(kw)
    return attn.attn_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"],
                             a["d"], a["scale"], a["qd"], a["kd"], a["vd"], a["causal"],
                             a["out_dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=64), E_HD), (dict(d=96), E_HD), (dict(out_dtype=3), E_DT), (dict(out_dtype=-1), E_DT),
    (dict(causal=2), E_CAUSAL), (dict(B=-1), E_SHAPE), (dict(N=-5), E_SHAPE),
    (dict(scale=float("inf")), E_SCALE), (dict(scale=float("nan")), E_SCALE),
    (dict(qd=0.0), E_SCALE), (dict(kd=-1.0), E_SCALE), (dict(vd=float("nan")), E_SCALE),
    (dict(vd=0.0), E_SCALE), (dict(kd=float("inf")), E_SCALE),
    (dict(scale=1e30, qd=1e30, kd=1e30), E_SCALE),
    (dict(q=0), E_NULL), (dict(lse=0), E_NULL), (dict(o=P[3] + 8), E_ALIGN),
    (dict(o=P[0]), E_ALIAS), (dict(lse=P[2] + 16), E_ALIAS), (dict(N=1 << 23), E_SHAPE),
])
def test_fwd_fp8_rejects(kw, code):
    assert fwd_fp8(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0), dict(N=0, q=0, o=0)])
def test_fwd_fp8_empty_is_noop(kw):
    assert fwd_fp8(**kw) == OK


def fwd_decode_fp8(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], ws=P[5], wsb=None, B=2, H=3, Nq=4, Nk=300,
             d=128, scale=0.1, qd=0.01, kd=0.02, vd=0.03, causal=1, out_dtype=1, nsplit=4, stream=0)
    a.update(kw)
    wsb = a["wsb"]
    if wsb is None:
        wsb = attn.attn_fwd_split_workspace_size(max(a["B"], 0), max(a["H"], 0), max(a["Nq"], 0), 128,
                                                 min(max(a["nsplit"], 1), 64))
    return attn.attn_fwd_decode_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], wsb, a["B"],
                                    a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["qd"], a["kd"],
                                    a["vd"], a["causal"], a["out_dtype"], a["nsplit"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(d=64), E_HD), (dict(out_dtype=3), E_DT), (dict(causal=2), E_CAUSAL),
    (dict(Nq=-1), E_SHAPE), (dict(Nk=-1), E_SHAPE), (dict(B=-1), E_SHAPE),
    (dict(qd=0.0), E_SCALE), (dict(vd=float("inf")), E_SCALE), (dict(scale=float("nan")), E_SCALE),
    (dict(nsplit=0), E_SPLIT), (dict(nsplit=65), E_SPLIT),
    (dict(q=0), E_NULL), (dict(ws=0), E_WS), (dict(wsb=16), E_WS), (dict(ws=P[5] + 8), E_ALIGN),
    (dict(o=P[1]), E_ALIAS), (dict(ws=P[0]), E_ALIAS),
])
def test_fwd_decode_fp8_rejects(kw, code):
    assert fwd_decode_fp8(**kw) == code


@pytest.mark.parametrize("kw", [dict(B=0), dict(Nq=0), dict(Nq=0, q=0, ws=0)])
def test_fwd_decode_fp8_empty_is_noop(kw):
    assert fwd_decode_fp8(**kw) == OK


# ---------------------------------------------------------------------------
# materialised standard attention (validation only)
# ---------------------------------------------------------------------------

def std_fwd(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], lse=P[4], ws=P[5], wsb=None, B=2, H=3, N=100,
             d=128, scale=0.1, causal=0, dtype=1, out_dtype=None, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    wsb = a["wsb"]
    if wsb is None:
        wsb = attn.attn_std_workspace_size(a["B"], a["H"], a["N"], a["d"], a["dtype"])
    return attn.attn_std_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"], wsb, a["B"], a["H"],
                             a["N"], a["d"], a["scale"], a["causal"], a["dtype"], od, a["stream"])


def test_std_workspace_size():
    # s in fp32 rounded up to 256 bytes, then p in 16 bits
    n = 2 * 3 * 100 * 100
    assert attn.attn_std_workspace_size(2, 3, 100, 128, 1) == (n * 4 + 255) // 256 * 256 + n * 2
    assert attn.attn_std_workspace_size(2, 3, 100, 64, 0) == (n * 4 + 255) // 256 * 256 + n * 2
    assert attn.attn_std_workspace_size(0, 3, 100, 64, 0) == 0
    assert attn.attn_std_workspace_size(1, 1, 40000, 64, 0) == 0      # N above ATTN_STD_MAX_N
    assert attn.attn_std_workspace_size(1, 1, 100, 96, 0) == 0        # bad d
    assert attn.attn_std_workspace_size(1, 1, 100, 64, 2) == 0        # fp32 is not an input type


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), E_NULL), (dict(lse=0), E_NULL), (dict(ws=0), E_WS),
    (dict(wsb=1000), E_WS), (dict(d=96), E_HD), (dict(dtype=2), E_DT), (dict(out_dtype=0), E_DT),
    (dict(N=40000), E_SHAPE), (dict(N=-1), E_SHAPE), (dict(causal=2), E_CAUSAL),
    (dict(scale=float("inf")), E_SCALE), (dict(o=P[3] + 8), E_ALIGN), (dict(ws=P[5] + 8), E_ALIGN),
    (dict(o=P[1]), E_ALIAS), (dict(ws=P[3]), E_ALIAS), (dict(lse=P[5] + 256), E_ALIAS),
])
def test_std_fwd_rejects(kw, code):
    assert std_fwd(**kw) == code


def test_std_fwd_empty_is_noop():
    assert std_fwd(B=0, q=0, k=0, v=0, o=0, lse=0, ws=0, wsb=0) == OK
    assert std_fwd(N=0, q=0, ws=0, wsb=0) == OK


def test_std_passes_reject():
    assert attn.attn_std_scores(0, P[1], P[2], 2, 3, 100, 128, 0.1, 1, 0) == E_NULL
    assert attn.attn_std_scores(P[0], P[1], P[2] + 4, 2, 3, 100, 128, 0.1, 1, 0) == E_ALIGN
    assert attn.attn_std_scores(P[0], P[1], P[0], 2, 3, 100, 128, 0.1, 1, 0) == E_ALIAS
    assert attn.attn_std_scores(P[0], P[1], P[2], 2, 3, 100, 80, 0.1, 1, 0) == E_HD
    assert attn.attn_std_softmax(P[0], 0, P[2], 2, 3, 100, 0, 1, 0) == E_NULL
    assert attn.attn_std_softmax(P[0], P[0], P[2], 2, 3, 100, 0, 1, 0) == E_ALIAS
    assert attn.attn_std_softmax(P[0], P[1], P[2], 2, 3, 100, 3, 1, 0) == E_CAUSAL
    assert attn.attn_std_softmax(P[0], P[1], P[2], 2, 3, 40000, 0, 1, 0) == E_SHAPE
    assert attn.attn_std_pv(P[0], P[1], 0, 2, 3, 100, 64, 1, 1, 0) == E_NULL
    assert attn.attn_std_pv(P[0], P[1], P[0], 2, 3, 100, 64, 1, 1, 0) == E_ALIAS
    assert attn.attn_std_pv(P[0], P[1], P[2], 2, 3, 100, 64, 1, 0, 0) == E_DT
    assert attn.attn_std_pv(P[0], P[1], P[2], 0, 3, 100, 64, 1, 1, 0) == OK


def test_mfma_probe_rejects():
    """The matrix-core rate probe validates before launching (no GPU needed)."""
    assert attn.attn_probe_mfma(0, 512, 100, 0) == E_NULL
    assert attn.attn_probe_mfma(P[0] + 4, 512, 100, 0) == E_ALIGN
    for wg, it in ((0, 100), (-1, 100), ((1 << 20) + 1, 100), (512, 0), (512, -3), (512, (1 << 24) + 1)):
        assert attn.attn_probe_mfma(P[0], wg, it, 0) == E_SHAPE, (wg, it)


def test_hbm_probe_rejects():
    """The HBM read probe validates before launching (no GPU needed)."""
    assert attn.attn_probe_hbm(0, 1 << 20, P[1], 64, 0) == E_NULL
    assert attn.attn_probe_hbm(P[0], 1 << 20, 0, 64, 0) == E_NULL
    assert attn.attn_probe_hbm(P[0] + 8, 1 << 20, P[1], 64, 0) == E_ALIGN
    assert attn.attn_probe_hbm(P[0], 1 << 20, P[1] + 4, 64, 0) == E_ALIGN
    for nb, wg in ((0, 64), (8, 64), (24, 64), ((1 << 42) + 16, 64), (1 << 20, 0), (1 << 20, (1 << 20) + 1)):
        assert attn.attn_probe_hbm(P[0], nb, P[1], wg, 0) == E_SHAPE, (nb, wg)
    # the sums may not land in the buffer being read
    assert attn.attn_probe_hbm(P[0], 1 << 20, P[0] + (1 << 19), 64, 0) == E_ALIAS


# ---------------------------------------------------------------------------
# backward without a workspace argument (validation only)
# ---------------------------------------------------------------------------

def bwd_noalloc(**kw):
    a = dict(q=P[0], k=P[1], v=P[2], o=P[3], dO=P[4], lse=P[5], dq=P[6], dk=P[7], dv=P[8],
             B=2, H=3, N=100, d=128, scale=0.1, causal=1, dtype=1, out_dtype=None, stream=0)
    a.update(kw)
    od = a["dtype"] if a["out_dtype"] is None else a["out_dtype"]
    return attn.attn_bwd_noalloc(a["q"], a["k"], a["v"], a["o"], a["dO"], a["lse"], a["dq"],
                                 a["dk"], a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"],
                                 a["causal"], a["dtype"], od, a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), E_NULL), (dict(dv=0), E_NULL), (dict(d=80), E_HD), (dict(dtype=3), E_DT),
    (dict(causal=5), E_CAUSAL), (dict(scale=float("nan")), E_SCALE), (dict(dk=P[7] + 4), E_ALIGN),
    (dict(dq=P[0]), E_ALIAS),
    # workspace rows past the fixed 16 MiB scratch: B*H*ceil(N/64)*64 > 2^21
    (dict(B=1, H=1, N=(1 << 21) + 1, d=64), E_WS), (dict(B=33, H=1, N=65536, d=64), E_WS),
])
def test_bwd_noalloc_rejects(kw, code):
    assert bwd_noalloc(**kw) == code


def test_bwd_noalloc_empty_is_noop():
    assert bwd_noalloc(B=0, q=0, k=0) == OK
    assert bwd_noalloc(N=0, dq=0) == OK
