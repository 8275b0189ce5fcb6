"""The measurement probes on the GPU.  attn_probe_mfma: its products are
those its operand definition gives (checked on the host in fp64), and its
timed rate is a plausible fraction of the published peak.  attn_probe_hbm:
every thread's checksum is the host's for the granules it reads, and its
timed read rate is plausible."""
import numpy as np
import pytest
import torch

import exact_io_aware_40_amd as attn
from tests._util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


def probe_values(x):
    """The probe's operand values for indices x (uint32): the MurmurHash3
    finaliser of x, keeping bit 15 (sign), bits 0..6 (mantissa) and bit 8 as
    the low exponent bit (exponent 126 or 127) of a bf16 number."""
    x = np.asarray(x, dtype=np.uint64) & 0xFFFFFFFF
    x ^= x >> 16
    x = (x * 0x85EBCA6B) & 0xFFFFFFFF
    x ^= x >> 13
    x = (x * 0xC2B2AE35) & 0xFFFFFFFF
    x ^= x >> 16
    bits = (x & 0x807F) | 0x3F00 | ((x >> 1) & 0x80)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def expected_lane_sums(rounds):
    """Every lane's sum of its 64 accumulators: chain j adds, per round,
    A_j (B_0 + B_1 + B_2 + B_3), with the 32x32x16 operand layout (lane l
    holds A[m = l % 32][k = 8 (l / 32) + e], B[k = 8 (l / 32) + e][n = l %
    32], and D[8 (r / 4) + 4 (l / 32) + r % 4][l % 32] for r = 0..15)."""
    lane = np.arange(64)

    def operand(j):   # [lane, e]
        return probe_values(64 * (8 * j + np.arange(8))[None, :] + lane[:, None])

    def as_a(x):
        A = np.zeros((32, 16))
        for l in range(64):
            A[l % 32, 8 * (l // 32):8 * (l // 32) + 8] = x[l]
        return A

    def as_b(x):
        Bm = np.zeros((16, 32))
        for l in range(64):
            Bm[8 * (l // 32):8 * (l // 32) + 8, l % 32] = x[l]
        return Bm

    bsum = sum(as_b(operand(j + 4)) for j in range(4))
    D = rounds * sum(as_a(operand(j)) @ bsum for j in range(4))
    Dabs = rounds * sum(np.abs(as_a(operand(j))) @ sum(np.abs(as_b(operand(j + 4))) for j in range(4))
                        for j in range(4))
    want, scale = np.zeros(64), np.zeros(64)
    for l in range(64):
        rows = [8 * (r // 4) + 4 * (l // 32) + r % 4 for r in range(16)]
        want[l] = sum(D[m, l % 32] for m in rows)
        scale[l] = sum(Dabs[m, l % 32] for m in rows)
    return want, scale


def test_probe_operands_are_normal_bf16():
    v = probe_values(np.arange(1 << 16))
    assert np.all((np.abs(v) >= 0.5) & (np.abs(v) < 2.0))
    assert 0.45 < np.mean(v > 0) < 0.55 and len(np.unique(v)) == 512


@pytest.mark.parametrize("rounds", [1, 3, 17])
def test_probe_products(rounds):
    announce(f"mfma probe rounds={rounds}")
    wg = 6
    out = torch.full((wg * 256,), float("nan"), dtype=torch.float32, device=DEV)
    st = attn.attn_probe_mfma(out.data_ptr(), wg, rounds, torch.cuda.current_stream().cuda_stream)
    assert st == 0, attn.attn_status_str(st)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(wg * 4, 64).astype(np.float64)
    want, scale = expected_lane_sums(rounds)
    # fp32 accumulation of products exact in fp32: the error is a few fp32
    # roundings of partial sums, far below 2^-16 of the terms' magnitudes
    err = np.abs(got - want[None, :])
    assert np.all(err <= 2.0 ** -16 * scale[None, :]), float((err / scale).max())
    assert np.array_equal(got, np.broadcast_to(got[0], got.shape))   # every wave the same


def test_probe_rate_is_plausible():
    announce("mfma probe rate")
    props = torch.cuda.get_device_properties(0)
    wg, rounds = 2 * props.multi_processor_count, 5000
    out = torch.empty(wg * 256, dtype=torch.float32, device=DEV)
    sp = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        assert attn.attn_probe_mfma(out.data_ptr(), wg, rounds, sp) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    assert attn.attn_probe_mfma(out.data_ptr(), wg, rounds, sp) == 0
    e1.record()
    e1.synchronize()
    ms = e0.elapsed_time(e1)
    tflops = wg * 4 * 16 * rounds * 32768 / (ms * 1e-3) / 1e12
    print(f"[probe] {wg} workgroups x {rounds} rounds: {ms:.3f} ms, {tflops:.0f} TFLOP/s", flush=True)
    assert 200.0 < tflops < 2600.0
    assert bool(torch.isfinite(out).all())


def expected_thread_sums(words, wg):
    """Thread 64 (4 b + w) + l's sum (mod 2^32) of the words of granule
    64 c + l of the 1 KiB chunks c of workgroup b's range (b C .. (b + 1) C,
    C = ceil(chunks / wg)) with c - b C = w mod 4."""
    g = words.reshape(-1, 4).astype(np.uint64).sum(axis=1) & 0xFFFFFFFF   # per 16-byte granule
    g = np.concatenate([g, np.zeros((-len(g)) % 64, dtype=np.uint64)]).reshape(-1, 64)   # [chunk, lane]
    per = -(-len(g) // wg)
    g = np.concatenate([g, np.zeros((wg * per - len(g), 64), dtype=np.uint64)]).reshape(wg, per, 64)
    g = np.concatenate([g, np.zeros((wg, (-per) % 4, 64), dtype=np.uint64)], axis=1).reshape(wg, -1, 4, 64)
    return (g.sum(axis=1) & 0xFFFFFFFF).astype(np.uint32).reshape(-1)


def test_expected_thread_sums_by_brute_force():
    rng = np.random.default_rng(7)
    for granules, wg in ((1, 1), (65, 1), (1000, 2), (3000, 5), (64 * 7 + 3, 3)):
        w = rng.integers(0, 1 << 32, size=4 * granules, dtype=np.uint64).astype(np.uint32)
        want = [0] * (256 * wg)
        nch = -(-granules // 64)
        per = -(-nch // wg)
        for gi in range(granules):
            c = gi // 64
            b = c // per
            t = 256 * b + 64 * ((c - b * per) % 4) + gi % 64
            want[t] = (want[t] + int(w[4 * gi:4 * gi + 4].astype(np.uint64).sum())) % (1 << 32)
        assert np.array_equal(expected_thread_sums(w, wg), np.array(want, dtype=np.uint32))


@pytest.mark.parametrize("granules,wg", [(1, 1), (255, 1), (1000003, 37), (1 << 20, 512), (777, 4096),
                                         (64 * 8 * 4 * 3 + 5, 1)])
def test_hbm_probe_sums(granules, wg):
    """Every thread's checksum equals the host's, for ragged sizes, fewer
    granules than threads, and more than four granules per thread."""
    announce(f"hbm probe granules={granules} wg={wg}")
    rng = np.random.default_rng(granules)
    words = rng.integers(0, 1 << 32, size=4 * granules, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    out = torch.full((wg * 256,), 0x5A5A5A5A, dtype=torch.int32, device=DEV)
    st = attn.attn_probe_hbm(buf.data_ptr(), 16 * granules, out.data_ptr(), wg,
                             torch.cuda.current_stream().cuda_stream)
    assert st == 0, attn.attn_status_str(st)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected_thread_sums(words, wg))


def test_hbm_probe_rate_is_plausible():
    announce("hbm probe rate")
    nbytes = 1 << 30
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
    wg = 16 * torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.empty(wg * 256, dtype=torch.int32, device=DEV)
    sp = torch.cuda.current_stream().cuda_stream
    for _ in range(3):
        assert attn.attn_probe_hbm(buf.data_ptr(), nbytes, out.data_ptr(), wg, sp) == 0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    assert attn.attn_probe_hbm(buf.data_ptr(), nbytes, out.data_ptr(), wg, sp) == 0
    e1.record()
    e1.synchronize()
    gbs = nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    print(f"[probe] hbm read {nbytes >> 20} MiB, {wg} workgroups: {gbs:.0f} GB/s", flush=True)
    assert 1000.0 < gbs < 9000.0
    assert bool((out == 0).all())
