"""The measurement probes on the GPU.  attn_probe_mfma: its products are
those its operand definition gives (checked on the host in fp64), and its
timed rate is a plausible fraction of the published peak.  attn_probe_hbm:
every thread's checksum is the host's for the granules it reads, and its
timed read rate is plausible."""
import numpy as np
import pytest
import torch

import exact_io_aware_40_amd as attn
from tests._probe_ref import expected_lane_sums, expected_thread_sums
from tests._util import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


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
