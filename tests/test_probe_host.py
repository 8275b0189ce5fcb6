"""The probes' host-side reference values (CPU only): the operand values
are normal bf16 numbers of either sign in [0.5, 2), and the per-thread
checksum formula of the HBM probe agrees with a direct loop over granules."""
import numpy as np

from tests._probe_ref import expected_thread_sums, probe_values


def test_probe_operands_are_normal_bf16():
    v = probe_values(np.arange(1 << 16))
    assert np.all((np.abs(v) >= 0.5) & (np.abs(v) < 2.0))
    assert 0.45 < np.mean(v > 0) < 0.55 and len(np.unique(v)) == 512


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
