"""Host-side reference values of the measurement probes (attn_probe_mfma,
attn_probe_hbm): what each thread of a launch must store, computed with
NumPy from the probes' definitions in include/attn.h."""
import numpy as np


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
