"""Pins for the fp64 CPU oracle.

Each test ties the oracle to something other than itself: values the pages
print, closed forms, invariants of the mathematics, an independent library
routine (torch's CPU scaled_dot_product_attention in fp64), an independent
materialised NumPy implementation, or finite differences.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import brute

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------------------
# The pages' worked examples
# ---------------------------------------------------------------------------

def _page_example():
    with open(os.path.join(GOLDEN, "online_softmax_8.json")) as f:
        return json.load(f)


def test_online_softmax_page_example():
    """Explainer Step 4: eight scores read two at a time; the result shown
    to two decimals is the full softmax."""
    g = _page_example()
    x = np.array(g["scores"])
    y, st = oracle.online_softmax(x, g["chunk"])
    assert len(st) == g["n_chunks"] == 4
    np.testing.assert_array_equal(np.round(y, 2), np.array(g["full_softmax_2dp"]))
    # running max after each chunk is the max of the prefix read so far
    np.testing.assert_array_equal(st[:, 0], [3.0, 3.0, 4.5, 4.5])
    # first chunk: empty history, no rescale ("none yet")
    assert math.isnan(st[0, 2])
    # chunk 2 (2.1 after 0.4) and chunk 4 keep the max: factor exactly 1
    assert st[1, 2] == 1.0 and st[3, 2] == 1.0
    # chunk 3 lifts the max from 3.0 to 4.5: factor e^(3.0 - 4.5)
    assert st[2, 2] == pytest.approx(math.exp(-1.5), rel=1e-15)
    # probabilities sum to one
    assert abs(y.sum() - 1.0) < 1e-15


@pytest.mark.parametrize("chunk", [1, 2, 3, 4, 5, 8, 100])
def test_online_softmax_chunk_invariance(chunk):
    """'Exact, not approximate': any chunking gives the one-shot softmax."""
    g = _page_example()
    x = np.array(g["scores"])
    y_ref, _ = oracle.online_softmax(x, len(x))
    y, _ = oracle.online_softmax(x, chunk)
    np.testing.assert_allclose(y, y_ref, rtol=0, atol=2e-16)


def test_attention_probe_exposes_softmax():
    """With q = e0, k_j = x_j e0, one-hot v_j = e_j and scale 1, row 0 of O
    is the softmax of the page's eight scores."""
    g = _page_example()
    x = np.array(g["scores"])
    N = d = 8
    q = np.zeros((N, d)); q[:, 0] = 1.0
    k = np.zeros((N, d)); k[:, 0] = x
    v = np.eye(N)
    o, lse = oracle.fwd(q, k, v, 1.0)
    np.testing.assert_array_equal(np.round(o[0], 2), np.array(g["full_softmax_2dp"]))
    y, _ = oracle.online_softmax(x, 2)
    np.testing.assert_allclose(o[0], y, rtol=0, atol=1e-15)
    # every row sees the same scores here
    np.testing.assert_allclose(o, np.tile(o[0], (N, 1)), rtol=0, atol=0)


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_equals_standard_page_check(causal):
    """Explainer Step 6: d = 8, four tiles of up to four keys; the tiled
    online-softmax output differs from standard attention only by rounding
    (the page shows 2.2e-16)."""
    N, d = 16, 8
    q, k, v = rand((N, d), 1), rand((N, d), 2), rand((N, d), 3)
    o_t, lse_t = oracle.fwd_online(q, k, v, 1 / math.sqrt(d), causal, tile=4)
    o, lse = oracle.fwd(q, k, v, 1 / math.sqrt(d), causal)
    assert np.abs(o_t - o).max() <= 1e-15
    assert np.abs(lse_t - lse).max() <= 1e-14
    o_b, lse_b, _ = brute.fwd(q, k, v, 1 / math.sqrt(d), causal)
    assert np.abs(o_t - o_b).max() <= 1e-15


# ---------------------------------------------------------------------------
# Closed forms and invariants of the forward
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_rows_of_p_sum_to_one(causal):
    """A column of ones in V comes out as ones: every row of P sums to 1."""
    B, H, N, d = 2, 3, 37, 16
    q, k, v = rand((B, H, N, d), 4) * 3, rand((B, H, N, d), 5) * 3, rand((B, H, N, d), 6)
    v[..., 0] = 1.0
    o, _ = oracle.fwd(q, k, v, 0.7, causal)
    assert np.abs(o[..., 0] - 1.0).max() <= 1e-15


@pytest.mark.parametrize("causal", [False, True])
def test_equal_scores_give_mean_v(causal):
    """Q = 0 makes every score equal: O is the mean of the visible V rows and
    lse = ln(number of visible keys)."""
    B, H, N, d = 1, 2, 29, 8
    q = np.zeros((B, H, N, d))
    k, v = rand((B, H, N, d), 7), rand((B, H, N, d), 8)
    o, lse = oracle.fwd(q, k, v, 0.5, causal)
    if causal:
        counts = np.arange(1, N + 1)
        mean = np.cumsum(v, axis=-2) / counts[:, None]
        np.testing.assert_allclose(lse, np.broadcast_to(np.log(counts), lse.shape), atol=1e-15)
    else:
        mean = np.broadcast_to(v.mean(axis=-2, keepdims=True), v.shape)
        np.testing.assert_allclose(lse, math.log(N), atol=1e-15)
    np.testing.assert_allclose(o, mean, rtol=0, atol=1e-15)


def test_single_key():
    """N = 1: the only key takes all the weight; lse is that key's score."""
    q, k, v = rand((3, 1, 16), 9), rand((3, 1, 16), 10), rand((3, 1, 16), 11)
    for causal in (False, True):
        o, lse = oracle.fwd(q, k, v, 0.25, causal)
        np.testing.assert_array_equal(o, v)
        np.testing.assert_allclose(lse[:, 0], 0.25 * np.sum(q[:, 0] * k[:, 0], axis=-1), rtol=1e-15)


def test_causal_row_zero_is_v0():
    q, k, v = rand((2, 20, 8), 12), rand((2, 20, 8), 13), rand((2, 20, 8), 14)
    o, _ = oracle.fwd(q, k, v, 1.0, True)
    np.testing.assert_array_equal(o[:, 0], v[:, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_affine_in_v(causal):
    """Rows of P sum to one, so O(a V + b) = a O(V) + b."""
    q, k, v = rand((2, 33, 8), 15), rand((2, 33, 8), 16), rand((2, 33, 8), 17)
    o, _ = oracle.fwd(q, k, v, 0.3, causal)
    o2, _ = oracle.fwd(q, k, 2.5 * v - 1.25, 0.3, causal)
    np.testing.assert_allclose(o2, 2.5 * o - 1.25, rtol=0, atol=1e-14)


def test_key_permutation_invariance():
    """Without a mask, reordering the (k_j, v_j) pairs changes nothing."""
    N, d = 41, 8
    q, k, v = rand((N, d), 18), rand((N, d), 19), rand((N, d), 20)
    perm = np.random.default_rng(21).permutation(N)
    o, lse = oracle.fwd(q, k, v, 0.4, False)
    o2, lse2 = oracle.fwd(q, k[perm], v[perm], 0.4, False)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse2, lse, rtol=0, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_shift_of_keys(causal):
    """Adding a vector c to every key adds scale*q_i.c to row i's scores:
    O is unchanged and lse moves by exactly that amount."""
    N, d = 23, 8
    q, k, v = rand((N, d), 22), rand((N, d), 23), rand((N, d), 24)
    c = rand((d,), 25) * 4
    o, lse = oracle.fwd(q, k, v, 0.6, causal)
    o2, lse2 = oracle.fwd(q, k + c, v, 0.6, causal)
    np.testing.assert_allclose(o2, o, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse2, lse + 0.6 * (q @ c), rtol=0, atol=1e-12)


def test_large_logits_are_stable():
    """Scores near +-1000 would overflow exp without the max subtraction
    (explainer Step 4: fp16 overflows above e^11.1); the oracle stays finite
    and matches the same problem with every score shifted down."""
    N, d = 16, 4
    q = np.zeros((N, d)); q[:, 0] = 1.0
    k = rand((N, d), 26); k[:, 0] = 1000.0 + np.arange(N) * 0.5
    v = rand((N, d), 27)
    o, lse = oracle.fwd(q, k, v, 1.0, False)
    k2 = k.copy(); k2[:, 0] -= 1000.0
    o2, lse2 = oracle.fwd(q, k2, v, 1.0, False)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    np.testing.assert_allclose(o, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse - 1000.0, lse2, rtol=0, atol=1e-12)


def test_row_subset_matches_full():
    B, H, N, d = 2, 2, 50, 8
    q, k, v = rand((B, H, N, d), 28), rand((B, H, N, d), 29), rand((B, H, N, d), 30)
    for causal in (False, True):
        o, lse = oracle.fwd(q, k, v, 0.35, causal)
        rows = np.array([0, 7, 49, 50, 123, 199])
        o_s, lse_s = oracle.fwd(q, k, v, 0.35, causal, rows=rows)
        np.testing.assert_array_equal(o_s, o.reshape(-1, d)[rows])
        np.testing.assert_array_equal(lse_s, lse.reshape(-1)[rows])


@pytest.mark.parametrize("shape", [(1, 1, 1, 4), (1, 2, 5, 8), (2, 1, 17, 16), (1, 3, 64, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_matches_materialised_brute_force(shape, causal):
    q, k, v = rand(shape, 31) * 2, rand(shape, 32) * 2, rand(shape, 33)
    o, lse = oracle.fwd(q, k, v, 0.8, causal)
    o_b, lse_b, _ = brute.fwd(q, k, v, 0.8, causal)
    assert np.abs(o - o_b).max() <= 1e-12
    assert np.abs(lse - lse_b).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_matches_torch_sdpa_fp64(causal):
    """torch's CPU scaled_dot_product_attention in fp64 is an independent
    library implementation of the same definition."""
    shape = (2, 3, 45, 16)
    q, k, v = rand(shape, 34), rand(shape, 35), rand(shape, 36)
    scale = 1 / math.sqrt(16)
    o, _ = oracle.fwd(q, k, v, scale, causal)
    t = [torch.from_numpy(a) for a in (q, k, v)]
    ref = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=scale)
    assert np.abs(o - ref.numpy()).max() <= 1e-13


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def _loss(q, k, v, dO, scale, causal):
    o, _ = oracle.fwd(q, k, v, scale, causal)
    return float(np.sum(o * dO))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N,d", [(1, 3), (5, 4), (8, 2)])
def test_backward_finite_differences(causal, N, d):
    """Central differences of L = sum(O * dO) pin the gradient formulas
    without restating them."""
    rng = np.random.default_rng(37 + N)
    q, k, v, dO = (rng.standard_normal((N, d)) for _ in range(4))
    scale = 0.9
    _, _, dq, dk, dv = oracle.bwd(q, k, v, dO, scale, causal)
    h = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], dO, scale, causal)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], dO, scale, causal)
            num[idx] = (lp - lm) / (2 * h)
        err = np.abs(num - g).max() / max(1.0, np.abs(g).max())
        assert err <= 1e-6, (name, err)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_invariants(causal):
    """Rows of dS sum to zero, so the key gradients sum to zero; the value
    gradients sum to the summed upstream gradient (rows of P sum to one)."""
    shape = (2, 2, 40, 8)
    q, k, v, dO = (rand(shape, s) for s in (40, 41, 42, 43))
    o, lse, dq, dk, dv = oracle.bwd(q, k, v, dO, 0.5, causal)
    assert np.abs(dk.sum(axis=-2)).max() <= 1e-12
    np.testing.assert_allclose(dv.sum(axis=-2), dO.sum(axis=-2), rtol=0, atol=1e-12)
    o_f, lse_f = oracle.fwd(q, k, v, 0.5, causal)
    np.testing.assert_array_equal(o, o_f)
    np.testing.assert_array_equal(lse, lse_f)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_with_stored_output(causal):
    """Given the exact forward output, D_i = dO_i . o_i equals
    sum_j P_ij dP_ij, so the gradients do not change; given a perturbed o,
    dv (which does not involve D) is unchanged and dq moves by exactly
    -scale * dD_i * sum_j P_ij k_j."""
    shape = (2, 2, 30, 8)
    q, k, v, dO = (rand(shape, s) for s in (60, 61, 62, 63))
    o, lse, dq, dk, dv = oracle.bwd(q, k, v, dO, 0.5, causal)
    _, _, dq2, dk2, dv2 = oracle.bwd(q, k, v, dO, 0.5, causal, o_in=o)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert np.abs(a - b).max() <= 1e-13
    eps = rand(shape, 64) * 1e-3
    _, _, dq3, dk3, dv3 = oracle.bwd(q, k, v, dO, 0.5, causal, o_in=o + eps)
    np.testing.assert_array_equal(dv3, dv)
    dD = np.sum(dO * eps, axis=-1)                       # change of D_i
    _, _, p = brute.fwd(q, k, v, 0.5, causal)
    np.testing.assert_allclose(dq3 - dq, -0.5 * dD[..., None] * (p @ k), rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float16])
def test_stored_o_allowance(causal, dtype):
    """The GPU tests' allowance for a backward fed a 16-bit o: the oracle's
    gradients from o rounded to the type, and from o moved by a whole ulp
    against the sign of dO (the largest change of D the bound admits), stay
    within it; the second reaches it (the bound is tight, not vacuous)."""
    from tests._util import stored_o_allowance, ulp
    shape = (2, 3, 40, 16)
    q, k, v, dO = (rand(shape, s) for s in (70, 71, 72, 73))
    o, lse, dq, dk, dv = oracle.bwd(q, k, v, dO, 0.3, causal)
    aq, ak = stored_o_allowance(q, k, dO, o, lse, 0.3, causal, dtype)
    o16 = torch.from_numpy(o).to(dtype).double().numpy()
    worst = o - ulp(o, dtype) * np.sign(dO)
    for o_in, tight in ((o16, False), (worst, True)):
        _, _, dq2, dk2, dv2 = oracle.bwd(q, k, v, dO, 0.3, causal, o_in=o_in)
        np.testing.assert_array_equal(dv2, dv)
        assert np.all(np.abs(dq2 - dq) <= aq * (1 + 1e-9) + 1e-15)
        assert np.all(np.abs(dk2 - dk) <= ak * (1 + 1e-9) + 1e-15)
        if tight:
            # dq_i's change is -scale e_i sum_j P_ij k_j: the bound uses |k|
            # inside the sum, so it is reached where one key dominates; the
            # sum over heads and rows reaches a fair fraction of it
            assert (np.abs(dq2 - dq).sum() / aq.sum()) > 0.2


def test_backward_single_key():
    """N = 1: P = 1 so dq = dk = 0 and dv = dO."""
    q, k, v, dO = (rand((3, 1, 8), s) for s in (44, 45, 46, 47))
    for causal in (False, True):
        _, _, dq, dk, dv = oracle.bwd(q, k, v, dO, 0.7, causal)
        assert np.abs(dq).max() == 0 and np.abs(dk).max() == 0
        np.testing.assert_array_equal(dv, dO)


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_brute_and_autograd(causal):
    shape = (2, 2, 33, 16)
    q, k, v, dO = (rand(shape, s) for s in (48, 49, 50, 51))
    scale = 0.25
    _, _, dq, dk, dv = oracle.bwd(q, k, v, dO, scale, causal)
    _, _, dq_b, dk_b, dv_b = brute.bwd(q, k, v, dO, scale, causal)
    for a, b in ((dq, dq_b), (dk, dk_b), (dv, dv_b)):
        assert np.abs(a - b).max() <= 1e-12
    t = [torch.from_numpy(a).requires_grad_(True) for a in (q, k, v)]
    out = torch.nn.functional.scaled_dot_product_attention(*t, is_causal=causal, scale=scale)
    out.backward(torch.from_numpy(dO))
    for a, tt in ((dq, t[0]), (dk, t[1]), (dv, t[2])):
        assert np.abs(a - tt.grad.numpy()).max() <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bounds", [[0, 37], [0, 5, 5, 37], [0, 1, 2, 3, 37], [0, 16, 20, 36, 37],
                                    [0, 0, 37, 37]])
def test_split_merge_equals_definition(causal, bounds):
    """Softmax per chunk of the keys, merged by the rescale rule in logsumexp
    form, gives the full softmax: for any chunking, including empty chunks
    and (causal) rows that see no key of a chunk."""
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((2, 37, 8)) for _ in range(3))
    o_ref, lse_ref, _ = brute.fwd(q, k, v, 0.3, causal)
    o, lse = brute.split_merge(q, k, v, 0.3, causal, bounds)
    np.testing.assert_allclose(o, o_ref, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse, lse_ref, atol=1e-12, rtol=0)


def test_split_merge_dropped_chunk_is_detected():
    """The check above is sharp: leaving one chunk out of the merge (a plausible
    mistake) changes O and lse."""
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((1, 20, 4)) for _ in range(3))
    o_ref, lse_ref, _ = brute.fwd(q, k, v, 0.5, False)
    o, lse = brute.split_merge(q, k, v, 0.5, False, [0, 10])   # keys 10..19 missing
    assert np.abs(lse - lse_ref).max() > 1e-3 and np.abs(o - o_ref).max() > 1e-3


# --------------------------------------------------------------------------
# Dropout on the probabilities: the pages fuse it into the kernel and have
# the backward regenerate the mask from the forward's PRNG state ("13% more
# FLOPs, 5.7x faster", section "The backward pass: recompute instead of
# read"; explainer Step 3 "Tiling").  The generator is Philox4x32-10; the
# mask is keep_ij = [byte_ij >= t], t = floor(256 p + 1/2), kept weights
# scaled by 256 / (256 - t).

def _kat():
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.json")) as f:
        return json.load(f)["vectors"]


def test_philox_known_answers():
    """Both generator implementations reproduce the published known-answer
    vectors of Philox4x32-10."""
    for vec in _kat():
        ctr = [int(x, 16) for x in vec["counter"]]
        key = [int(x, 16) for x in vec["key"]]
        want = [int(x, 16) for x in vec["output"]]
        assert list(oracle.philox4x32_10(ctr, key)) == want
        assert list(brute.philox4x32_10(np.array([ctr], np.uint32), key)[0]) == want


@pytest.mark.parametrize("p,seed,offset", [(0.1, 0, 0), (0.25, 2**40 + 17, 3), (0.5, 2**64 - 1, 2**32 - 1),
                                           (0.9, 12345, 77)])
def test_dropout_mask_two_implementations(p, seed, offset):
    """The C oracle's mask and the vectorised NumPy one (written separately
    from the same definition) agree bit for bit, on every head."""
    kb = brute.dropout_keep(p, seed, offset, 3, 97)
    for bh in range(3):
        np.testing.assert_array_equal(oracle.dropout_keep(p, seed, offset, bh, 97).astype(bool), kb[bh])


@pytest.mark.parametrize("p", [0.0, 0.1, 0.25, 0.5, 0.9])
def test_dropout_keep_fraction(p):
    """The kept fraction is 1 - t/256 within five binomial standard
    deviations, overall and per key column group of 32; p = 0 keeps all."""
    t = math.floor(256 * p + 0.5)
    q = 1 - t / 256
    keep = oracle.dropout_keep(p, 2024, 1, 5, 512).astype(np.float64)
    if t == 0:
        assert keep.all()
        return
    n = keep.size
    assert abs(keep.mean() - q) <= 5 * math.sqrt(q * (1 - q) / n)
    cols = keep.reshape(512, 16, 32).mean(axis=(0, 2))
    assert np.abs(cols - q).max() <= 5 * math.sqrt(q * (1 - q) / (512 * 32))


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_zero_is_plain_attention(causal):
    """p = 0 keeps every weight with factor 1: forward and backward equal the
    plain oracle bit for bit."""
    shape = (2, 3, 45, 8)
    q, k, v, dO = (rand(shape, s) for s in (60, 61, 62, 63))
    o, lse = oracle.fwd(q, k, v, 0.4, causal)
    od, lsed = oracle.fwd(q, k, v, 0.4, causal, dropout=(0.0, 5, 6))
    np.testing.assert_array_equal(o, od)
    np.testing.assert_array_equal(lse, lsed)
    plain = oracle.bwd(q, k, v, dO, 0.4, causal)
    drop = oracle.bwd(q, k, v, dO, 0.4, causal, dropout=(0.0, 5, 6))
    for a, b in zip(plain, drop):
        np.testing.assert_array_equal(a, b)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("p", [0.1, 0.5])
def test_dropout_oracle_vs_brute(causal, p):
    """Row-by-row C oracle against the materialised NumPy version."""
    rng = np.random.default_rng(64)
    q, k, v, dO = (rng.standard_normal((3, 70, 8)) for _ in range(4))
    ob, lb, dqb, dkb, dvb = brute.bwd_dropout(q, k, v, dO, 0.35, causal, p, 99, 5)
    oc, lc, dqc, dkc, dvc = oracle.bwd(q, k, v, dO, 0.35, causal, dropout=(p, 99, 5))
    of, lf = oracle.fwd(q, k, v, 0.35, causal, dropout=(p, 99, 5))
    for a, b in ((ob, oc), (lb, lc), (dqb, dqc), (dkb, dkc), (dvb, dvc), (of, oc), (lf, lc)):
        assert np.abs(a - b).max() <= 1e-12


def _loss_drop(q, k, v, dO, scale, causal, drop):
    o, _ = oracle.fwd(q, k, v, scale, causal, dropout=drop)
    return float(np.sum(o * dO))


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_backward_finite_differences(causal):
    """The mask does not depend on Q, K, V, so central differences of
    L = sum(O * dO) with dropout pin the dropout gradients."""
    rng = np.random.default_rng(65)
    N, d, scale, drop = 40, 3, 0.8, (0.3, 7, 11)
    q, k, v, dO = (rng.standard_normal((N, d)) for _ in range(4))
    keep = oracle.dropout_keep(*drop, 0, N)
    assert 0 < keep.mean() < 1
    _, _, dq, dk, dv = oracle.bwd(q, k, v, dO, scale, causal, dropout=drop)
    h = 1e-6
    pick = np.random.default_rng(66)
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(12):
            idx = (int(pick.integers(N)), int(pick.integers(d)))
            args = {"q": q, "k": k, "v": v}
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args[name] = xp
            lp = _loss_drop(args["q"], args["k"], args["v"], dO, scale, causal, drop)
            args[name] = xm
            lm = _loss_drop(args["q"], args["k"], args["v"], dO, scale, causal, drop)
            num = (lp - lm) / (2 * h)
            assert abs(num - g[idx]) <= 1e-6 * max(1.0, abs(g[idx])), (name, idx, num, g[idx])


def test_dropout_is_unbiased():
    """The kept weights are scaled so that E[keep r] = 1: averaged over many
    seeds, the dropout output approaches the plain output (six standard
    errors of the Bernoulli mask's variance)."""
    rng = np.random.default_rng(67)
    N, d, p = 8, 4, 0.3
    q, k, v = (rng.standard_normal((1, N, d)) for _ in range(3))
    o, _ = oracle.fwd(q, k, v, 0.7, False)
    _, _, prob = brute.fwd(q, k, v, 0.7, False)
    t = math.floor(256 * p + 0.5)
    keepq = 1 - t / 256
    n = 3000
    acc = np.zeros_like(o)
    for seed in range(n):
        acc += oracle.fwd(q, k, v, 0.7, False, dropout=(p, seed, 0))[0]
    mean = acc / n
    var = ((prob[..., :, :, None] ** 2) * (v[..., None, :, :] ** 2)).sum(axis=-2) * (1 - keepq) / keepq
    assert (np.abs(mean - o) <= 6 * np.sqrt(var / n) + 1e-12).all()


@pytest.mark.parametrize("causal", [False, True])
def test_dropout_delta_identity(causal):
    """With dropout, D_i = sum_j P_ij dP_ij equals dO_i . O_i of the dropout
    output: the backward from the stored output gives the same gradients."""
    shape = (2, 33, 8)
    q, k, v, dO = (rand(shape, s) for s in (68, 69, 70, 71))
    drop = (0.2, 8, 9)
    o, _, dq, dk, dv = oracle.bwd(q, k, v, dO, 0.6, causal, dropout=drop)
    _, _, dq2, dk2, dv2 = oracle.bwd(q, k, v, dO, 0.6, causal, o_in=o, dropout=drop)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert np.abs(a - b).max() <= 1e-12


# --------------------------------------------------------------------------
# Queries and keys of different lengths (Flash-Decoding's shape: a few new
# queries against a long key/value cache; explainer "Common questions").

@pytest.mark.parametrize("causal", [False, True])
def test_rect_square_is_plain_forward(causal):
    """Nq = Nk is the square definition, bit for bit."""
    shape = (2, 3, 41, 8)
    q, k, v = (rand(shape, s) for s in (80, 81, 82))
    o, lse = oracle.fwd(q, k, v, 0.3, causal)
    o2, lse2 = oracle.fwd_rect(q, k, v, 0.3, causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, lse2)


@pytest.mark.parametrize("Nq", [1, 5, 64])
def test_rect_queries_are_the_last_positions(Nq):
    """Under the causal mask, Nq queries against Nk keys are the last Nq rows
    of the square problem whose queries continue the same sequence: this pins
    the mask's alignment."""
    Nk, d = 64, 8
    q_all, k, v = (rand((2, Nk, d), s) for s in (83, 84, 85))
    o_sq, lse_sq = oracle.fwd(q_all, k, v, 0.4, True)
    o, lse = oracle.fwd_rect(q_all[:, Nk - Nq:], k, v, 0.4, True)
    assert np.abs(o - o_sq[:, Nk - Nq:]).max() <= 1e-13
    assert np.abs(lse - lse_sq[:, Nk - Nq:]).max() <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Nq,Nk", [(1, 1), (1, 50), (7, 50), (50, 7), (33, 100)])
def test_rect_vs_brute(causal, Nq, Nk):
    """Row by row C oracle against the materialised rectangular softmax,
    including rows that see no key (Nq > Nk, causal): o = 0, lse = -inf."""
    rng = np.random.default_rng(86)
    q = rng.standard_normal((3, Nq, 8))
    k, v = (rng.standard_normal((3, Nk, 8)) for _ in range(2))
    o, lse = oracle.fwd_rect(q, k, v, 0.5, causal)
    ob, lb = brute.fwd_rect(q, k, v, 0.5, causal)
    assert np.abs(o - ob).max() <= 1e-12
    fin = np.isfinite(lb)
    np.testing.assert_array_equal(np.isfinite(lse), fin)
    assert np.abs(lse[fin] - lb[fin]).max(initial=0.0) <= 1e-12
    if causal and Nq > Nk:
        assert (~fin).sum() == 3 * (Nq - Nk) and (o[~fin] == 0).all()


def test_rect_single_query_sees_every_key():
    """One query at the end of the sequence sees all keys under either mask,
    and equals the softmax-weighted mean written out directly."""
    rng = np.random.default_rng(87)
    q = rng.standard_normal((1, 1, 6))
    k, v = (rng.standard_normal((1, 300, 6)) for _ in range(2))
    oc, lc = oracle.fwd_rect(q, k, v, 0.7, True)
    on, ln = oracle.fwd_rect(q, k, v, 0.7, False)
    s = 0.7 * (k[0] @ q[0, 0])
    w = np.exp(s - s.max())
    np.testing.assert_allclose(oc[0, 0], (w[:, None] * v[0]).sum(0) / w.sum(), rtol=0, atol=1e-13)
    np.testing.assert_array_equal(oc, on)
    np.testing.assert_array_equal(lc, ln)
