"""The seeded input generator: determinism, shapes, the outlier recipe."""
import numpy as np
import torch

from exact_io_aware_40_amd import inputs


def test_workload_table():
    w = inputs.WORKLOADS
    assert [x.name for x in w.values()] == [
        "tiny_fwd", "gpt2_medium_fwd", "llama7b_layer_fwd", "long_context_fwd", "recompute_bwd"]
    assert w["llama7b_layer_fwd"].flops() == 4 * 4 * 32 * 4096 ** 2 * 128 / 2
    assert w["recompute_bwd"].flops() == 2.5 * 4 * 8 * 16 * 2048 ** 2 * 128 / 2
    assert w["gpt2_medium_fwd"].flops() == 4 * 64 * 16 * 1024 ** 2 * 64


def test_deterministic_and_distinct():
    w = inputs.WORKLOADS["tiny_fwd"]
    a, b = inputs.make_inputs(w), inputs.make_inputs(w)
    for name in ("q", "k", "v"):
        assert a[name].dtype == torch.float16 and a[name].shape == (1, 2, 256, 64)
        assert torch.equal(a[name], b[name])
        assert inputs.checksum(a[name]) == inputs.checksum(b[name])
    assert not torch.equal(a["q"], a["k"])
    c = inputs.make_inputs(w, seed=99)
    assert not torch.equal(a["q"], c["q"])


def test_values_look_standard_normal():
    x = inputs.normal((1 << 16,), 1, 0, torch.float32).numpy()
    assert abs(x.mean()) < 0.02 and abs(x.std() - 1) < 0.02


def test_outlier_rows_recipe():
    w = inputs.WORKLOADS["llama7b_layer_fwd"]
    shape = (1, 2, 256, 128)
    t = inputs.make_inputs(w, shape=shape)
    base = inputs.normal(shape, w.seed, inputs.TENSOR_IDS["k"], torch.bfloat16)
    rows = inputs.outlier_rows(2 * 256, 0.01, w.seed)
    assert len(rows) == 5 and len(np.unique(rows)) == 5
    kf, bf = t["k"].view(-1, 128), base.view(-1, 128)
    assert torch.equal(kf[rows], bf[rows] * 8)          # exact in bf16
    others = np.setdiff1d(np.arange(512), rows)
    assert torch.equal(kf[others], bf[others])
    assert len(inputs.outlier_rows(4 * 32 * 4096, 0.01, w.seed)) == 5242


def test_backward_workload_has_upstream_gradient():
    w = inputs.WORKLOADS["recompute_bwd"]
    t = inputs.make_inputs(w, shape=(1, 1, 64, 128))
    assert set(t) == {"q", "k", "v", "dO"} and t["dO"].dtype == torch.bfloat16
