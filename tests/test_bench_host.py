"""Host logic of bench.py (CPU only): the algorithmic byte counts, the HBM
entry and its no-N^2-traffic flag, and the derivations from rocprofv3
counter files (written here as small synthetic CSV files in rocprofv3's
column layout), so that the figures the bench line reports follow from the
counters as stated."""
import csv
import importlib.util
import os
import types

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def bench():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def nbytes(*shape, dtype=torch.bfloat16):
    return torch.empty(shape, dtype=dtype).nbytes


def test_algorithmic_bytes_are_the_tensors_moved(bench):
    """Each kernel's algorithmic bytes are the sizes of the tensors it must
    read and write once: forward q, k, v -> o, lse; dq kernel q, k, v, dO,
    o, lse -> dq and the two per-row workspace values; dk/dv kernel q, k, v,
    dO and the workspace -> dk, dv."""
    w = types.SimpleNamespace(B=2, H=3, N=50, d=64)
    t = nbytes(2, 3, 50, 64)
    rows = nbytes(2, 3, 50, dtype=torch.float32)
    a = bench.algorithmic_bytes(w)
    assert a["fwd_kernel"] == {"read": 3 * t, "write": t + rows}
    assert a["dq_kernel"] == {"read": 5 * t + rows, "write": t + 2 * rows}
    assert a["dkdv_kernel"] == {"read": 4 * t + 2 * rows, "write": 2 * t}


def test_hbm_entry_flag_decided_by_writes(bench):
    alg = {"read": 1000.0, "write": 400.0}
    n2 = 1.0e6
    ok = bench.hbm_entry(1000.0, 400.0, alg, n2, 1.0)
    assert ok["no_n2_traffic"] and ok["read_ratio"] == 1.0 and ok["excess_read_bytes"] == 0.0
    # 1000 + 400 bytes in 1 ms
    assert ok["gbs"] == pytest.approx(1400.0 / 1e-3 / 1e9)
    # re-read input tiles: many more reads, outputs written once -> still no N x N traffic
    reread = bench.hbm_entry(50.0 * 1000.0 + 1.0e6, 400.0, alg, n2, 1.0)
    assert reread["no_n2_traffic"] and reread["excess_read_bytes"] == pytest.approx(49000.0 + 1.0e6)
    # a tenth of an N x N matrix written beyond the outputs
    assert not bench.hbm_entry(1000.0, 400.0 + 0.1 * n2, alg, n2, 1.0)["no_n2_traffic"]
    # writes more than 10% above the outputs
    assert not bench.hbm_entry(1000.0, 441.0, alg, n2, 1.0)["no_n2_traffic"]


COLS = ["Correlation_Id", "Dispatch_Id", "Agent_Id", "Queue_Id", "Process_Id", "Thread_Id", "Grid_Size",
        "Kernel_Id", "Kernel_Name", "Workgroup_Size", "LDS_Block_Size", "Scratch_Size", "VGPR_Count",
        "Accum_VGPR_Count", "SGPR_Count", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_pmc(d, dispatches, xcc=8):
    """dispatches: [(kernel name, {counter: value}, start ns, end ns)]."""
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "p_counter_collection.csv"), "w", newline="") as f:
        wr = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        wr.writerow(COLS)
        for i, (name, ctrs, t0, t1) in enumerate(dispatches, 1):
            for c, v in ctrs.items():
                wr.writerow([i, i, "Agent 1", 1, 1, 1, 1024, 1, name, 256, 0, 0, 128, 0, 64, c, float(v), t0, t1])
    with open(os.path.join(d, "p_agent_info.csv"), "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Node_Id", "Agent_Type", "Num_Xcc"])
        wr.writerow([1, "CPU", 0])
        wr.writerow([2, "GPU", xcc])


FWD = "_ZN4attn12_GLOBAL__N_110fwd_kernelIDF16bDF16bLi128ELb1ELb0ELb0EEEvNS_7FwdArgsE"


def test_derive_counters(bench, tmp_path):
    """Averages over dispatches and the derived figures: busy cycles over
    (GRBM active cycles per XCD x 1024 SIMDs), the vector ALU's issue share
    (SQ_ACTIVE_INST_VALU in units of four cycles), the clock, the FLOPs of
    the products (512 per MOPS unit), instructions per product."""
    g, busy, act, mops, nmf, valu, lds = 8.0e6, 4.0e8, 9.0e7, 1.0e9, 1.5e7, 9.0e7, 2.0e7
    d1 = [(FWD, {"GRBM_GUI_ACTIVE": g, "SQ_VALU_MFMA_BUSY_CYCLES": busy, "SQ_INSTS_VALU_MFMA_MOPS_BF16": mops,
                 "SQ_INSTS_VALU_MFMA_BF16": nmf, "SQ_INSTS_VALU": valu, "SQ_INSTS_LDS": lds}, 0, 500000),
          (FWD, {"GRBM_GUI_ACTIVE": 3 * g, "SQ_VALU_MFMA_BUSY_CYCLES": 3 * busy, "SQ_INSTS_VALU_MFMA_MOPS_BF16": mops,
                 "SQ_INSTS_VALU_MFMA_BF16": nmf, "SQ_INSTS_VALU": valu, "SQ_INSTS_LDS": lds}, 0, 500000)]
    d2 = [(FWD, {"GRBM_GUI_ACTIVE": 2 * g, "SQ_ACTIVE_INST_VALU": act}, 0, 500000)] * 2
    write_pmc(str(tmp_path / "p1"), d1)
    write_pmc(str(tmp_path / "p2"), d2)
    e = bench.derive_counters([str(tmp_path / "p1"), str(tmp_path / "p2")])["fwd_kernel"]
    g_mean = (g + 3 * g + 2 * g + 2 * g) / 4          # GRBM_GUI_ACTIVE appears in both passes
    per_xcd = g_mean / 8
    assert e["dispatches"] == 2
    assert e["active_cycles_per_xcd"] == pytest.approx(per_xcd)
    assert e["clock_ghz"] == pytest.approx(per_xcd / 500000)
    assert e["mfma_busy_frac"] == pytest.approx(2 * busy / (per_xcd * 1024))
    assert e["valu_active_frac"] == pytest.approx(4 * act / (per_xcd * 1024))
    assert e["mfma_flop_by_mops"] == pytest.approx(512 * mops)
    assert e["mfma_tflops_by_mops"] == pytest.approx(512 * mops / 500e-6 / 1e12)
    assert e["lds_insts_per_mfma"] == pytest.approx(lds / nmf)
    assert e["valu_insts_per_mfma"] == pytest.approx((valu - nmf) / nmf)


def test_derive_traffic(bench, tmp_path):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) scaled by the copy
    kernel's bytes over its own reading."""
    copy = "void at::native::vectorized_elementwise_kernel<4, at::native::neg_kernel_cuda>(...)"
    fetch = [(copy, {"FETCH_SIZE": bench.COPY_BYTES / 1024 / 2}, 0, 1), (FWD, {"FETCH_SIZE": 1000.0}, 0, 1),
             (FWD, {"FETCH_SIZE": 3000.0}, 0, 1)]
    write = [(copy, {"WRITE_SIZE": bench.COPY_BYTES / 1024}, 0, 1), (FWD, {"WRITE_SIZE": 500.0}, 0, 1)]
    write_pmc(str(tmp_path / "f"), fetch)
    write_pmc(str(tmp_path / "w"), write)
    e = bench.derive_traffic(str(tmp_path / "f"), str(tmp_path / "w"))["fwd_kernel"]
    assert e["fetch_size_factor"] == pytest.approx(2.0)
    assert e["write_size_factor"] == pytest.approx(1.0)
    assert e["fetch_size_bytes"] == pytest.approx(2.0 * 2000.0 * 1024)
    assert e["write_size_bytes"] == pytest.approx(500.0 * 1024)
    assert e["bytes"] == pytest.approx(2.0 * 2000.0 * 1024 + 500.0 * 1024)


def test_derive_traffic_needs_the_copy(bench, tmp_path):
    write_pmc(str(tmp_path / "f"), [(FWD, {"FETCH_SIZE": 1000.0}, 0, 1)])
    write_pmc(str(tmp_path / "w"), [(FWD, {"WRITE_SIZE": 500.0}, 0, 1)])
    with pytest.raises(SystemExit):
        bench.derive_traffic(str(tmp_path / "f"), str(tmp_path / "w"))
