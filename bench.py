#!/usr/bin/env python3
"""Benchmark of the exact fused attention path on one MI355X.

One step is one pass of the whole hot path over one batch: the fused
forward (O and lse) followed by the recomputing backward (dq, dk, dv) on
the seven-billion-parameter-layer-shaped workload (B=4, H=32, N=4096,
d=128, bf16, causal, 1% of K rows x8), inputs resident in HBM.

Prints ONE JSON line: TFLOP/s of the step (credited FLOPs: forward
4*B*H*N^2*d/2 under the causal mask, backward 2.5x that), with a per-phase
and per-kernel breakdown, the roofline of the dominant kernel measured live
with HIP events on the launch stream, and the fp64 oracle timed on the host
cores on a bounded sample (its forward rows also compared with the GPU's).

Each kernel has its own entry point (attn_fwd, attn_bwd_dq, attn_bwd_dkdv;
attn_bwd is the last two in order), so the events bracket one kernel each.
A kernel's algorithmic FLOPs are those of the products its algorithm
performs per (batch, head), halved under the causal mask: the forward
4 N^2 d (S, P.V); the dq kernel 6 N^2 d (S and dP recomputed, dS.K); the
dk/dv kernel 8 N^2 d (S and dP recomputed, P^T.dO, dS^T.Q).

Counter support: --copy-calibration adds a plain copy of known size
(torch.neg over 512 MiB) before the warm-up, and --traffic FETCH_DIR
WRITE_DIR turns two rocprofv3 --pmc runs (FETCH_SIZE, then WRITE_SIZE) of
such a command into profiles/traffic.json: HBM bytes per launch of each
kernel, each counter scaled by the copy's known bytes over its reading.

The default run also times the other workloads' forward and step, and the
matrix cores' sustained bf16 rate on this board (attn_probe_mfma: products
only, two workgroups per CU), against which each kernel's rate is stated
beside the published 2.5 PFLOP/s; --no-other-workloads skips both.

Side measurements (not the headline line): --decode NQ times a decode step
against the HBM roofline and the measured one-pass read rate (--hbm-ceiling
prints that rate alone), --dropout P the dropout path, and --fp8 the E4M3
forward (attn_fwd_fp8) on the same workload quantised per tensor, against the
dense fp8 matrix peak.
"""
import argparse
import hashlib
import json
import re
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import exact_io_aware_40_amd as attn  # noqa: E402
from exact_io_aware_40_amd import inputs  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16/fp16 matrix peak
PEAK_FP8_TFLOPS = 5000.0     # MI355X dense fp8 matrix peak
PEAK_HBM_GBS = 8000.0
# the sources each kernel is built from: the fused kernels' and the
# materialised baseline's counter data are keyed separately
KERNEL_SOURCES = {
    "fused": ["exact_io_aware_40_amd/csrc/attn_fwd_kernel.h",
              "exact_io_aware_40_amd/csrc/attn_fwd.hip",
              "exact_io_aware_40_amd/csrc/attn_decode.hip",
              "exact_io_aware_40_amd/csrc/attn_bwd.hip",
              "exact_io_aware_40_amd/csrc/attn_common.h"],
    "standard": ["exact_io_aware_40_amd/csrc/attn_std.hip",
                 "exact_io_aware_40_amd/csrc/attn_common.h"],
}


def _family(kernel: str) -> str:
    return "standard" if kernel.startswith("std_") else "fused"


def source_hash(family: str = "fused") -> str:
    """Hash of a kernel family's sources with comments removed and
    whitespace collapsed, and of the compiler flags they are built with: it
    keys the committed counter data, which stays valid across edits of
    comments and layout only."""
    from exact_io_aware_40_amd.csrc import build as hip_build
    h = hashlib.sha256()
    for p in KERNEL_SOURCES[family]:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    flags = [f for f in hip_build.FLAGS if not f.startswith(ROOT) and f != "-I"]
    h.update(" ".join(flags).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps before the timed ones (default 50, about 0.1 s on the default "
                         "workload: the shader clock needs that long under load to settle after the "
                         "idle input generation; 5 steps read about 2%% slow)")
    ap.add_argument("--workload", default="llama7b_layer_fwd",
                    help="shape of the batch (default: the 7B-layer-shaped workload)")
    ap.add_argument("--phase", choices=["step", "fwd", "bwd"], default="step",
                    help="time the whole step (default) or one phase only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="approximate CPU time budget of each oracle sample")
    ap.add_argument("--no-parity", action="store_true",
                    help="do not compare the GPU output on the CPU baseline's rows")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run a 512 MiB copy (read + write) first, for counter scaling")
    ap.add_argument("--dropout", type=float, default=None, metavar="P",
                    help="time the dropout path instead (attn_fwd_dropout, attn_bwd_dropout) "
                         "with probability P; the backward's two kernels are then timed together")
    ap.add_argument("--decode", type=int, default=None, metavar="NQ",
                    help="time a decode step instead: attn_fwd_decode of NQ new queries against "
                         "a 16384-key cache (B=16, H=32, d=128, bf16, causal), against the HBM "
                         "roofline")
    ap.add_argument("--nsplit", type=int, default=None,
                    help="key chunks of the decode step (default: 4 for the 16-bit cache, 8 for the 8-bit one, "
                         "the faster of the two for each at 1 to 16 queries)")
    ap.add_argument("--fp8", action="store_true",
                    help="time the E4M3 forward (attn_fwd_fp8) on the workload quantised per "
                         "tensor, against the dense fp8 matrix peak; with --decode, the E4M3 "
                         "decode step (attn_fwd_decode_fp8)")
    ap.add_argument("--traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json from two rocprofv3 --pmc output dirs")
    ap.add_argument("--counters", nargs="+", metavar="PMC_DIR",
                    help="write profiles/counters.json from rocprofv3 --pmc output dirs")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the context measurements: the other workloads' forward and step "
                         "timings and the matrix-core ceiling")
    ap.add_argument("--ceiling", action="store_true",
                    help="only measure the matrix cores' sustained bf16 rate (attn_probe_mfma)")
    ap.add_argument("--hbm-ceiling", action="store_true",
                    help="only measure the HBM read rate of a plain one-pass read (attn_probe_hbm)")
    ap.add_argument("--other-steps", type=int, default=10,
                    help="timed steps of each other workload")
    ap.add_argument("--standard", action="store_true",
                    help="time the materialised standard attention (S and P written to HBM) "
                         "against the fused forward on the workload (default: the GPT-2-medium shape)")
    return ap.parse_args()


KERNELS = ("fwd_kernel", "dq_kernel", "dkdv_kernel", "std_scores_kernel", "std_softmax_kernel",
           "std_pv_kernel")
COPY_BYTES = 512 << 20


def _pmc_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows += list(csv.DictReader(open(f)))
    return rows


def derive_traffic(fetch_dir, write_dir):
    """Per-launch HBM bytes of each kernel from FETCH_SIZE / WRITE_SIZE (KiB
    per dispatch), scaled by copy-bytes / counter-reading of the copy."""
    res = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        per = {}
        for r in _pmc_rows(d):
            if r["Counter_Name"] != counter:
                continue
            name = r["Kernel_Name"]
            key = next((k for k in KERNELS if k in name), "copy" if "neg" in name else None)
            if key:
                per.setdefault(key, []).append(float(r["Counter_Value"]) * 1024.0)
        if "copy" not in per:
            raise SystemExit(f"no copy-calibration dispatch found in {d}")
        factor = COPY_BYTES / (sum(per["copy"]) / len(per["copy"]))
        for k in KERNELS:
            if k in per:
                e = res.setdefault(k, {})
                e[counter.lower() + "_raw_bytes"] = sum(per[k]) / len(per[k])
                e[counter.lower() + "_factor"] = factor
                e[counter.lower() + "_bytes"] = factor * sum(per[k]) / len(per[k])
    for k, e in res.items():
        e["bytes"] = e.get("fetch_size_bytes", 0.0) + e.get("write_size_bytes", 0.0)
    return res


def write_traffic(fetch_dir, write_dir, workload):
    """profiles/traffic.json from the two rocprofv3 --pmc runs (derive_traffic),
    keyed by the kernels' source hash."""
    res = derive_traffic(fetch_dir, write_dir)
    for k, e in res.items():
        e["source_hash"] = source_hash(_family(k))
    path = os.path.join(ROOT, "profiles", "traffic.json")
    rec = {}
    if os.path.exists(path):
        rec = json.load(open(path))
    rec.setdefault(workload, {}).update(res)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(rec[workload], indent=1))


def mfma_ceiling(dev, rounds=15000, reps=5):
    """The matrix cores' sustained bf16 rate on this board: attn_probe_mfma
    (only products, on pseudo-random operands that change from one product
    to the next, four chains per wave, two workgroups per CU) timed with HIP
    events on the launch stream, median of `reps` launches after two warm-up
    ones, at whatever clock the board holds under that load (the probe runs
    right after the timed steps, on a warm board)."""
    props = torch.cuda.get_device_properties(dev)
    wg = 2 * props.multi_processor_count
    buf = torch.empty(wg * 256, dtype=torch.float32, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream

    def launch():
        st = attn.attn_probe_mfma(buf.data_ptr(), wg, rounds, sp)
        if st != 0:
            raise RuntimeError(attn.attn_status_str(st))

    for _ in range(2):
        launch()
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        launch()
        e1.record()
        e1.synchronize()
        ms.append(e0.elapsed_time(e1))
    med = float(np.median(ms))
    tflops = wg * 4 * 16 * rounds * 32768 / (med * 1e-3) / 1e12
    return {"tflops": tflops, "frac_of_spec": tflops / PEAK_BF16_TFLOPS, "workgroups": wg, "rounds": rounds,
            "ms_median": med, "launches": reps,
            "kernel": "mfma_probe_kernel: v_mfma_f32_32x32x16_bf16 only, pseudo-random bf16 operands changing "
                      "between products, 4 chains per wave, 2 waves per SIMD"}


def hbm_ceiling(dev, nbytes=4 << 30, reps=5, wg_per_cu=(2, 4, 8, 16)):
    """The rate at which this board streams a buffer from HBM:
    attn_probe_hbm (each workgroup streams a contiguous range with the
    kernels' non-temporal direct-to-LDS copies, eight 1 KiB chunks in flight
    per wave, a checksum kept) over `nbytes`, for a few grid sizes, each the
    median of `reps` launches after two warm-up ones; the best of them."""
    props = torch.cuda.get_device_properties(dev)
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device=dev)
    sp = torch.cuda.current_stream(dev).cuda_stream
    sweep = {}
    for m in wg_per_cu:
        wg = m * props.multi_processor_count
        out = torch.empty(wg * 256, dtype=torch.int32, device=dev)

        def launch():
            st = attn.attn_probe_hbm(buf.data_ptr(), nbytes, out.data_ptr(), wg, sp)
            if st != 0:
                raise RuntimeError(attn.attn_status_str(st))

        for _ in range(2):
            launch()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            e1.synchronize()
            ms.append(e0.elapsed_time(e1))
        sweep[wg] = nbytes / (float(np.median(ms)) * 1e-3) / 1e9
        del out
    best = max(sweep, key=sweep.get)
    del buf
    torch.cuda.empty_cache()
    return {"gbs": sweep[best], "frac_of_spec": sweep[best] / PEAK_HBM_GBS, "bytes": nbytes,
            "workgroups": best, "gbs_by_workgroups": sweep, "launches": reps,
            "kernel": "hbm_probe_kernel: one pass over the buffer, a contiguous range per workgroup, non-temporal direct-to-LDS copies, eight 1 KiB chunks in flight per wave"}


def cpu_baseline(w, t, scale, budget_s, gpu_out=None):
    """The fp64 oracle on this host's cores over a bounded sample of the
    same workload: query rows drawn from many heads for the forward, whole
    heads for the backward, each sized to about `budget_s` seconds.
    With gpu_out = (o, lse) of the timed forward, the oracle's rows are also
    compared with the GPU's (max |gpu - oracle| in the result's "parity").
    Returns the JSON object."""
    import oracle
    cores = oracle.default_threads()
    B, H, N, d = w.B, w.H, w.N, w.d
    BH = B * H
    rng = np.random.default_rng(12345)
    q3, k3, v3 = (t[x].reshape(BH, N, d) for x in ("q", "k", "v"))
    heads = np.sort(rng.choice(BH, size=min(BH, 32), replace=False))
    sub = lambda x, hs: x[torch.from_numpy(hs)].double().numpy()  # noqa: E731
    qs, ks, vs = sub(q3, heads), sub(k3, heads), sub(v3, heads)
    # forward: calibrate on a small batch of rows, then size the sample
    n_cal = 32 * cores
    rows = rng.choice(len(heads) * N, size=n_cal, replace=False)
    t0 = time.perf_counter()
    oracle.fwd(qs, ks, vs, scale, w.causal, rows=rows, threads=cores)
    t_cal = time.perf_counter() - t0
    n_rows = int(min(len(heads) * N, max(n_cal, n_cal * budget_s / max(t_cal, 1e-3))))
    rows = rng.choice(len(heads) * N, size=n_rows, replace=False)
    t0 = time.perf_counter()
    o_ref, l_ref = oracle.fwd(qs, ks, vs, scale, w.causal, rows=rows, threads=cores)
    t_fwd = time.perf_counter() - t0
    parity = None
    if gpu_out is not None:
        o, lse = gpu_out
        grow = torch.from_numpy(heads[rows // N] * N + rows % N).to(o.device)
        og = o.reshape(-1, d)[grow].double().cpu().numpy()
        lg = lse.reshape(-1)[grow].double().cpu().numpy()
        # o is stored in the input type: half of its spacing at the exact value
        # is a rounding error no 16-bit output can avoid, so the excess of
        # |gpu - oracle| over tol + that half spacing is reported as well
        mant = 7 if w.dtype == "bf16" else 10
        ao = np.abs(o_ref)
        ex = np.floor(np.log2(np.where(ao > 0, ao, 1.0)))
        if w.dtype != "bf16":
            ex = np.maximum(ex, -14)   # fp16 subnormal spacing
        tol = 1.5e-2 if w.dtype == "bf16" else 2e-3
        err = np.abs(og - o_ref)
        excess = err - (tol + np.ldexp(0.5, (ex - mant).astype(np.int64)))
        # the exact values' own rounding to the output type: elements that no
        # output of that type can bring within the literal tolerance
        own = np.abs(torch.from_numpy(o_ref).to(w.torch_dtype).double().numpy() - o_ref)
        beyond = err > tol
        parity = {"rows": int(len(rows)), "max_abs_o": float(err.max()),
                  "max_abs_lse": float(np.abs(lg - l_ref).max()), "tol_o": tol, "tol_lse": 1e-3,
                  "o_elements": int(err.size),
                  "o_elements_beyond_tol": int(beyond.sum()),
                  "o_exact_values_beyond_tol_by_own_rounding": int((own > tol).sum()),
                  "o_beyond_tol_where_own_rounding_is_beyond_tol": int((beyond & (own > tol)).sum()),
                  "o_beyond_tol_within_tol_plus_half_ulp": int((beyond & (excess <= 0)).sum()),
                  "max_excess_o_over_tol_plus_half_ulp": float(excess.max())}
    i = rows % N
    keys = (i + 1) if w.causal else np.full_like(i, N)
    f_fwd = float(np.sum(4.0 * keys * d))
    del qs, ks, vs
    # backward: batches of whole heads (one per thread) until the budget is spent
    g3 = inputs.normal((B, H, N, d), w.seed, inputs.TENSOR_IDS["dO"], w.torch_dtype).reshape(BH, N, d)
    order = rng.permutation(BH)
    t_bwd, nh = 0.0, 0
    while nh < BH and t_bwd < budget_s:
        hs = np.sort(order[nh:nh + cores])
        args = [sub(x, hs) for x in (q3, k3, v3, g3)]
        t0 = time.perf_counter()
        oracle.bwd(*args, scale, w.causal, threads=cores)
        t_bwd += time.perf_counter() - t0
        nh += len(hs)
    f_bwd = nh * 2.5 * 4.0 * N * N * d * (0.5 if w.causal else 1.0)
    val = (f_fwd + f_bwd) / (t_fwd + t_bwd) / 1e12
    return {
        "value": val, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
        "sample": (f"{n_rows} query rows from {len(heads)} heads (forward, {t_fwd:.1f} s) and "
                   f"{nh} whole heads (backward, {t_bwd:.1f} s) of {w.name}; fp64, one thread "
                   f"per row or head; credited FLOPs as on the GPU"),
        "fwd_tflops": f_fwd / t_fwd / 1e12, "bwd_tflops": f_bwd / t_bwd / 1e12,
        **({} if parity is None else {"parity": parity}),
    }


DROP_STATE = (2024, 17)   # generator seed and offset of the dropout path


def bench_decode(args):
    """One decode step per call: attn_fwd_decode (split kernel and merge).
    Algorithmic bytes: K and V read once, q read, o and lse written, and the
    fp32 partials written and read back by the merge.  With --fp8 the step
    is attn_fwd_decode_fp8 on E4M3 q, k, v (inputs.make_decode_fp8_inputs),
    one byte per element read, bf16 output.  Unless --no-other-workloads,
    the rate of a plain one-pass HBM read (attn_probe_hbm) is measured after
    the timed calls, and the roofline also states the step against it."""
    dev = torch.device("cuda:0")
    B, H, Nk, d, Nq = 16, 32, 16384, 128, int(args.decode)
    ns = int(args.nsplit) if args.nsplit is not None else (8 if args.fp8 else 4)
    f8 = bool(args.fp8)
    if f8:
        x, desc = inputs.make_decode_fp8_inputs(B, H, Nq, Nk, d, seed=12)
        qd, kd, vd = (x[n].to(dev) for n in "qkv")
    else:
        g = torch.Generator(device="cpu").manual_seed(11)
        q = torch.randn((B, H, Nq, d), generator=g).to(torch.bfloat16)
        k = torch.randn((B, H, Nk, d), generator=g).to(torch.bfloat16)
        v = torch.randn((B, H, Nk, d), generator=g).to(torch.bfloat16)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    need = attn.attn_fwd_split_workspace_size(B, H, Nq, d, ns)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def call():
        if f8:
            st = attn.attn_fwd_decode_fp8(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                                          lse.data_ptr(), ws.data_ptr(), ws.numel(), B, H, Nq, Nk, d,
                                          scale, desc[0], desc[1], desc[2], 1, attn.ATTN_BF16, ns, sp)
        else:
            st = attn.attn_fwd_decode(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), ws.data_ptr(), ws.numel(), B, H, Nq, Nk, d, scale,
                                      1, attn.ATTN_BF16, attn.ATTN_BF16, ns, sp)
        if st:
            raise attn.AttnError(st, "attn_fwd_decode_fp8" if f8 else "attn_fwd_decode")

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    BH = B * H
    esz = 1 if f8 else 2                      # bytes per input element
    kv = 2 * BH * Nk * d * esz
    partial = ns * BH * Nq * (d + 1) * 4 * 2
    byts = kv + BH * Nq * d * (esz + 2) + BH * Nq * 4 + partial
    ms = float(per.mean())
    gbs = byts / (ms * 1e-3) / 1e9
    out = {
        "metric": "decode step: K/V cache read GB/s at 1 GPU + % of HBM peak",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3" if f8 else "bf16", "data": "synthetic",
        "config": {"workload": f"decode: B={B} H={H} Nq={Nq} Nk={Nk} d={d} "
                               f"{'E4M3 q, k, v' if f8 else 'bf16'} causal, nsplit={ns}; step = "
                               f"{'attn_fwd_decode_fp8' if f8 else 'attn_fwd_decode'} (split kernel + merge)"},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": None, "bytes_per_call": byts,
                     "call_ms": ms},
    }
    if not args.no_other_workloads:
        # the rate a plain one-pass read of HBM reaches on this board
        del qd, kd, vd, ws
        torch.cuda.empty_cache()
        c = hbm_ceiling(dev)
        out["hbm_read_ceiling"] = c
        out["roofline"]["frac_of_measured_ceiling"] = gbs / c["gbs"]
    print(json.dumps(out), flush=True)


def bench_fp8(args):
    """The E4M3 forward, one launch per call, on the workload's inputs
    quantised per tensor (inputs.make_fp8_inputs); bf16 output.  FLOPs as
    for the 16-bit forward: 4 B H N^2 d, halved under the causal mask."""
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[args.workload]
    if w.d != 128:
        print("the fp8 forward takes d = 128", file=sys.stderr)
        sys.exit(2)
    x, ds = inputs.make_fp8_inputs(w)
    q, k, v = (x[n].to(dev) for n in "qkv")
    B, H, N, d = w.B, w.H, w.N, w.d
    scale = 1.0 / math.sqrt(d)
    o = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = stream.cuda_stream

    def call():
        st = attn.attn_fwd_fp8(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               B, H, N, d, scale, ds[0], ds[1], ds[2], int(w.causal), attn.ATTN_BF16, sp)
        if st:
            raise attn.AttnError(st, "attn_fwd_fp8")

    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    wall0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(args.steps):
        call()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])
    flops = 4.0 * B * H * N * N * d * (0.5 if w.causal else 1.0)
    ms = float(per.mean())
    tf = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": "fp8 (E4M3) attention forward TFLOP/s at 1 GPU + % of fp8 MFMA peak",
        "value": flops / (wall / args.steps) / 1e12, "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / args.steps, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": f"{w.name} quantised per tensor to E4M3: B={B} H={H} N={N} d={d} "
                               f"{'causal' if w.causal else 'non-causal'}, bf16 output; "
                               f"step = fwd_kernel (8-bit)"},
        "roofline": {"bound": "mfma", "kernel": "fwd_kernel<fp8e4m3>", "achieved": tf,
                     "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": tf / PEAK_FP8_TFLOPS,
                     "traffic": None, "flops_per_launch": flops, "launch_ms": ms,
                     "launch_ms_min": float(per.min())},
        "kernel_source_hash": source_hash(),
    }
    c = _committed("counters.json", w.name + "_fp8", "fwd_kernel")
    if c:
        # matrix pipes against vector ALU over a profiled launch (8-bit
        # products take 64 busy cycles each, 2048 FLOP per clock per SIMD)
        out["roofline"]["counters"] = {x: c[x] for x in ("mfma_busy_frac", "valu_active_frac",
                                                         "clock_ghz", "duration_ns_median") if x in c}
    print(json.dumps(out), flush=True)


class StepRunner:
    """The step's launches on one workload, inputs resident on the GPU: the
    forward (attn_fwd), then the backward's two kernels (attn_bwd_dq,
    attn_bwd_dkdv), or their dropout forms."""

    def __init__(self, w, dev, dropout=None, t=None):
        self.w = w
        self.scale = 1.0 / math.sqrt(w.d)
        if t is None:
            t = inputs.make_inputs(w)
        if "dO" not in t:
            t["dO"] = inputs.normal((w.B, w.H, w.N, w.d), w.seed, inputs.TENSOR_IDS["dO"],
                                    w.torch_dtype)
        self.t = t
        q, k, v, dO = (t[x].to(dev) for x in ("q", "k", "v", "dO"))
        B, H, N, d = w.B, w.H, w.N, w.d
        code = attn.ATTN_BF16 if w.dtype == "bf16" else attn.ATTN_F16
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
        ws = torch.empty(max(256, attn.attn_bwd_workspace_size(B, H, N, d, code)), dtype=torch.uint8,
                         device=dev)
        self.stream = torch.cuda.current_stream(dev)
        sp = self.stream.cuda_stream
        causal = int(w.causal)
        scale = self.scale
        nb = ws.numel()
        self.o, self.lse = o, lse
        self.bufs = (q, k, v, dO, o, lse, dq, dk, dv, ws)

        def fwd():
            st = attn.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                               B, H, N, d, scale, causal, code, code, sp)
            if st:
                raise attn.AttnError(st, "attn_fwd")

        def bwd_dq():
            st = attn.attn_bwd_dq(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                  dO.data_ptr(), lse.data_ptr(), dq.data_ptr(), ws.data_ptr(),
                                  nb, B, H, N, d, scale, causal, code, code, sp)
            if st:
                raise attn.AttnError(st, "attn_bwd_dq")

        def bwd_dkdv():
            st = attn.attn_bwd_dkdv(q.data_ptr(), k.data_ptr(), v.data_ptr(), dO.data_ptr(),
                                    dk.data_ptr(), dv.data_ptr(), ws.data_ptr(), nb, B, H, N,
                                    d, scale, causal, code, code, sp)
            if st:
                raise attn.AttnError(st, "attn_bwd_dkdv")

        self.drop = drop = None if dropout is None else (dropout,) + DROP_STATE

        def fwd_drop():
            st = attn.attn_fwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), B, H, N, d, scale, causal, drop[0], drop[1],
                                       drop[2], code, code, sp)
            if st:
                raise attn.AttnError(st, "attn_fwd_dropout")

        def bwd_drop():
            st = attn.attn_bwd_dropout(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                       dO.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                       dv.data_ptr(), ws.data_ptr(), nb, B, H, N, d, scale,
                                       causal, drop[0], drop[1], drop[2], code, code, sp)
            if st:
                raise attn.AttnError(st, "attn_bwd_dropout")

        half = 0.5 if w.causal else 1.0
        unit = B * H * N * N * d * half
        self.f_fwd = 4.0 * unit
        self.f_bwd = 2.5 * self.f_fwd                 # credited: five N^2 d products
        self.algo = {"fwd_kernel": 4.0 * unit, "dq_kernel": 6.0 * unit, "dkdv_kernel": 8.0 * unit,
                     "bwd_kernels": 14.0 * unit}
        if drop is None:
            self.calls = {"step": [("fwd_kernel", fwd), ("dq_kernel", bwd_dq), ("dkdv_kernel", bwd_dkdv)],
                          "fwd": [("fwd_kernel", fwd)],
                          "bwd": [("dq_kernel", bwd_dq), ("dkdv_kernel", bwd_dkdv)]}
        else:
            self.calls = {"step": [("fwd_kernel", fwd_drop), ("bwd_kernels", bwd_drop)],
                          "fwd": [("fwd_kernel", fwd_drop)],
                          "bwd": [("bwd_kernels", bwd_drop)]}
        self.fwd = fwd_drop if drop is not None else fwd

    def settle(self, phase, seconds):
        """Run the phase's launches, untimed, for about `seconds`."""
        if phase == "bwd":
            self.fwd()
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                for _, fn in self.calls[phase]:
                    fn()
            torch.cuda.synchronize()

    def time(self, phase, steps, warmup):
        """Warm up, then time `steps` passes of the phase's launches, an event
        after every call on the launch stream.  Returns (wall ms per step,
        kernels, phases, credited FLOPs per step)."""
        calls = self.calls[phase]
        if phase == "bwd":
            self.fwd()
        for _ in range(warmup):
            for _, fn in calls:
                fn()
        torch.cuda.synchronize()
        nc = len(calls)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nc + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        for st_ in range(steps):
            ev[st_][0].record(self.stream)
            for j_, (_, fn) in enumerate(calls):
                fn()
                ev[st_][j_ + 1].record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        per = np.array([[ev[s_][j_].elapsed_time(ev[s_][j_ + 1]) for j_ in range(nc)]
                        for s_ in range(steps)])  # ms
        algo = self.algo
        kernels = {}
        for j_, (nm, _) in enumerate(calls):
            m = float(per[:, j_].mean())
            kernels[nm] = {"ms_mean": m, "ms_median": float(np.median(per[:, j_])), "ms_min": float(per[:, j_].min()),
                           "algorithmic_tflop": algo[nm] / 1e12,
                           "tflops": algo[nm] / (m * 1e-3) / 1e12,
                           "frac_of_peak": algo[nm] / (m * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        phases = {}
        if "fwd_kernel" in kernels:
            m = kernels["fwd_kernel"]["ms_mean"]
            phases["fwd"] = {"ms_mean": m, "tflops": self.f_fwd / (m * 1e-3) / 1e12,
                             "frac_of_peak": self.f_fwd / (m * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}
        if "dq_kernel" in kernels or "bwd_kernels" in kernels:
            m = (kernels["bwd_kernels"]["ms_mean"] if "bwd_kernels" in kernels
                 else kernels["dq_kernel"]["ms_mean"] + kernels["dkdv_kernel"]["ms_mean"])
            phases["bwd"] = {"ms_mean": m, "tflops": self.f_bwd / (m * 1e-3) / 1e12,
                             "frac_of_peak": self.f_bwd / (m * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                             "flops": "credited 2.5x forward"}
        flops_step = {"step": self.f_fwd + self.f_bwd, "fwd": self.f_fwd, "bwd": self.f_bwd}[phase]
        return wall * 1e3 / steps, kernels, phases, flops_step


def algorithmic_bytes(w):
    """HBM bytes each kernel must move at least (inputs read once, outputs
    written once), split into reads and writes."""
    e = 2
    BH, N, d = w.B * w.H, w.N, w.d
    t = BH * N * d * e
    r = BH * N * 4
    return {"fwd_kernel": {"read": 3 * t, "write": t + r},
            "dq_kernel": {"read": 5 * t + r, "write": t + 2 * r},
            "dkdv_kernel": {"read": 4 * t + 2 * r, "write": 2 * t}}


def _counter_rows(dirs):
    rows = []
    for d in dirs:
        rows += _pmc_rows(d)
    return rows


SIMDS = 256 * 4   # MI355X: 256 compute units of four SIMDs


def _num_xcc(dirs):
    """XCDs of the profiled GPU (rocprofv3's agent info), default 8."""
    import csv
    import glob
    for d in dirs:
        for f in glob.glob(os.path.join(d, "**", "*agent_info.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r.get("Agent_Type") == "GPU" and r.get("Num_Xcc"):
                    return int(r["Num_Xcc"])
    return 8


def derive_counters(dirs):
    """Per kernel from rocprofv3 --pmc output dirs (any counter set per
    dir): every counter averaged over its dispatches
    (each value summed over the GPU's blocks), plus derived figures:
      - the dispatch's duration and the shader clock GRBM_GUI_ACTIVE implies
        (it counts on every XCD, so it is divided by their number);
      - the matrix pipes' busy fraction: busy cycles summed over SIMDs over
        (active cycles per XCD x SIMDs), rocprofv3's MfmaUtil;
      - the products' FLOPs by the MOPS counters (x 512), their rate, and
        that rate against 2.5 PFLOP/s and against the peak at the clock the
        dispatch ran at (1024 FLOP per clock per SIMD);
      - LDS and other vector instructions per product."""
    xcc = _num_xcc(dirs)
    per, dur = {}, {}
    for r in _counter_rows(dirs):
        name = r["Kernel_Name"]
        key = next((k for k in KERNELS if k in name), None)
        if key is None:
            continue
        per.setdefault(key, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        dur.setdefault(key, {})[(d_id := (r.get("Dispatch_Id"), r.get("Start_Timestamp")))] = (
            float(r["End_Timestamp"]) - float(r["Start_Timestamp"]))
    res = {}
    for k, cs in per.items():
        e = {c: sum(v) / len(v) for c, v in cs.items()}
        e["dispatches"] = min(len(v) for v in cs.values())   # per pass (GRBM_GUI_ACTIVE is in every pass)
        ns = sorted(dur[k].values())
        e["duration_ns_median"] = ns[len(ns) // 2]
        g = e.get("GRBM_GUI_ACTIVE")
        if g:
            e["num_xcc"] = xcc
            e["active_cycles_per_xcd"] = g / xcc
            e["clock_ghz"] = g / xcc / e["duration_ns_median"]
        if g and "SQ_VALU_MFMA_BUSY_CYCLES" in e:
            e["mfma_busy_frac"] = e["SQ_VALU_MFMA_BUSY_CYCLES"] / (g / xcc * SIMDS)
        mops = e.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) + e.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0)
        if mops:
            f = mops * 512.0
            e["mfma_flop_by_mops"] = f
            e["mfma_tflops_by_mops"] = f / (e["duration_ns_median"] * 1e-9) / 1e12
            e["mfma_frac_of_2500_tflops"] = e["mfma_tflops_by_mops"] / PEAK_BF16_TFLOPS
            if "clock_ghz" in e:
                e["mfma_frac_of_clock_peak"] = (e["mfma_tflops_by_mops"] * 1e12
                                                / (e["clock_ghz"] * 1e9 * SIMDS * 1024.0))
        va = valu_active_frac(e)
        if va is not None:
            e["valu_active_frac"] = va
        nmf = e.get("SQ_INSTS_VALU_MFMA_BF16", 0.0) + e.get("SQ_INSTS_VALU_MFMA_F16", 0.0)
        if nmf and "SQ_INSTS_LDS" in e:
            e["lds_insts_per_mfma"] = e["SQ_INSTS_LDS"] / nmf
        if nmf and "SQ_INSTS_VALU" in e:
            e["valu_insts_per_mfma"] = (e["SQ_INSTS_VALU"] - nmf) / nmf
        res[k] = e
    return res


def write_counters(dirs, workload):
    """profiles/counters.json from rocprofv3 --pmc output dirs
    (derive_counters), keyed by the kernels' source hash."""
    res = derive_counters(dirs)
    for k, e in res.items():
        e["source_hash"] = source_hash(_family(k))
    path = os.path.join(ROOT, "profiles", "counters.json")
    rec = json.load(open(path)) if os.path.exists(path) else {}
    rec.setdefault(workload, {}).update(res)
    with open(path, "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)
    print(json.dumps(rec[workload], indent=1))


def _committed(name, workload, kernel):
    """A kernel's entry of profiles/<name>.json if taken with the current
    sources and flags, else None."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        entry = json.load(open(path)).get(workload, {}).get(kernel)
    except (ValueError, OSError):
        return None
    if entry and entry.get("source_hash") == source_hash(_family(kernel)):
        return entry
    return None


def hbm_entry(rd, wr, alg, n2, ms):
    """A kernel's counter bytes read (rd) and written (wr) per launch against
    its algorithmic bytes (alg: {"read", "write"}), one N x N matrix in 16
    bits (n2) and its launch time in ms."""
    return {
        "read_bytes": rd, "write_bytes": wr,
        "algorithmic_read_bytes": alg["read"], "algorithmic_write_bytes": alg["write"],
        "read_ratio": rd / alg["read"], "write_ratio": wr / alg["write"],
        "gbs": (rd + wr) / (ms * 1e-3) / 1e9,
        "frac_of_hbm_peak": (rd + wr) / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "n2_matrix_bytes": n2,
        # reads beyond the algorithmic bytes are tiles of the inputs fetched
        # again by other workgroups (L2 misses); their total grows as
        # N^2 d^2 / (tile size) and can reach N^2 itself
        "excess_read_bytes": rd - alg["read"],
        # S or P in HBM would have to be written there first: every kernel of
        # the step writing within 10% of its outputs, and far less than one
        # N x N matrix beyond them, rules it out
        "no_n2_traffic": bool(wr <= 1.1 * alg["write"] and wr - alg["write"] < 0.05 * n2),
    }


def attach_counters(w, kernels):
    """Per kernel: HBM bytes from the committed FETCH/WRITE counters against
    the algorithmic bytes (and the GB/s they mean at the live launch time),
    whether any N x N traffic reached HBM, and the matrix pipes' counter
    utilisation.  Entries taken with other sources or flags are left out."""
    alg = algorithmic_bytes(w)
    n2 = w.B * w.H * w.N * w.N * 2 * (0.5 if w.causal else 1.0)   # one S (or P) in 16 bits
    for k, kern in kernels.items():
        tr = _committed("traffic.json", w.name, k)
        if tr and k in alg:
            kern["hbm"] = hbm_entry(tr.get("fetch_size_bytes", 0.0), tr.get("write_size_bytes", 0.0),
                                    alg[k], n2, kern["ms_mean"])
        c = _committed("counters.json", w.name, k)
        if c:
            kern["counters"] = {x: c[x] for x in ("mfma_busy_frac", "mfma_flop_by_mops",
                                                  "mfma_frac_of_clock_peak", "clock_ghz",
                                                  "lds_insts_per_mfma", "valu_insts_per_mfma",
                                                  "SQ_LDS_BANK_CONFLICT") if x in c}
            if "mfma_flop_by_mops" in c:
                kern["counters"]["mfma_tflops_by_mops"] = (c["mfma_flop_by_mops"]
                                                           / (kern["ms_mean"] * 1e-3) / 1e12)
            if "valu_active_frac" in c:
                kern["counters"]["valu_active_frac"] = c["valu_active_frac"]


def valu_active_frac(e):
    """The SIMDs' vector-ALU issue cycles over their active cycles.
    SQ_ACTIVE_INST_VALU counts in units of four cycles, the time a SIMD
    takes to issue one plain wave64 vector instruction (a fit over the
    forward and both backward kernels gives 1.00 unit per plain
    instruction, 2.00 per transcendental and 1.00 per matrix product)."""
    if "SQ_ACTIVE_INST_VALU" in e and "active_cycles_per_xcd" in e:
        return e["SQ_ACTIVE_INST_VALU"] * 4.0 / (e["active_cycles_per_xcd"] * SIMDS)
    return None


OTHER_WORKLOADS = ("gpt2_medium_fwd", "long_context_fwd", "recompute_bwd")


def bench_standard(args):
    """The materialised standard attention (attn_std_scores, attn_std_softmax,
    attn_std_pv: S and P written to HBM in full and read back) against the
    fused forward (attn_fwd) on the same inputs, one pass of each per step.
    Default workload: the GPT-2-medium shape of the pages' comparison.
    Algorithmic HBM bytes per head: the standard passes move S (fp32)
    written and read, P (16-bit) written and read -- the explainer's 4 N^2
    elements -- plus Q, K, V read and O, lse written; the fused forward only
    the latter.  Their FETCH/WRITE counters go to profiles/traffic.json
    under the workload's name with --copy-calibration and --traffic."""
    dev = torch.device("cuda:0")
    name = args.workload if args.workload != "llama7b_layer_fwd" else "gpt2_medium_fwd"
    w = inputs.WORKLOADS[name]
    t = inputs.make_inputs(w)
    q, k, v = (t[x].to(dev) for x in ("q", "k", "v"))
    B, H, N, d = w.B, w.H, w.N, w.d
    BH = B * H
    code = attn.ATTN_BF16 if w.dtype == "bf16" else attn.ATTN_F16
    scale = 1.0 / math.sqrt(d)
    causal = int(w.causal)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=dev)
    o2 = torch.empty_like(q)
    lse2 = torch.empty_like(lse)
    need = attn.attn_std_workspace_size(B, H, N, d, code)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    sbytes = (BH * N * N * 4 + 255) // 256 * 256
    sp_ = ws.data_ptr()
    pp_ = sp_ + sbytes
    stream = torch.cuda.current_stream(dev)
    st_ = stream.cuda_stream

    def ck(st, nm):
        if st:
            raise attn.AttnError(st, nm)

    calls = [
        ("std_scores_kernel", lambda: ck(attn.attn_std_scores(q.data_ptr(), k.data_ptr(), sp_, B, H, N, d,
                                                              scale, code, st_), "attn_std_scores")),
        ("std_softmax_kernel", lambda: ck(attn.attn_std_softmax(sp_, pp_, lse2.data_ptr(), B, H, N, causal,
                                                                code, st_), "attn_std_softmax")),
        ("std_pv_kernel", lambda: ck(attn.attn_std_pv(pp_, v.data_ptr(), o2.data_ptr(), B, H, N, d, code,
                                                      code, st_), "attn_std_pv")),
        ("fwd_kernel", lambda: ck(attn.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                                lse.data_ptr(), B, H, N, d, scale, causal, code, code,
                                                st_), "attn_fwd")),
    ]
    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    for _ in range(args.warmup):
        for _, fn in calls:
            fn()
    torch.cuda.synchronize()
    nc = len(calls)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(nc + 1)] for _ in range(args.steps)]
    for st in range(args.steps):
        ev[st][0].record(stream)
        for j, (_, fn) in enumerate(calls):
            fn()
            ev[st][j + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([[ev[s_][j].elapsed_time(ev[s_][j + 1]) for j in range(nc)]
                    for s_ in range(args.steps)])
    e = 2
    io = BH * N * d * e
    alg = {"std_scores_kernel": {"read": 2 * io, "write": BH * N * N * 4},
           "std_softmax_kernel": {"read": BH * N * N * 4, "write": BH * N * N * e + BH * N * 4},
           "std_pv_kernel": {"read": BH * N * N * e + io, "write": io},
           "fwd_kernel": {"read": 3 * io, "write": io + BH * N * 4}}
    kern = {}
    for j, (nm, _) in enumerate(calls):
        m = float(per[:, j].mean())
        b = alg[nm]["read"] + alg[nm]["write"]
        kern[nm] = {"ms_mean": m, "ms_min": float(per[:, j].min()),
                    "algorithmic_read_bytes": alg[nm]["read"], "algorithmic_write_bytes": alg[nm]["write"],
                    "algorithmic_gbs": b / (m * 1e-3) / 1e9,
                    "frac_of_hbm_peak": b / (m * 1e-3) / 1e9 / PEAK_HBM_GBS}
        tr = _committed("traffic.json", w.name, nm)
        if tr:
            kern[nm]["counter_read_bytes"] = tr.get("fetch_size_bytes")
            kern[nm]["counter_write_bytes"] = tr.get("write_size_bytes")
    std_ms = sum(kern[n]["ms_mean"] for n in ("std_scores_kernel", "std_softmax_kernel", "std_pv_kernel"))
    fused_ms = kern["fwd_kernel"]["ms_mean"]
    std_bytes = sum(alg[n]["read"] + alg[n]["write"] for n in ("std_scores_kernel", "std_softmax_kernel",
                                                                 "std_pv_kernel"))
    fused_bytes = alg["fwd_kernel"]["read"] + alg["fwd_kernel"]["write"]
    flops = 4.0 * BH * N * N * d * (0.5 if w.causal else 1.0)
    out = {
        "metric": "materialised standard attention vs fused forward: ms and HBM bytes at 1 GPU",
        "value": std_ms / fused_ms, "unit": "x (standard time / fused time)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.describe()}; standard = attn_std_scores + "
                               f"attn_std_softmax + attn_std_pv (S fp32, P {w.dtype} in HBM); "
                               f"fused = attn_fwd"},
        "standard_ms": std_ms, "fused_ms": fused_ms,
        "standard_algorithmic_bytes": std_bytes, "fused_algorithmic_bytes": fused_bytes,
        "byte_ratio": std_bytes / fused_bytes,
        "standard_tflops": flops / (std_ms * 1e-3) / 1e12, "fused_tflops": flops / (fused_ms * 1e-3) / 1e12,
        "elements_per_head_standard": 4 * N * N + 4 * N * d, "elements_per_head_fused": 4 * N * d,
        "roofline": {"bound": "hbm", "kernel": "std_softmax_kernel",
                     "achieved": kern["std_softmax_kernel"]["algorithmic_gbs"], "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": kern["std_softmax_kernel"]["frac_of_hbm_peak"],
                     "traffic": None},
        "kernels": kern,
    }
    tr = _committed("traffic.json", w.name, "std_softmax_kernel")
    if tr:
        out["roofline"]["traffic"] = tr.get("bytes")
    print(json.dumps(out), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU and has no multi-GPU path: every (batch, head) "
              "is independent, so heads shard across GPUs without communication. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.traffic:
        write_traffic(args.traffic[0], args.traffic[1], args.workload)
        return
    if args.counters:
        write_counters(args.counters, args.workload)
        return
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.decode is not None or args.fp8:
        if args.decode is None:
            bench_fp8(args)
        else:
            bench_decode(args)
        return
    if args.standard:
        bench_standard(args)
        return
    if args.hbm_ceiling:
        c = hbm_ceiling(torch.device("cuda:0"), reps=max(1, args.steps))
        print(json.dumps({"metric": "HBM read rate (one pass over a 4 GiB buffer) at 1 GPU",
                          "value": c["gbs"], "unit": "GB/s", "n_gpus": 1, "steps": c["launches"],
                          "warmup": 2, "ms_per_step": c["bytes"] / (c["gbs"] * 1e9) * 1e3,
                          "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "i32",
                          "data": "synthetic",
                          "config": {"workload": "attn_probe_hbm: " + c["kernel"], "bytes": c["bytes"],
                                     "workgroups": c["workgroups"]},
                          "frac_of_peak": c["frac_of_spec"], "gbs_by_workgroups": c["gbs_by_workgroups"]}),
              flush=True)
        return
    if args.ceiling:
        c = mfma_ceiling(torch.device("cuda:0"), reps=max(1, args.steps))
        print(json.dumps({"metric": "bf16 matrix-core sustained rate (products only) at 1 GPU",
                          "value": c["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": c["launches"],
                          "warmup": 2, "ms_per_step": c["ms_median"], "higher_is_better": True,
                          "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
                          "config": {"workload": "attn_probe_mfma: " + c["kernel"],
                                     "workgroups": c["workgroups"], "rounds": c["rounds"]},
                          "frac_of_peak": c["frac_of_spec"]}), flush=True)
        return
    dev = torch.device("cuda:0")
    w = inputs.WORKLOADS[args.workload]
    run = StepRunner(w, dev, dropout=args.dropout)
    drop = run.drop

    if args.copy_calibration:
        src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(2):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst

    ms_step, kernels, phases, flops_step = run.time(args.phase, args.steps, args.warmup)
    value = flops_step / (ms_step * 1e-3) / 1e12
    if drop is None:
        attach_counters(w, kernels)

    # roofline of the dominant kernel (longest mean launch)
    dom = max(kernels, key=lambda k_: kernels[k_]["ms_mean"])
    traffic = kernels[dom].get("hbm", {})
    traffic = traffic.get("read_bytes", 0.0) + traffic.get("write_bytes", 0.0) if traffic else None
    achieved = kernels[dom]["tflops"]
    roofline = {"bound": "mfma", "kernel": dom, "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS, "traffic": traffic,
                "flops_per_launch": run.algo[dom], "launch_ms": kernels[dom]["ms_mean"]}
    names = [nm for nm, _ in run.calls[args.phase]]
    B, H, N, d = w.B, w.H, w.N, w.d

    out = {
        "metric": "attention fwd/bwd TFLOP/s at 1 GPU + % of bf16 MFMA peak",
        "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: {w.describe()}; step = {' + '.join(names)}"
                               + ("" if drop is None else f"; dropout p={drop[0]} (seed, offset)={DROP_STATE}"),
                   "global_batch": B, "seq_len": N, "heads": H, "head_dim": d,
                   "causal": w.causal, "parallelism": "none (1 GPU)"},
        "frac_of_peak": value / PEAK_BF16_TFLOPS,
        "phases": phases,
        "kernels": kernels,
        "roofline": roofline,
        "kernel_source_hash": source_hash(),
    }
    if not args.no_other_workloads:
        # the matrix cores' sustained rate on this board: each kernel's rate
        # against it, beside the published peak
        ceil = mfma_ceiling(dev)
        out["mfma_ceiling"] = ceil
        out["frac_of_measured_ceiling"] = value / ceil["tflops"]
        roofline["frac_of_measured_ceiling"] = achieved / ceil["tflops"]
        for rec in list(phases.values()) + list(kernels.values()):
            if "tflops" in rec:
                rec["frac_of_measured_ceiling"] = rec["tflops"] / ceil["tflops"]
    o, lse = run.o, run.lse
    if not args.no_cpu_baseline and drop is None:
        torch.cuda.synchronize()
        out["cpu_baseline"] = cpu_baseline(w, run.t, float(np.float32(run.scale)), args.cpu_seconds,
                                           gpu_out=None if args.no_parity else (o, lse))
    if not args.no_other_workloads and drop is None and args.phase == "step":
        # the other workloads' forward alone and whole step, for context (not the headline)
        del run
        others = {}
        for name in OTHER_WORKLOADS:
            if name == w.name:
                continue
            wo = inputs.WORKLOADS[name]
            r = StepRunner(wo, dev)
            # untimed passes for about 0.1 s first, so that the clock has settled
            # after the idle gap of the input generation
            r.settle("step", 0.1)
            fms, fk, fph, ff = r.time("fwd", args.other_steps, 3)
            sms, sk, sph, sf = r.time("step", args.other_steps, 3)
            attach_counters(wo, sk)
            fkm = fk["fwd_kernel"]["ms_mean"]
            others[name] = {"workload": wo.describe(), "steps": args.other_steps, "warmup": "0.1 s, then 3",
                            "fwd_alone_ms": fms, "fwd_alone_tflops": ff / (fms * 1e-3) / 1e12,
                            "fwd_alone_kernel_ms": fkm, "fwd_alone_kernel_tflops": ff / (fkm * 1e-3) / 1e12,
                            "step_ms": sms, "step_tflops": sf / (sms * 1e-3) / 1e12,
                            "step_frac_of_peak": sf / (sms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
                            "phases_in_step": sph, "kernels_in_step": sk}
            del r
            torch.cuda.empty_cache()
        out["other_workloads"] = others
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
