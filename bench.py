#!/usr/bin/env python3
"""Engram forward throughput on one MI355X at the Engram-27B scale.

One step = one forward pass of the whole hot path (hash -> row gather ->
MFMA key/value projection with the fused gate partial sums -> gate + causal
conv) over B x T = 32 x 4096 synthetic Zipf(1.0) tokens, 16 bf16 tables of
~4.45M x 80 (5.7B parameters) resident in HBM, hidden 2560.  Prints one JSON
line with tokens/s, the roofline of the dominant kernel, the HBM figures of
the memory-bound kernels and the oracle timed on the host cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_F32_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_units(wl, N):
    """Algorithmic bytes / flops per launch of each forward kernel."""
    es = 2 if wl.dtype == "bf16" else 4
    J, d, dm = wl.J, wl.hidden, wl.d_mem
    nkt = d // 256
    return {
        "hash": {"bound": "hbm", "bytes": N * 4 + N * J * 4},
        "gather": {"bound": "hbm", "bytes": N * J * 4 + 2 * N * dm * es},
        "proj_gemm": {"bound": "mfma", "flops": 2 * N * dm * 2 * d,
                      "bytes": N * dm * es + 2 * d * dm * es + 2 * N * d * es + N * nkt * 12},
        # the same projection reading the table rows itself (row gather fused)
        "gather_proj_gemm": {"bound": "mfma", "flops": 2 * N * dm * 2 * d,
                             "bytes": N * J * 4 + N * dm * es + 2 * d * dm * es + 2 * N * d * es
                             + N * nkt * 12},
        "gate_conv": {"bound": "hbm", "bytes": 2 * N * d * es + N * nkt * 12},
    }


def cpu_baseline(inp, budget_s: float):
    """The oracle, as it stands, on sampled positions of the same workload."""
    import numpy as np

    import oracle
    from tests import harness as H
    wl = inp.wl
    p = oracle.Problem.from_inputs(inp)
    cores = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    pos_all = H.sample_positions(wl.B, wl.T, 1 << 16, seed=99)
    done = 0
    t0 = time.perf_counter()
    chunk = 64
    while done < pos_all.size and time.perf_counter() - t0 < budget_s:
        p.forward(pos_all[done:done + chunk], want=("y",))
        done += min(chunk, pos_all.size - done)
        chunk = min(chunk * 2, 1024)
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} sampled token positions of the {wl.name} workload "
                      f"(each: hash, gather, both projections, gate of 4 tokens, conv), {dt:.1f} s"}


def copy_calibration(nbytes: int):
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    ms = []
    for _ in range(5):
        start.record()
        dst.copy_(src)
        end.record()
        torch.cuda.synchronize()
        ms.append(start.elapsed_time(end))
    best = min(ms)
    print(json.dumps({"copy_bytes": nbytes, "best_ms": best,
                      "GBps_read_plus_write": round(2 * nbytes / (best * 1e-3) / 1e9, 1)}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="engram27b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--fused-gather", action="store_true",
                    help="let the projection read the table rows itself (ENGRAM_FLAG_FUSED_GATHER) "
                         "instead of gathering e into the workspace first")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 5 times (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the multi-GPU table sharding is a design note, not a code path", file=sys.stderr)
        sys.exit(2)

    import torch

    import hashed_gram_embedding_canon_amd as eg
    import synth
    from tests import harness as H

    wl = synth.get_workload(args.workload)
    N = wl.n_tokens
    log(f"[bench] {wl.name}: B={wl.B} T={wl.T} J={wl.J} D={wl.dim} d={wl.hidden} "
        f"table params={wl.table_params / 1e9:.2f}B; generating inputs")
    t = time.perf_counter()
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp, flags=eg.ENGRAM_FLAG_FUSED_GATHER if args.fused_gather else 0)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM after {time.perf_counter() - t:.1f} s")
    y = torch.empty(wl.B, wl.T, wl.hidden, dtype=dp.tdtype, device="cuda")
    ws = dp.workspace(eg.ENGRAM_OP_FORWARD)
    saved = None
    for _ in range(args.warmup):
        dp.forward(saved, ws=ws, y=y)
    torch.cuda.synchronize()
    log(f"[bench] warmup done ({args.warmup} steps)")

    eg.engram_profile_reset()
    eg.engram_profile_enable(True)
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        dp.forward(saved, ws=ws, y=y)
    end.record()
    torch.cuda.synchronize()
    eg.engram_profile_enable(False)
    prof = eg.engram_profile_read()
    ms = start.elapsed_time(end) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step")

    units = kernel_units(wl, N)
    kernels = {}
    for name, (count, tot_ms) in prof.items():
        avg = tot_ms / max(count, 1)
        u = units.get(name, {})
        ent = {"launches": count, "avg_ms": round(avg, 5)}
        if "bytes" in u:
            ent["alg_GBps"] = round(u["bytes"] / (avg * 1e-3) / 1e9, 1)
            ent["hbm_frac"] = round(ent["alg_GBps"] / HBM_PEAK_GBS, 4)
        if "flops" in u:
            ent["TFLOPs"] = round(u["flops"] / (avg * 1e-3) / 1e12, 1)
        kernels[name] = ent
    dom = max(prof.items(), key=lambda kv: kv[1][1])[0] if prof else None
    roof = None
    if dom is not None:
        u = units[dom]
        avg_s = prof[dom][1] / prof[dom][0] * 1e-3
        if u["bound"] == "mfma":
            peak = MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS
            ach = u["flops"] / avg_s / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(ach / peak, 4), "traffic": None}
        else:
            ach = u["bytes"] / avg_s / 1e9
            roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": None}
    mem_names = [k for k in ("gather", "gate_conv") if k in prof]
    mem_ms = sum(prof[k][1] / prof[k][0] for k in mem_names)
    mem_bytes = sum(units[k]["bytes"] for k in mem_names)
    es = 2 if wl.dtype == "bf16" else 4
    alg_per_token = wl.J * wl.dim * es + 2 * wl.hidden * es + 4  # rows + h + Y + token id

    out = {
        "metric": "Engram fwd tokens/s + achieved HBM GB/s (gather+gate+conv), 27B-scale table",
        "value": round(N / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "row_gather": "fused into projection" if args.fused_gather else "gathered into workspace", "batch": wl.B, "seq_len": wl.T, "tables": wl.J,
                   "rows_per_table": list(wl.rows[:1]) + ["..."], "dim": wl.dim,
                   "d_mem": wl.d_mem, "hidden": wl.hidden, "table_params": wl.table_params,
                   "zipf_s": wl.zipf_s, "vocab": wl.vocab, "canon_vocab": wl.canon_vocab},
        "roofline": roof,
        "hbm_gather_gate_conv": {"kernels": mem_names, "alg_GBps": round(mem_bytes / (mem_ms * 1e-3) / 1e9, 1) if mem_ms else None,
                                 "frac": round(mem_bytes / (mem_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4) if mem_ms else None,
                                 "ms": round(mem_ms, 4)},
        "end_to_end_alg_GBps": round(alg_per_token * N / (ms * 1e-3) / 1e9, 1),
        "kernels": kernels,
    }
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on host cores for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
