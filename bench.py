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
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
MFMA_FP8_PEAK_TFLOPS = 5000.0
MFMA_F32_PEAK_TFLOPS = 157.3


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_units(wl, N):
    """Algorithmic bytes / flops per launch of each forward kernel: the bytes a
    kernel must move (each input read once, each output written once) and the
    multiply-adds of its contraction.  With M branches the projection has
    (M+1)*d outputs and reads M hidden states; gate + conv reads v once and
    writes one Y per branch."""
    es = 2 if wl.dtype == "bf16" else 4
    J, d, dm, M = wl.J, wl.hidden, wl.d_mem, wl.branches
    nkt = d // 256
    proj_bytes = N * dm * es + (M + 1) * d * dm * es + (M + 1) * N * d * es + M * N * nkt * 12
    return {
        "hash": {"bound": "hbm", "bytes": N * 4 + N * J * 4},
        "gather": {"bound": "hbm", "bytes": N * J * 4 + 2 * N * dm * es},
        # hash and gather in one kernel: token ids in, rows in, e out (no indices)
        "hash_gather": {"bound": "hbm", "bytes": N * 4 + 2 * N * dm * es},
        # the same with rows repeated inside a 16-token tile read once (the
        # algorithmic bytes count every token's rows, as for hash_gather)
        "dedup_gather": {"bound": "hbm", "bytes": N * 4 + 2 * N * dm * es},
        "proj_gemm": {"bound": "mfma", "flops": 2 * N * dm * (M + 1) * d, "bytes": proj_bytes},
        # the same projection reading the table rows itself (row gather fused)
        "gather_proj_gemm": {"bound": "mfma", "flops": 2 * N * dm * (M + 1) * d,
                             "bytes": N * J * 4 + proj_bytes},
        # v is read once for all branches; each branch writes its own Y
        "gate_conv": {"bound": "hbm", "bytes": (M + 1) * N * d * es + M * N * nkt * 12},
        # FP8 projection: E4M3 e and W (one byte each) with their fp32 scales
        "proj_gemm_fp8": {"bound": "mfma_fp8", "flops": 2 * N * dm * (M + 1) * d,
                          "bytes": N * dm + N * 4 + (M + 1) * d * (dm + 4) + (M + 1) * N * d * es
                          + M * N * nkt * 12},
        "quant_w": {"bound": "hbm", "bytes": (M + 1) * d * (dm * es + dm + 4)},
        # indices + bf16 rows in, E4M3 e and its scale out
        "gather_quant": {"bound": "hbm", "bytes": N * J * 4 + N * dm * es + N * dm + N * 4},
    }


def cpu_baseline(inp, budget_s: float):
    """The oracle, as it stands, on sampled positions of the same workload."""
    import numpy as np

    import oracle
    from tests import harness as H
    wl = inp.wl
    p = oracle.Problem.from_inputs(inp)
    cores = int(oracle._load().oracle_threads())  # the threads its OpenMP loops use
    host = ""
    try:
        with open("/proc/cpuinfo") as fh:
            host = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
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
                      f"(each: hash, gather, both projections, gate of 4 tokens, conv), {dt:.1f} s",
            "host_cpu": host}


# ------------------------------------------------------------ rocprofv3 summaries
def kernel_key(name: str) -> str:
    """The bench's name for a rocprofv3 kernel name (empty for other kernels)."""
    base = name.split("(")[0]
    if "gemm_kernel<" in base:
        targs = base.split("<", 1)[1].rstrip(">").replace(" ", "").split(",")
        gt, epi, gather = targs[0], targs[1], targs[2]
        if epi == "1":
            return "de_gemm"
        if gt == "3":
            return "proj_gemm_fp8"
        return "gather_proj_gemm" if gather == "true" else "proj_gemm"
    if "gemm_tn_kernel" in base or "tn_reduce_kernel" in base:
        return "dw_gemm"
    if "colsum64_kernel" in base or "param_finish_kernel" in base:
        return "bwd_param_sums"
    if "bwd_gate_conv_kernel<" in base:
        targs = base.split("<", 1)[1].rstrip(">").replace(" ", "").split(",")
        return "bwd_gate_conv_params" if targs[2] == "true" else "bwd_gate_conv"
    if "quant_rows_kernel" in base:
        return "quant_w"
    if "bwd_scale_kernel" in base:
        return "bwd_scale"
    if "scale_rows_kernel" in base:
        return "scale_rows"
    for key in ("hash_gather", "dedup_gather", "gather_quant", "gate_conv", "gather", "hash",
                "transpose_w", "atomic_scatter"):
        if f"engram::{key}_kernel" in base:
            return key
    # the per-GPU steps of the sharded exchange
    if "owner_bounds_kernel" in base or "shard_pack_kernel" in base or "remap_kernel" in base:
        return "shard_pack"
    if "serve_kernel" in base:
        return "shard_serve"
    if "grad_add_kernel" in base:
        return "shard_reduce"
    if "seg_inverse_kernel" in base:
        return "shard_dedup"
    for key in ("sort_", "seg_"):
        if "engram::" + key in base:
            return "sorted_scatter"
    if "copyBuffer" in base or "engram::stream_copy_kernel" in base:
        return "copy"
    return ""


def code_tokens(src: str) -> str:
    """C/C++ source without its comments and with whitespace runs collapsed:
    what the compiler sees, so edits of comments do not count as changes."""
    import re
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def csrc_digest(root: str | None = None) -> str:
    """sha256 over the code of the library sources (comments excluded);
    traffic figures are tied to it."""
    import hashlib
    root = root or ROOT
    h = hashlib.sha256()
    d = os.path.join(root, "hashed_gram_embedding_canon_amd", "csrc")
    files = [os.path.join(d, f) for f in sorted(os.listdir(d)) if f.endswith((".hip", ".h"))]
    for path in files + [os.path.join(root, "include", "engram.h")]:
        with open(path, encoding="utf-8") as fh:
            h.update(os.path.basename(path).encode() + b"\0" + code_tokens(fh.read()).encode())
    return h.hexdigest()[:16]


# bench names made of several dispatches per call: the kernel that runs once per call
GROUP_LEADER = {"sorted_scatter": "sort_hist_kernel<true>", "dw_gemm": "gemm_tn_kernel",
                "bwd_param_sums": "param_finish_kernel", "shard_pack": "owner_bounds_kernel"}
# names whose leader is the last dispatch of a call (the others' is the first)
GROUP_LEADER_LAST = {"bwd_param_sums"}


def _pmc_per_kernel(csv_dir: str, counter: str) -> dict:
    """Counter value per call of each bench kernel (summed over the dispatches
    of one call where a bench name covers several kernels)."""
    import csv
    import glob
    total: dict = {}
    calls: dict = {}
    for path in glob.glob(os.path.join(csv_dir, "*counter_collection.csv")):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                if r["Counter_Name"] != counter:
                    continue
                k = kernel_key(r["Kernel_Name"])
                if not k:
                    continue
                total[k] = total.get(k, 0.0) + float(r["Counter_Value"])
                leader = GROUP_LEADER.get(k)
                if leader is None or leader in r["Kernel_Name"]:
                    calls[k] = calls.get(k, 0) + 1
    return {k: total[k] / calls[k] for k in total if calls.get(k)}


def summarize_trace(trace_dir: str) -> str:
    """Per-kernel durations of a rocprofv3 --kernel-trace run (bench kernels
    only; the dispatches in a row of one multi-dispatch bench name count as
    one call)."""
    import csv
    import glob
    import statistics
    rows = []
    for path in glob.glob(os.path.join(trace_dir, "*kernel_trace.csv")):
        with open(path) as fh:
            rows += [r for r in csv.DictReader(fh)]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    calls: dict = {}
    names: dict = {}
    prev_key, prev_name, cur = None, "", None
    for r in rows:
        k = kernel_key(r["Kernel_Name"])
        if not k or k == "copy":
            prev_key = None
            continue
        ns = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        names.setdefault(k, set()).add(r["Kernel_Name"].split("(")[0])
        lead = GROUP_LEADER.get(k, "")
        new_call = (lead in prev_name) if k in GROUP_LEADER_LAST else (lead in r["Kernel_Name"])
        if k == prev_key and lead and not new_call:
            cur[-1] += ns  # a later dispatch of the same call
        else:
            cur = calls.setdefault(k, [])
            cur.append(ns)
        prev_key, prev_name = k, r["Kernel_Name"]
    lines = [f"{'kernel':<21} {'calls':>5} {'mean_us':>9} {'median_us':>10} {'min_us':>9} {'max_us':>9}  kernels"]
    for k, v in sorted(calls.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{k:<21} {len(v):>5} {statistics.mean(v) / 1e3:>9.2f} {statistics.median(v) / 1e3:>10.2f} "
                     f"{min(v) / 1e3:>9.2f} {max(v) / 1e3:>9.2f}  {'; '.join(sorted(names[k]))}")
    return "\n".join(lines)


def summarize_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, copy_bytes) -> str:
    """HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE (KiB), each scaled by
    what the same counter reads for a plain device copy of copy_bytes."""
    fetch = _pmc_per_kernel(fetch_dir, "FETCH_SIZE")
    write = _pmc_per_kernel(write_dir, "WRITE_SIZE")
    cf = _pmc_per_kernel(copy_fetch_dir, "FETCH_SIZE")["copy"]
    cw = _pmc_per_kernel(copy_write_dir, "WRITE_SIZE")["copy"]
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    out = [f"source {csrc_digest()}",
           f"copy_calibration bytes {copy_bytes} fetch_kib {cf:.1f} write_kib {cw:.1f} "
           f"fetch_scale {f_scale:.4f} write_scale {w_scale:.4f}",
           f"{'kernel':<21} {'fetch_kib':>14} {'write_kib':>14} {'traffic_bytes':>16}"]
    for k in sorted(set(fetch) & set(write)):
        if k == "copy":
            continue
        t = fetch[k] * 1024.0 * f_scale + write[k] * 1024.0 * w_scale
        out.append(f"{k:<21} {fetch[k]:>14.1f} {write[k]:>14.1f} {t:>16.0f}")
    return "\n".join(out)


def summarize_pmc(csv_dir: str) -> str:
    """Mean per dispatch of every counter of a rocprofv3 --pmc run, for the
    MFMA kernels (the weight-gradient GEMM without its chunk-sum kernel)."""
    import csv
    import glob
    vals: dict = {}
    for path in glob.glob(os.path.join(csv_dir, "*counter_collection.csv")):
        with open(path) as fh:
            for r in csv.DictReader(fh):
                k = kernel_key(r["Kernel_Name"])
                if k not in ("proj_gemm", "proj_gemm_fp8", "gather_proj_gemm", "de_gemm", "dw_gemm"):
                    continue
                if k == "dw_gemm" and "gemm_tn_kernel" not in r["Kernel_Name"]:
                    continue
                vals.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    counters = sorted({c for v in vals.values() for c in v})
    lines = [f"{'kernel':<16} {'dispatches':>10} " + " ".join(f"{c:>28}" for c in counters)]
    for k, v in sorted(vals.items()):
        n = max(len(x) for x in v.values())
        lines.append(f"{k:<16} {n:>10} " + " ".join(
            f"{(sum(v[c]) / len(v[c]) if c in v else float('nan')):>28.6g}" for c in counters))
    return "\n".join(lines)


def traffic_from_profile(workload: str) -> dict:
    """{kernel: HBM bytes per launch} from profiles/traffic_<workload>.txt when
    that file was taken from the current sources, else {}."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(path):
        return {}
    rows, src = {}, None
    with open(path) as fh:
        for ln in fh:
            parts = ln.split()
            if not parts or ln.startswith("#"):
                continue
            if parts[0] == "source":
                src = parts[1]
            elif len(parts) == 4 and parts[0] not in ("kernel", "copy_calibration"):
                rows[parts[0]] = float(parts[3])
    return rows if src == csrc_digest() else {}


def backward_units(wl, N):
    """Algorithmic bytes / flops per launch of each table-gradient backward
    kernel.  With M branches the elementwise backward runs once per branch
    (dv gathers over them in fp32) and the contractions run over (M+1)d."""
    es = 2 if wl.dtype == "bf16" else 4
    eg_ = 2 if wl.dtype == "bf16" else 4          # fp16 / fp32 GEMM operands
    J, d, dm, D, M = wl.J, wl.hidden, wl.d_mem, wl.dim, wl.branches
    # dv per launch: written once (one branch), or fp32 first / add / last over M launches
    dv = N * d * eg_ if M == 1 else (N * d * (4 + 8 * (M - 2) + 4) + N * d * eg_) / M
    return {
        # bf16: the per-token fp16 range factors from dy (every branch), v and the stats
        "bwd_scale": {"bound": "hbm", "bytes": (M + 1) * N * d * es + M * N * 16 + N * 4},
        # dy, v, k, h in; stats; dk out, dv
        "bwd_gate_conv": {"bound": "hbm", "bytes": 4 * N * d * es + N * 16 + N * d * eg_ + dv},
        "transpose_w": {"bound": "hbm", "bytes": (M + 1) * d * dm * (es + eg_)},
        "de_gemm": {"bound": "mfma", "flops": 2 * N * (M + 1) * d * dm,
                    "bytes": N * (M + 1) * d * eg_ + (M + 1) * d * dm * eg_ + N * dm * 4},
        # idx + de in, at most one fp32 row + key per (token, table) out
        "sorted_scatter": {"bound": "hbm", "bytes": N * J * 4 + N * dm * 4 + N * J * (D * 4 + 8)},
        "atomic_scatter": {"bound": "hbm", "bytes": N * J * 4 + N * dm * 4 + N * J * D * 4},
    }


def training_units(wl, N):
    """The training backward's extra kernels (parameter and hidden-state
    gradients) on top of backward_units."""
    es = 2 if wl.dtype == "bf16" else 4
    eg_ = 2 if wl.dtype == "bf16" else 4
    J, d, dm, taps = wl.J, wl.hidden, wl.d_mem, wl.taps
    nblk = wl.B * ((wl.T + 63) // 64)
    u = backward_units(wl, N)
    # dh written and the per-workgroup conv / RMSNorm-scale sums
    u["bwd_gate_conv_params"] = {"bound": "hbm", "bytes": u["bwd_gate_conv"]["bytes"] + N * d * es
                                 + nblk * d * (taps + 1) * 4}
    # rows gathered again: indices + rows in, e out
    u["gather"] = {"bound": "hbm", "bytes": N * J * 4 + 2 * N * dm * es}
    # dW = [dk|dv]^T e: both token-major operands once, dW once
    M = wl.branches
    u["dw_gemm"] = {"bound": "mfma", "flops": 2 * N * (M + 1) * d * dm,
                    "bytes": N * (M + 1) * d * eg_ + N * dm * es + (M + 1) * d * dm * 4}
    u["bwd_param_sums"] = {"bound": "hbm", "bytes": nblk * d * (taps + 1) * 4}
    return u


def bench_backward(dp, inp, steps: int) -> dict:
    """Backward of the same workload: the table gradients by sorted segmented
    reduce (sparse rows) and by the dense-atomic variant, and the training
    backward (sorted table gradients plus dW_KV, conv taps, RMSNorm scales and
    dh, e gathered again); per-kernel times and rates."""
    import torch

    import hashed_gram_embedding_canon_amd as eg
    from tests import harness as H
    wl, N = dp.wl, dp.N
    import numpy as np
    saved = dp.alloc_saved(("idx", "stats", "k", "v"))
    dp.forward(saved)
    M = wl.branches
    dy = H.to_dev(inp.dy if M == 1 else np.ascontiguousarray(np.stack([inp.dy_branch(m) for m in range(M)])))
    ws = dp.workspace(eg.ENGRAM_OP_BACKWARD_PARAMS)
    res = {}
    for mode, label in ((eg.ENGRAM_GRAD_SORTED_SPARSE, "sorted_sparse"),
                        (eg.ENGRAM_GRAD_ATOMIC_DENSE, "atomic_dense"),
                        (eg.ENGRAM_GRAD_SORTED_SPARSE, "training")):
        training = label == "training"
        units = training_units(wl, N) if training else backward_units(wl, N)
        out = dp.backward(saved, dy, mode, ws=ws)  # warm-up; allocates the outputs
        pgrads, pg = None, None
        if training:
            pgrads = dp.backward_params(saved, dy, ws=ws)
            pg = eg.make_param_grad(**pgrads)
        torch.cuda.synchronize()
        tg = eg.engram_table_grad()
        tg.mode = mode
        if mode == eg.ENGRAM_GRAD_SORTED_SPARSE:
            tg.keys, tg.rows, tg.count = (out["keys"].data_ptr(), out["rows"].data_ptr(),
                                          out["count"].data_ptr())
        else:
            for j, t in enumerate(out["dense"]):
                tg.dense[j] = t.data_ptr()
        zero_ms = None
        if mode == eg.ENGRAM_GRAD_ATOMIC_DENSE:
            z0, z1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            z0.record()
            for t in out["dense"]:
                t.zero_()
            z1.record()
            torch.cuda.synchronize()
            zero_ms = z0.elapsed_time(z1)
        sv = eg.make_saved(**saved)
        eg.engram_profile_reset()
        eg.engram_profile_enable(True)
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(steps):
            if training:
                eg.engram_backward(dp.cfg, dp.params, dp.hidden, dy, B=dp.B, T=dp.T, saved=sv,
                                   table_out=tg, param_out=pg, workspace=ws)
            else:
                eg.engram_backward_table_grad(dp.cfg, dp.params, dp.hidden, dy, B=dp.B, T=dp.T,
                                              saved=sv, out=tg, workspace=ws)
        t1.record()
        torch.cuda.synchronize()
        eg.engram_profile_enable(False)
        prof = eg.engram_profile_read()
        ms = t0.elapsed_time(t1) / steps
        kern = {}
        for name, (count, tot) in prof.items():
            avg = tot / max(count, 1)
            ent = {"launches": count, "avg_ms": round(avg, 5)}
            u = units.get(name, {})
            if "bytes" in u and u["bound"] == "hbm":
                ent["alg_GBps"] = round(u["bytes"] / (avg * 1e-3) / 1e9, 1)
                ent["hbm_frac"] = round(ent["alg_GBps"] / HBM_PEAK_GBS, 4)
            if "flops" in u:
                ent["TFLOPs"] = round(u["flops"] / (avg * 1e-3) / 1e12, 1)
            kern[name] = ent
        entry = {"ms_per_step": round(ms, 4), "tokens_per_s": round(N / (ms * 1e-3), 1),
                 "kernels": kern}
        if mode == eg.ENGRAM_GRAD_SORTED_SPARSE:
            entry["unique_rows"] = int(out["count"].item())
            entry["token_table_pairs"] = N * wl.J
        if zero_ms is not None:
            entry["zero_dense_ms_excluded"] = round(zero_ms, 3)
            entry["note"] = "accumulates into the caller's dense fp32 tables without zeroing them"
        if training:
            entry["note"] = ("table gradients (sorted) + dW_KV, conv taps, RMSNorm scales, dh; "
                             "e gathered again from the tables")
        res[label] = entry
        del out, pgrads
        torch.cuda.empty_cache()
    return res


def bench_host(args):
    """Tables in host memory: the prefetch planner (indices ahead of time, then
    gather into pinned staging and async copy on a side stream) overlapped
    with k stand-in [N,4096]x[4096,4096] bf16 GEMMs, then the compact-mode
    forward.  exposed copy = (GEMMs + prefetch + forward) - (GEMMs + forward)."""
    import dataclasses

    import numpy as np
    import torch

    import hashed_gram_embedding_canon_amd as eg
    import synth
    from synth.workloads import primes_from
    from tests import harness as H
    base = synth.get_workload("host100b")
    wl = dataclasses.replace(base, rows=tuple(primes_from(args.host_rows, base.J)))
    N, J = wl.n_tokens, wl.J
    es = 2 if wl.dtype == "bf16" else 4
    log(f"[bench-host] {J} tables of ~{args.host_rows} x {wl.dim} in host memory "
        f"({wl.table_params / 1e9:.1f}B parameters); B={wl.B} T={wl.T} d={wl.hidden}")
    inp = synth.Inputs(wl)
    host_tables = []
    for j in range(J):  # a full-size table takes tens of seconds to generate
        host_tables.append(inp.table(j))
        log(f"[bench-host] table {j + 1}/{J} generated ({host_tables[-1].nbytes / 1e9:.1f} GB)")
    dp = H.DeviceProblem(inp, upload_tables=False)
    cap = N * J
    counts = np.zeros(J, np.int64)
    uniq = np.zeros(cap, np.int32)
    inv_h = torch.empty(N, J, dtype=torch.int32, pin_memory=True)
    staging = torch.empty(cap * wl.dim * es, dtype=torch.uint8, pin_memory=True)
    rows_dev = torch.empty(cap * wl.dim * es, dtype=torch.uint8, device="cuda")
    inv_dev = torch.empty(N, J, dtype=torch.int32, device="cuda")
    side = torch.cuda.Stream()
    ev = torch.cuda.Event(enable_timing=True)
    ev.record()
    plan = eg.engram_compact()
    plan.capacity_rows = cap
    plan.counts, plan.uniq_host = counts.ctypes.data, uniq.ctypes.data
    plan.inverse_host, plan.staging_host = inv_h.data_ptr(), staging.data_ptr()
    plan.rows_dev, plan.inverse_dev = rows_dev.data_ptr(), inv_dev.data_ptr()
    plan.ready_event = ev.cuda_event
    tok, canon = inp.tokens, inp.canon_map
    # 1. indices ahead of time (host threads)
    t = time.perf_counter()
    eg.engram_prefetch_plan(dp.cfg, canon, tok, B=wl.B, T=wl.T, host_tables=None, plan=plan)
    plan_ms = (time.perf_counter() - t) * 1e3
    plan.flags = eg.ENGRAM_PLAN_REUSE
    copy_bytes = int(plan.total_rows) * wl.dim * es + N * J * 4

    def prefetch():
        eg.engram_prefetch_plan(dp.cfg, canon, tok, B=wl.B, T=wl.T, host_tables=host_tables,
                                plan=plan, side_stream=side)

    # 2. gather + copy alone
    prefetch()
    torch.cuda.synchronize()
    s0 = torch.cuda.Event(enable_timing=True)
    s0.record(side)
    t = time.perf_counter()
    prefetch()
    host_ms = (time.perf_counter() - t) * 1e3
    torch.cuda.synchronize()
    copy_ms = s0.elapsed_time(ev)
    # the compact forward against the forward over the same tables in HBM
    # (uploaded for this check only)
    y_c = torch.empty(wl.B, wl.T, wl.hidden, dtype=dp.tdtype, device="cuda")
    dp.forward(compact=plan, y=y_c)
    log("[bench-host] uploading the tables once to check the compact forward against them")
    dev_tables = [H.to_dev(tb) for tb in host_tables]
    params_full = eg.make_params(canon_map=dp.canon, tables=dev_tables, w_kv=dp.w_kv, conv_w=dp.conv_w)
    y_full = torch.empty_like(y_c)
    eg.engram_forward(dp.cfg, params_full, dp.tokens, dp.hidden, y_full, B=wl.B, T=wl.T,
                      workspace=dp.workspace(eg.ENGRAM_OP_FORWARD))
    torch.cuda.synchronize()
    compact_identical = bool(torch.equal(y_c, y_full))
    del dev_tables, params_full, y_full, y_c
    torch.cuda.empty_cache()
    log(f"[bench-host] compact forward bit-identical to the HBM-table forward: {compact_identical}")
    # 3. compact forward alone, and the stand-in GEMM
    y = torch.empty(wl.B, wl.T, wl.hidden, dtype=dp.tdtype, device="cuda")
    ws = dp.workspace(eg.ENGRAM_OP_FORWARD)
    g = torch.Generator(device="cuda").manual_seed(7)
    xa = torch.randn(N, 4096, device="cuda", dtype=torch.bfloat16, generator=g)
    wg = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16, generator=g)
    yg = torch.empty(N, 4096, device="cuda", dtype=torch.bfloat16)

    def timed(fn, reps=3):
        out = []
        for _ in range(reps):
            torch.cuda.synchronize()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            fn()
            a1.record()
            torch.cuda.synchronize()
            out.append(a0.elapsed_time(a1))
        return float(np.median(out))

    fwd = lambda: dp.forward(compact=plan, ws=ws, y=y)  # noqa: E731
    for _ in range(2):
        fwd()
        torch.matmul(xa, wg, out=yg)
    fwd_ms = timed(fwd)
    gemm_ms = timed(lambda: torch.matmul(xa, wg, out=yg))
    sweep = []
    for k in (1, 2, 4, 8):
        def only():
            for _ in range(k):
                torch.matmul(xa, wg, out=yg)
            fwd()

        def overlapped():
            for _ in range(k):
                torch.matmul(xa, wg, out=yg)
            prefetch()
            fwd()
        t_only = timed(only)
        t_ovl = timed(overlapped)
        sweep.append({"gemms": k, "gemms_forward_ms": round(t_only, 3), "with_prefetch_ms": round(t_ovl, 3),
                      "exposed_copy_ms": round(max(0.0, t_ovl - t_only), 3),
                      "tokens_per_s": round(N / (t_ovl * 1e-3), 1)})
    ring = bench_ring(args, wl, inp, dp, host_tables, staging, inv_h, inv_dev, side, ev, y, ws,
                      lambda: torch.matmul(xa, wg, out=yg), timed)
    out = {
        "metric": "host-table Engram forward: tokens/s and exposed copy time",
        "workload": wl.name, "batch": wl.B, "seq_len": wl.T, "tables": J,
        "rows_per_table": list(wl.rows[:1]) + ["..."], "dim": wl.dim, "hidden": wl.hidden,
        "table_params": wl.table_params, "unique_rows": int(plan.total_rows),
        "compact_forward_bit_identical": compact_identical,
        "plan_ahead_ms": round(plan_ms, 2), "gather_host_ms": round(host_ms, 2),
        "h2d_copy_ms": round(copy_ms, 3), "copy_bytes": copy_bytes,
        "h2d_GBps": round(copy_bytes / (copy_ms * 1e-3) / 1e9, 1),
        "compact_forward_ms": round(fwd_ms, 3), "standin_gemm_ms": round(gemm_ms, 3),
        "tokens_per_s_forward_only": round(N / (fwd_ms * 1e-3), 1),
        "sweep": sweep,
        "row_ring": ring,
        "note": ("tables at the stated size (~48.8M rows each)" if args.host_rows >= 48_800_000 else
                 f"table rows reduced from ~48.8M to ~{args.host_rows} per table; the rows copied per "
                 "forward depend on the token stream, not the table size"),
    }
    print(json.dumps(out), flush=True)


def bench_ring(args, wl, inp, dp, host_tables, staging, inv_h, inv_dev, side, ev, y, ws, gemm,
               timed) -> dict:
    """Successive batches of one token stream, each planned ahead and then
    gathered + copied behind two stand-in GEMMs, without and with the HBM row
    ring (rows an earlier batch copied are not copied again)."""
    import numpy as np
    import torch

    import hashed_gram_embedding_canon_amd as eg
    import synth
    N, J = wl.n_tokens, wl.J
    es = 2 if wl.dtype == "bf16" else 4
    rb = wl.dim * es
    cap = N * J
    R = args.ring_factor * cap
    rows_dev = torch.empty(R * rb, dtype=torch.uint8, device="cuda")
    ring_pos = np.full(int(inp.table_rows.sum()), -1, np.int64)
    counts = np.zeros(J, np.int64)
    uniq = np.zeros(cap, np.int32)
    res = {"ring_rows": R, "ring_GiB": round(R * rb / 2**30, 2), "batches": args.ring_batches,
           "standin_gemms": 2}
    for mode in ("no_ring", "ring"):
        plan = eg.engram_compact()
        plan.capacity_rows = cap
        plan.counts, plan.uniq_host = counts.ctypes.data, uniq.ctypes.data
        plan.inverse_host, plan.staging_host = inv_h.data_ptr(), staging.data_ptr()
        plan.rows_dev, plan.inverse_dev = rows_dev.data_ptr(), inv_dev.data_ptr()
        plan.ready_event = ev.cuda_event
        if mode == "ring":
            ring_pos.fill(-1)
            plan.ring_rows, plan.ring_pos, plan.ring_head = R, ring_pos.ctypes.data, 0
        per = []
        for k in range(args.ring_batches):
            tok = synth.zipf_tokens(synth.seed_of(wl.cfg, synth.S_TOKENS), N, wl.vocab, wl.zipf_s,
                                    offset=k * N).reshape(wl.B, wl.T)
            plan.flags = 0
            eg.engram_prefetch_plan(dp.cfg, inp.canon_map, tok, B=wl.B, T=wl.T, host_tables=None,
                                    plan=plan)
            plan.flags = eg.ENGRAM_PLAN_REUSE
            torch.cuda.synchronize()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s0 = torch.cuda.Event(enable_timing=True)
            a0.record()
            gemm()
            gemm()
            s0.record(side)
            eg.engram_prefetch_plan(dp.cfg, inp.canon_map, tok, B=wl.B, T=wl.T,
                                    host_tables=host_tables, plan=plan, side_stream=side)
            dp.forward(compact=plan, ws=ws, y=y)
            a1.record()
            torch.cuda.synchronize()
            t_ovl = a0.elapsed_time(a1)
            copy_ms = s0.elapsed_time(ev)

            def only():
                gemm()
                gemm()
                dp.forward(compact=plan, ws=ws, y=y)
            t_only = timed(only)
            copied = int(plan.total_rows)  # with the ring, the plan keeps its misses only
            hits = int(plan.ring_hits) if mode == "ring" else 0
            per.append({"distinct_rows": copied + hits, "copied_rows": copied,
                        "copy_ms": round(copy_ms, 3), "exposed_copy_ms": round(max(0.0, t_ovl - t_only), 3)})
        later = per[1:] if len(per) > 1 else per
        res[mode] = {"per_batch": per,
                     "mean_copied_rows_after_first": round(float(np.mean([p["copied_rows"] for p in later])), 1),
                     "mean_exposed_copy_ms_after_first": round(float(np.mean([p["exposed_copy_ms"] for p in later])), 3)}
    res["copied_rows_reduction"] = round(1.0 - res["ring"]["mean_copied_rows_after_first"]
                                         / res["no_ring"]["mean_copied_rows_after_first"], 4)
    return res


def bench_shard(args):
    """Tables sharded over G GPUs, the device steps of one GPU at the 27B
    shape: G GPUs are emulated in one process (GPU r with batch r of the
    stream); GPU 0 is timed as sender (dedup + requests grouped by owner,
    gradient rows grouped by owner) and as owner (serve the requests of all
    G GPUs from its 1/G shard, add the gradient rows of all G GPUs), and its
    forward runs on the served rows.  The All-to-All is a device copy here;
    its bytes are reported with the time they take over xGMI links."""
    import numpy as np
    import torch

    import hashed_gram_embedding_canon_amd as eg
    import synth
    from tests import harness as H
    G = args.shard_gpus
    wl = synth.get_workload("engram27b_bwd")
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    N, J, D = dp.N, wl.J, wl.dim
    es = 2 if wl.dtype == "bf16" else 4
    rb = D * es
    S = [(int(m) + G - 1) // G for m in inp.table_rows]
    shards0 = [dp.tables[j].view(-1)[: min(S[j], int(inp.table_rows[j])) * D] for j in range(J)]
    ws = torch.empty(eg.engram_workspace_size(dp.cfg, 1, N, eg.ENGRAM_OP_SHARD), dtype=torch.uint8,
                     device="cuda")
    dy = H.to_dev(inp.dy)
    cap = N * J
    log(f"[bench-shard] G={G}: requests, gradients and forwards of {G} emulated GPUs")
    ranks = []
    for r in range(G):
        tok = synth.zipf_tokens(synth.seed_of(wl.cfg, synth.S_TOKENS), N, wl.vocab, wl.zipf_s,
                                offset=r * N).reshape(dp.B, dp.T)
        dp.tokens_host, dp.tokens = tok, H.to_dev(tok)
        saved = dp.alloc_saved(("idx", "stats", "k", "v"))
        dp.forward(saved)
        send_ids = torch.empty(cap, dtype=torch.int32, device="cuda")
        counts = torch.empty(G, dtype=torch.int64, device="cuda")
        inverse = torch.empty(N, J, dtype=torch.int32, device="cuda")
        eg.engram_shard_requests(dp.cfg, G, saved["idx"], N, send_ids, counts, inverse, workspace=ws)
        sp = dp.backward(saved, dy, eg.ENGRAM_GRAD_SORTED_SPARSE)
        gids = torch.empty(cap, dtype=torch.int32, device="cuda")
        grows = torch.empty(cap, D, dtype=torch.float32, device="cuda")
        gcounts = torch.empty(G, dtype=torch.int64, device="cuda")
        eg.engram_shard_grads(dp.cfg, G, sp["keys"], sp["rows"], sp["count"], cap, gids, grows, gcounts,
                              workspace=ws)
        c, gc = counts.cpu().numpy(), gcounts.cpu().numpy()
        keep = {"c": c, "gc": gc}
        # what GPU 0 receives as owner: block 0 of every GPU
        keep["req0"] = send_ids[: c[0]].clone()
        keep["g0"] = (gids[: gc[0]].clone(), grows[: gc[0]].clone())
        if r == 0:
            keep.update(tok=tok, saved=saved, send_ids=send_ids, inverse=inverse, sp=sp, gids=gids,
                        grows=grows, gcounts_dev=gcounts)
        else:
            del saved, sp, gids, grows
        ranks.append(keep)
        torch.cuda.empty_cache()
    r0 = ranks[0]
    # owner 0: requests of all GPUs in GPU order, and their gradient rows
    recv = torch.cat([rk["req0"] for rk in ranks])
    served = torch.empty(recv.numel() * rb, dtype=torch.uint8, device="cuda")
    gids0 = torch.cat([rk["g0"][0] for rk in ranks])
    grows0 = torch.cat([rk["g0"][1] for rk in ranks]).contiguous()
    gblocks = [int(rk["gc"][0]) for rk in ranks]
    shard_grads = [torch.zeros(S[j] * D, dtype=torch.float32, device="cuda") for j in range(J)]
    # GPU 0's replies: block 0 of each owner; owner 0's is served above, the
    # others' are the same rows read from the whole tables (an owner's serve
    # is the same kernel on its shard)
    offs = np.concatenate([[0], np.cumsum(r0["c"])])
    parts = []
    for o in range(G):
        ids_o = r0["send_ids"][offs[o]: offs[o + 1]]
        out = torch.empty(max(ids_o.numel(), 1) * rb, dtype=torch.uint8, device="cuda")
        sh = [dp.tables[j].view(-1)[o * S[j] * D: min((o + 1) * S[j], int(inp.table_rows[j])) * D]
              for j in range(J)]
        eg.engram_shard_serve(dp.cfg, G, sh, ids_o, ids_o.numel(), out)
        parts.append(out[: ids_o.numel() * rb])
    replies = torch.cat(parts)
    plan = eg.engram_compact()
    plan.rows_dev, plan.inverse_dev = replies.data_ptr(), r0["inverse"].data_ptr()
    dp.tokens_host, dp.tokens = r0["tok"], H.to_dev(r0["tok"])
    y_ref = dp.forward()
    y = dp.forward(compact=plan)
    torch.cuda.synchronize()
    bit_identical = bool(torch.equal(y, y_ref))
    fwd_ws = dp.workspace(eg.ENGRAM_OP_FORWARD)
    steps = args.steps
    timings = {}

    def run(label, fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        eg.engram_profile_reset()
        eg.engram_profile_enable(True)
        a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a0.record()
        for _ in range(steps):
            fn()
        a1.record()
        torch.cuda.synchronize()
        eg.engram_profile_enable(False)
        prof = {k: round(tot / max(n, 1), 5) for k, (n, tot) in eg.engram_profile_read().items()}
        timings[label] = {"ms": round(a0.elapsed_time(a1) / steps, 4), "kernels_avg_ms": prof}

    run("sender_requests", lambda: eg.engram_shard_requests(dp.cfg, G, r0["saved"]["idx"], N, r0["send_ids"],
                                                            torch.empty(G, dtype=torch.int64, device="cuda"),
                                                            torch.empty(N, J, dtype=torch.int32, device="cuda"),
                                                            workspace=ws))
    run("owner_serve", lambda: eg.engram_shard_serve(dp.cfg, G, shards0, recv, recv.numel(), served))
    y_out = torch.empty_like(y)
    run("forward_served_rows", lambda: dp.forward(compact=plan, ws=fwd_ws, y=y_out))
    run("forward_whole_tables", lambda: dp.forward(ws=fwd_ws, y=y_out))
    run("sender_grad_rows", lambda: eg.engram_shard_grads(dp.cfg, G, r0["sp"]["keys"], r0["sp"]["rows"],
                                                          r0["sp"]["count"], cap, r0["gids"], r0["grows"],
                                                          r0["gcounts_dev"], workspace=ws))
    run("owner_grad_reduce", lambda: eg.engram_shard_reduce(dp.cfg, G, shard_grads, gids0, grows0, gblocks))
    # bytes GPU 0 moves over the fabric per step (to or from the other G-1 GPUs)
    c0 = r0["c"]
    recv_from = [int(rk["c"][0]) for rk in ranks]
    g_out = r0["gc"]
    send, recv_b = [], []
    for o in range(1, G):
        # to peer o: requests, replies to its requests, gradient rows of its rows
        send.append(int(c0[o]) * 4 + recv_from[o] * rb + int(g_out[o]) * (4 + 4 * D))
        # from peer o: replies, its requests, its gradient rows of GPU 0's rows
        recv_b.append(int(c0[o]) * rb + recv_from[o] * 4 + int(ranks[o]["gc"][0]) * (4 + 4 * D))
    per_peer = [max(a, b) for a, b in zip(send, recv_b)]
    link = 153e9
    out = {
        "metric": "table-sharded Engram step, device side of one of G GPUs",
        "workload": wl.name, "gpus_emulated": G, "tokens_per_gpu": N, "tables": J,
        "shard_rows_per_table": S[0], "distinct_rows_requested": int(c0.sum()),
        "rows_served_by_owner": int(recv.numel()), "grad_rows_received_by_owner": int(gids0.numel()),
        "forward_bit_identical": bit_identical, "timings": timings,
        "fabric_bytes_sent": int(sum(send)), "fabric_bytes_received": int(sum(recv_b)),
        "fabric_ms_at_153GBps_per_link": round(max(per_peer) / link * 1e3, 3),
        "note": "one GPU; the All-to-All transfers are device copies here, their time modelled "
                "as the largest per-peer volume over one xGMI link (pairwise exchange, 7 links)",
    }
    print(json.dumps(out), flush=True)


def device_copy_rate(nbytes: int, reps: int = 10) -> dict:
    """The library's plain device copy (engram_device_copy) of nbytes: read +
    write bytes over its median time, the achievable-bandwidth reference."""
    import torch

    import hashed_gram_embedding_canon_amd as eg
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(2):
        eg.engram_device_copy(dst, src, nbytes)
    torch.cuda.synchronize()
    ms = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        eg.engram_device_copy(dst, src, nbytes)
        b.record()
        torch.cuda.synchronize()
        ms.append(a.elapsed_time(b))
    med = statistics.median(ms)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_copied": nbytes, "median_ms": round(med, 4),
            "GBps": round(2 * nbytes / (med * 1e-3) / 1e9, 1),
            "frac_of_peak": round(2 * nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}


def copy_calibration(nbytes: int):
    """Five copies of nbytes by the library's copy kernel: the reference
    dispatches that scale the FETCH_SIZE / WRITE_SIZE counters."""
    r = device_copy_rate(nbytes, reps=5)
    print(json.dumps({"copy_bytes": nbytes, "median_ms": r["median_ms"],
                      "GBps_read_plus_write": r["GBps"]}), flush=True)


def bench_library_gemm(args):
    """The three contractions of the 27B shape as plain library products
    (torch.matmul on hipBLASLt, no epilogue work) beside this library's
    kernels, in one process, passes alternated: the projection e W_KV
    (bf16 out; ours adds the gate sums and reads h), de = [dk|dv] W_KV^T
    (fp16 operands, fp16 out; ours writes fp32) and dW = [dk|dv]^T e over the
    tokens (bf16; ours sums token chunks in fp32)."""
    import statistics

    import torch

    import hashed_gram_embedding_canon_amd as eg
    import synth
    from tests import harness as H
    wl = synth.get_workload("engram27b")
    N, dm, d = wl.n_tokens, wl.d_mem, wl.hidden
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    dp.forward(bufs)
    dy = H.to_dev(inp.dy)
    g = torch.Generator(device="cuda").manual_seed(5)
    e = torch.randn(N, dm, device="cuda", dtype=torch.bfloat16, generator=g)
    w = torch.randn(dm, 2 * d, device="cuda", dtype=torch.bfloat16, generator=g)
    x16 = torch.randn(N, 2 * d, device="cuda", dtype=torch.float16, generator=g)
    wt16 = torch.randn(2 * d, dm, device="cuda", dtype=torch.float16, generator=g)
    xt = torch.randn(2 * d, N, device="cuda", dtype=torch.bfloat16, generator=g)  # contiguous
    lib = {"projection": lambda: torch.matmul(e, w), "de": lambda: torch.matmul(x16, wt16),
           "dW": lambda: torch.matmul(xt, e)}
    y = torch.empty(wl.B, wl.T, d, dtype=dp.tdtype, device="cuda")
    ws_f = dp.workspace(eg.ENGRAM_OP_FORWARD)
    ws_b = dp.workspace(eg.ENGRAM_OP_BACKWARD_PARAMS)
    res = {f"hipblaslt_{k}": [] for k in lib}
    res.update({"ours_proj_gemm": [], "ours_de_gemm": [], "ours_dw_gemm": []})
    tg = eg.engram_table_grad()
    tg.mode = eg.ENGRAM_GRAD_SORTED_SPARSE
    cap = N * wl.J
    kb = torch.empty(cap, dtype=torch.int64, device="cuda")
    rb = torch.empty(cap, wl.dim, dtype=torch.float32, device="cuda")
    cb = torch.empty(1, dtype=torch.int64, device="cuda")
    tg.keys, tg.rows, tg.count = kb.data_ptr(), rb.data_ptr(), cb.data_ptr()
    pres = {"w_kv": torch.empty(2 * d, dm, device="cuda")}
    pg = eg.make_param_grad(**pres)
    sv = eg.make_saved(**bufs)
    for r in range(args.steps if args.steps < 20 else 5):
        for k, fn in lib.items():
            for _ in range(2):
                fn()
            a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a0.record()
            for _ in range(5):
                fn()
            a1.record()
            torch.cuda.synchronize()
            res[f"hipblaslt_{k}"].append(a0.elapsed_time(a1) / 5)
        eg.engram_profile_reset()
        eg.engram_profile_enable(True)
        for _ in range(5):
            dp.forward(ws=ws_f, y=y)
            eg.engram_backward(dp.cfg, dp.params, dp.hidden, dy, B=dp.B, T=dp.T, saved=sv, table_out=tg,
                               param_out=pg, workspace=ws_b)
        torch.cuda.synchronize()
        eg.engram_profile_enable(False)
        prof = eg.engram_profile_read()
        for k in ("proj_gemm", "de_gemm", "dw_gemm"):
            n, tot = prof[k]
            res[f"ours_{k}"].append(tot / n)
        log(f"[bench-lib] pass {r}: " + ", ".join(f"{k} {v[-1]:.3f}" for k, v in res.items()))
    med = {k: round(statistics.median(v), 4) for k, v in res.items()}
    print(json.dumps({"metric": "27B-shape contractions: hipBLASLt plain products beside this library's kernels",
                      "shapes": {"projection": [N, dm, 2 * d], "de": [N, 2 * d, dm], "dW": [2 * d, N, dm]},
                      "median_ms": med, "passes": len(res["ours_proj_gemm"])}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--settle-ms", type=float, default=150.0,
                    help="untimed forward steps for this long before the warmup steps, so that "
                         "the GPU clock is past its power-management transient (0: none)")
    ap.add_argument("--workload", default="engram27b")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the table-gradient backward block")
    ap.add_argument("--backward-steps", type=int, default=5)
    ap.add_argument("--fused-gather", action="store_true",
                    help="let the projection read the table rows itself (ENGRAM_FLAG_FUSED_GATHER) "
                         "instead of gathering e into the workspace first")
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the three 27B-shape contractions as hipBLASLt products beside ours")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run a plain device-to-device copy of BYTES, 5 times (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--summarize-trace", metavar="DIR",
                    help="print the kernel table of a rocprofv3 --kernel-trace --stats csv run")
    ap.add_argument("--summarize-pmc", metavar="DIR",
                    help="print per-dispatch counter means of the MFMA kernels of a rocprofv3 --pmc csv run")
    ap.add_argument("--summarize-traffic", nargs=4,
                    metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"),
                    help="print HBM bytes per dispatch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE "
                         "csv runs of the bench and of --copy-calibration")
    ap.add_argument("--calibration-bytes", type=int, default=1 << 30)
    ap.add_argument("--branches", type=int, default=1,
                    help="M branches sharing the tables and W_V (own W_K, hidden state, gate, Y)")
    ap.add_argument("--dedup", action="store_true",
                    help="read rows repeated inside a 16-token gather tile once (ENGRAM_FLAG_GATHER_DEDUP)")
    ap.add_argument("--token-stream", choices=("zipf", "repeat"), default="zipf",
                    help="i.i.d. Zipf tokens, or the Zipf stream with local repetition of short segments")
    ap.add_argument("--fp8", action="store_true",
                    help="the projection as one E4M3 matmul (ENGRAM_FLAG_FP8_PROJ); not the headline")
    ap.add_argument("--shard-gpus", type=int, default=8,
                    help="GPUs the tables are sharded over for --workload shard27b")
    ap.add_argument("--ring-batches", type=int, default=8,
                    help="successive batches for the row-ring measurement of --workload host100b")
    ap.add_argument("--ring-factor", type=int, default=16,
                    help="HBM row ring size in units of one batch's capacity (N*J rows)")
    ap.add_argument("--host-rows", type=int, default=4_880_000,
                    help="rows per host table for --workload host100b")
    args = ap.parse_args()
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace))
        return
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc))
        return
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, args.calibration_bytes))
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(f"bench.py: the Engram path runs on one GPU only (asked for --gpus {args.gpus}); "
              "table sharding over several GPUs has its per-GPU steps here (--workload shard27b) "
              "but no multi-GPU run", file=sys.stderr)
        sys.exit(2)

    if args.workload == "shard27b":
        bench_shard(args)
        return
    if args.workload == "host100b":
        bench_host(args)
        return
    if args.library_gemm:
        bench_library_gemm(args)
        return

    import torch

    import hashed_gram_embedding_canon_amd as eg
    import synth
    from tests import harness as H

    wl = synth.get_workload(args.workload)
    if args.branches != 1:
        import dataclasses
        wl = dataclasses.replace(wl, branches=args.branches)
        args.no_cpu_baseline = True  # the oracle baseline is timed on one branch
    N = wl.n_tokens
    log(f"[bench] {wl.name}: B={wl.B} T={wl.T} J={wl.J} D={wl.dim} d={wl.hidden} "
        f"table params={wl.table_params / 1e9:.2f}B; generating inputs")
    t = time.perf_counter()
    inp = synth.Inputs(wl)
    flags = ((eg.ENGRAM_FLAG_FUSED_GATHER if args.fused_gather else 0) |
             (eg.ENGRAM_FLAG_FP8_PROJ if args.fp8 else 0) |
             (eg.ENGRAM_FLAG_GATHER_DEDUP if args.dedup else 0))
    dp = H.DeviceProblem(inp, flags=flags)
    torch.cuda.synchronize()
    log(f"[bench] inputs resident in HBM after {time.perf_counter() - t:.1f} s")
    lead = (wl.B, wl.T) if wl.branches == 1 else (wl.branches, wl.B, wl.T)
    y = torch.empty(*lead, wl.hidden, dtype=dp.tdtype, device="cuda")
    ws = dp.workspace(eg.ENGRAM_OP_FORWARD)
    saved = None
    # one distinct token batch per timed step (consecutive stretches of the
    # seeded Zipf stream), all resident in HBM before timing: a step never
    # finds the previous step's rows in the caches
    draw = synth.repeat_tokens if args.token_stream == "repeat" else synth.zipf_tokens
    batches = [H.to_dev(draw(synth.seed_of(wl.cfg, synth.S_TOKENS), N, wl.vocab, wl.zipf_s,
                             offset=k * N).reshape(wl.B, wl.T)) for k in range(args.steps)]

    def step(i):
        dp.tokens = batches[i % len(batches)]
        dp.forward(saved, ws=ws, y=y)

    # After any idle period of 0.1 s or more the GPU's power management first
    # boosts, then throttles below its steady clock and settles within ~15
    # steps (~30 ms): the first steps after idle run up to 25 % slower.  Forward
    # steps over the same batches run untimed for --settle-ms first, so the
    # timed steps measure the steady state of a running job.
    settle_steps = 0
    t = time.perf_counter()
    while (time.perf_counter() - t) * 1e3 < args.settle_ms:
        for _ in range(5):
            step(settle_steps)
            settle_steps += 1
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] settle ({settle_steps} steps) and warmup ({args.warmup} steps) done; "
        f"{len(batches)} distinct token batches resident")

    # headline: no library timing events inside; one event between steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    evs[0].record()
    for i in range(args.steps):
        step(i)
        evs[i + 1].record()
    torch.cuda.synchronize()
    step_ms = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    log(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step (median {statistics.median(step_ms):.3f}, "
        f"min {min(step_ms):.3f})")
    # per-kernel durations: a second pass over the same batches with the
    # library's event pairs around every launch (on the launch stream)
    eg.engram_profile_reset()
    eg.engram_profile_enable(True)
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    k0.record()
    for i in range(args.steps):
        step(i)
    k1.record()
    torch.cuda.synchronize()
    eg.engram_profile_enable(False)
    prof = eg.engram_profile_read()
    prof_pass_ms = k0.elapsed_time(k1) / args.steps
    dp.tokens = batches[0]
    copy_ref = device_copy_rate(256 << 20)

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
    # the counters were taken on the default configuration (one branch, bf16
    # projection, rows gathered first): other configurations report none
    traffic = (traffic_from_profile(wl.name)
               if wl.branches == 1 and flags == 0 and args.token_stream == "zipf" else {})
    for name, ent in kernels.items():
        if name in traffic:
            ent["counter_bytes"] = int(traffic[name])
            ent["counter_GBps"] = round(traffic[name] / (ent["avg_ms"] * 1e-3) / 1e9, 1)
    dom = max(prof.items(), key=lambda kv: kv[1][1])[0] if prof else None
    roof = None
    if dom is not None:
        u = units[dom]
        avg_s = prof[dom][1] / prof[dom][0] * 1e-3
        if u["bound"] in ("mfma", "mfma_fp8"):
            peak = (MFMA_FP8_PEAK_TFLOPS if u["bound"] == "mfma_fp8" else
                    MFMA_BF16_PEAK_TFLOPS if wl.dtype == "bf16" else MFMA_F32_PEAK_TFLOPS)
            ach = u["flops"] / avg_s / 1e12
            roof = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1), "peak": peak,
                    "unit": "TFLOP/s", "frac": round(ach / peak, 4),
                    "traffic": int(traffic[dom]) if dom in traffic else None}
        else:
            ach = u["bytes"] / avg_s / 1e9
            roof = {"kernel": dom, "bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                    "traffic": int(traffic[dom]) if dom in traffic else None}
    mem_names = [k for k in ("hash_gather", "dedup_gather", "gather", "gather_quant", "gate_conv")
                 if k in prof]
    mem_ms = sum(prof[k][1] / prof[k][0] for k in mem_names)
    mem_bytes = sum(units[k]["bytes"] for k in mem_names)
    es = 2 if wl.dtype == "bf16" else 4
    alg_per_token = wl.J * wl.dim * es + 2 * wl.hidden * es + 4  # rows + h + Y + token id
    hbm_block = {"kernels": mem_names, "ms": round(mem_ms, 4), "target_frac": 0.6}
    if mem_ms:
        hbm_block["alg_GBps"] = round(mem_bytes / (mem_ms * 1e-3) / 1e9, 1)
        hbm_block["frac"] = round(hbm_block["alg_GBps"] / HBM_PEAK_GBS, 4)
        hbm_block["meets_target"] = hbm_block["frac"] >= 0.6
        hbm_block["frac_of_device_copy"] = round(hbm_block["alg_GBps"] / copy_ref["GBps"], 4)
        if all(k in traffic for k in mem_names):
            cb = sum(traffic[k] for k in mem_names)
            hbm_block["counter_GBps"] = round(cb / (mem_ms * 1e-3) / 1e9, 1)
            hbm_block["counter_frac"] = round(hbm_block["counter_GBps"] / HBM_PEAK_GBS, 4)

    out = {
        "metric": "Engram fwd tokens/s + achieved HBM GB/s (gather+gate+conv), 27B-scale table",
        "value": round(N / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_steps": settle_steps,
        "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(statistics.median(step_ms), 4),
        "ms_per_step_min": round(min(step_ms), 4),
        "token_batches": len(batches),
        "kernel_pass_ms_per_step": round(prof_pass_ms, 4),
        "hbm_peak_GBps": HBM_PEAK_GBS,
        "device_copy": copy_ref,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("fp8 e4m3 projection, bf16 elsewhere" if args.fp8 else
                  "bf16" if wl.dtype == "bf16" else "f32"),
        "data": "synthetic",
        "config": {"workload": wl.name, "token_stream": args.token_stream,
                   "gather": "lds dedup" if args.dedup else "plain", "branches": wl.branches, "row_gather": "fused into projection" if args.fused_gather else "gathered into workspace", "batch": wl.B, "seq_len": wl.T, "tables": wl.J,
                   "rows_per_table": list(wl.rows[:1]) + ["..."], "dim": wl.dim,
                   "d_mem": wl.d_mem, "hidden": wl.hidden, "table_params": wl.table_params,
                   "zipf_s": wl.zipf_s, "vocab": wl.vocab, "canon_vocab": wl.canon_vocab},
        "roofline": roof,
        "hbm_gather_gate_conv": hbm_block,
        "end_to_end_alg_GBps": round(alg_per_token * N / (ms * 1e-3) / 1e9, 1),
        "kernels": kernels,
    }
    if not args.no_backward:
        log(f"[bench] backward (table gradients; training), {args.backward_steps} steps per mode")
        out["backward"] = bench_backward(dp, inp, args.backward_steps)
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on host cores for ~{args.cpu_seconds:.0f} s")
        out["cpu_baseline"] = cpu_baseline(inp, args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
