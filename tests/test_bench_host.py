"""Host logic of bench.py (no GPU): kernel-name mapping, grouping of
multi-dispatch calls in a kernel trace, counter summaries, the source digest
that ties counter bytes to the sources, the algorithmic units, and the
refusal of more than one GPU."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
import synth  # noqa: E402


@pytest.mark.parametrize("name,key", [
    ("void engram::gemm_kernel<0, 0, false, 128>(engram::GemmArgs)", "proj_gemm"),
    ("void engram::gemm_kernel<0, 0, true, 128>(engram::GemmArgs)", "gather_proj_gemm"),
    ("void engram::gemm_kernel<3, 0, false, 128>(engram::GemmArgs)", "proj_gemm_fp8"),
    ("void engram::gemm_kernel<1, 1, false, 128>(engram::GemmArgs)", "de_gemm"),
    ("void engram::gemm_tn_kernel<1>(engram::GemmTnArgs)", "dw_gemm"),
    ("engram::tn_reduce_kernel(float const*, float*, long, int)", "dw_gemm"),
    ("void engram::bwd_gate_conv_kernel<true, 4, false, 1024, false>(engram::BwdArgs)", "bwd_gate_conv"),
    ("void engram::bwd_gate_conv_kernel<true, 4, true, 768, false>(engram::BwdArgs)", "bwd_gate_conv_params"),
    ("void engram::gate_conv_kernel<8, true, 4>(engram::GateConvArgs)", "gate_conv"),
    ("engram::gather_kernel(int const*, unsigned char*, unsigned int, engram::GatherArgs)", "gather"),
    ("engram::hash_gather_kernel(int const*, int const*, int, unsigned int, engram::GatherArgs)",
     "hash_gather"),
    ("engram::hash_kernel(int const*, int const*, long, int, int*, engram::HashArgs)", "hash"),
    ("engram::gather_quant_kernel(int const*, long, engram::GatherArgs, int, unsigned char*, float*)",
     "gather_quant"),
    ("void engram::quant_rows_kernel<true>(unsigned char const*, long, int, unsigned char*, float*)", "quant_w"),
    ("void engram::sort_hist_kernel<true>(int const*, unsigned int const*, unsigned int*, long, int, int, int)",
     "sorted_scatter"),
    ("void engram::seg_reduce_kernel<0>(engram::ScatterArgs)", "sorted_scatter"),
    ("engram::owner_bounds_kernel(x)", "shard_pack"),
    ("engram::serve_kernel(x)", "shard_serve"),
    ("engram::grad_add_kernel(x)", "shard_reduce"),
    ("__amd_rocclr_copyBuffer", "copy"),
    ("void at::native::vectorized_elementwise_kernel<4>(x)", ""),
])
def test_kernel_key(name, key):
    assert bench.kernel_key(name) == key


def _trace(tmp_path, rows):
    path = tmp_path / "run_kernel_trace.csv"
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        t = 0
        for name, ns in rows:
            w.writerow({"Kernel_Name": name, "Start_Timestamp": t, "End_Timestamp": t + ns})
            t += ns + 100
    return str(tmp_path)


def _calls(summary, key):
    for ln in summary.splitlines():
        parts = ln.split()
        if parts and parts[0] == key:
            return int(parts[1]), float(parts[2])
    raise KeyError(key)


def test_trace_groups_calls_at_their_leader(tmp_path):
    """Back-to-back calls of a multi-dispatch name stay separate calls: a new
    call starts at the leader dispatch (or after it, for a leader that comes
    last)."""
    pack = ["engram::owner_bounds_kernel(x)", "engram::shard_pack_kernel(x)"]
    sums = ["engram::colsum64_kernel(x)", "engram::colsum64_kernel(x)", "engram::param_finish_kernel(x)"]
    rows = [(n, 1000) for n in pack * 3] + [(n, 2000) for n in sums * 2]
    rows += [("void engram::gemm_tn_kernel<1>(x)", 5000), ("engram::tn_reduce_kernel(x)", 1000)]
    s = bench.summarize_trace(_trace(tmp_path, rows))
    assert _calls(s, "shard_pack") == (3, 2.0)       # 3 calls of 2 dispatches x 1 us
    assert _calls(s, "bwd_param_sums") == (2, 6.0)   # 2 calls of 3 dispatches x 2 us
    assert _calls(s, "dw_gemm") == (1, 6.0)


def test_pmc_summary_means_per_dispatch(tmp_path):
    path = tmp_path / "run_counter_collection.csv"
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for v in (40.0, 60.0):
            w.writerow({"Kernel_Name": "void engram::gemm_kernel<0, 0, false, 128>(x)",
                        "Counter_Name": "MfmaUtil", "Counter_Value": v})
        w.writerow({"Kernel_Name": "engram::tn_reduce_kernel(x)", "Counter_Name": "MfmaUtil",
                    "Counter_Value": 1.0})  # the chunk sum is not the dW GEMM
        w.writerow({"Kernel_Name": "void engram::gemm_tn_kernel<1>(x)", "Counter_Name": "MfmaUtil",
                    "Counter_Value": 44.0})
    s = bench.summarize_pmc(str(tmp_path)).splitlines()
    rows = {ln.split()[0]: ln.split() for ln in s[1:]}
    assert rows["proj_gemm"][1] == "2" and float(rows["proj_gemm"][2]) == 50.0
    assert rows["dw_gemm"][1] == "1" and float(rows["dw_gemm"][2]) == 44.0


def test_traffic_follows_the_source_digest(tmp_path, monkeypatch):
    """Counter bytes are used only while the profile's source digest is the
    digest of the current sources."""
    prof = tmp_path / "profiles"
    prof.mkdir()
    body = "kernel fetch_kib write_kib traffic_bytes\nproj_gemm 1.0 2.0 4096\n"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "csrc_digest", lambda: "abc")
    (prof / "traffic_w.txt").write_text("# header\nsource abc\n" + body)
    assert bench.traffic_from_profile("w") == {"proj_gemm": 4096.0}
    (prof / "traffic_w.txt").write_text("# header\nsource old\n" + body)
    assert bench.traffic_from_profile("w") == {}
    assert bench.traffic_from_profile("missing") == {}


def test_digest_covers_the_sources():
    d = bench.csrc_digest()
    assert len(d) == 16 and d == bench.csrc_digest()


def test_projection_units_at_the_27b_scale():
    """2 N d_mem 2d FLOP and the bytes the forward kernels must move."""
    wl = synth.get_workload("engram27b")
    u = bench.kernel_units(wl, wl.n_tokens)
    assert u["proj_gemm"]["flops"] == 2 * 131072 * 1280 * 5120
    # gather: indices, rows read, e written (64 + 2560 + 2560 bytes per token)
    assert u["gather"]["bytes"] == 131072 * (64 + 2560 + 2560)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_digest_ignores_comments_only():
    a = "int f(int x) { // the input\n  return x + 1; /* one more */ }\n"
    b = "int f(int x) {\n  /* changed words */ return x + 1;   }  // other\n"
    c = "int f(int x) { return x + 2; }"
    assert bench.code_tokens(a) == bench.code_tokens(b) != bench.code_tokens(c)
