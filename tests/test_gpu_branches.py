"""GPU parity of the multi-branch forward ("DeepSeek AI II", section
"DeepSeek Engram", multi-branch integration): one projection GEMM over
[W_K^(0); ...; W_K^(M-1); W_V], a gate and an output per branch, v shared.
Each branch is checked against the single-branch oracle on its own W_K and
hidden state."""
import dataclasses

import numpy as np
import pytest

import synth
from tests import harness as H

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


@pytest.mark.parametrize("dtype,M,B,T", [("f32", 3, 2, 300), ("bf16", 2, 3, 77), ("f32", 1, 1, 64),
                                         ("bf16", 4, 1, 513), ("bf16", 8, 1, 130)])  # 8: the most
def test_tiny_branches_full(torch, oracle_lib, dtype, M, B, T):
    wl = dataclasses.replace(synth.get_workload("tiny"), dtype=dtype, branches=M).with_shape(B, T)
    print(f"[branches tiny {dtype}] M={M} B={B} T={T}", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    y = dp.forward(bufs)
    torch.cuda.synchronize()
    ys = y.reshape(M, -1, wl.hidden) if M > 1 else y.reshape(1, -1, wl.hidden)
    stats = bufs["stats"].reshape(M, -1, 4)
    for m in range(M):
        p = H.oracle_problem(inp, branch=m)
        if m == 0:
            assert np.array_equal(bufs["idx"].cpu().numpy(), p.hash())
        ref = p.forward(want=("y", "alpha"))
        err = H.rel_max_err(H.to_host_f64(ys[m]), ref["y"])
        a_err = float(np.abs(stats[m, :, 0].cpu().numpy() - ref["alpha"]).max())
        print(f"  branch {m}: max-abs-err/max|ref| = {err:.3e}, alpha err {a_err:.2e}", flush=True)
        assert err <= TOL[dtype], (m, err)
        assert a_err <= (1e-5 if dtype == "f32" else 1e-2), (m, a_err)


def test_one_branch_matches_default_config(torch):
    """branches = 1 and the default (0) run the same kernels: identical Y."""
    wl = synth.get_workload("tiny").with_shape(2, 300)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    y1 = dp.forward()
    dp.cfg.c.branches = 0
    y0 = dp.forward()
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_small_bf16_branches_sampled(torch, oracle_lib):
    wl = dataclasses.replace(synth.get_workload("small"), branches=3).with_shape(2, 2048)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("stats",))
    y = dp.forward(bufs).reshape(3, -1, wl.hidden)
    torch.cuda.synchronize()
    pos = H.sample_positions(dp.B, dp.T, 128, seed=21)
    for m in range(3):
        p = H.oracle_problem(inp, branch=m)
        ref = p.forward(pos, want=("y", "alpha"))
        got = H.to_host_f64(y[m][torch.as_tensor(pos, device=y.device)])
        err = H.rel_max_err(got, ref["y"])
        print(f"  small branch {m}: max-abs-err/max|ref| = {err:.3e}", flush=True)
        assert err <= TOL["bf16"], (m, err)


@pytest.mark.parametrize("dtype,M,B,T", [("f32", 2, 1, 300), ("bf16", 3, 2, 150), ("f32", 8, 1, 70)])
def test_branch_backward(torch, oracle_lib, dtype, M, B, T):
    """Training backward with M branches: the loss is the sum of the branches'
    <G^(m), Y^(m)>, so the table, W_V and conv gradients are the sums of the
    single-branch oracle's over the branches, and dW_K^(m), the RMSNorm
    scales and dh are branch m's own."""
    import hashed_gram_embedding_canon_amd as eg
    wl = dataclasses.replace(synth.get_workload("tiny"), dtype=dtype, branches=M).with_shape(B, T)
    print(f"[branch bwd {dtype}] M={M} B={B} T={T}", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    dp.forward(bufs)
    dy = H.to_dev(np.ascontiguousarray(np.stack([inp.dy_branch(m) for m in range(M)])))
    table = dp.backward(bufs, dy, eg.ENGRAM_GRAD_SORTED_DENSE)["dense"]
    pg = dp.backward_params(bufs, dy)
    torch.cuda.synchronize()
    d = wl.hidden
    ref_tab = None
    ref = {"w_kv": np.zeros(((M + 1) * d, wl.d_mem)), "conv_w": 0.0, "gamma_q": [], "gamma_k": [],
           "hidden": []}
    for m in range(M):
        p = H.oracle_problem(inp, branch=m)
        dym = inp.dy_branch(m)
        tg = p.table_grad_dense(dym)
        ref_tab = tg if ref_tab is None else [a + b for a, b in zip(ref_tab, tg)]
        g = p.backward_params(dym)
        ref["w_kv"][m * d:(m + 1) * d] = g["w_k"]
        ref["w_kv"][M * d:] += g["w_v"]
        ref["conv_w"] = ref["conv_w"] + g["conv_w"]
        for k in ("gamma_q", "gamma_k"):
            ref[k].append(g[k])
        ref["hidden"].append(g["h"])
    got_tab = np.concatenate([t.cpu().numpy().astype(np.float64).ravel() for t in table])
    err = H.rel_l2(got_tab, np.concatenate([r.ravel() for r in ref_tab]))
    print(f"  table grads rel L2 {err:.2e}", flush=True)
    assert err <= 1e-3, err
    bf = dtype == "bf16"
    for k in ("w_kv", "conv_w", "gamma_q", "gamma_k", "hidden"):
        r = np.asarray(ref[k], np.float64)
        got = H.to_host_f64(pg[k]).reshape(r.shape)
        if k == "hidden" and bf:
            e = H.rel_max_err(got, r)
            bar = 1e-2
        else:
            e = H.rel_l2(got, r)
            bar = 5e-3 if bf else 1e-5
        print(f"  {k}: {e:.2e}", flush=True)
        assert e <= bar, (k, e)


def test_engram27b_four_branches_sampled(torch, oracle_lib):
    """The 27B-scale forward with M = 4 branches, as the bench runs it: every
    branch's Y and gate against the oracle at sampled positions."""
    wl = dataclasses.replace(synth.get_workload("engram27b"), branches=4)
    print("[engram27b, 4 branches] generating and uploading 5.7B table parameters", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("stats",))
    y = dp.forward(bufs).reshape(4, -1, wl.hidden)
    torch.cuda.synchronize()
    pos = H.sample_positions(dp.B, dp.T, 64, seed=23)
    ipos = torch.as_tensor(pos, device=y.device)
    for m in range(4):
        p = H.oracle_problem(inp, branch=m)
        ref = p.forward(pos, want=("y", "alpha"))
        err = H.rel_max_err(H.to_host_f64(y[m][ipos]), ref["y"])
        a_err = float(np.abs(bufs["stats"][m][ipos, 0].cpu().numpy() - ref["alpha"]).max())
        print(f"  branch {m}: max-abs-err/max|ref| = {err:.3e}, alpha err {a_err:.2e}", flush=True)
        assert err <= TOL["bf16"] and a_err <= 1e-2, (m, err, a_err)
    del dp, bufs, y
    torch.cuda.empty_cache()
