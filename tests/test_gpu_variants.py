"""Configurations beyond the workloads' own: other conv widths, three N-gram
orders with two heads, 16-byte table rows.  Forward against the oracle at
every position (max |err| / max |ref| <= 1e-5 fp32, <= 1e-2 bf16), table
gradients (relative L2 <= 1e-3) and the parameter gradients (the bars of the
parameter-gradient tests).  d_mem = J*D is a multiple of 256 in every case,
as the library requires."""
import dataclasses

import numpy as np
import pytest

import synth
from synth.workloads import primes_from
from tests import harness as H

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 1e-2}


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


CASES = [
    # dtype, taps, orders, heads, dim, B, T
    ("f32", 1, (2, 3), 4, 32, 2, 130),
    ("bf16", 2, (2, 3), 4, 32, 2, 200),
    ("bf16", 7, (2, 3, 4), 2, 128, 1, 333),
    ("bf16", 4, (2, 3), 16, 8, 2, 150),   # 16-byte rows, 32 tables (the most), d_mem 256
    ("f32", 8, (2, 3), 4, 32, 1, 70),
]


def test_d_mem_must_tile_by_256(torch):
    """d_mem = J * D must be a multiple of 256 (the feature tiles of the de
    contraction): 6 tables of 64 are refused before any launch."""
    import hashed_gram_embedding_canon_amd as eg
    wl = dataclasses.replace(synth.get_workload("tiny"), dtype="bf16", orders=(2, 3, 4), heads=2, dim=64,
                             rows=tuple(primes_from(10007, 6))).with_shape(1, 64)
    dp = H.DeviceProblem(synth.Inputs(wl))
    with pytest.raises(eg.EngramError, match="status 2"):
        dp.forward()


@pytest.mark.parametrize("dtype,taps,orders,heads,dim,B,T", CASES)
def test_config_variants(torch, oracle_lib, dtype, taps, orders, heads, dim, B, T):
    import hashed_gram_embedding_canon_amd as eg
    J = len(orders) * heads
    base = synth.get_workload("tiny")
    wl = dataclasses.replace(base, dtype=dtype, taps=taps, orders=orders, heads=heads, dim=dim,
                             rows=tuple(primes_from(10007, J)), w_std=(J * dim) ** -0.5).with_shape(B, T)
    print(f"[variant {dtype}] taps={taps} orders={orders} heads={heads} D={dim} d_mem={wl.d_mem} "
          f"B={B} T={T}", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    bufs = dp.alloc_saved(("idx", "stats", "k", "v"))
    y = dp.forward(bufs)
    torch.cuda.synchronize()
    p = H.oracle_problem(inp)
    ref = p.forward(want=("y",))["y"]
    assert np.array_equal(bufs["idx"].cpu().numpy(), p.hash())
    err = H.rel_max_err(H.to_host_f64(y).reshape(ref.shape), ref)
    print(f"  forward {err:.2e}", flush=True)
    assert err <= TOL[dtype], err
    dy = H.to_dev(inp.dy)
    dense = dp.backward(bufs, dy, eg.ENGRAM_GRAD_SORTED_DENSE)["dense"]
    torch.cuda.synchronize()
    ref_t = p.table_grad_dense(inp.dy)
    got = np.concatenate([t.cpu().numpy().astype(np.float64).ravel() for t in dense])
    err = H.rel_l2(got, np.concatenate([r.ravel() for r in ref_t]))
    print(f"  table grads {err:.2e}", flush=True)
    assert err <= 1e-3, err
    g = dp.backward_params(bufs, dy)
    torch.cuda.synchronize()
    r = p.backward_params(inp.dy)
    refs = {"w_kv": np.concatenate([r["w_k"], r["w_v"]]), "conv_w": r["conv_w"],
            "gamma_q": r["gamma_q"], "gamma_k": r["gamma_k"], "hidden": r["h"]}
    bf = dtype == "bf16"
    for k, rv in refs.items():
        gv = H.to_host_f64(g[k]).reshape(rv.shape)
        e = H.rel_max_err(gv, rv) if (k == "hidden" and bf) else H.rel_l2(gv, rv)
        bar = (1e-2 if k == "hidden" else 5e-3) if bf else 1e-5
        print(f"  {k} {e:.2e}", flush=True)
        assert e <= bar, (k, e)
