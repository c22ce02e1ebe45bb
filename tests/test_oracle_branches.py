"""Multi-branch gating ("DeepSeek AI II", section "DeepSeek Engram",
multi-branch integration): the branches share the tables and W_V, each has its
own W_K and hidden state.  The oracle of branch m is the single-branch oracle
on (W_K^(m), h^(m)); these tests pin what ties the branches together."""
import dataclasses

import numpy as np

import synth
from tests import harness as H


def _inp(M, B=1, T=64):
    wl = dataclasses.replace(synth.get_workload("tiny"), branches=M).with_shape(B, T)
    return synth.Inputs(wl)


def test_branch_arrays_extend_the_single_branch_streams():
    inp = _inp(3)
    one = synth.Inputs(synth.get_workload("tiny").with_shape(1, 64))
    assert np.array_equal(inp.w_k_branch(0), one.w_k)
    assert np.array_equal(inp.hidden_branch(0), one.hidden)
    # distinct branches draw distinct values from the same streams
    assert not np.array_equal(inp.w_k_branch(1), inp.w_k_branch(0))
    assert not np.array_equal(inp.hidden_branch(2), inp.hidden_branch(1))


def test_value_is_shared_gates_differ(oracle_lib):
    """With the conv taps at zero, Y^(m) = alpha^(m) v with one shared v, so
    Y^(1) / Y^(0) equals alpha^(1) / alpha^(0) in every feature."""
    import oracle
    inp = _inp(2)
    zero = np.zeros_like(inp.conv_w)
    outs = []
    for m in range(2):
        p = oracle.Problem.from_inputs(inp, conv_w=zero, h=inp.hidden_branch(m),
                                       w_k=oracle.widen(inp.w_k_branch(m)))
        outs.append(p.forward(want=("y", "alpha")))
    y0, y1 = outs[0]["y"], outs[1]["y"]
    a0, a1 = outs[0]["alpha"], outs[1]["alpha"]
    assert not np.allclose(a0, a1)
    ratio = a1 / a0
    mask = np.abs(y0) > 1e-12
    got = (y1[mask] / y0[mask])
    want = np.broadcast_to(ratio[:, None], y0.shape)[mask]
    assert np.allclose(got, want, rtol=1e-10, atol=0)


def test_identical_branches_give_identical_outputs(oracle_lib):
    inp = _inp(2)
    import oracle
    p0 = H.oracle_problem(inp, branch=0)
    same = oracle.Problem.from_inputs(inp, w_k=oracle.widen(inp.w_k_branch(0)), h=inp.hidden_branch(0))
    assert np.array_equal(p0.forward(want=("y",))["y"], same.forward(want=("y",))["y"])
