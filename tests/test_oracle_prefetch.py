"""Pins of the oracle's prefetch plan: per-table sorted unique rows and the
inverse map (the pages: indices are known from the token ids before the
forward pass, so the needed rows can be fetched ahead of time)."""
import numpy as np

import synth


def test_plan_matches_numpy_unique(oracle_lib):
    wl = synth.get_workload("tiny").with_shape(2, 300)
    inp = synth.Inputs(wl)
    p = oracle_lib.Problem.from_inputs(inp)
    idx = p.hash()
    uniq, counts, inv = oracle_lib.prefetch_plan(idx)
    base = 0
    for j in range(wl.J):
        u, iv = np.unique(idx[:, j], return_inverse=True)
        assert counts[j] == u.size
        assert np.array_equal(uniq[base:base + u.size], u)
        assert np.array_equal(inv[:, j], iv)
        assert np.array_equal(u[inv[:, j]], idx[:, j])
        base += u.size


def test_plan_edge_cases(oracle_lib):
    idx = np.zeros((5, 3), np.int32)
    uniq, counts, inv = oracle_lib.prefetch_plan(idx)
    assert list(counts) == [1, 1, 1] and (inv == 0).all() and list(uniq) == [0, 0, 0]
    idx = np.zeros((0, 2), np.int32)
    uniq, counts, inv = oracle_lib.prefetch_plan(idx)
    assert list(counts) == [0, 0] and inv.shape == (0, 2)
