"""Pins of the oracle's forward: gather, projections, gate, conv, composition.

What the pages fix ("DeepSeek AI II", section "DeepSeek Engram"): e_t is
the concatenation of the retrieved rows; e_t feeds the key and value
projections; query h_t and key k_t pass through RMSNorm before a scalar gate
alpha_t in (0,1); the gated value alpha_t v_t is refined by a short depthwise
causal convolution and added residually.  Checked against exact table rows,
numpy matmul, closed forms of the gate, the conv's impulse response and
locality/causality invariants.
"""
import numpy as np
import pytest

import synth
from tests.oracle_cases import small_problem


@pytest.fixture(scope="module")
def tiny(oracle_lib):
    wl = synth.get_workload("tiny").with_shape(2, 96)
    inp = synth.Inputs(wl)
    return wl, inp, oracle_lib.Problem.from_inputs(inp)


def test_gather_is_exact_concat_of_rows(tiny):
    wl, inp, p = tiny
    pos = np.arange(0, wl.B * wl.T, 7)
    out = p.forward(pos, want=("e",))
    idx = p.hash(pos)
    for q in range(pos.size):
        for j in range(wl.J):
            row = synth.as_float(inp.tables[j][idx[q, j]]).astype(np.float64)
            assert np.array_equal(out["e"][q, j * wl.dim:(j + 1) * wl.dim], row)


def test_projection_matches_numpy_matmul(tiny):
    wl, inp, p = tiny
    pos = np.arange(0, wl.B * wl.T, 5)
    out = p.forward(pos, want=("e", "k", "v"))
    wk = synth.as_float(inp.w_k).astype(np.float64)
    wv = synth.as_float(inp.w_v).astype(np.float64)
    k_ref = out["e"] @ wk.T
    v_ref = out["e"] @ wv.T
    assert np.abs(out["k"] - k_ref).max() <= 1e-12 * np.abs(k_ref).max()
    assert np.abs(out["v"] - v_ref).max() <= 1e-12 * np.abs(v_ref).max()


def test_gate_half_when_dot_is_zero(oracle_lib):
    p, _ = small_problem(oracle_lib, d=8)
    rng = synth.normal_stream(31, 16, 1.0, "f64")
    h, k = rng[:8], rng[8:]
    assert p.gate_value(np.zeros(8), k) == 0.5
    assert p.gate_value(h, np.zeros(8)) == 0.5
    # orthogonal (after the RMSNorm scales) h and k: <g_q h, g_k k> = 0
    gq, gk = p.gamma_q, p.gamma_k
    kk = k.copy()
    kk -= (np.dot(gq * h, gk * kk) / np.dot(gq * h, gk * (gq * h))) * (gq * h)
    assert abs(p.gate_value(h, kk) - 0.5) < 1e-15


def test_gate_closed_forms(oracle_lib):
    p, _ = small_problem(oracle_lib, d=8, gammas=False, eps=1e-6)
    h = synth.normal_stream(32, 8, 1.0, "f64")
    a = p.gate_value(h, h)
    ms = np.mean(h * h)
    s = np.sqrt(8.0) * ms / (ms + 1e-6)
    assert abs(a - 1.0 / (1.0 + np.exp(-s))) < 1e-15
    # antisymmetry: sigma(-s) = 1 - sigma(s)
    k = synth.normal_stream(33, 8, 1.0, "f64")
    assert abs(p.gate_value(-h, k) - (1.0 - p.gate_value(h, k))) < 1e-15
    assert 0.0 < p.gate_value(h, k) < 1.0
    # scale invariance of RMSNorm (exact with eps = 0)
    p0, _ = small_problem(oracle_lib, d=8, gammas=False, eps=0.0)
    base = p0.gate_value(h, k)
    for c in (1e-3, 0.5, 7.0, 1e4):
        assert abs(p0.gate_value(c * h, k) - base) < 1e-14
        assert abs(p0.gate_value(h, c * k) - base) < 1e-14


def test_conv_impulse_response_is_kernel(oracle_lib):
    p, _ = small_problem(oracle_lib, d=8, taps=4)
    T = 9
    vt = np.zeros((T, 8))
    vt[0] = 1.0
    z, y = p.conv(vt)
    for t in range(T):
        want = p.conv_w[:, t] if t < 4 else np.zeros(8)
        assert np.array_equal(z[t], want)
    silu = z / (1.0 + np.exp(-z))
    assert np.allclose(y, silu + vt, rtol=0, atol=1e-15)


def test_conv_identity_linearity_causality(oracle_lib):
    p, _ = small_problem(oracle_lib, d=8, taps=4)
    T = 12
    x1 = synth.normal_stream(40, T * 8, 1.0, "f64").reshape(T, 8)
    x2 = synth.normal_stream(41, T * 8, 1.0, "f64").reshape(T, 8)
    z1, _ = p.conv(x1)
    z2, _ = p.conv(x2)
    z12, _ = p.conv(2.0 * x1 - 3.0 * x2)
    assert np.abs(z12 - (2.0 * z1 - 3.0 * z2)).max() < 1e-13
    # causality: changing x at t0 leaves z before t0 untouched
    x3 = x1.copy()
    x3[6] += 1.0
    z3, _ = p.conv(x3)
    assert np.array_equal(z3[:6], z1[:6]) and not np.array_equal(z3[6], z1[6])
    # w = delta at tap 0 -> z = x
    q, _ = small_problem(oracle_lib, d=8, taps=4)
    q.conv_w[:] = 0.0
    q.conv_w[:, 0] = 1.0
    z, y = q.conv(x1)
    assert np.array_equal(z, x1)


def test_forward_composition_special_cases(oracle_lib):
    # conv taps all zero -> y = alpha v; W_K = 0 -> alpha = 1/2
    p, _ = small_problem(oracle_lib)
    p.conv_w[:] = 0.0
    out = p.forward(want=("y", "alpha", "v"))
    assert np.abs(out["y"] - out["alpha"][:, None] * out["v"]).max() < 1e-15
    p.w_k[:] = 0.0
    out = p.forward(want=("y", "alpha", "v"))
    assert (out["alpha"] == 0.5).all()
    assert np.abs(out["y"] - 0.5 * out["v"]).max() < 1e-15


def test_forward_locality(oracle_lib):
    """Y_t depends on canonical ids t-5..t and hidden states t-3..t only (orders<=3, taps 4)."""
    p, _ = small_problem(oracle_lib, B=1, T=16, vocab=50, canon=40)
    t = 10
    base = p.forward(np.array([t]))["y"][0]

    def y_with(tokens=None, h=None):
        q, _ = small_problem(oracle_lib, B=1, T=16, vocab=50, canon=40)
        if tokens is not None:
            q.tokens[:] = tokens
        if h is not None:
            q.h[:] = h
        return q.forward(np.array([t]))["y"][0]

    for tp, changes in ((t + 1, False), (t - 6, False), (t - 5, True), (t, True)):
        tok = p.tokens.copy()
        # pick a raw id with a different canonical id
        cur = p.canon_map[tok[0, tp]]
        tok[0, tp] = int(np.nonzero(p.canon_map != cur)[0][0])
        y = y_with(tokens=tok)
        assert (not np.array_equal(y, base)) == changes, tp
    for tp, changes in ((t - 4, False), (t + 1, False), (t - 3, True), (t, True)):
        h = p.h.copy()
        h[0, tp] += 1.0
        y = y_with(h=h)
        assert (not np.array_equal(y, base)) == changes, tp


def test_identical_contexts_identical_rows(oracle_lib):
    """Same canonical 3-gram context -> same e_t (deterministic retrieval)."""
    wl = synth.get_workload("tiny").with_shape(2, 96)
    inp = synth.Inputs(wl)
    tok = inp.tokens.copy()
    tok[0, 50:53] = tok[0, 10:13]   # repeat a trigram inside a sequence
    tok[1, 30:33] = tok[0, 10:13]   # and across sequences
    p = oracle_lib.Problem.from_inputs(inp, tokens=tok)
    canon = inp.canon_map[tok].reshape(-1)
    T = wl.T
    pos = np.arange(wl.B * wl.T)
    e = p.forward(pos, want=("e",))["e"]
    seen = {}
    hits = 0
    for q in pos:
        b, t = divmod(int(q), T)
        ctx = tuple(int(canon[b * T + t - i]) if t - i >= 0 else wl.pad_id for i in range(3))
        if ctx in seen:
            assert np.array_equal(e[seen[ctx]], e[q])
            hits += 1
        else:
            seen[ctx] = q
    assert hits >= 2
