"""Pins of the oracle's table-gradient backward.

The pages ("DeepSeek AI II", system-efficiency section) state that in
training the gradients of the gathered rows are sent back to the rows they
came from; the backward itself is derived by the chain rule.  Pinned by
central finite differences of L = sum <G, Y> in float64, by conservation of
the summed gradient, by linearity in G, and by torch's CPU autograd.
"""
import numpy as np
import pytest

import synth
from tests.oracle_cases import small_problem


def _loss(p, dy):
    y = p.forward(want=("y",))["y"]
    return float(np.sum(y * dy.reshape(y.shape)))


def test_finite_differences(oracle_lib):
    p, dy = small_problem(oracle_lib, B=2, T=10, D=3, d=6, rows=[5, 7, 11, 13])
    grads = p.table_grad_dense(dy)
    idx = p.hash()
    h = 1e-5
    checked = 0
    worst = 0.0
    for j in range(p.J):
        for r in np.unique(idx[:, j])[:3]:
            for c in range(p.dim):
                orig = p.tables[j][r, c]
                p.tables[j][r, c] = orig + h
                lp = _loss(p, dy)
                p.tables[j][r, c] = orig - h
                lm = _loss(p, dy)
                p.tables[j][r, c] = orig
                fd = (lp - lm) / (2 * h)
                an = grads[j][r, c]
                worst = max(worst, abs(fd - an) / max(1e-3, abs(an)))
                checked += 1
    assert checked >= 30
    assert worst < 1e-6, worst
    # rows never addressed get no gradient
    for j in range(p.J):
        untouched = np.setdiff1d(np.arange(p.table_rows[j]), idx[:, j])
        assert np.all(grads[j][untouched] == 0.0)


def test_conservation_and_linearity(oracle_lib):
    p, dy = small_problem(oracle_lib, B=2, T=12, D=4, d=8)
    de = p.backward_de(dy)
    grads = p.table_grad_dense(dy)
    for j in range(p.J):
        assert np.allclose(grads[j].sum(0), de[:, j * p.dim:(j + 1) * p.dim].sum(0), rtol=1e-12, atol=1e-12)
    dy2 = synth.normal_stream(99, dy.size, 1.0, "f64").reshape(dy.shape)
    g2 = p.table_grad_dense(dy2)
    g12 = p.table_grad_dense(2.0 * dy - 0.5 * dy2)
    for j in range(p.J):
        assert np.abs(g12[j] - (2.0 * grads[j] - 0.5 * g2[j])).max() < 1e-12


def test_rows_match_dense(oracle_lib):
    p, dy = small_problem(oracle_lib, B=2, T=12, D=4, d=8, rows=[31, 37, 41, 43])
    grads = p.table_grad_dense(dy)
    idx = p.hash()
    rj, rr = [], []
    for j in range(p.J):
        for r in np.unique(idx[:, j])[:2]:
            rj.append(j)
            rr.append(int(r))
    rj.append(0)
    rr.append(int(np.setdiff1d(np.arange(p.table_rows[0]), idx[:, 0])[0]))  # a row never hit
    out, npos = p.table_grad_rows(dy, idx, rj, rr)
    for q, (j, r) in enumerate(zip(rj, rr)):
        assert np.abs(out[q] - grads[j][r]).max() < 1e-13
    assert np.all(out[-1] == 0.0) and npos > 0


def test_autograd_cross_check(oracle_lib):
    """de_t from the hand-derived backward equals torch CPU float64 autograd."""
    torch = pytest.importorskip("torch")
    p, dy = small_problem(oracle_lib, B=2, T=9, D=4, d=8)
    e = torch.tensor(p.forward(want=("e",))["e"].reshape(p.B, p.T, -1), requires_grad=True)
    wk, wv = torch.tensor(p.w_k), torch.tensor(p.w_v)
    h = torch.tensor(p.h)
    gq, gk = torch.tensor(p.gamma_q), torch.tensor(p.gamma_k)
    w = torch.tensor(p.conv_w)
    d = p.hidden
    k = e @ wk.T
    v = e @ wv.T
    qh = gq * h / torch.sqrt((h * h).mean(-1, keepdim=True) + p.eps)
    kh = gk * k / torch.sqrt((k * k).mean(-1, keepdim=True) + p.eps)
    a = torch.sigmoid((qh * kh).sum(-1, keepdim=True) / d ** 0.5)
    vt = a * v
    z = torch.zeros_like(vt)
    for i in range(p.taps):
        z[:, i:] = z[:, i:] + w[:, i] * vt[:, : p.T - i]
    y = torch.nn.functional.silu(z) + vt
    (y * torch.tensor(dy)).sum().backward()
    de = p.backward_de(dy)
    ref = e.grad.reshape(-1, p.d_mem).numpy()
    assert np.abs(de - ref).max() <= 1e-12 * np.abs(ref).max()
    assert np.abs(p.forward(want=("y",))["y"] - y.detach().reshape(-1, d).numpy()).max() < 1e-12
