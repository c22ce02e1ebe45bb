"""Pins of the oracle's parameter and hidden-state gradients.

Training ("DeepSeek AI II", section "DeepSeek Engram" with its
system-efficiency part) updates the projections, the conv and the RMSNorm
scales along with the tables; the gradients are the chain rule through the
forward.  Pinned by central finite differences of L = sum <G, Y> in float64,
by torch's CPU autograd, by the scale invariance of RMSNorm, by the
bilinearity of the gate score in the two RMSNorm scales, and by the locality
of the conv (a sparse G touches a few positions only).
"""
import numpy as np
import pytest

from tests.oracle_cases import small_problem


def _loss(p, dy):
    y = p.forward(want=("y",))["y"]
    return float(np.sum(y * dy.reshape(y.shape)))


def _fd(p, dy, arr, index, h=1e-5):
    orig = arr[index]
    arr[index] = orig + h
    lp = _loss(p, dy)
    arr[index] = orig - h
    lm = _loss(p, dy)
    arr[index] = orig
    return (lp - lm) / (2 * h)


def test_finite_differences(oracle_lib):
    p, dy = small_problem(oracle_lib, B=2, T=9, D=3, d=6)
    g = p.backward_params(dy)
    rng = np.random.default_rng(7)
    worst = 0.0
    checks = []
    for name, arr in (("w_k", p.w_k), ("w_v", p.w_v)):
        for _ in range(12):
            checks.append((name, arr, (int(rng.integers(p.hidden)), int(rng.integers(p.d_mem)))))
    for c in range(p.hidden):
        for i in range(p.taps):
            checks.append(("conv_w", p.conv_w, (c, i)))
        checks.append(("gamma_q", p.gamma_q, (c,)))
        checks.append(("gamma_k", p.gamma_k, (c,)))
    for name, arr, index in checks:
        fd = _fd(p, dy, arr, index)
        an = g[name][index]
        worst = max(worst, abs(fd - an) / max(1e-3, abs(an)))
    assert worst < 1e-6, worst
    # the hidden state enters through the gate's query only
    worst = 0.0
    for _ in range(20):
        b, t, c = int(rng.integers(p.B)), int(rng.integers(p.T)), int(rng.integers(p.hidden))
        fd = _fd(p, dy, p.h, (b, t, c))
        an = g["h"][b * p.T + t, c]
        worst = max(worst, abs(fd - an) / max(1e-3, abs(an)))
    assert worst < 1e-6, worst


def test_autograd_cross_check(oracle_lib):
    torch = pytest.importorskip("torch")
    p, dy = small_problem(oracle_lib, B=2, T=9, D=4, d=8)
    e = torch.tensor(p.forward(want=("e",))["e"].reshape(p.B, p.T, -1))
    wk = torch.tensor(p.w_k, requires_grad=True)
    wv = torch.tensor(p.w_v, requires_grad=True)
    h = torch.tensor(p.h, requires_grad=True)
    gq = torch.tensor(p.gamma_q, requires_grad=True)
    gk = torch.tensor(p.gamma_k, requires_grad=True)
    w = torch.tensor(p.conv_w, requires_grad=True)
    d = p.hidden
    k = e @ wk.T
    v = e @ wv.T
    qh = gq * h / torch.sqrt((h * h).mean(-1, keepdim=True) + p.eps)
    kh = gk * k / torch.sqrt((k * k).mean(-1, keepdim=True) + p.eps)
    a = torch.sigmoid((qh * kh).sum(-1, keepdim=True) / d ** 0.5)
    vt = a * v
    z = torch.zeros_like(vt)
    for i in range(p.taps):
        z = z + torch.nn.functional.pad(w[:, i] * vt[:, : p.T - i], (0, 0, i, 0))
    y = torch.nn.functional.silu(z) + vt
    (y * torch.tensor(dy)).sum().backward()
    g = p.backward_params(dy)
    for name, ref in (("w_k", wk.grad), ("w_v", wv.grad), ("conv_w", w.grad), ("gamma_q", gq.grad),
                      ("gamma_k", gk.grad), ("h", h.grad.reshape(-1, d))):
        ref = ref.numpy()
        assert np.abs(g[name] - ref).max() <= 1e-12 * np.abs(ref).max(), name


def test_sparse_upstream_gradient_touches_few_positions(oracle_lib):
    """With G nonzero at a few tokens only, the sums over the positions
    s-taps+1..s of those tokens equal the sums over every position."""
    p, dy = small_problem(oracle_lib, B=2, T=16, D=3, d=6)
    keep = [(0, 0), (0, 9), (1, 15), (1, 4)]
    sp = np.zeros_like(dy)
    for b, t in keep:
        sp[b, t] = dy[b, t]
    full = p.backward_params(sp)
    pos = sorted({b * p.T + u for b, t in keep for u in range(max(0, t - p.taps + 1), t + 1)})
    part = p.backward_params(sp, pos=np.array(pos))
    for name in ("w_k", "w_v", "conv_w", "gamma_q", "gamma_k"):
        scale = np.abs(full[name]).max()
        assert scale > 0 and np.abs(part[name] - full[name]).max() <= 1e-14 * scale, name
    assert np.array_equal(part["h"], full["h"][pos])
    untouched = np.setdiff1d(np.arange(p.B * p.T), pos)
    assert np.all(full["h"][untouched] == 0.0)


def test_rmsnorm_scale_invariance(oracle_lib):
    """With eps = 0 the gate does not change when h_t is scaled, so dh_t is
    orthogonal to h_t."""
    p, dy = small_problem(oracle_lib, B=2, T=8, D=4, d=8, eps=0.0)
    dh = p.backward_params(dy, want=("h",))["h"]
    h = p.h.reshape(-1, p.hidden)
    dots = np.einsum("nc,nc->n", dh, h)
    assert np.abs(dots).max() <= 1e-12 * np.abs(dh).max() * np.abs(h).max() * p.hidden
    assert np.abs(dh).max() > 1e-3


def test_gamma_bilinearity(oracle_lib):
    """The score is linear in each RMSNorm scale, so sum_c g_q dL/dg_q and
    sum_c g_k dL/dg_k both equal sum_t dL/ds_t s_t."""
    p, dy = small_problem(oracle_lib, B=2, T=10, D=4, d=8)
    g = p.backward_params(dy, want=("gamma_q", "gamma_k"))
    a = float(p.gamma_q @ g["gamma_q"])
    b = float(p.gamma_k @ g["gamma_k"])
    assert abs(a) > 1e-6
    assert abs(a - b) <= 1e-12 * abs(a)
