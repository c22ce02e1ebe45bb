"""Pins of the oracle's E4M3 quantization and its FP8 projection mode.

The pages fuse W_V and the M key projections into one dense FP8 matmul
("DeepSeek AI II", section "DeepSeek Engram", multi-branch integration).
The OCP E4M3 format is pinned against torch's float8_e4m3fn (an independent
implementation): every code's value, and round-to-nearest-even on random,
midpoint and subnormal inputs.  The per-row scale maps the row's largest
magnitude to 448; the FP8 forward equals the plain forward whenever the
quantization is exact.
"""
import numpy as np
import pytest

import synth
from tests.oracle_cases import small_problem


def test_decode_matches_torch(oracle_lib):
    torch = pytest.importorskip("torch")
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle_lib.e4m3_decode(int(c)) for c in codes])
    finite = (codes & 0x7F) != 0x7F
    assert np.array_equal(got[finite], ref[finite])
    assert np.isnan(ref[~finite]).all()
    assert got[finite].max() == 448.0 and oracle_lib.e4m3_decode(1) == 2.0 ** -9


def test_encode_matches_torch(oracle_lib):
    torch = pytest.importorskip("torch")
    finite = [c for c in range(256) if (c & 0x7F) != 0x7F]
    vals = np.array(sorted({oracle_lib.e4m3_decode(c) for c in finite}))
    mids = (vals[1:] + vals[:-1]) / 2          # ties: exactly between two codes
    rnd = synth.unit_stream(5, 20000).astype(np.float64) * 2 - 1
    xs = np.concatenate([vals, mids, rnd * 448.0, rnd * 2.0 ** -6, rnd * 3.0]).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle_lib.e4m3_encode(float(x)) for x in xs], np.uint8)
    # torch keeps the sign of zero; the oracle does too
    assert np.array_equal(got, ref)
    # representable values round-trip; ties go to the even mantissa
    assert all(oracle_lib.e4m3_decode(oracle_lib.e4m3_encode(v)) == v for v in vals)
    # 432 lies between 416 and 448, 17 between 16 and 18, 19 between 18 and 20
    assert oracle_lib.e4m3_encode(432.0) == 0x7E and oracle_lib.e4m3_encode(17.0) == 0x58
    assert oracle_lib.e4m3_encode(19.0) == 0x5A
    # beyond the largest finite value: saturation
    assert oracle_lib.e4m3_encode(1e6) == 0x7E and oracle_lib.e4m3_encode(-500.0) == 0xFE


def test_row_scale(oracle_lib):
    x = synth.normal_stream(7, 6 * 300, 0.02, "f32").reshape(6, 300)
    x[3] = 0.0
    codes, scales, deq = oracle_lib.quantize_rows(x)
    for r in range(6):
        if r == 3:
            assert scales[r] == 1.0 and not codes[r].any()
            continue
        amax = np.float32(np.abs(x[r]).max())
        assert scales[r] == np.float32(amax / np.float32(448.0))
        assert (codes[r] & 0x7F).max() == 0x7E      # the largest magnitude becomes 448
        # each value within half a step of its E4M3 neighbourhood (relative 2^-4)
        assert np.all(np.abs(deq[r] - x[r]) <= np.abs(x[r]) * 2.0 ** -4 + scales[r] * 2.0 ** -10)


def test_fp8_forward_is_exact_when_quantization_is(oracle_lib):
    """With every table row, weight row and token row holding 448 and
    otherwise E4M3 values, all scales are 1 and the FP8 forward equals the
    plain forward."""
    p, dy = small_problem(oracle_lib, B=2, T=9, D=4, d=8)
    pick = np.array([0.25, -0.5, 1.0, 2.0, -3.0, 0.125, 6.0, -0.75])
    for j, t in enumerate(p.tables):
        t[:] = pick[(np.arange(t.size) * 7 + j) % pick.size].reshape(t.shape)
    p.tables[0][:, 0] = 448.0        # every token's e row reaches 448
    for w in (p.w_k, p.w_v):
        w[:] = pick[(np.arange(w.size) * 5) % pick.size].reshape(w.shape) / 64.0
        w[:, 1] = 448.0
    plain = p.forward(want=("y", "k", "v"))
    import oracle
    q = oracle.Problem(orders=p.orders, heads=p.heads, mult=p.mult, table_rows=p.table_rows,
                       pad_id=p.pad_id, canon_map=p.canon_map, tokens=p.tokens, tables=p.tables,
                       w_k=p.w_k, w_v=p.w_v, h=p.h, conv_w=p.conv_w, gamma_q=p.gamma_q,
                       gamma_k=p.gamma_k, eps=p.eps, fp8=True)
    f8 = q.forward(want=("y", "k", "v"))
    for k in ("y", "k", "v"):
        assert np.array_equal(f8[k], plain[k]), k


def test_fp8_forward_differs_when_inexact(oracle_lib):
    """On ordinary data the FP8 projection rounds e and W: k moves by about
    the E4M3 step, not by more."""
    p, dy = small_problem(oracle_lib, B=2, T=9, D=4, d=8)
    import oracle
    q = oracle.Problem(orders=p.orders, heads=p.heads, mult=p.mult, table_rows=p.table_rows,
                       pad_id=p.pad_id, canon_map=p.canon_map, tokens=p.tokens, tables=p.tables,
                       w_k=p.w_k, w_v=p.w_v, h=p.h, conv_w=p.conv_w, gamma_q=p.gamma_q,
                       gamma_k=p.gamma_k, eps=p.eps, fp8=True)
    a = p.forward(want=("k",))["k"]
    b = q.forward(want=("k",))["k"]
    rel = np.abs(a - b).max() / np.abs(a).max()
    assert 1e-4 < rel < 0.2
