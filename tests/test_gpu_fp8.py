"""FP8 projection on the GPU: E4M3 codes and scales bit-exact against the
oracle's quantization (the same fp32 scale and quotient, round to nearest
even)."""
import numpy as np
import pytest

import synth
from tests import harness as H

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    return torch


def _quantize(torch, x):
    import hashed_gram_embedding_canon_amd as eg
    rows, cols = x.shape
    codes = torch.empty(rows, cols, dtype=torch.uint8, device="cuda")
    scales = torch.empty(rows, dtype=torch.float32, device="cuda")
    dt = eg.ENGRAM_BF16 if x.dtype == np.uint16 else eg.ENGRAM_F32
    eg.engram_quantize_fp8(H.to_dev(x), dt, rows, cols, codes, scales)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def test_quantize_matches_oracle(torch, oracle_lib):
    w = synth.normal_stream(11, 512 * 256, 0.05, "bf16").reshape(512, 256)
    # fp32 rows spanning many binades, so that many quotients are E4M3 subnormals
    u = synth.unit_stream(12, 64 * 1024).reshape(64, 1024)
    x = ((u * 2 - 1) * np.exp2(np.floor(synth.unit_stream(13, 64 * 1024) * 40) - 30).reshape(64, 1024)).astype(np.float32)
    x[5] = 0.0
    x[6] = 1e-3
    x[6, 17] = 3e4
    for arr in (w, x):
        codes, scales = _quantize(torch, arr)
        rc, rs, _ = oracle_lib.quantize_rows(arr)
        assert np.array_equal(scales, rs)
        mism = np.argwhere(codes != rc)
        assert mism.size == 0, (mism[:5], codes[tuple(mism[0])], rc[tuple(mism[0])])


def _fp8_problem(inp, branch=0, tokens=None):
    import oracle
    over = {"fp8": True}
    if branch:
        over["w_k"] = oracle.widen(inp.w_k_branch(branch))
        over["h"] = inp.hidden_branch(branch)
    if tokens is not None:
        over["tokens"] = tokens
    return oracle.Problem.from_inputs(inp, **over)


@pytest.mark.parametrize("B,T,M", [(2, 300, 1), (3, 77, 1), (1, 256, 2)])
def test_fp8_forward_matches_oracle(torch, oracle_lib, B, T, M):
    """Y, the saved k and the gates of the FP8 projection against the oracle
    in its FP8 mode (the same E4M3 codes and scales), to the bf16 bars."""
    import dataclasses
    import hashed_gram_embedding_canon_amd as eg
    wl = dataclasses.replace(synth.get_workload("tiny"), dtype="bf16", branches=M).with_shape(B, T)
    print(f"[fp8 forward] B={B} T={T} M={M}", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp, flags=eg.ENGRAM_FLAG_FP8_PROJ)
    bufs = dp.alloc_saved(("idx", "stats", "k"))
    y = dp.forward(bufs)
    torch.cuda.synchronize()
    for m in range(M):
        p = _fp8_problem(inp, branch=m)
        if m == 0:  # the indices the quantizing gather hashed and saved
            assert np.array_equal(bufs["idx"].cpu().numpy(), p.hash())
        ref = p.forward(want=("y", "k", "alpha"))
        ym = y if M == 1 else y[m]
        km = bufs["k"] if M == 1 else bufs["k"][m]
        sm = bufs["stats"] if M == 1 else bufs["stats"][m]
        ey = H.rel_max_err(H.to_host_f64(ym).reshape(ref["y"].shape), ref["y"])
        ek = H.rel_max_err(H.to_host_f64(km).reshape(ref["k"].shape), ref["k"])
        ea = np.abs(sm[:, 0].cpu().numpy().astype(np.float64) - ref["alpha"]).max()
        print(f"  branch {m}: y {ey:.2e} k {ek:.2e} alpha {ea:.2e}", flush=True)
        assert ey <= 1e-2 and ek <= 1e-2 and ea <= 1e-3, (ey, ek, ea)


def test_fp8_small_sampled(torch, oracle_lib):
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload("small").with_shape(8, 4096)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp, flags=eg.ENGRAM_FLAG_FP8_PROJ)
    y = dp.forward()
    torch.cuda.synchronize()
    pos = H.sample_positions(wl.B, wl.T, 96)
    ref = _fp8_problem(inp).forward(pos, want=("y",))["y"]
    got = H.to_host_f64(y).reshape(-1, wl.hidden)[pos]
    err = H.rel_max_err(got, ref)
    print(f"  small fp8: {err:.2e}", flush=True)
    assert err <= 1e-2, err


def test_fp8_rejects_fused_gather(torch):
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload("tiny").with_shape(1, 64)
    import dataclasses
    wl = dataclasses.replace(wl, dtype="bf16")
    dp = H.DeviceProblem(synth.Inputs(wl), flags=eg.ENGRAM_FLAG_FP8_PROJ | eg.ENGRAM_FLAG_FUSED_GATHER)
    with pytest.raises(eg.EngramError, match="status 2"):
        dp.forward()


def test_fp8_concurrent_streams(torch):
    """The FP8 projection (four-deep stage ring) with batch slices on three
    streams at once: Y bit-identical to one forward over the batch."""
    import hashed_gram_embedding_canon_amd as eg
    from tests.test_gpu_forward import _forward_on_streams
    wl = synth.get_workload("small").with_shape(8, 4096)
    dp = H.DeviceProblem(synth.Inputs(wl), flags=eg.ENGRAM_FLAG_FP8_PROJ)
    y_ref = dp.forward()
    torch.cuda.synchronize()
    for rep in range(3):
        y = _forward_on_streams(torch, dp, y_ref, chunks=8, streams=3)
        bad = int((y != y_ref).reshape(dp.N, -1).any(dim=1).sum())
        print(f"  rep {rep}: tokens differing {bad}", flush=True)
        assert bad == 0


def test_fp8_engram27b_sampled(torch, oracle_lib):
    """The FP8 projection at the 27B scale, as the bench's --fp8 run: Y against
    the oracle's FP8 mode at sampled positions."""
    import hashed_gram_embedding_canon_amd as eg
    wl = synth.get_workload("engram27b")
    print("[engram27b fp8] generating and uploading 5.7B table parameters", flush=True)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp, flags=eg.ENGRAM_FLAG_FP8_PROJ)
    y = dp.forward()
    torch.cuda.synchronize()
    pos = H.sample_positions(wl.B, wl.T, 96, seed=31)
    ref = _fp8_problem(inp).forward(pos, want=("y",))["y"]
    got = H.to_host_f64(y).reshape(-1, wl.hidden)[pos]
    err = H.rel_max_err(got, ref)
    print(f"  engram27b fp8: {err:.2e}", flush=True)
    assert err <= 1e-2, err
    del dp, y
    torch.cuda.empty_cache()
