"""GPU parity of the forward pass against the oracle, through the C ABI.

Bit-exact: hash indices and gathered rows.  Floating point: max-abs-error /
max|ref| <= 1e-5 for the fp32 path, <= 1e-2 for the bf16 path (bf16 tables,
weights, hidden states and outputs; fp32 accumulation and gate math).  At the
small/27B/40B scales the oracle is evaluated on sampled positions, which is
exact to the definition: Y_t depends on canonical ids t-5..t and hidden
states t-3..t only.
"""
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


def _run_full(torch, wl, tokens=None, hidden=None, saved=("idx", "stats", "e"), flags=0):
    """Forward with the requested saved tensors.  By default the library
    gathers e (into saved e or its workspace) and runs the projection on it;
    with ENGRAM_FLAG_FUSED_GATHER and no saved e the projection reads the table
    rows itself."""
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp, tokens=tokens, flags=flags)
    if hidden is not None:
        dp.hidden = H.to_dev(hidden)
    bufs = dp.alloc_saved(saved)
    y = dp.forward(bufs)
    torch.cuda.synchronize()
    return inp, dp, bufs, y


@pytest.mark.parametrize("B,T", [(1, 512), (3, 77), (2, 1), (1, 3), (5, 257), (2, 300)])
def test_tiny_fp32_full(torch, oracle_lib, B, T):
    wl = synth.get_workload("tiny").with_shape(B, T)
    print(f"[tiny fp32] B={B} T={T}", flush=True)
    inp, dp, bufs, y = _run_full(torch, wl)
    p = H.oracle_problem(inp)
    idx_ref = p.hash()
    assert np.array_equal(bufs["idx"].cpu().numpy(), idx_ref)
    ref = p.forward(want=("y", "alpha", "e"))
    assert np.array_equal(H.to_host_f64(bufs["e"]), ref["e"])  # gathered rows, bit-exact
    got = H.to_host_f64(y).reshape(-1, wl.hidden)
    err = H.rel_max_err(got, ref["y"])
    assert err <= TOL["f32"], err
    a_err = np.abs(bufs["stats"][:, 0].cpu().numpy() - ref["alpha"]).max()
    assert a_err <= 1e-5, a_err


def test_tiny_repeated_ngrams_give_identical_rows(torch):
    wl = synth.get_workload("tiny").with_shape(2, 96)
    inp = synth.Inputs(wl)
    tok = inp.tokens.copy()
    tok[0, 50:53] = tok[0, 10:13]
    tok[1, 30:33] = tok[0, 10:13]
    inp2, dp, bufs, y = _run_full(torch, wl, tokens=tok)
    e = bufs["e"].cpu().numpy().reshape(2, 96, -1)
    assert np.array_equal(e[0, 52], e[0, 12]) and np.array_equal(e[1, 32], e[0, 12])


def test_deterministic_and_hash_entry_point(torch):
    wl = synth.get_workload("tiny").with_shape(2, 300)
    inp, dp, bufs, y = _run_full(torch, wl)
    y2 = dp.forward(dp.alloc_saved(()))
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    idx = dp.hash()
    torch.cuda.synchronize()
    assert torch.equal(idx, bufs["idx"])


@pytest.mark.parametrize("name,dtype,B,T", [("tiny", "f32", 3, 77), ("tiny", "bf16", 2, 513),
                                             ("tiny", "f32", 1, 512), ("small", "bf16", 2, 1024)])
def test_fused_gather_matches_materialized(torch, oracle_lib, name, dtype, B, T):
    """The projection fed straight from the tables gives bit-identical Y to the
    one fed from the gathered e (saved or workspace), and matches the oracle."""
    import hashed_gram_embedding_canon_amd as eg
    wl = dataclasses.replace(synth.get_workload(name), dtype=dtype).with_shape(B, T)
    inp, dp, bufs, y_mat = _run_full(torch, wl, saved=("idx", "e"), flags=eg.ENGRAM_FLAG_FUSED_GATHER)
    y_fused = dp.forward(dp.alloc_saved(("idx",)))
    dp.cfg.c.flags = 0
    y_ws = dp.forward(dp.alloc_saved(("idx",)))
    torch.cuda.synchronize()
    assert torch.equal(y_fused, y_mat)
    assert torch.equal(y_ws, y_mat)
    if name == "tiny":
        ref = H.oracle_problem(inp).forward(want=("y",))["y"]
        err = H.rel_max_err(H.to_host_f64(y_fused).reshape(-1, wl.hidden), ref)
        assert err <= TOL[dtype], err


def test_empty_batch_is_a_noop(torch):
    wl = synth.get_workload("tiny").with_shape(1, 8)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    import hashed_gram_embedding_canon_amd as eg
    y = torch.full((1, 8, wl.hidden), 7.0, device="cuda")
    eg.engram_forward(dp.cfg, dp.params, dp.tokens, dp.hidden, y, B=0, T=8,
                      workspace=dp.workspace(0))
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())


def _sampled_check(torch, oracle_lib, dp, inp, bufs, y, n_pos, seed):
    wl = inp.wl
    pos = H.sample_positions(dp.B, dp.T, n_pos, seed=seed)
    p = H.oracle_problem(inp)
    idx_all = p.hash()
    assert np.array_equal(bufs["idx"].cpu().numpy(), idx_all)  # every index, bit-exact
    ref = p.forward(pos, want=("y", "alpha"))
    yy = y.reshape(-1, wl.hidden)[torch.as_tensor(pos, device=y.device)]
    got = H.to_host_f64(yy)
    err = H.rel_max_err(got, ref["y"])
    alpha = bufs["stats"][torch.as_tensor(pos, device=y.device), 0].cpu().numpy()
    a_err = float(np.abs(alpha - ref["alpha"]).max())
    # gathered rows at the sampled positions, bit-exact
    e = bufs["e"][torch.as_tensor(pos, device=y.device)].view(torch.int16).cpu().numpy()
    e = e.view(np.uint16).reshape(len(pos), wl.J, wl.dim)
    for j in range(wl.J):
        rows = inp.table(j)[idx_all[pos, j]]
        assert np.array_equal(e[:, j, :], rows), j
    return err, a_err


@pytest.mark.parametrize("B,T", [(3, 77), (2, 513), (1, 2)])
def test_tiny_bf16_ragged(torch, oracle_lib, B, T):
    """bf16 kernels on ragged token counts (partial 256-token GEMM tiles, short sequences)."""
    wl = dataclasses.replace(synth.get_workload("tiny"), name="tiny_bf16", dtype="bf16").with_shape(B, T)
    inp, dp, bufs, y = _run_full(torch, wl)
    p = H.oracle_problem(inp)
    assert np.array_equal(bufs["idx"].cpu().numpy(), p.hash())
    ref = p.forward(want=("y", "alpha", "e"))
    assert np.array_equal(H.to_host_f64(bufs["e"]), ref["e"])
    err = H.rel_max_err(H.to_host_f64(y).reshape(-1, wl.hidden), ref["y"])
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("heads,dim", [(4, 32), (6, 64)])
def test_bf16_short_memory(torch, oracle_lib, heads, dim):
    """bf16 projections over a memory vector of 4 and 12 K stages of 64
    values (e_t of 256 values: 8 tables of 32; 768 values: 12 tables of 64):
    the projection peels its first two stages (whose first step starts the
    accumulators) and runs its last two with no, or with four, passes of the
    stage loop between them."""
    wl = dataclasses.replace(synth.get_workload("tiny"), name=f"tiny_bf16_h{heads}", dtype="bf16",
                             heads=heads, dim=dim, rows=(10007,) * (2 * heads)).with_shape(2, 300)
    assert wl.d_mem == 2 * heads * dim
    inp, dp, bufs, y = _run_full(torch, wl)
    p = H.oracle_problem(inp)
    assert np.array_equal(bufs["idx"].cpu().numpy(), p.hash())
    ref = p.forward(want=("y", "alpha", "e"))
    assert np.array_equal(H.to_host_f64(bufs["e"]), ref["e"])
    err = H.rel_max_err(H.to_host_f64(y).reshape(-1, wl.hidden), ref["y"])
    a_err = float(np.abs(bufs["stats"][:, 0].cpu().numpy() - ref["alpha"]).max())
    print(f"  d_mem = {wl.d_mem}: max-abs-err/max|ref| = {err:.3e}, alpha err {a_err:.2e}", flush=True)
    assert err <= TOL["bf16"] and a_err <= 1e-2, (err, a_err)


@pytest.mark.parametrize("B,T", [(1, 4196), (2, 2048), (2, 2085)])
def test_bf16_tiles_per_workgroup(torch, oracle_lib, B, T):
    """bf16 forward where the persistent projection gives workgroups several
    tiles each (d = 2560: 20 feature tiles; 16 or 17 token tiles), so every
    tile but a workgroup's last loads the next one's first K stage early;
    with a ragged last token tile (4196 and 4170 tokens) that tile is loaded
    by its own prologue.  Every position against the oracle."""
    wl = dataclasses.replace(synth.get_workload("tiny"), name="tiny_bf16_tiles", dtype="bf16",
                             hidden=2560).with_shape(B, T)
    print(f"[bf16 tiles per workgroup] B={B} T={T}", flush=True)
    inp, dp, bufs, y = _run_full(torch, wl, saved=("idx", "stats"))
    p = H.oracle_problem(inp)
    ref = p.forward(want=("y", "alpha"))
    err = H.rel_max_err(H.to_host_f64(y).reshape(-1, wl.hidden), ref["y"])
    a_err = float(np.abs(bufs["stats"][:, 0].cpu().numpy() - ref["alpha"]).max())
    print(f"  max-abs-err/max|ref| = {err:.3e}, alpha err {a_err:.2e}", flush=True)
    assert err <= TOL["bf16"] and a_err <= 1e-2, (err, a_err)


@pytest.mark.parametrize("B,T", [(8, 4096)])
def test_small_bf16(torch, oracle_lib, B, T):
    wl = synth.get_workload("small").with_shape(B, T)
    print(f"[small bf16] B={B} T={T}", flush=True)
    inp, dp, bufs, y = _run_full(torch, wl)
    err, a_err = _sampled_check(torch, oracle_lib, dp, inp, bufs, y, 384, seed=11)
    print(f"  max-abs-err/max|ref| = {err:.3e}, alpha err {a_err:.2e}", flush=True)
    assert err <= TOL["bf16"], err
    assert a_err <= 1e-2


@pytest.fixture(scope="module")
def c27(torch):
    wl = synth.get_workload("engram27b")
    print("[engram27b] generating and uploading 5.7B table parameters", flush=True)
    inp, dp, bufs, y = _run_full(torch, wl)
    yield inp, dp, bufs, y
    del dp, bufs, y
    torch.cuda.empty_cache()


def test_engram27b_forward(torch, oracle_lib, c27):
    inp, dp, bufs, y = c27
    err, a_err = _sampled_check(torch, oracle_lib, dp, inp, bufs, y, 4096, seed=12)
    print(f"  engram27b max-abs-err/max|ref| = {err:.3e}, alpha err {a_err:.2e}", flush=True)
    assert err <= TOL["bf16"], err
    assert a_err <= 1e-2


def _forward_on_streams(torch, dp, y_like, chunks=8, streams=3):
    """Forwards of `chunks` batch slices issued round-robin on `streams` torch
    streams at once (each stream with its own workspace) -> Y."""
    import hashed_gram_embedding_canon_amd as eg
    bc = dp.B // chunks
    sts = [torch.cuda.Stream() for _ in range(streams)]
    ws = [torch.empty(eg.engram_workspace_size(dp.cfg, bc, dp.T, eg.ENGRAM_OP_FORWARD), dtype=torch.uint8,
                      device="cuda")
          for _ in range(streams)]
    y = torch.full_like(y_like, float("nan"))
    ev = torch.cuda.Event()
    ev.record()
    for st in sts:
        st.wait_event(ev)
    for c in range(chunks):
        sl = slice(c * bc, (c + 1) * bc)
        eg.engram_forward(dp.cfg, dp.params, dp.tokens[sl], dp.hidden[sl], y[sl], B=bc, T=dp.T,
                          workspace=ws[c % streams], stream=sts[c % streams])
    torch.cuda.synchronize()
    return y


def test_engram27b_concurrent_streams(torch, c27):
    """Slices of the batch run on three streams at once give Y bit-identical to
    one forward over the whole batch.  Kernels of other streams slow the
    placeholder h loads that the projection's value tiles issue in their last
    K stage; those loads land in LDS rows the value epilogue then writes, so
    the epilogue waits for them (without that wait, late loads overwrote
    pieces of v under this load)."""
    inp, dp, bufs, y_ref = c27
    for rep in range(4):
        y = _forward_on_streams(torch, dp, y_ref)
        bad = int((y != y_ref).reshape(dp.N, -1).any(dim=1).sum())
        print(f"  rep {rep}: tokens differing {bad}", flush=True)
        assert bad == 0


@pytest.fixture(scope="module")
def c40(torch):
    wl = synth.get_workload("engram40b")
    print("[engram40b] generating and uploading 18.5B table parameters", flush=True)
    inp, dp, bufs, y = _run_full(torch, wl)
    yield inp, dp, bufs, y
    del dp, bufs, y
    torch.cuda.empty_cache()


def test_engram40b_forward(torch, oracle_lib, c40):
    """Engram-40B scale (4 x 32768 tokens, 16 tables of ~9.03M x 128, d = 4096)
    on sampled positions, exact to the definition by locality."""
    inp, dp, bufs, y = c40
    err, a_err = _sampled_check(torch, oracle_lib, dp, inp, bufs, y, 4096, seed=13)
    print(f"  engram40b max-abs-err/max|ref| = {err:.3e}, alpha err {a_err:.2e}", flush=True)
    assert err <= TOL["bf16"], err
    assert a_err <= 1e-2


def test_widest_hidden_forward(torch, oracle_lib):
    """The widest hidden state the forward takes in bf16 (d = 8192: the gate +
    conv workgroup is 1024 lanes of 8 features), against the oracle at every
    position; the backward stops at d = 4096 and says so."""
    import hashed_gram_embedding_canon_amd as eg
    wl = dataclasses.replace(synth.get_workload("tiny"), name="tiny_wide", dtype="bf16",
                             hidden=8192).with_shape(1, 100)
    inp, dp, bufs, y = _run_full(torch, wl, saved=("idx", "stats", "k", "v"))
    p = H.oracle_problem(inp)
    ref = p.forward(want=("y", "alpha"))
    err = H.rel_max_err(H.to_host_f64(y).reshape(-1, wl.hidden), ref["y"])
    a_err = float(np.abs(bufs["stats"][:, 0].cpu().numpy() - ref["alpha"]).max())
    print(f"  d = 8192: max-abs-err/max|ref| = {err:.3e}, alpha err {a_err:.2e}", flush=True)
    assert err <= TOL["bf16"] and a_err <= 1e-2, (err, a_err)
    dy = H.to_dev(np.zeros((1, 100, wl.hidden), np.float32).astype(np.uint16))
    with pytest.raises(eg.EngramError, match="status 2"):
        dp.backward(bufs, dy, eg.ENGRAM_GRAD_SORTED_SPARSE)
