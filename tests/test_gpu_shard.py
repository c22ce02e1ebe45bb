"""Table-sharded row exchange on one GPU: G GPUs are emulated in one process
(each with its own batch of the token stream; the All-to-All is a device copy
between their buffers, the RCCL transfer the library leaves to its caller).

Bit-exact: the send order and inverse map against their plain definition
(numpy), every GPU's forward over the rows served by the owners against the
forward over the whole tables, and each owner's summed gradient against the
same per-GPU gradient rows added in the same order.  The summed gradient
also matches the oracle's at sampled rows (relative L2 <= 1e-3).
"""
import dataclasses

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


def _shard_rows(table_rows, G):
    return [(int(m) + G - 1) // G for m in table_rows]


def _requests(torch, dp, idx, G, N=None):
    import hashed_gram_embedding_canon_amd as eg
    N, J = dp.N if N is None else N, dp.wl.J
    send_ids = torch.empty(max(N * J, 1), dtype=torch.int32, device="cuda")
    counts = torch.empty(G, dtype=torch.int64, device="cuda")
    inverse = torch.empty(N, J, dtype=torch.int32, device="cuda")
    ws = torch.empty(eg.engram_workspace_size(dp.cfg, 1, N, eg.ENGRAM_OP_SHARD), dtype=torch.uint8,
                     device="cuda")
    eg.engram_shard_requests(dp.cfg, G, idx, N, send_ids, counts, inverse, workspace=ws)
    return send_ids, counts, inverse


def _reference_order(idx, table_rows, G):
    """The send order by its definition: distinct (table, row) keys sorted by
    (owner, table, row); ids (j << 27) | (row - owner * S_j); inverse = the
    position of each token's key."""
    N, J = idx.shape
    S = _shard_rows(table_rows, G)
    keys = np.unique((np.arange(J, dtype=np.int64)[None, :] << 32) | idx.astype(np.int64))
    j = keys >> 32
    row = keys & 0xFFFFFFFF
    owner = row // np.asarray(S, np.int64)[j]
    order = np.lexsort((row, j, owner))
    ids = ((j[order] << 27) | (row[order] - owner[order] * np.asarray(S, np.int64)[j[order]])).astype(np.uint32)
    counts = np.bincount(owner, minlength=G)
    pos = np.empty(keys.size, np.int64)
    pos[order] = np.arange(keys.size)
    tok = (np.arange(J, dtype=np.int64)[None, :] << 32) | idx.astype(np.int64)
    inverse = pos[np.searchsorted(keys, tok)]
    return ids, counts, inverse


@pytest.mark.parametrize("name,B,T,G,rows", [("tiny", 2, 300, 1, None), ("tiny", 2, 300, 3, None),
                                              ("small", 2, 2048, 8, None), ("tiny", 2, 300, 3, 251)])
def test_requests_match_definition(torch, name, B, T, G, rows):
    wl = synth.get_workload(name).with_shape(B, T)
    if rows is not None:  # one 8-bit digit pass sorts the row ids
        wl = dataclasses.replace(wl, rows=(rows,) * wl.J)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    idx = dp.hash()
    send_ids, counts, inverse = _requests(torch, dp, idx, G)
    torch.cuda.synchronize()
    ids_ref, counts_ref, inv_ref = _reference_order(idx.cpu().numpy(), inp.table_rows, G)
    assert np.array_equal(counts.cpu().numpy(), counts_ref)
    assert np.array_equal(send_ids[: ids_ref.size].cpu().numpy().view(np.uint32), ids_ref)
    assert np.array_equal(inverse.cpu().numpy(), inv_ref)


def test_requests_many_sort_blocks(torch):
    """300001 tokens of seeded row ids (more than 64 sort blocks per table):
    send order, counts and inverse map exact."""
    wl = synth.get_workload("tiny").with_shape(1, 300)
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    N, J, G = 300_001, wl.J, 3
    rows = np.asarray(inp.table_rows, np.uint64)
    u = synth.u64_stream(31, N * J).reshape(N, J)
    # half the tokens on 64 rows per table, half anywhere: long and short segments
    hot = (u >> np.uint64(40)) % np.uint64(2) == 0
    idx = np.where(hot, u % np.uint64(64), u % rows[None, :]).astype(np.int32)
    print(f"[shard requests] N={N} J={J} G={G}", flush=True)
    send_ids, counts, inverse = _requests(torch, dp, H.to_dev(idx), G, N)
    torch.cuda.synchronize()
    ids_ref, counts_ref, inv_ref = _reference_order(idx, inp.table_rows, G)
    assert np.array_equal(counts.cpu().numpy(), counts_ref)
    assert np.array_equal(send_ids[: ids_ref.size].cpu().numpy().view(np.uint32), ids_ref)
    assert np.array_equal(inverse.cpu().numpy(), inv_ref)


def _emulate(torch, wl, G, backward=False):
    """G GPUs, GPU r with stream batch r; returns per-GPU results."""
    import hashed_gram_embedding_canon_amd as eg
    inp = synth.Inputs(wl)
    dp = H.DeviceProblem(inp)
    N, J = dp.N, wl.J
    es = 2 if wl.dtype == "bf16" else 4
    rb = wl.dim * es
    S = _shard_rows(inp.table_rows, G)
    # GPU g's shard of table j: rows [g S_j, (g+1) S_j) of the full device table (a view)
    shards = [[dp.tables[j].view(-1)[g * S[j] * wl.dim: min((g + 1) * S[j], int(inp.table_rows[j])) * wl.dim]
               for j in range(J)] for g in range(G)]
    ranks = []
    for r in range(G):
        tok = synth.zipf_tokens(synth.seed_of(wl.cfg, synth.S_TOKENS), N, wl.vocab, wl.zipf_s,
                                offset=r * N).reshape(dp.B, dp.T)
        dp.tokens_host, dp.tokens = tok, H.to_dev(tok)
        saved = dp.alloc_saved(("idx", "stats", "k", "v"))
        y_ref = dp.forward(saved)
        send_ids, counts, inverse = _requests(torch, dp, saved["idx"], G)
        ranks.append({"tok": tok, "saved": saved, "y_ref": y_ref, "send_ids": send_ids,
                      "counts": counts.cpu().numpy(), "inverse": inverse})
    offs = [np.concatenate([[0], np.cumsum(rk["counts"])]) for rk in ranks]
    # All-to-All of requests: owner o receives block o of every GPU, in GPU order
    replies = []
    for o in range(G):
        recv = torch.cat([rk["send_ids"][offs[r][o]: offs[r][o + 1]] for r, rk in enumerate(ranks)])
        out = torch.empty(max(recv.numel(), 1) * rb, dtype=torch.uint8, device="cuda")
        eg.engram_shard_serve(dp.cfg, G, shards[o], recv, recv.numel(), out)
        replies.append((out, [int(rk["counts"][o]) for rk in ranks]))
    # All-to-All of replies: GPU r receives its block from every owner, in owner order
    for r, rk in enumerate(ranks):
        parts = []
        for o, (out, cnt) in enumerate(replies):
            start = sum(cnt[:r])
            parts.append(out[start * rb:(start + cnt[r]) * rb])
        rows = torch.cat(parts) if parts else torch.empty(0, dtype=torch.uint8, device="cuda")
        plan = eg.engram_compact()
        plan.rows_dev, plan.inverse_dev = rows.data_ptr(), rk["inverse"].data_ptr()
        rk["rows"] = rows
        dp.tokens_host, dp.tokens = rk["tok"], H.to_dev(rk["tok"])
        rk["y"] = dp.forward(compact=plan)
    if backward:
        D = wl.dim
        dy = H.to_dev(inp.dy)
        sg = [[torch.zeros(S[j] * D, dtype=torch.float32, device="cuda") for j in range(J)]
              for _ in range(G)]
        dense_ref = [torch.zeros(int(m), D, dtype=torch.float32, device="cuda") for m in inp.table_rows]
        ws = torch.empty(eg.engram_workspace_size(dp.cfg, 1, 1, eg.ENGRAM_OP_SHARD), dtype=torch.uint8,
                         device="cuda")
        for r, rk in enumerate(ranks):
            dp.tokens_host, dp.tokens = rk["tok"], H.to_dev(rk["tok"])
            sp = dp.backward(rk["saved"], dy, eg.ENGRAM_GRAD_SORTED_SPARSE)
            # the same rows added into whole dense tables, GPU after GPU
            out = eg.engram_table_grad()
            out.mode = eg.ENGRAM_GRAD_SORTED_DENSE
            for j, t in enumerate(dense_ref):
                out.dense[j] = t.data_ptr()
            eg.engram_backward_table_grad(dp.cfg, dp.params, dp.hidden, dy, B=dp.B, T=dp.T,
                                          saved=eg.make_saved(**rk["saved"]), out=out,
                                          workspace=dp.workspace(eg.ENGRAM_OP_BACKWARD))
            cap = N * J
            gids = torch.empty(cap, dtype=torch.int32, device="cuda")
            grows = torch.empty(cap, D, dtype=torch.float32, device="cuda")
            gcounts = torch.empty(G, dtype=torch.int64, device="cuda")
            eg.engram_shard_grads(dp.cfg, G, sp["keys"], sp["rows"], sp["count"], cap, gids, grows,
                                  gcounts, workspace=ws)
            rk["gids"], rk["grows"], rk["gcounts"] = gids, grows, gcounts.cpu().numpy()
        for o in range(G):
            blocks = []
            for rk in ranks:
                g0 = int(np.sum(rk["gcounts"][:o]))
                blocks.append((rk["gids"][g0: g0 + rk["gcounts"][o]], rk["grows"][g0: g0 + rk["gcounts"][o]]))
            ids = torch.cat([b[0] for b in blocks])
            rows = torch.cat([b[1] for b in blocks]).contiguous()
            eg.engram_shard_reduce(dp.cfg, G, sg[o], ids, rows, [b[0].numel() for b in blocks])
        torch.cuda.synchronize()
        return inp, dp, ranks, S, sg, dense_ref
    torch.cuda.synchronize()
    return inp, dp, ranks


@pytest.mark.parametrize("name,B,T,G", [("tiny", 2, 300, 3), ("small", 2, 2048, 4)])
def test_sharded_forward_bit_identical(torch, name, B, T, G):
    wl = synth.get_workload(name).with_shape(B, T)
    print(f"[shard fwd {name}] B={B} T={T} G={G}", flush=True)
    inp, dp, ranks = _emulate(torch, wl, G)
    for r, rk in enumerate(ranks):
        assert torch.equal(rk["y"], rk["y_ref"]), r


@pytest.mark.parametrize("dtype,G", [("f32", 3), ("bf16", 4)])
def test_sharded_table_grads(torch, oracle_lib, dtype, G):
    wl = dataclasses.replace(synth.get_workload("tiny"), dtype=dtype).with_shape(2, 300)
    print(f"[shard bwd {dtype}] G={G}", flush=True)
    inp, dp, ranks, S, sg, dense_ref = _emulate(torch, wl, G, backward=True)
    D = wl.dim
    for o in range(G):
        for j in range(wl.J):
            lo, hi = o * S[j], min((o + 1) * S[j], int(inp.table_rows[j]))
            got = sg[o][j].view(S[j], D)[: hi - lo]
            assert torch.equal(got, dense_ref[j][lo:hi]), (o, j)
    # oracle at sampled rows: the sum over the GPUs' batches
    import oracle
    rng = np.random.default_rng(3)
    rj, rr = [], []
    idx_all = [oracle.Problem.from_inputs(inp, tokens=rk["tok"]).hash() for rk in ranks]
    for _ in range(24):
        j = int(rng.integers(wl.J))
        r = int(idx_all[int(rng.integers(G))][int(rng.integers(dp.N)), j])
        rj.append(j)
        rr.append(r)
    ref = np.zeros((len(rj), D))
    for rk, idx in zip(ranks, idx_all):
        p = oracle.Problem.from_inputs(inp, tokens=rk["tok"])
        out, _ = p.table_grad_rows(inp.dy, idx, rj, rr)
        ref += out
    got = np.stack([dense_ref[j][r].cpu().numpy().astype(np.float64) for j, r in zip(rj, rr)])
    err = H.rel_l2(got, ref)
    print(f"  rel L2 vs oracle {err:.2e}", flush=True)
    assert err <= 1e-3, err
