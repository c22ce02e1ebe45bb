"""Device-side set-up shared by the GPU tests and the bench: uploads the
seeded ``synth`` arrays and calls the library through its binding."""
from __future__ import annotations

import numpy as np

import synth


def torch_mod():
    import torch
    return torch


def to_dev(a: np.ndarray, device="cuda"):
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def to_host_f64(t) -> np.ndarray:
    torch = torch_mod()
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


class DeviceProblem:
    """One workload on the GPU: config, parameters, tokens and hidden states."""

    def __init__(self, inp: synth.Inputs, device="cuda", upload_tables=True, tokens=None, flags=0):
        import hashed_gram_embedding_canon_amd as eg
        torch = torch_mod()
        self.eg = eg
        wl = inp.wl
        self.wl, self.inp, self.device = wl, inp, device
        self.dtype_code = eg.ENGRAM_BF16 if wl.dtype == "bf16" else eg.ENGRAM_F32
        self.tdtype = torch.bfloat16 if wl.dtype == "bf16" else torch.float32
        self.cfg = eg.Config(vocab=wl.vocab, canon_vocab=wl.canon_vocab, orders=wl.orders,
                             heads=wl.heads, dim=wl.dim, hidden=wl.hidden,
                             table_rows=inp.table_rows, multipliers=inp.multipliers,
                             dtype=self.dtype_code, conv_kernel=wl.taps, rms_eps=wl.rms_eps,
                             pad_id=wl.pad_id, flags=flags, branches=wl.branches)
        self.tokens_host = np.ascontiguousarray(inp.tokens if tokens is None else tokens, dtype=np.int32)
        self.B, self.T = self.tokens_host.shape
        self.tokens = to_dev(self.tokens_host, device)
        self.canon = to_dev(inp.canon_map, device)
        self.tables = [to_dev(inp.table(j), device) for j in range(wl.J)] if upload_tables else []
        M = self.M = wl.branches
        self.w_kv = torch.cat([to_dev(inp.w_k_branch(m), device) for m in range(M)]
                              + [to_dev(inp.w_v, device)], 0).contiguous()
        self.conv_w = to_dev(inp.conv_w, device)
        hids = []
        for m in range(M):
            hid = inp.hidden_branch(m)
            hids.append(hid if tokens is None else hid[: self.B, : self.T])
        hid = hids[0] if M == 1 else np.stack(hids)
        self.hidden = to_dev(np.ascontiguousarray(hid), device)
        self.params = eg.make_params(canon_map=self.canon, tables=self.tables, w_kv=self.w_kv,
                                     conv_w=self.conv_w)

    @property
    def N(self):
        return self.B * self.T

    def workspace(self, op):
        torch = torch_mod()
        n = self.eg.engram_workspace_size(self.cfg, self.B, self.T, op)
        return torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)

    def alloc_saved(self, want=("idx", "stats", "k", "v", "e")):
        torch = torch_mod()
        wl, N = self.wl, self.N
        bufs = {}
        if "idx" in want:
            bufs["idx"] = torch.empty(N, wl.J, dtype=torch.int32, device=self.device)
        lead = (N,) if self.M == 1 else (self.M, N)
        if "stats" in want:
            bufs["stats"] = torch.empty(*lead, 4, dtype=torch.float32, device=self.device)
        if "k" in want:
            bufs["k"] = torch.empty(*lead, wl.hidden, dtype=self.tdtype, device=self.device)
        if "v" in want:
            bufs["v"] = torch.empty(N, wl.hidden, dtype=self.tdtype, device=self.device)
        if "e" in want:
            bufs["e"] = torch.empty(N, wl.d_mem, dtype=self.tdtype, device=self.device)
        return bufs

    def forward(self, saved_bufs=None, compact=None, ws=None, y=None):
        torch = torch_mod()
        eg = self.eg
        if y is None:
            lead = (self.B, self.T) if self.M == 1 else (self.M, self.B, self.T)
            y = torch.empty(*lead, self.wl.hidden, dtype=self.tdtype, device=self.device)
        if ws is None:
            ws = self.workspace(eg.ENGRAM_OP_FORWARD)
        saved = eg.make_saved(**saved_bufs) if saved_bufs else None
        eg.engram_forward(self.cfg, self.params, self.tokens, self.hidden, y, B=self.B, T=self.T,
                          saved=saved, compact=compact, workspace=ws)
        return y

    def hash(self):
        torch = torch_mod()
        idx = torch.empty(self.N, self.wl.J, dtype=torch.int32, device=self.device)
        self.eg.engram_hash_indices(self.cfg, self.canon, self.tokens, idx, B=self.B, T=self.T)
        return idx

    def backward(self, saved_bufs, dy, mode, ws=None):
        """Returns dict: sparse -> keys, rows, count; dense -> list of [M_j, D] fp32 tensors."""
        torch = torch_mod()
        eg = self.eg
        wl = self.wl
        out = eg.engram_table_grad()
        out.mode = mode
        res = {}
        if mode == eg.ENGRAM_GRAD_SORTED_SPARSE:
            cap = self.N * wl.J
            res["keys"] = torch.empty(max(cap, 1), dtype=torch.int64, device=self.device)
            res["rows"] = torch.empty(max(cap, 1), wl.dim, dtype=torch.float32, device=self.device)
            res["count"] = torch.zeros(1, dtype=torch.int64, device=self.device)
            out.keys, out.rows, out.count = (res["keys"].data_ptr(), res["rows"].data_ptr(),
                                             res["count"].data_ptr())
        else:
            res["dense"] = [torch.zeros(int(m), wl.dim, dtype=torch.float32, device=self.device)
                            for m in self.inp.table_rows]
            for j, t in enumerate(res["dense"]):
                out.dense[j] = t.data_ptr()
        if ws is None:
            ws = self.workspace(eg.ENGRAM_OP_BACKWARD)
        eg.engram_backward_table_grad(self.cfg, self.params, self.hidden, dy, B=self.B, T=self.T,
                                      saved=eg.make_saved(**saved_bufs), out=out, workspace=ws)
        return res


    def backward_params(self, saved_bufs, dy, want=("w_kv", "conv_w", "gamma_q", "gamma_k", "hidden"),
                        ws=None):
        """engram_backward with parameter gradients only -> dict of tensors."""
        torch = torch_mod()
        eg, wl = self.eg, self.wl
        d, M = wl.hidden, self.M
        lead = () if M == 1 else (M,)
        shapes = {"w_kv": (((M + 1) * d, wl.d_mem), torch.float32),
                  "conv_w": ((d, wl.taps), torch.float32),
                  "gamma_q": (lead + (d,), torch.float32), "gamma_k": (lead + (d,), torch.float32),
                  "hidden": (lead + (self.B, self.T, d), self.tdtype)}
        res = {k: torch.full(shapes[k][0], float("nan"), dtype=shapes[k][1], device=self.device)
               for k in want}
        pg = eg.make_param_grad(**res)
        if ws is None:
            ws = self.workspace(eg.ENGRAM_OP_BACKWARD_PARAMS)
        eg.engram_backward(self.cfg, self.params, self.hidden, dy, B=self.B, T=self.T,
                           saved=eg.make_saved(**saved_bufs), param_out=pg, workspace=ws)
        return res


def oracle_problem(inp: synth.Inputs, tokens=None, hidden=None, branch=0):
    """The oracle's problem for one branch: its W_K and hidden state, the shared
    tables, W_V and conv."""
    import oracle
    over = {}
    if tokens is not None:
        over["tokens"] = tokens
    if hidden is not None:
        over["h"] = hidden
    elif branch:
        over["h"] = inp.hidden_branch(branch)
    if branch:
        over["w_k"] = oracle.widen(inp.w_k_branch(branch))
    return oracle.Problem.from_inputs(inp, **over)


def rel_max_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / max |ref|"""
    den = np.abs(ref).max()
    return float(np.abs(got - ref).max() / (den if den > 0 else 1.0))


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def sample_positions(B: int, T: int, n: int, seed: int = 7) -> np.ndarray:
    """Sorted distinct flat positions: every sequence start and end, plus seeded picks."""
    fixed = set()
    for b in range(B):
        for t in (0, 1, 2, 3, T - 1):
            if 0 <= t < T:
                fixed.add(b * T + t)
    picks = synth.u64_stream(seed, 4 * n) % np.uint64(max(B * T, 1))
    out = list(fixed)
    for p in picks:
        if len(out) >= max(n, len(fixed)):
            break
        out.append(int(p))
    return np.unique(np.asarray(out, dtype=np.int64))
