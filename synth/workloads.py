"""Workload shapes: the tiny fp32 case, the small bf16 model, the Engram-27B
scale (forward and backward), the Engram-40B scale and the host-resident
100B-parameter table.  Sizes only; the arrays come from ``synth.Inputs``."""
from __future__ import annotations

from dataclasses import dataclass, field, replace


@dataclass(frozen=True)
class Workload:
    name: str
    cfg: int              # index that seeds the streams (seed = 1000*cfg + stream)
    canon_cfg: int        # index that seeds the canonical surjection
    B: int
    T: int
    vocab: int
    canon_vocab: int
    zipf_s: float
    orders: tuple
    heads: int
    dim: int              # D, columns per table row
    dtype: str            # 'f32' or 'bf16' for tables, weights, hidden, output
    rows: tuple           # prime row count of each table, j = order_idx*heads + head
    hidden: int           # d
    taps: int = 4
    table_std: float = 0.02
    w_std: float = 0.0    # 0 -> 1/sqrt(d_mem)
    conv_std: float = 0.5
    rms_eps: float = 1e-6
    pad_id: int = 0
    branches: int = 1     # M residual branches (own W_K and hidden state each)
    note: str = field(default="", compare=False)

    @property
    def J(self) -> int:
        return len(self.orders) * self.heads

    @property
    def max_order(self) -> int:
        return max(self.orders)

    @property
    def d_mem(self) -> int:
        return self.J * self.dim

    @property
    def n_tokens(self) -> int:
        return self.B * self.T

    @property
    def table_params(self) -> int:
        return sum(self.rows) * self.dim

    def with_shape(self, B: int, T: int) -> "Workload":
        return replace(self, B=B, T=T)

    def __post_init__(self):
        if self.w_std == 0.0:
            object.__setattr__(self, "w_std", self.d_mem ** -0.5)


def primes_from(start: int, count: int) -> list[int]:
    """The first `count` primes >= start (trial division)."""
    out = []
    n = max(2, start)
    while len(out) < count:
        if n < 4:
            ok = n >= 2
        elif n % 2 == 0:
            ok = False
        else:
            ok = True
            f = 3
            while f * f <= n:
                if n % f == 0:
                    ok = False
                    break
                f += 2
        if ok:
            out.append(n)
        n += 1
    return out


def _primes(start, count):
    return tuple(primes_from(start, count))


def _mk():
    out = {}
    out["tiny"] = Workload(
        name="tiny", cfg=0, canon_cfg=0, B=1, T=512, vocab=4096, canon_vocab=3200, zipf_s=1.1,
        orders=(2, 3), heads=4, dim=32, dtype="f32", rows=(10007,) * 8, hidden=256,
        note="tiny fp32 forward: 1x512 tokens, 8 tables of 10007x32")
    out["small"] = Workload(
        name="small", cfg=1, canon_cfg=1, B=8, T=4096, vocab=131072, canon_vocab=100930, zipf_s=1.0,
        orders=(2, 3), heads=8, dim=64, dtype="bf16", rows=_primes(7_812_500, 16), hidden=2048,
        note="small-model bf16 forward: 8x4096 tokens, 16 tables of ~7.81M x 64")
    out["engram27b"] = Workload(
        name="engram27b", cfg=2, canon_cfg=1, B=32, T=4096, vocab=131072, canon_vocab=100930,
        zipf_s=1.0, orders=(2, 3), heads=8, dim=80, dtype="bf16", rows=_primes(4_450_000, 16),
        hidden=2560, note="Engram-27B scale: 5.7B bf16 table params, 32x4096 tokens")
    out["engram27b_bwd"] = replace(out["engram27b"], name="engram27b_bwd", cfg=3,
                                   note="Engram-27B scale forward + table-gradient backward")
    out["engram40b"] = Workload(
        name="engram40b", cfg=4, canon_cfg=1, B=4, T=32768, vocab=131072, canon_vocab=100930,
        zipf_s=1.0, orders=(2, 3), heads=8, dim=128, dtype="bf16", rows=_primes(9_030_000, 16),
        hidden=4096, note="Engram-40B scale: 18.5B bf16 table params, 4x32768 tokens")
    out["host100b"] = replace(out["engram40b"], name="host100b", rows=_primes(48_800_000, 16),
                              note="100B-parameter bf16 table in pinned host memory")
    return out


WORKLOADS = _mk()


def get_workload(name: str) -> Workload:
    return WORKLOADS[name]
