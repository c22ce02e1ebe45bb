"""Small float64 problems for the oracle pins (seeded through ``synth``)."""
import numpy as np

import synth


def small_problem(oracle, *, B=2, T=10, vocab=20, canon=15, orders=(2, 3), heads=2, D=4, d=8,
                  rows=None, taps=4, seed=4242, table_std=0.5, w_std=0.3, conv_std=0.5,
                  gammas=True, eps=1e-6, dtype="f64"):
    J = len(orders) * heads
    rows = list(rows) if rows is not None else synth.primes_from(7, J)
    s = seed
    tokens = (synth.u64_stream(s + 1, B * T) % np.uint64(vocab)).astype(np.int32).reshape(B, T)
    cmap = synth.random_surjection(s + 2, vocab, canon)
    mult = (synth.u64_stream(s + 3, J * max(orders)) | np.uint64(1)).reshape(J, max(orders))
    offs = np.concatenate([[0], np.cumsum(np.asarray(rows) * D)[:-1]])
    tables = [synth.normal_stream(s + 4, r * D, table_std, dtype, offset=int(o)).reshape(r, D)
              for r, o in zip(rows, offs)]
    d_mem = J * D
    w_k = synth.normal_stream(s + 5, d * d_mem, w_std, dtype).reshape(d, d_mem)
    w_v = synth.normal_stream(s + 6, d * d_mem, w_std, dtype).reshape(d, d_mem)
    h = synth.normal_stream(s + 7, B * T * d, 1.0, dtype).reshape(B, T, d)
    conv_w = synth.normal_stream(s + 8, d * taps, conv_std, "f64").reshape(d, taps)
    gq = gk = None
    if gammas:
        gq = 1.0 + 0.5 * synth.unit_stream(s + 10, d)
        gk = 1.0 + 0.5 * synth.unit_stream(s + 11, d)
    dy = synth.normal_stream(s + 9, B * T * d, 1.0, dtype).reshape(B, T, d)
    p = oracle.Problem(orders=orders, heads=heads, mult=mult, table_rows=rows, pad_id=0,
                       canon_map=cmap, tokens=tokens, tables=tables, w_k=w_k, w_v=w_v, h=h,
                       conv_w=conv_w, gamma_q=gq, gamma_k=gk, eps=eps)
    return p, dy
