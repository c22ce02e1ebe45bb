"""Pins of the oracle's canonicalisation and multi-head hash.

The pages ("DeepSeek AI II", section "DeepSeek Engram") fix: raw ids are
mapped by a surjection to canonical ids; the suffix N-gram of canonical ids
is hashed by K independent multiply-XOR heads per order into tables of
prime size; retrieval depends on the token ids only.  Checked here against
hand-derived values, Python big-integer brute force, and invariants.
"""
import os

import numpy as np
import pytest

import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hash_hand.txt")
M64 = 1 << 64


def _single(oracle, M, m, cs, order):
    """idx at the last position of a one-sequence problem holding ids cs (oldest first)."""
    vocab = max(cs) + 1
    tokens = np.asarray([cs], dtype=np.int32)
    mult = np.asarray([m], dtype=np.uint64)
    tab = np.zeros((M, 1), np.float32)
    p = oracle.Problem(orders=(order,), heads=1, mult=mult, table_rows=[M], pad_id=0,
                       canon_map=np.arange(vocab, dtype=np.int32), tokens=tokens, tables=[tab])
    return int(p.hash(np.asarray([len(cs) - 1]))[0, 0])


def test_hand_derived_values(oracle_lib):
    rows = [ln.split() for ln in open(GOLDEN) if ln.strip() and not ln.startswith("#")]
    assert len(rows) == 7
    for M, m0, m1, m2, c0, c1, c2, order, want in rows:
        M, order, want = int(M), int(order), int(want)
        m = [int(m0), int(m1), int(m2)]
        cs = [int(c2), int(c1), int(c0)][3 - order:]
        assert _single(oracle_lib, M, m, cs, order) == want


def test_modulus_fixture_arithmetic():
    # 2^64 mod 10007 = 3798 by Python's modular exponentiation
    assert pow(2, 64, 10007) == 3798
    assert pow(2, 12, 13) == 1


def _bigint_hash(mult_row, cs_newest_first, M):
    x = 0
    for m, c in zip(mult_row, cs_newest_first):
        x ^= (int(m) * int(c)) % M64
    return x % M


def test_brute_force_tiny_vocab(oracle_lib):
    """All 2- and 3-grams over 8 canonical ids (plus padding) vs big-int arithmetic."""
    V = 8
    heads = 3
    orders = (2, 3)
    J = len(orders) * heads
    rows = synth.primes_from(11, J)
    mult = (synth.u64_stream(777, J * 3) | np.uint64(1)).reshape(J, 3)
    # one sequence per trigram (a, b, c): positions 0,1,2 see (pad,pad,a), (pad,a,b), (a,b,c)
    grams = np.array([(a, b, c) for a in range(V) for b in range(V) for c in range(V)], np.int32)
    tokens = grams  # [512, 3]
    tabs = [np.zeros((r, 1), np.float32) for r in rows]
    pad = 5
    p = oracle_lib.Problem(orders=orders, heads=heads, mult=mult, table_rows=rows, pad_id=pad,
                           canon_map=np.arange(V, dtype=np.int32), tokens=tokens, tables=tabs)
    idx = p.hash().reshape(len(grams), 3, J)
    for s, (a, b, c) in enumerate(grams):
        ctx = {0: [a, pad, pad], 1: [b, a, pad], 2: [c, b, a]}  # newest first
        for t in range(3):
            j = 0
            for n in orders:
                for _ in range(heads):
                    want = _bigint_hash(mult[j, :n], ctx[t][:n], rows[j])
                    assert idx[s, t, j] == want, (s, t, j)
                    j += 1


def _tiny_problem(oracle, B=4, T=256):
    wl = synth.get_workload("tiny").with_shape(B, T)
    inp = synth.Inputs(wl)
    return wl, inp, oracle.Problem(orders=wl.orders, heads=wl.heads, mult=inp.multipliers,
                                   table_rows=inp.table_rows, pad_id=wl.pad_id,
                                   canon_map=inp.canon_map, tokens=inp.tokens, tables=inp.tables)


def test_range_and_prime_sizes(oracle_lib):
    import sympy
    wl, inp, p = _tiny_problem(oracle_lib)
    idx = p.hash()
    assert idx.min() >= 0
    assert (idx < inp.table_rows[None, :]).all()
    for m in inp.table_rows:
        assert sympy.isprime(int(m))


def test_identical_ngrams_identical_slots(oracle_lib):
    """Deterministic addressing: equal canonical suffix N-grams give equal indices."""
    wl, inp, p = _tiny_problem(oracle_lib, B=4, T=512)
    canon = inp.canon_map[inp.tokens]
    idx = p.hash().reshape(wl.B, wl.T, wl.J)
    seen = {}
    hits = 0
    for b in range(wl.B):
        for t in range(wl.T):
            ctx = tuple(int(canon[b, t - i]) if t - i >= 0 else wl.pad_id for i in range(3))
            j = 0
            for n in wl.orders:
                key = (n, ctx[:n])
                cur = tuple(idx[b, t, j:j + wl.heads])
                if key in seen:
                    assert seen[key] == cur
                    hits += 1
                else:
                    seen[key] = cur
                j += wl.heads
    assert hits > 100  # Zipf streams repeat short N-grams


def test_canonical_equivalence(oracle_lib):
    """Raw ids with the same canonical id address the same rows."""
    wl, inp, p = _tiny_problem(oracle_lib, B=1, T=64)
    cmap = inp.canon_map
    tok = inp.tokens.copy()
    # replace every token by another raw id with the same canonical id, where one exists
    by_canon = {}
    for raw, c in enumerate(cmap):
        by_canon.setdefault(int(c), []).append(raw)
    swapped = 0
    for t in range(tok.shape[1]):
        alts = [r for r in by_canon[int(cmap[tok[0, t]])] if r != tok[0, t]]
        if alts:
            tok[0, t] = alts[0]
            swapped += 1
    assert swapped > 5
    q = oracle_lib.Problem(orders=wl.orders, heads=wl.heads, mult=inp.multipliers,
                           table_rows=inp.table_rows, pad_id=wl.pad_id, canon_map=cmap,
                           tokens=tok, tables=inp.tables)
    assert (q.hash() == p.hash()).all()


def test_order_sensitivity_and_padding(oracle_lib):
    """(a,b) and (b,a) differ for the sampled multipliers; position 0 sees the pad id."""
    V = 64
    mult = (synth.u64_stream(99, 3) | np.uint64(1)).reshape(1, 3)
    M = 1000003
    tab = [np.zeros((M, 1), np.float32)]
    ident = np.arange(V, dtype=np.int32)
    diff = 0
    for a in range(1, V):
        b = (a * 7) % V
        if a == b:
            continue
        pa = oracle_lib.Problem(orders=(2,), heads=1, mult=mult, table_rows=[M], pad_id=0,
                                canon_map=ident, tokens=np.array([[a, b], [b, a]], np.int32), tables=tab)
        i = pa.hash(np.array([1, 3]))
        diff += int(i[0, 0] != i[1, 0])
    assert diff >= 60
    # padding: position 0 of [x, ...] equals position 1 of [pad, x, ...]
    pad = 17
    seq = np.array([[9, 4, 33]], np.int32)
    seq2 = np.array([[pad, 9, 4, 33]], np.int32)
    for order in (2, 3):
        p1 = oracle_lib.Problem(orders=(order,), heads=1, mult=mult, table_rows=[M], pad_id=pad,
                                canon_map=ident, tokens=seq, tables=tab)
        p2 = oracle_lib.Problem(orders=(order,), heads=1, mult=mult, table_rows=[M], pad_id=pad,
                                canon_map=ident, tokens=seq2 if order == 2 else np.array([[pad, pad, 9, 4, 33]], np.int32),
                                tables=tab)
        off = 1 if order == 2 else 2
        assert p1.hash(np.array([0]))[0, 0] == p2.hash(np.array([off]))[0, 0]


def test_heads_spread_uniformly(oracle_lib):
    """Distinct bigrams land near-uniformly in a small prime table (chi-square)."""
    V = 128
    M = 101
    mult = (synth.u64_stream(5, 3) | np.uint64(1)).reshape(1, 3)
    grams = np.array([(a, b) for a in range(V) for b in range(V)], np.int32)
    p = oracle_lib.Problem(orders=(2,), heads=1, mult=mult, table_rows=[M], pad_id=0,
                           canon_map=np.arange(V, dtype=np.int32), tokens=grams,
                           tables=[np.zeros((M, 1), np.float32)])
    idx = p.hash(np.arange(len(grams)) * 2 + 1)[:, 0]
    counts = np.bincount(idx, minlength=M)
    exp = len(grams) / M
    chi2 = ((counts - exp) ** 2 / exp).sum()
    assert chi2 < 200  # dof 100; a biased hash gives thousands
