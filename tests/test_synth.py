"""Checks of the seeded input generators against their published definitions."""
import numpy as np

import synth


def test_splitmix64_reference_vector():
    # splitmix64 from state 0 (Steele, Lea, Flood 2014; Vigna's reference code)
    got = [int(x) for x in synth.u64_stream(0, 3)]
    assert got == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def test_element_indexing_and_offsets():
    a = synth.u64_stream(12345, 100)
    b = synth.u64_stream(12345, 40, offset=60)
    assert np.array_equal(a[60:], b)
    n = synth.normal_stream(7, 50, 1.0, "f64")
    assert np.array_equal(n[10:], synth.normal_stream(7, 40, 1.0, "f64", offset=10))


def test_normal_moments_and_bf16_rounding():
    x = synth.normal_stream(3, 200000, 0.02, "f64")
    assert abs(x.mean()) < 3e-4 and abs(x.std() - 0.02) < 3e-4
    f = synth.normal_stream(3, 1000, 0.02, "f32")
    bf = synth.normal_stream(3, 1000, 0.02, "bf16")
    assert np.array_equal(bf, synth.f32_to_bf16(f))
    w = synth.bf16_to_f32(bf)
    assert np.all(np.abs(w - f) <= np.abs(f) * 2.0 ** -8)


def test_zipf_frequencies():
    V, s = 64, 1.0
    x = synth.zipf_tokens(11, 400000, V, s)
    assert x.min() >= 0 and x.max() < V
    p = np.arange(1, V + 1, dtype=np.float64) ** -s
    p /= p.sum()
    counts = np.bincount(x, minlength=V)
    chi2 = ((counts - p * x.size) ** 2 / (p * x.size)).sum()
    assert chi2 < 120  # dof 63


def test_surjection():
    m = synth.random_surjection(5, 4096, 3200)
    assert m.min() >= 0 and m.max() < 3200
    assert np.unique(m).size == 3200  # every canonical id has a preimage
    assert 1 - 100930 / 131072 > 0.22  # the configured reduction is about 23 %


def test_primes():
    import sympy
    assert not sympy.isprime(7812503) and 17 * 181 * 2539 == 7812503
    ps = synth.primes_from(4_450_000, 16)
    assert all(sympy.isprime(q) for q in ps)
    assert ps[0] == sympy.nextprime(4_450_000 - 1)
    for a, b in zip(ps, ps[1:]):
        assert sympy.nextprime(a) == b
    assert sympy.isprime(10007)
