"""Pins of the oracle's NTT/INTT: evaluation definition (Horner), convolution theorem, round trip, linearity."""
import numpy as np
import pytest

from oracle.chain import chain_primes, min_root
from oracle.ntt import intt, ntt, ntt_definition
from tests.bigint_helpers import brv, horner_eval, negacyclic_mul


def _setup(n, bits, count):
    qs = chain_primes(n, bits, count)
    return qs, [min_root(q, n) for q in qs]


@pytest.mark.parametrize("n,bits", [(16, 20), (16, 32), (64, 32), (256, 30), (1024, 32)])
def test_ntt_matches_evaluation_definition_every_index(n, bits):
    qs, psis = _setup(n, bits, 3)
    rng = np.random.default_rng(n + bits)
    a = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    a[0, :] = np.uint64(qs[0] - 1)  # all q-1 limb
    out = ntt(a, qs, psis)
    logn = n.bit_length() - 1
    for i, (q, psi) in enumerate(zip(qs, psis)):
        for j in range(n):
            x = pow(psi, 2 * brv(j, logn) + 1, q)
            assert int(out[i, j]) == horner_eval(a[i], x, q)


@pytest.mark.parametrize("n,bits,count", [(1 << 12, 30, 2), (1 << 16, 32, 2)])
def test_ntt_matches_evaluation_definition_sampled(n, bits, count):
    qs, psis = _setup(n, bits, count)
    rng = np.random.default_rng(5)
    a = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    out = ntt(a, qs, psis)
    logn = n.bit_length() - 1
    for i, (q, psi) in enumerate(zip(qs, psis)):
        for j in list(rng.integers(0, n, 24)) + [0, n - 1]:
            x = pow(psi, 2 * brv(int(j), logn) + 1, q)
            assert int(out[i, j]) == horner_eval(a[i], x, q)


@pytest.mark.parametrize("n,bits", [(16, 32), (64, 30), (256, 32)])
def test_convolution_theorem(n, bits):
    qs, psis = _setup(n, bits, 2)
    rng = np.random.default_rng(11)
    a = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    b = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    q = np.array(qs, dtype=np.uint64).reshape(-1, 1)
    prod = intt(ntt(a, qs, psis) * ntt(b, qs, psis) % q, qs, psis)
    for i, qq in enumerate(qs):
        assert prod[i].tolist() == negacyclic_mul(a[i], b[i], qq)


@pytest.mark.parametrize("n,bits,count", [(1 << 12, 30, 6), (1 << 16, 32, 4), (32, 32, 3)])
def test_round_trip_and_linearity(n, bits, count):
    qs, psis = _setup(n, bits, count)
    rng = np.random.default_rng(3)
    a = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    b = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    q = np.array(qs, dtype=np.uint64).reshape(-1, 1)
    assert np.array_equal(intt(ntt(a, qs, psis), qs, psis), a)
    assert np.array_equal(ntt(intt(a, qs, psis), qs, psis), a)
    assert np.array_equal(ntt((a + b) % q, qs, psis), (ntt(a, qs, psis) + ntt(b, qs, psis)) % q)


def test_ntt_special_inputs():
    n = 1 << 12
    qs, psis = _setup(n, 30, 2)
    # constant polynomial c maps to c everywhere; X maps to the evaluation points themselves
    a = np.zeros((2, n), dtype=np.uint64)
    a[:, 0] = 7
    assert np.all(ntt(a, qs, psis) == 7)
    a[:, 0] = 0
    a[:, 1] = 1
    out = ntt(a, qs, psis)
    for i, (q, psi) in enumerate(zip(qs, psis)):
        for j in (0, 1, 2, n - 1):
            assert int(out[i, j]) == pow(psi, 2 * brv(j, 12) + 1, q)
    # batch dimension is independent
    rng = np.random.default_rng(0)
    x = np.stack([np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs]) for _ in range(3)])
    assert np.array_equal(ntt(x, qs, psis)[1], ntt(x[1], qs, psis))


@pytest.mark.parametrize("n,bits", [(16, 20), (64, 32), (128, 30)])
def test_ntt_definition_matches_horner_every_index(n, bits):
    # the O(N^2) definition (a table of powers of psi) against Horner evaluation in Python integers
    qs, psis = _setup(n, bits, 2)
    rng = np.random.default_rng(n)
    logn = n.bit_length() - 1
    for q, psi in zip(qs, psis):
        a = rng.integers(0, q, n, dtype=np.uint64)
        a[-1] = q - 1
        out = ntt_definition(a, q, psi)
        for j in range(n):
            assert int(out[j]) == horner_eval(a, pow(psi, 2 * brv(j, logn) + 1, q), q)


@pytest.mark.parametrize("n,bits,count", [(16, 32, 3), (256, 30, 2), (1024, 32, 2), (4096, 30, 1)])
def test_fast_ntt_equals_definition_every_index(n, bits, count):
    # merged-twist Cooley-Tukey reaches the definition's values, every index, up to N = 2^12
    qs, psis = _setup(n, bits, count)
    rng = np.random.default_rng(n + count)
    a = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    fast = ntt(a, qs, psis)
    for i, (q, psi) in enumerate(zip(qs, psis)):
        assert np.array_equal(fast[i], ntt_definition(a[i], q, psi)), i
