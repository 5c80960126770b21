"""Pins of the oracle's Galois automorphisms: ring homomorphism, composition, NTT-domain form."""
import numpy as np
import pytest

from oracle.automorph import automorph_coeff, automorph_ntt, ntt_permutation
from oracle.chain import chain_primes, min_root
from oracle.ntt import intt, ntt
from tests.bigint_helpers import brv, horner_eval, negacyclic_mul


def _setup(n, bits, count):
    qs = chain_primes(n, bits, count)
    return qs, [min_root(q, n) for q in qs]


def _substitute(a, g, q):
    """a(X^g) mod (X^N + 1, q) by direct substitution of every monomial."""
    n = len(a)
    out = [0] * n
    for k, c in enumerate(a):
        e = k * g % (2 * n)
        if e < n:
            out[e] += int(c)
        else:
            out[e - n] -= int(c)
    return [x % q for x in out]


@pytest.mark.parametrize("g", [1, 3, 5, 25, 31, 63])
def test_coeff_automorphism_definition_and_homomorphism(g):
    n = 32
    qs, _ = _setup(n, 32, 2)
    rng = np.random.default_rng(g)
    a = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    b = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    sa, sb = automorph_coeff(a, g, qs), automorph_coeff(b, g, qs)
    for i, q in enumerate(qs):
        assert sa[i].tolist() == _substitute(a[i], g, q)
        ab = negacyclic_mul(a[i], b[i], q)
        assert automorph_coeff(np.array([ab], dtype=np.uint64), g, [q])[0].tolist() == negacyclic_mul(sa[i], sb[i], q)


def test_composition():
    n = 64
    qs, _ = _setup(n, 30, 1)
    a = np.random.default_rng(1).integers(0, qs[0], (1, n), dtype=np.uint64)
    for g1, g2 in [(5, 5), (5, 25), (3, 127), (125, 77)]:
        lhs = automorph_coeff(automorph_coeff(a, g2, qs), g1, qs)
        assert np.array_equal(lhs, automorph_coeff(a, g1 * g2 % (2 * n), qs))
        p = ntt_permutation(g1, n)[ntt_permutation(g2, n)]
        # applying pi_g1 after pi_g2 on indices: sigma_g1(sigma_g2(x))[j] = x[pi_g2[pi_g1[j]]]
        assert np.array_equal(ntt_permutation(g2, n)[ntt_permutation(g1, n)], ntt_permutation(g1 * g2 % (2 * n), n))
        assert sorted(p.tolist()) == list(range(n))


@pytest.mark.parametrize("n,bits", [(16, 32), (256, 30), (1 << 12, 30), (1 << 16, 32)])
def test_ntt_domain_automorphism(n, bits):
    qs, psis = _setup(n, bits, 2)
    rng = np.random.default_rng(n)
    a = np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in qs])
    for g in (5, 5**3 % (2 * n), 2 * n - 1):
        lhs = intt(automorph_ntt(ntt(a, qs, psis), g), qs, psis)
        assert np.array_equal(lhs, automorph_coeff(a, g, qs))
    if n <= 256:
        # NTT(sigma(a))[j] = a(psi^((2 brv(j) + 1) g)) directly
        logn = n.bit_length() - 1
        s = automorph_ntt(ntt(a, qs, psis), 5)
        for j in range(n):
            x = pow(psis[0], (2 * brv(j, logn) + 1) * 5, qs[0])
            assert int(s[0, j]) == horner_eval(a[0], x, qs[0])


def test_permutation_keeps_aligned_blocks_together():
    # the high bits of pi(j) depend only on the high bits of j: aligned blocks map to aligned blocks
    n = 1 << 12
    for g in (5, 25, 8191):
        p = ntt_permutation(g, n)
        for blk in (64, 1024):
            tgt = p.reshape(-1, blk) // blk
            assert np.all(tgt == tgt[:, :1])
