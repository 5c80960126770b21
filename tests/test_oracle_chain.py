"""Pins of the oracle's prime chain, roots and CRT against brute force and number theory."""
import random

import pytest

from oracle.chain import chain_primes, centered, crt, min_root
from tests.bigint_helpers import is_prime_trial

CHAINS = [(1 << 12, 30, 6), (1 << 16, 32, 48), (1 << 4, 30, 4), (1 << 10, 32, 5)]


@pytest.mark.parametrize("n,bits,count", CHAINS)
def test_chain_is_the_largest_qualifying_primes(n, bits, count):
    ps = chain_primes(n, bits, count)
    assert len(ps) == count and ps == sorted(ps, reverse=True)
    # every member qualifies, and every skipped candidate of the progression is composite
    cand = (1 << bits) - 1
    cand -= (cand - 1) % (2 * n)
    found = []
    while len(found) < count:
        assert cand < 1 << bits and cand % (2 * n) == 1
        if is_prime_trial(cand):
            found.append(cand)
        cand -= 2 * n
    assert found == ps


def test_chain_known_extremes():
    # N = 2^12 primes sit below 2^30 (floor(2^32/q) = 4); every N = 2^16 prime exceeds 2^31
    small = chain_primes(1 << 12, 30, 6)
    assert all(2**29 < q < 2**30 and 2**32 // q == 4 for q in small)
    big = chain_primes(1 << 16, 32, 48)
    assert all(2**31 < q < 2**32 for q in big)


def _scan_root(q, n):
    """The definition written out: first x >= 2 with x^N = -1 (mod q), by linear scan."""
    x = 2
    while pow(x, n, q) != q - 1:
        x += 1
    return x


@pytest.mark.parametrize("n,bits,count", [(1 << 12, 30, 6), (1 << 4, 20, 4), (1 << 10, 28, 5), (1 << 16, 32, 48)])
def test_min_root_is_the_smallest_negacyclic_root(n, bits, count):
    qs = chain_primes(n, bits, count)
    for q in qs:  # all 48 primes of the 2^16 chain: ~5 s of scanning
        psi = min_root(q, n)
        assert pow(psi, n, q) == q - 1
        assert psi == _scan_root(q, n)


def test_min_root_small_ring_32bit_primes():
    # the scan is too slow here; the root must still be a primitive 2N-th root
    for n in (1 << 4, 1 << 6):
        for q in chain_primes(n, 32, 3):
            psi = min_root(q, n)
            assert pow(psi, n, q) == q - 1 and pow(psi, 2 * n, q) == 1


def test_crt_reconstruction_property():
    rng = random.Random(7)
    mods = chain_primes(1 << 16, 32, 12)
    big = 1
    for m in mods:
        big *= m
    for _ in range(200):
        x = rng.randrange(big)
        res = [x % m for m in mods]
        assert crt(res, mods) == x
        c = centered(x, big)
        assert -big // 2 < c <= big // 2 and (c - x) % big == 0
