"""Prime chain, minimal negacyclic roots and big-integer CRT (oracle; test infrastructure only).

The pages fix only "a 32-bit RNS CKKS chain" (Perseus summary on ai4snews,
"Interpretation" paragraph 2 and "Perspective" paragraph 1).  They are silent on
which primes, on their order and on the roots of unity, so this module takes
the plainest readings:

* chain: the L+K largest primes q < 2**bits with q = 1 (mod 2N), in descending
  order; the first L are the ciphertext primes q_0..q_{L-1}, the next K the
  special primes p_0..p_{K-1};
* root: psi_t is the smallest integer x >= 2 with x**N = -1 (mod q_t), i.e. the
  smallest primitive 2N-th root of unity.
"""
from __future__ import annotations

from functools import reduce

import sympy


def chain_primes(n: int, bits: int, count: int) -> list[int]:
    """The `count` largest primes q < 2**bits with q = 1 (mod 2n), descending.

    Scans downward over the arithmetic progression 1 + k*2n.
    """
    step = 2 * n
    q = 2**bits - step + 1  # largest value = 1 (mod 2n) below 2**bits (2n divides 2**bits)
    out: list[int] = []
    while len(out) < count:
        if q <= step:
            raise ValueError("not enough primes")
        if sympy.isprime(q):
            out.append(q)
        q -= step
    return out


def min_root(q: int, n: int) -> int:
    """Smallest x >= 2 with x**n = -1 (mod q).

    For n a power of two these x are exactly the primitive 2n-th roots of unity,
    i.e. the odd powers of any one of them; the minimum over that set is taken.
    """
    h = 2
    while True:
        w = pow(h, (q - 1) // (2 * n), q)
        if pow(w, n, q) == q - 1:
            break
        h += 1
    w2 = w * w % q
    best, x = w, w
    for _ in range(n - 1):
        x = x * w2 % q
        best = min(best, x)
    return best


def crt(residues: list[int], moduli: list[int]) -> int:
    """The unique X in [0, prod(moduli)) with X = r_i (mod m_i), by the textbook CRT formula."""
    m = reduce(lambda a, b: a * b, moduli, 1)
    x = 0
    for r, mi in zip(residues, moduli):
        mhat = m // mi
        x += int(r) * mhat * pow(mhat, -1, mi)
    return x % m


def centered(x: int, m: int) -> int:
    """Representative of x mod m in (-m/2, m/2]."""
    x %= m
    return x - m if x > m // 2 else x
