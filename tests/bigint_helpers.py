"""Plain Python-integer helpers the pins use to check the oracle independently of it."""
from __future__ import annotations


def small_primes(limit: int) -> list[int]:
    sieve = bytearray([1]) * (limit + 1)
    sieve[0:2] = b"\x00\x00"
    for i in range(2, int(limit**0.5) + 1):
        if sieve[i]:
            sieve[i * i::i] = bytearray(len(sieve[i * i::i]))
    return [i for i in range(limit + 1) if sieve[i]]


_SP = small_primes(1 << 16)


def is_prime_trial(n: int) -> bool:
    """Trial division by every prime up to 2**16: exact for n < 2**32."""
    assert n < 1 << 32
    if n < 2:
        return False
    for p in _SP:
        if p * p > n:
            return True
        if n % p == 0:
            return n == p
    return True


def brv(j: int, logn: int) -> int:
    return int(format(j, f"0{logn}b")[::-1], 2) if logn else 0


def horner_eval(coeffs, x: int, q: int) -> int:
    acc = 0
    for c in reversed(list(coeffs)):
        acc = (acc * x + int(c)) % q
    return acc


def negacyclic_mul(a, b, q: int) -> list[int]:
    """Schoolbook product in Z_q[X]/(X^N+1)."""
    n = len(a)
    out = [0] * n
    for i in range(n):
        ai = int(a[i])
        if ai == 0:
            continue
        for k in range(n):
            v = ai * int(b[k])
            if i + k < n:
                out[i + k] += v
            else:
                out[i + k - n] -= v
    return [x % q for x in out]
