"""Negacyclic NTT and its inverse over one prime per limb (oracle; test infrastructure only).

The pages name no transform; the key-switching path runs on RNS limbs of
Z_q[X]/(X^N+1) (Perseus summary on ai4snews, "Interpretation" paragraph 2:
"32-bit RNS CKKS chain").  Reading adopted for the transform and its order:

    NTT(a)[j] = sum_{n<N} a[n] * psi**((2*brv(j)+1)*n)  (mod q)

with brv the log2(N)-bit reversal, i.e. the evaluations of a at the odd powers
of psi stored in bit-reversed order, and INTT its exact inverse.  `ntt_definition`
is that formula written out (O(N^2)); `ntt`/`intt` are the merged-twist
Cooley-Tukey / Gentleman-Sande forms of Longa and Naehrig (2016), which reach
the same values.  All arrays are numpy uint64 with shape [..., limbs, N] and a
per-limb prime list.
"""
from __future__ import annotations

import numpy as np


def brv(j: int, logn: int) -> int:
    """Reverse the low `logn` bits of j."""
    r = 0
    for _ in range(logn):
        r = (r << 1) | (j & 1)
        j >>= 1
    return r


def brv_array(n: int) -> np.ndarray:
    logn = n.bit_length() - 1
    return np.array([brv(j, logn) for j in range(n)], dtype=np.int64)


def ntt_definition(a: np.ndarray, q: int, psi: int) -> np.ndarray:
    """NTT of one length-N vector straight from the definition (O(N^2), small N only)."""
    n = a.shape[-1]
    two_n = 2 * n
    pw = np.array([pow(psi, e, q) for e in range(two_n)], dtype=np.uint64)
    e = (2 * brv_array(n) + 1)[:, None] * np.arange(n)[None, :] % two_n
    prod = (pw[e] * (a.astype(np.uint64) % q)[None, :]) % q  # each product < 2**64
    return (prod.sum(axis=1, dtype=np.uint64) % q).astype(np.uint64)


def _tables(n: int, qs: list[int], psis: list[int], inverse: bool) -> np.ndarray:
    """[limbs, N] table psi**(+-brv(k)) mod q."""
    r = brv_array(n)
    rows = []
    for q, psi in zip(qs, psis):
        base = pow(psi, -1, q) if inverse else psi
        pw = [1] * n
        for k in range(1, n):
            pw[k] = pw[k - 1] * base % q
        rows.append(np.array(pw, dtype=np.uint64)[r])
    return np.stack(rows)


def ntt(a: np.ndarray, qs: list[int], psis: list[int]) -> np.ndarray:
    """Forward transform of every limb: a[..., i, :] over prime qs[i] (natural order in, bit-reversed out)."""
    a = np.array(a, dtype=np.uint64, copy=True)
    n = a.shape[-1]
    nl = a.shape[-2]
    assert nl == len(qs) == len(psis)
    tw = _tables(n, qs, psis, inverse=False)
    q = np.array(qs, dtype=np.uint64)
    lead = a.shape[:-2]
    m = 1
    while m < n:
        t = n // (2 * m)
        v = a.reshape(lead + (nl, m, 2, t))
        qb = q.reshape((nl, 1, 1))
        s = tw[:, m:2 * m].reshape((nl, m, 1))
        u = v[..., 0, :].copy()
        w = v[..., 1, :] * s % qb
        v[..., 0, :] = (u + w) % qb
        v[..., 1, :] = (u + qb - w) % qb
        m *= 2
    return a


def intt(a: np.ndarray, qs: list[int], psis: list[int]) -> np.ndarray:
    """Inverse transform of every limb (bit-reversed order in, natural order out), scaled by N^-1."""
    a = np.array(a, dtype=np.uint64, copy=True)
    n = a.shape[-1]
    nl = a.shape[-2]
    assert nl == len(qs) == len(psis)
    tw = _tables(n, qs, psis, inverse=True)
    q = np.array(qs, dtype=np.uint64)
    lead = a.shape[:-2]
    m = n // 2
    while m >= 1:
        t = n // (2 * m)
        v = a.reshape(lead + (nl, m, 2, t))
        qb = q.reshape((nl, 1, 1))
        s = tw[:, m:2 * m].reshape((nl, m, 1))
        u = v[..., 0, :].copy()
        w = v[..., 1, :].copy()
        v[..., 0, :] = (u + w) % qb
        v[..., 1, :] = (u + qb - w) % qb * s % qb
        m //= 2
    ninv = np.array([pow(n, -1, qq) for qq in qs], dtype=np.uint64).reshape((nl, 1))
    return a * ninv % q.reshape((nl, 1))
