"""Galois automorphisms sigma_g: a(X) -> a(X^g) in Z_q[X]/(X^N+1) (oracle; test infrastructure only).

The pages do not describe rotations at this level; the key-switching kernels
they speak of (Perseus summary on ai4snews, "Interpretation" paragraph 2) are
the ones behind rotations.  Readings adopted: g is odd and below 2N; in the
coefficient domain coefficient n moves to n*g mod 2N, negated when that index
is >= N; in the NTT domain (bit-reversed evaluation order) sigma_g is the pure
index permutation out[j] = in[pi(j)] with 2*brv(pi(j))+1 = (2*brv(j)+1)*g mod 2N.
"""
from __future__ import annotations

import numpy as np

from .ntt import brv_array


def automorph_coeff(a: np.ndarray, g: int, qs: list[int]) -> np.ndarray:
    """sigma_g on coefficient-domain limbs a[..., limbs, N] (definition: X^n -> X^(n*g))."""
    n = a.shape[-1]
    assert g % 2 == 1 and 0 < g < 2 * n
    a = np.asarray(a, dtype=np.uint64)
    q = np.array(qs, dtype=np.uint64).reshape((len(qs), 1))
    out = np.zeros_like(a)
    idx = np.arange(n) * g % (2 * n)
    neg = idx >= n
    dst = np.where(neg, idx - n, idx)
    out[..., dst[~neg]] = a[..., np.nonzero(~neg)[0]]
    out[..., dst[neg]] = (q - a[..., np.nonzero(neg)[0]]) % q
    return out


def ntt_permutation(g: int, n: int) -> np.ndarray:
    """pi with NTT(sigma_g(a))[j] = NTT(a)[pi[j]] in bit-reversed evaluation order."""
    assert g % 2 == 1 and 0 < g < 2 * n
    r = brv_array(n)  # brv is an involution: r[r[k]] = k
    e = (2 * r + 1) * g % (2 * n)
    return r[(e - 1) // 2]


def automorph_ntt(a: np.ndarray, g: int) -> np.ndarray:
    """sigma_g on NTT-domain limbs a[..., N]."""
    return np.asarray(a)[..., ntt_permutation(g, a.shape[-1])]
