"""Ciphertext multiply, relinearise and rescale (oracle; test infrastructure only).

The pages name these operations only in passing: a CKKS ciphertext spends
multiplication depth, relinearisation is one of the key-switches the backend
runs, and bootstrapping restores the depth (Perseus abstract on paperdot;
EncryptedLLM summary on lpnh, "Core problem" paragraph).  The steps follow the
RNS variant of CKKS (Cheon, Han, Kim, Kim and Song, SAC 2018).  Readings adopted
where the pages are silent:

* the tensor product is taken in the NTT domain, limb by limb:
  d0 = x0*y0, d1 = x0*y1 + x1*y0, d2 = x1*y1 (mod q_i);
* relinearisation is the key-switch of `ks` with Galois element 1 and a key whose
  source secret is s^2 (the negacyclic square of s):
  (e0, e1) = (d0 + ModDown(acc_b), d1 + ModDown(acc_a));
* rescaling drops the last active prime q_{l-1} with the floor convention of
  ModDown: c_i <- (c_i - NTT_i([INTT_{l-1}(c_{l-1})] mod q_i)) * q_{l-1}^-1 mod q_i
  for i < l-1, so a coefficient C in [0, Q_l) becomes floor(C / q_{l-1}).
"""
from __future__ import annotations

import numpy as np

from .chain import centered
from .ks import inner_product, keygen
from .chacha import expand_key_a
from .ntt import intt, ntt
from .params import Params
from .rns import moddown, modup


def _qcol(primes: list[int]) -> np.ndarray:
    return np.array(primes, dtype=np.uint64).reshape((-1, 1))


def square_secret(s: np.ndarray, pr: Params) -> np.ndarray:
    """s*s in Z[X]/(X^N+1) as signed integers (|coefficient| <= N for ternary s).

    Computed through one chain prime q > 2N and centred, which is exact because
    every coefficient of the product lies in [-N, N]."""
    q, psi = pr.primes[0], pr.psis[0]
    sh = ntt(np.mod(s.astype(np.int64), q).astype(np.uint64).reshape(1, -1), [q], [psi])
    sq = intt(sh * sh % np.uint64(q), [q], [psi])[0]
    return np.array([centered(int(v), q) for v in sq.tolist()], dtype=np.int64)


def relin_keygen(pr: Params, s: np.ndarray, errors: list[np.ndarray], seed: bytes):
    """Relinearisation key (key_b, key_a): the key-switching key from s^2 to s."""
    return keygen(pr, s, square_secret(s, pr), errors, seed)


def tensor(x: np.ndarray, y: np.ndarray, level: int, pr: Params):
    """(d0, d1, d2), each [..., l, N]: the NTT-domain tensor product of x, y [..., 2, l, N]."""
    q = _qcol(pr.primes[:level])
    x0, x1 = x[..., 0, :, :], x[..., 1, :, :]
    y0, y1 = y[..., 0, :, :], y[..., 1, :, :]
    d0 = x0 * y0 % q
    d1 = (x0 * y1 % q + x1 * y0 % q) % q
    d2 = x1 * y1 % q
    return d0, d1, d2


def relinearize(pr: Params, d0: np.ndarray, d1: np.ndarray, d2: np.ndarray, level: int,
                key_b: np.ndarray, key_a: np.ndarray) -> np.ndarray:
    """[..., 2, l, N]: (d0 + ModDown(acc_b), d1 + ModDown(acc_a)) with acc from ModUp(d2) and the key."""
    q = _qcol(pr.primes[:level])
    digits = modup(d2, level, pr)
    acc_b, acc_a = inner_product(digits, key_b, key_a, 1, level, pr)
    e0 = (d0 + moddown(acc_b, level, pr)) % q
    e1 = (d1 + moddown(acc_a, level, pr)) % q
    return np.stack([e0, e1], axis=-3)


def rescale(pr: Params, ct: np.ndarray, level: int) -> np.ndarray:
    """Drop q_{l-1}: [..., 2, l, N] -> [..., 2, l-1, N] (NTT domain, floor convention)."""
    assert level >= 2
    ql = pr.primes[level - 1]
    qs = pr.primes[:level - 1]
    q = _qcol(qs)
    last = intt(ct[..., level - 1:level, :], [ql], [pr.psis[level - 1]])  # coefficients in [0, q_{l-1})
    y = ntt(last % q, qs, pr.psis[:level - 1])
    inv = _qcol([pow(ql, -1, qi) for qi in qs])
    return (ct[..., :level - 1, :] + q - y) % q * inv % q


def mul_relin_rescale(pr: Params, x: np.ndarray, y: np.ndarray, level: int, key_b: np.ndarray,
                      key_a: np.ndarray | None = None, seed: bytes | None = None) -> np.ndarray:
    """Rescale(Relinearise(x (x) y)): [..., 2, l, N] x2 -> [..., 2, l-1, N]; a stored or from the seed."""
    if key_a is None:
        key_a = expand_key_a(seed, pr.primes, pr.dnum, pr.n)
    d0, d1, d2 = tensor(x, y, level, pr)
    return rescale(pr, relinearize(pr, d0, d1, d2, level, key_b, key_a), level)
