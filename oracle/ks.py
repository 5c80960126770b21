"""Key generation, inner product, key-switch and hoisted key-switch (oracle; test infrastructure only).

The method of the pages: the key-switching key is a pair (b, a) whose half a is
uniformly random, so it is regenerated from a seed by counter-mode ChaCha12
inside the kernels that use the key instead of being stored (Perseus summary on
ai4snews, "Interpretation" paragraph 2).  The surrounding algorithm is hybrid
key-switching (Han and Ki, CT-RSA 2020) on RNS-CKKS (Cheon et al., SAC 2018).
Readings adopted where the pages are silent:

* keys and ciphertexts live in the NTT domain; key rows are indexed by the
  absolute prime index t, so one key serves every level;
* key row j encrypts the gadget P*g_j*s_src under s, with g_j the CRT idempotent
  of digit j over the full chain: b_j = -a_j*s + e_j + [t in digit j]*[P]_{q_t}*s_src;
* the automorphism sigma_g is applied after ModUp, to the NTT-domain extended
  digits and to c0, so that one ModUp serves many rotations bit-identically;
* output ct' = (sigma_g(c0) + ModDown(acc_b), ModDown(acc_a)).
"""
from __future__ import annotations

from math import prod

import numpy as np

from .automorph import automorph_coeff, automorph_ntt
from .chacha import expand_key_a
from .chain import centered, crt
from .ntt import intt, ntt
from .params import Params
from .rns import moddown, modup


def to_ntt_all(poly: np.ndarray, pr: Params, idx: list[int]) -> np.ndarray:
    """NTT of one signed integer polynomial reduced modulo every prime in idx -> [len(idx), N]."""
    qs = [pr.primes[t] for t in idx]
    res = np.stack([np.mod(poly.astype(np.int64), q).astype(np.uint64) for q in qs])
    return ntt(res, qs, [pr.psis[t] for t in idx])


def keygen(pr: Params, s: np.ndarray, s_src: np.ndarray, errors: list[np.ndarray], seed: bytes):
    """(key_b, key_a), each [dnum][L+K][N]: a from the seed, b = -a*s + e_j + gadget_j*s_src."""
    allidx = list(range(pr.L + pr.K))
    key_a = expand_key_a(seed, pr.primes, pr.dnum, pr.n)
    sh = to_ntt_all(s, pr, allidx)
    srch = to_ntt_all(s_src, pr, allidx)
    q = np.array(pr.primes, dtype=np.uint64).reshape((-1, 1))
    big_p = pr.P
    key_b = np.empty_like(key_a)
    for j in range(pr.dnum):
        eh = to_ntt_all(errors[j], pr, allidx)
        b = (q - key_a[j] * sh % q + eh) % q
        for t in pr.digit(j, pr.L):
            b[t] = (b[t] + np.uint64(big_p % pr.primes[t]) * srch[t]) % q[t]
        key_b[j] = b
    return key_b, key_a


def inner_product(digits: np.ndarray, key_b: np.ndarray, key_a: np.ndarray, g: int, level: int, pr: Params):
    """acc_b, acc_a [..., l+K, N]: sum over digits of sigma_g(digit_j)[t] * key_{b,a}[j][t]."""
    ext = pr.ext(level)
    q = np.array([pr.primes[t] for t in ext], dtype=np.uint64).reshape((-1, 1))
    sd = automorph_ntt(digits, g)
    acc_b = np.zeros(digits.shape[:-3] + (len(ext), pr.n), dtype=np.uint64)
    acc_a = np.zeros_like(acc_b)
    for j in range(digits.shape[-3]):
        acc_b = (acc_b + sd[..., j, :, :] * key_b[j][ext] % q) % q
        acc_a = (acc_a + sd[..., j, :, :] * key_a[j][ext] % q) % q
    return acc_b, acc_a


def finish(ct: np.ndarray, acc_b: np.ndarray, acc_a: np.ndarray, g: int, level: int, pr: Params) -> np.ndarray:
    q = np.array(pr.primes[:level], dtype=np.uint64).reshape((-1, 1))
    out0 = (automorph_ntt(ct[..., 0, :, :], g) + moddown(acc_b, level, pr)) % q
    out1 = moddown(acc_a, level, pr)
    return np.stack([out0, out1], axis=-3)


def keyswitch(pr: Params, ct: np.ndarray, level: int, key_b: np.ndarray, g: int,
              key_a: np.ndarray | None = None, seed: bytes | None = None) -> np.ndarray:
    """Key-switch ct [..., 2, l, N] under (key_b, a) with Galois element g; a stored or from the seed."""
    if key_a is None:
        key_a = expand_key_a(seed, pr.primes, pr.dnum, pr.n)
    digits = modup(ct[..., 1, :, :], level, pr)
    acc_b, acc_a = inner_product(digits, key_b, key_a, g, level, pr)
    return finish(ct, acc_b, acc_a, g, level, pr)


def keyswitch_hoisted(pr: Params, ct: np.ndarray, level: int, keys: list) -> np.ndarray:
    """One ModUp of ct [2, l, N], then one inner product + ModDown per (key_b, key_a, g): [n_keys, 2, l, N]."""
    digits = modup(ct[1], level, pr)
    outs = []
    for key_b, key_a, g in keys:
        acc_b, acc_a = inner_product(digits, key_b, key_a, g, level, pr)
        outs.append(finish(ct, acc_b, acc_a, g, level, pr))
    return np.stack(outs)


def noise_bound(pr: Params, level: int, b_err: int = 19) -> float:
    """Bound on |Dec_s(ct') - (sigma(c0) + sigma(c1)*s_src)|_inf, from the digit, error and rounding sizes."""
    big_p = pr.P
    s = sum(len(pr.digit(j, level)) * prod(pr.primes[i] for i in pr.digit(j, level))
            for j in range(pr.n_digits(level)))
    return pr.n * b_err * s / big_p + 1 + pr.n + pr.K + pr.K * pr.n


def switch_error(pr: Params, ct: np.ndarray, out: np.ndarray, level: int, s: np.ndarray,
                 s_src: np.ndarray, g: int) -> int:
    """max |Delta| with Delta = [Dec_s(out) - (sigma_g(c0) + sigma_g(c1)*s_src)] mod Q_l, centred (big-int CRT)."""
    idx = list(range(level))
    qs = pr.primes[:level]
    q = np.array(qs, dtype=np.uint64).reshape((-1, 1))
    sh = to_ntt_all(s, pr, idx)
    srch = to_ntt_all(s_src, pr, idx)
    dec = (out[0] + out[1] * sh % q) % q
    ref = (automorph_ntt(ct[0], g) + automorph_ntt(ct[1], g) * srch % q) % q
    delta = intt((dec + q - ref) % q, qs, pr.psis[:level])
    big_q = prod(qs)
    worst = 0
    cols = delta.T.tolist()
    for col in cols:
        worst = max(worst, abs(centered(crt(col, qs), big_q)))
    return worst


def decrypt_coeffs(pr: Params, ct: np.ndarray, level: int, s: np.ndarray) -> list[int]:
    """Centred big-integer coefficients of c0 + c1*s mod Q_l (used by small tests)."""
    qs = pr.primes[:level]
    q = np.array(qs, dtype=np.uint64).reshape((-1, 1))
    sh = to_ntt_all(s, pr, list(range(level)))
    m = intt((ct[0] + ct[1] * sh % q) % q, qs, pr.psis[:level])
    big_q = prod(qs)
    return [centered(crt(col, qs), big_q) for col in m.T.tolist()]


def rotation_source(s: np.ndarray, g: int, pr: Params) -> np.ndarray:
    """s_src = sigma_g(s) as a signed integer polynomial (the secret a rotation key switches from)."""
    n = pr.n
    out = np.zeros(n, dtype=np.int64)
    idx = np.arange(n) * g % (2 * n)
    neg = idx >= n
    out[np.where(neg, idx - n, idx)] = np.where(neg, -s, s)
    return out
