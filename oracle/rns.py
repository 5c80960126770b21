"""ModUp and ModDown by fast base conversion (oracle; test infrastructure only).

The pages name the kernels that use the key but not the conversions around
them (Perseus summary on ai4snews, "Interpretation" paragraph 2).  These are the
hybrid key-switching steps of Han and Ki (CT-RSA 2020) with the fast base
conversion of Bajard, Eynard, Hasan and Zucca (SAC 2016).  Readings adopted:

* ModUp leaves the overflow u*Q~_j (0 <= u < alpha'_j) in place: no correction;
* ModDown is floor-type: the special-prime part is taken in [0, p_k), no P/2
  offset, and the conversion overflow v*P (0 <= v < K) is left in;
* inputs and outputs are in the NTT domain, bit-reversed order, canonical residues.
"""
from __future__ import annotations

from math import prod

import numpy as np

from .ntt import intt, ntt
from .params import Params


def modup(c1_hat: np.ndarray, level: int, pr: Params) -> np.ndarray:
    """Extended digits [..., d_l, l+K, N] of c1_hat [..., l, N].

    Per digit j with primes D: x = INTT(c1); y_i = x_i * [(Q~/q_i)^-1]_{q_i};
    z_t = sum_i y_i * [Q~/q_i]_{q_t} for every extended-basis prime t not in D;
    digit[t] = NTT_t(z_t), and digit[t] = c1_hat[t] for t in D.
    """
    qs = pr.primes
    x = intt(c1_hat, qs[:level], pr.psis[:level])
    ext = pr.ext(level)
    lead = c1_hat.shape[:-2]
    out = np.empty(lead + (pr.n_digits(level), len(ext), pr.n), dtype=np.uint64)
    for j in range(pr.n_digits(level)):
        dig = pr.digit(j, level)
        qt = prod(qs[i] for i in dig)
        y = {i: x[..., i, :] * np.uint64(pow(qt // qs[i], -1, qs[i])) % np.uint64(qs[i]) for i in dig}
        targets = [e for e, t in enumerate(ext) if t not in dig]
        z = np.empty(lead + (len(targets), pr.n), dtype=np.uint64)
        for k, e in enumerate(targets):
            qtar = np.uint64(qs[ext[e]])
            acc = np.zeros(lead + (pr.n,), dtype=np.uint64)
            for i in dig:
                acc += y[i] * np.uint64((qt // qs[i]) % qs[ext[e]]) % qtar
            z[..., k, :] = acc % qtar
        zh = ntt(z, [qs[ext[e]] for e in targets], [pr.psis[ext[e]] for e in targets])
        for k, e in enumerate(targets):
            out[..., j, e, :] = zh[..., k, :]
        for i in dig:
            out[..., j, i, :] = c1_hat[..., i, :]
    return out


def moddown(x_hat: np.ndarray, level: int, pr: Params) -> np.ndarray:
    """[..., l, N] from an extended-basis polynomial x_hat [..., l+K, N] (q limbs then p limbs).

    x = INTT over the special primes; y_k = x_k * [(P/p_k)^-1]_{p_k};
    z_i = sum_k y_k * [P/p_k]_{q_i}; out_i = (x_hat_i - NTT_i(z_i)) * [P^-1]_{q_i}.
    """
    qs, ps = pr.primes[:level], pr.p
    big_p = pr.P
    xp = intt(x_hat[..., level:, :], ps, pr.psis[pr.L:])
    y = [xp[..., k, :] * np.uint64(pow(big_p // pk, -1, pk)) % np.uint64(pk) for k, pk in enumerate(ps)]
    lead = x_hat.shape[:-2]
    z = np.empty(lead + (level, pr.n), dtype=np.uint64)
    for i, qi in enumerate(qs):
        acc = np.zeros(lead + (pr.n,), dtype=np.uint64)
        for k, pk in enumerate(ps):
            acc += y[k] * np.uint64((big_p // pk) % qi) % np.uint64(qi)
        z[..., i, :] = acc % np.uint64(qi)
    zh = ntt(z, qs, pr.psis[:level])
    q = np.array(qs, dtype=np.uint64).reshape((level, 1))
    pinv = np.array([pow(big_p, -1, qi) for qi in qs], dtype=np.uint64).reshape((level, 1))
    return (x_hat[..., :level, :] + q - zh) % q * pinv % q
