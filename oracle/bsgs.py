"""Double-hoisted baby-step/giant-step linear transform (oracle; test infrastructure only).

The pages name bootstrapping as the cost centre of encrypted inference (Perseus
summary on ai4snews, "Synopsis"; Sylph summary on rrmt.cn, "Technical details"
item 3) without giving its steps.  The linear transforms of bootstrapping
(CoeffsToSlots, SlotsToCoeffs) are sums of plaintext-diagonal products of
rotations, evaluated baby-step/giant-step with two hoisting steps (Bossuat,
Mouchet, Troncoso-Pastoriza and Hubaux, Eurocrypt 2021).  Readings adopted
where the pages are silent:

* inputs: one ciphertext ct at level l; n1 baby steps k = 0..n1-1 and n2 giant
  steps j = 0..n2-1; baby step 0 and giant step 0 are the identity, every other
  step has its own key-switching key and Galois element (chosen by the caller);
  plaintext diagonals D[j][k] are given in the NTT domain over the extended
  basis q_0..q_{l-1}, p_0..p_{K-1} (the layout of an extended digit);
* first hoist: one ModUp of c1 serves every baby step; baby step k in the
  extended basis is R_k = (P*sigma_k(c0) + acc_b^k, acc_a^k) (acc from the inner
  product of sigma_k(digits) with key k; the P*sigma_k(c0) term is zero on the
  special primes), and R_0 = (P*c0, P*c1);
* second hoist: per giant step, S_j = sum_k D[j][k] * R_k stays in the extended
  basis and is brought down by a single ModDown (the floor ModDown of `rns`);
* giant step j rotates ModDown(S_j) by a full key-switch with its key (the
  key-switch of `ks`), and the result is out = sum_j of the rotated terms.
"""
from __future__ import annotations

import numpy as np

from .automorph import automorph_ntt
from .chacha import expand_key_a
from .ks import inner_product, keyswitch
from .params import Params
from .rns import moddown, modup


def _qcol(primes: list[int]) -> np.ndarray:
    return np.array(primes, dtype=np.uint64).reshape((-1, 1))


def _key_a(pr: Params, key: dict) -> np.ndarray:
    return key["a"] if key.get("a") is not None else expand_key_a(key["seed"], pr.primes, pr.dnum, pr.n)


def baby_steps(pr: Params, ct: np.ndarray, level: int, baby_keys: list[dict]) -> list[np.ndarray]:
    """[R_0, ..., R_{n1-1}], each [2, l+K, N] in the extended basis (NTT domain).

    baby_keys[k-1] = {"b": key_b, "a": key_a or None, "seed": seed or None, "g": Galois element} for k >= 1."""
    ext = pr.ext(level)
    q = _qcol([pr.primes[t] for t in ext])
    p_mod = _qcol([pr.P % pr.primes[t] if e < level else 0 for e, t in enumerate(ext)])
    lift = lambda c: np.concatenate([c, np.zeros((pr.K, pr.n), dtype=np.uint64)], axis=0) * p_mod % q
    out = [np.stack([lift(ct[0]), lift(ct[1])])]
    digits = modup(ct[1], level, pr)
    for key in baby_keys:
        acc_b, acc_a = inner_product(digits, key["b"], _key_a(pr, key), key["g"], level, pr)
        out.append(np.stack([(lift(automorph_ntt(ct[0], key["g"])) + acc_b) % q, acc_a]))
    return out


def linear_transform(pr: Params, ct: np.ndarray, level: int, diags: np.ndarray, baby_keys: list[dict],
                     giant_keys: list[dict]) -> np.ndarray:
    """sum_j Rot_j(ModDown(sum_k D[j][k] * R_k)) -> [2, l, N]; diags [n2][n1][l+K][N]."""
    n2, n1 = diags.shape[:2]
    assert len(baby_keys) == n1 - 1 and len(giant_keys) == n2 - 1
    ext = pr.ext(level)
    qe = _qcol([pr.primes[t] for t in ext])
    ql = _qcol(pr.primes[:level])
    rs = baby_steps(pr, ct, level, baby_keys)
    out = np.zeros((2, level, pr.n), dtype=np.uint64)
    for j in range(n2):
        s = np.zeros((2, len(ext), pr.n), dtype=np.uint64)
        for k in range(n1):
            s = (s + diags[j, k] * rs[k] % qe) % qe
        term = moddown(s, level, pr)
        if j > 0:
            key = giant_keys[j - 1]
            term = keyswitch(pr, term, level, key["b"], key["g"], key_a=_key_a(pr, key))
        out = (out + term) % ql
    return out
