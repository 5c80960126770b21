"""Seeded synthetic inputs for the five key-switching workloads.

This module only draws random numbers; it holds none of the method's
arithmetic, so the GPU path and the CPU oracle can both consume its output.
Each workload c draws from numpy Generator(PCG64(1000 + c)) in a fixed order:

1. the ternary secret s (uniform over {-1, 0, 1});
2. the second secret s' of a relinearisation-style key, when the workload has one;
3. for the mixed stream: every ciphertext's level (uniform over 8..36) and key
   index (uniform over the 33 keys);
4. per key, in key-list order: a 32-byte ChaCha seed, then one error polynomial
   per digit (normal with sigma 3.2, rounded, |e| > 19 redrawn);
5. ciphertext residues, uniform in [0, q_i), per ciphertext, component, prime.

The level sweep reuses the single-switch workload's secret and key and draws
only its ciphertexts.  Primes are passed in: they are parameters of the chain,
computed elsewhere.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

SIGMA = 3.2
ERR_BOUND = 19


@dataclass
class Workload:
    """Shape of one workload: ring, chain split, digits, levels, batch and Galois elements."""
    ident: int
    name: str
    log_n: int
    L: int
    K: int
    dnum: int
    bits: int
    levels: list[int]
    batch: int
    galois: list[int]              # Galois element of each key, in key-list order
    relin_key: int | None = None   # index of the key that switches from an independent s'
    mixed: bool = False            # mixed stream: one level and one key per ciphertext

    @property
    def n(self) -> int:
        return 1 << self.log_n


def _pow5(k: int, two_n: int) -> int:
    return pow(5, k, two_n)


WORKLOADS = {
    1: Workload(1, "tiny key-switch N=2^12, 4+2 primes <2^30, dnum 2, relinearisation-style key",
                12, 4, 2, 2, 30, [4], 1, [1], relin_key=0),
    2: Workload(2, "single key-switch N=2^16, 36+12 primes <2^32, dnum 3, batch 8, rotation g=5",
                16, 36, 12, 3, 32, [36], 8, [5]),
    3: Workload(3, "level sweep N=2^16, batch 16 at levels 36/24/12/4, key of the single-switch workload",
                16, 36, 12, 3, 32, [36, 24, 12, 4], 16, [5]),
    4: Workload(4, "hoisted rotations N=2^16, one ciphertext at level 36, 16 keys g=5^k",
                16, 36, 12, 3, 32, [36], 1, [_pow5(k, 1 << 17) for k in range(1, 17)]),
    5: Workload(5, "mixed stream N=2^16, 64 ciphertexts at levels 8..36, 32 rotation keys + 1 relinearisation key",
                16, 36, 12, 3, 32, list(range(8, 37)), 64,
                [_pow5(k, 1 << 17) for k in range(1, 33)] + [1], relin_key=32, mixed=True),
}


@dataclass
class KeyDraw:
    seed: bytes
    errors: list[np.ndarray]
    galois: int


@dataclass
class Draw:
    """Everything a workload draws; ciphertexts are NTT-domain residues [2][l][N] (uint32)."""
    s: np.ndarray
    s_prime: np.ndarray | None
    keys: list[KeyDraw]
    cts: list[np.ndarray] = field(default_factory=list)
    levels: list[int] = field(default_factory=list)
    key_index: list[int] = field(default_factory=list)


def ternary(rng: np.random.Generator, n: int) -> np.ndarray:
    return rng.integers(-1, 2, n).astype(np.int64)


def gaussian(rng: np.random.Generator, n: int) -> np.ndarray:
    e = np.rint(rng.normal(0.0, SIGMA, n))
    bad = np.abs(e) > ERR_BOUND
    while bad.any():
        e[bad] = np.rint(rng.normal(0.0, SIGMA, int(bad.sum())))
        bad = np.abs(e) > ERR_BOUND
    return e.astype(np.int64)


def residues(rng: np.random.Generator, primes: list[int], n: int) -> np.ndarray:
    """[len(primes)][N] uint32, each row uniform in [0, q)."""
    return np.stack([rng.integers(0, q, n, dtype=np.uint64) for q in primes]).astype(np.uint32)


def _keys(rng, wl: Workload) -> list[KeyDraw]:
    out = []
    for g in wl.galois:
        seed = rng.bytes(32)
        errs = [gaussian(rng, wl.n) for _ in range(wl.dnum)]
        out.append(KeyDraw(seed, errs, g))
    return out


def draw(ident: int, primes: list[int], ct_count: int | None = None) -> Draw:
    """Draw workload `ident`; `ct_count` limits how many ciphertexts are drawn (prefix of the full draw)."""
    wl = WORKLOADS[ident]
    n = wl.n
    if ident == 3:
        base = draw(2, primes, ct_count=0)
        rng = np.random.Generator(np.random.PCG64(1000 + ident))
        d = Draw(base.s, None, base.keys)
        total = wl.batch * len(wl.levels)
        want = total if ct_count is None else min(ct_count, total)
        for k in range(want):
            lvl = wl.levels[k // wl.batch]
            d.cts.append(np.stack([residues(rng, primes[:lvl], n) for _ in range(2)]))
            d.levels.append(lvl)
            d.key_index.append(0)
        return d
    rng = np.random.Generator(np.random.PCG64(1000 + ident))
    s = ternary(rng, n)
    s_prime = ternary(rng, n) if wl.relin_key is not None else None
    if wl.mixed:
        levels = [int(v) for v in rng.integers(8, 37, wl.batch)]
        kidx = [int(v) for v in rng.integers(0, len(wl.galois), wl.batch)]
    else:
        levels = [wl.levels[0]] * wl.batch
        kidx = [0] * wl.batch
    d = Draw(s, s_prime, _keys(rng, wl))
    want = wl.batch if ct_count is None else min(ct_count, wl.batch)
    for k in range(want):
        d.cts.append(np.stack([residues(rng, primes[:levels[k]], n) for _ in range(2)]))
    d.levels = levels[:want]
    d.key_index = kidx[:want]
    return d


def uniform_key_rows(seed: int, primes: list[int], dnum: int, n: int) -> np.ndarray:
    """Stand-in key half [dnum][L+K][N] of uniform residues (same distribution as a real b-half)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.stack([residues(rng, primes, n) for _ in range(dnum)])
