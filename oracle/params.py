"""Parameter set of one prime chain (oracle; test infrastructure only).

Readings adopted where the pages are silent (they fix only a 32-bit RNS CKKS
chain, Perseus summary on ai4snews, "Interpretation" paragraph 2):

* level l = number of active ciphertext primes, always the prefix q_0..q_{l-1};
* digit width alpha = ceil(L/dnum); digit j holds primes j*alpha .. min((j+1)*alpha, l)-1
  at level l, so the last digit may be partial and there are ceil(l/alpha) digits;
* at level l the extended basis is q_0..q_{l-1} followed by p_0..p_{K-1}; limb e of
  an extended polynomial is absolute prime index e if e < l, else L + (e - l).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from math import prod

from .chain import chain_primes, min_root


@dataclass
class Params:
    n: int
    L: int
    K: int
    dnum: int
    bits: int
    primes: list[int] = field(default_factory=list)
    psis: list[int] = field(default_factory=list)

    @classmethod
    def make(cls, log_n: int, L: int, K: int, dnum: int, bits: int) -> "Params":
        n = 1 << log_n
        primes = chain_primes(n, bits, L + K)
        return cls(n=n, L=L, K=K, dnum=dnum, bits=bits, primes=primes,
                   psis=[min_root(q, n) for q in primes])

    @property
    def alpha(self) -> int:
        return -(-self.L // self.dnum)

    @property
    def q(self) -> list[int]:
        return self.primes[:self.L]

    @property
    def p(self) -> list[int]:
        return self.primes[self.L:]

    @property
    def P(self) -> int:
        return prod(self.p)

    def n_digits(self, level: int) -> int:
        return -(-level // self.alpha)

    def digit(self, j: int, level: int) -> list[int]:
        """Absolute indices of the ciphertext primes of digit j at this level."""
        return list(range(j * self.alpha, min((j + 1) * self.alpha, level)))

    def ext(self, level: int) -> list[int]:
        """Absolute prime index of each limb of the extended basis at this level."""
        return list(range(level)) + list(range(self.L, self.L + self.K))
