"""Pins of the oracle's ModUp and ModDown against their big-integer closed forms.

ModUp (fast base conversion without correction): with x = CRT_{Q~}(x_i) in [0, Q~)
there is one integer u with 0 <= u < alpha' such that every output limb is
x + u*Q~ modulo its prime.  ModDown (floor type): with X = CRT_{PQ}(acc) and
[X]_P = X mod P there is one integer v with 0 <= v < K such that
out = (X - [X]_P - v*P)/P modulo every q_i.
"""
import numpy as np
import pytest

from oracle.chain import crt
from oracle.ntt import intt, ntt
from oracle.params import Params
from oracle.rns import moddown, modup


def _small(log_n=4, L=6, K=3, dnum=2, bits=32):
    return Params.make(log_n, L, K, dnum, bits)


@pytest.mark.parametrize("pr_args,level", [((4, 6, 3, 2, 32), 6), ((4, 6, 3, 2, 32), 4), ((4, 6, 3, 2, 32), 2),
                                           ((5, 5, 2, 3, 30), 5), ((5, 5, 2, 3, 30), 3), ((12, 4, 2, 2, 30), 4)])
def test_modup_closed_form(pr_args, level):
    pr = Params.make(*pr_args)
    rng = np.random.default_rng(level)
    qs = pr.primes[:level]
    c1 = np.stack([rng.integers(0, q, pr.n, dtype=np.uint64) for q in qs])
    c1[0, :3] = [0, qs[0] - 1, 1]
    digits = modup(c1, level, pr)
    ext = pr.ext(level)
    x = intt(c1, qs, pr.psis[:level])
    coeff = np.stack([intt(digits[j], [pr.primes[t] for t in ext], [pr.psis[t] for t in ext])
                      for j in range(pr.n_digits(level))])
    cols = range(pr.n) if pr.n <= 64 else np.random.default_rng(1).integers(0, pr.n, 48)
    for j in range(pr.n_digits(level)):
        dig = pr.digit(j, level)
        qt = 1
        for i in dig:
            qt *= pr.primes[i]
        for c in cols:
            xi = [int(x[i, c]) for i in dig]
            xv = crt(xi, [pr.primes[i] for i in dig])
            ys = [xi[k] * pow(qt // pr.primes[i], -1, pr.primes[i]) % pr.primes[i] for k, i in enumerate(dig)]
            s = sum(y * (qt // pr.primes[i]) for y, i in zip(ys, dig))
            assert (s - xv) % qt == 0
            u = (s - xv) // qt
            assert 0 <= u < len(dig)
            for e, t in enumerate(ext):
                assert int(coeff[j, e, c]) == (xv + u * qt) % pr.primes[t]


@pytest.mark.parametrize("pr_args,level", [((4, 6, 3, 2, 32), 6), ((4, 6, 3, 2, 32), 1), ((5, 5, 2, 3, 30), 4),
                                           ((12, 4, 2, 2, 30), 4)])
def test_moddown_closed_form(pr_args, level):
    pr = Params.make(*pr_args)
    rng = np.random.default_rng(10 + level)
    ext = pr.ext(level)
    mods = [pr.primes[t] for t in ext]
    xc = np.stack([rng.integers(0, m, pr.n, dtype=np.uint64) for m in mods])
    xc[:, 0] = 0
    xhat = ntt(xc, mods, [pr.psis[t] for t in ext])
    out = intt(moddown(xhat, level, pr), pr.primes[:level], pr.psis[:level])
    big_p = pr.P
    cols = range(pr.n) if pr.n <= 64 else np.random.default_rng(2).integers(0, pr.n, 48)
    for c in cols:
        X = crt([int(v) for v in xc[:, c]], mods)
        xp = X % big_p
        ys = [int(xc[level + k, c]) * pow(big_p // pk, -1, pk) % pk for k, pk in enumerate(pr.p)]
        s = sum(y * (big_p // pk) for y, pk in zip(ys, pr.p))
        assert (s - xp) % big_p == 0
        v = (s - xp) // big_p
        assert 0 <= v < pr.K
        ref = (X - xp - v * big_p)
        assert ref % big_p == 0
        ref //= big_p
        for i in range(level):
            assert int(out[i, c]) == ref % pr.primes[i]


def test_modup_digit_structure():
    pr = Params.make(4, 36, 12, 3, 32)
    assert pr.alpha == 12 and pr.n_digits(36) == 3 and pr.n_digits(24) == 2 and pr.n_digits(4) == 1
    assert pr.digit(0, 4) == [0, 1, 2, 3] and pr.digit(2, 30) == list(range(24, 30))
    assert pr.ext(8) == list(range(8)) + list(range(36, 48))
    pr1 = Params.make(12, 4, 2, 2, 30)
    assert pr1.alpha == 2 and pr1.n_digits(4) == 2 and pr1.n_digits(3) == 2 and pr1.n_digits(2) == 1
