"""Seeded random cases of the other entry points against the oracle, bit for bit: the NTT
pair, ModUp, ModDown, hoisted key-switches, multi-item streams, multiply-relinearise-
rescale and the BSGS linear transform, each on randomly drawn small chains (ring 2^12
or 2^13, 2..6 ciphertext primes, any dnum, 30- to 32-bit primes), with random levels,
batch and group sizes (hoisted keys in chunks of max_batch, multi-item streams split
into groups) and keys whose a-half is stored or regenerated.
"""
import functools

import numpy as np
import pytest

from tests.gpu_common import announce, first_mismatch, gpu, host, rand_limbs

pytestmark = pytest.mark.gpu

from oracle import bsgs as obsgs  # noqa: E402
from oracle import ks as oks  # noqa: E402
from oracle import mult as omult  # noqa: E402
from oracle.ntt import intt, ntt  # noqa: E402
from oracle.params import Params  # noqa: E402
from oracle.rns import moddown, modup  # noqa: E402
from rns_ckks_key_amd import synth  # noqa: E402
from rns_ckks_key_amd.api import Context  # noqa: E402

N_CASES = 10


def _shape(rng):
    log_n = int(rng.choice([12, 13]))
    L = int(rng.integers(2, 7))
    dnum = int(rng.integers(1, L + 1))
    alpha = -(-L // dnum)
    K = alpha + int(rng.integers(0, 3))
    bits = int(rng.choice([30, 31, 32]))
    return log_n, L, K, dnum, bits


@functools.lru_cache(maxsize=None)
def _params(shape):
    return Params.make(*shape)


def _ctx(shape, max_batch):
    pr = _params(shape)
    return Context(shape[0], shape[1], shape[2], shape[3], pr.primes, max_batch)


def _key(pr, rng, g):
    s = synth.ternary(rng, pr.n)
    s_src = synth.ternary(rng, pr.n) if g == 1 else oks.rotation_source(s, g, pr)
    errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
    seed = rng.bytes(32)
    kb, ka = oks.keygen(pr, s, s_src, errs, seed)
    return kb, ka, seed


def _galois(rng, n):
    return 1 if rng.integers(0, 6) == 0 else int(rng.integers(0, n)) * 2 + 1


def _ct(rng, pr, level, lead=()):
    return rand_limbs(rng, pr.primes[:level], pr.n, lead + (2,))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_ntt_modup_moddown(case):
    rng = np.random.default_rng(7100 + case)
    shape = _shape(rng)
    pr = _params(shape)
    level = int(rng.integers(1, shape[1] + 1))
    batch = int(rng.integers(1, 6))
    announce(f"random ntt/modup/moddown case {case}: {shape} level={level} batch={batch}")
    ctx = _ctx(shape, batch)
    try:
        first = int(rng.integers(0, shape[1] + shape[2]))
        nl = int(rng.integers(1, shape[1] + shape[2] - first + 1))
        a = rand_limbs(rng, pr.primes[first:first + nl], pr.n, (batch,))
        t = gpu(a)
        ctx.ntt_fwd(t, first)
        got = host(t)
        for b in range(batch):
            want = ntt(a[b], pr.primes[first:first + nl], pr.psis[first:first + nl])
            assert np.array_equal(got[b], want), ("ntt", b, first_mismatch(got[b], want))
        ctx.ntt_inv(t, first)
        assert np.array_equal(host(t), a)
        assert np.array_equal(intt(got[0], pr.primes[first:first + nl], pr.psis[first:first + nl]), a[0])
        c1 = rand_limbs(rng, pr.primes[:level], pr.n, (batch,))
        got = host(ctx.modup(gpu(c1), level))
        want = modup(c1, level, pr)
        assert np.array_equal(got, want), ("modup", first_mismatch(got, want))
        x = rand_limbs(rng, [pr.primes[t] for t in pr.ext(level)], pr.n, (batch,))
        got = host(ctx.moddown(gpu(x), level))
        want = moddown(x, level, pr)
        assert np.array_equal(got, want), ("moddown", first_mismatch(got, want))
    finally:
        ctx.close()


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_hoisted(case):
    rng = np.random.default_rng(7200 + case)
    shape = _shape(rng)
    pr = _params(shape)
    level = int(rng.integers(1, shape[1] + 1))
    n_keys = int(rng.integers(1, 21))
    max_batch = int(rng.choice([1, 2, 4, 16]))
    announce(f"random hoisted case {case}: {shape} level={level} keys={n_keys} max_batch={max_batch}")
    keys, dev = [], []
    for _ in range(n_keys):
        g = _galois(rng, pr.n)
        kb, ka, seed = _key(pr, rng, g)
        stored = bool(rng.integers(0, 2))
        keys.append((kb, ka, g))
        dev.append((gpu(kb), g, None if stored else seed, gpu(ka) if stored else None))
    ct = _ct(rng, pr, level)
    ctx = _ctx(shape, max_batch)
    try:
        got = host(ctx.keyswitch_hoisted(gpu(ct), level, dev))
    finally:
        ctx.close()
    want = oks.keyswitch_hoisted(pr, ct, level, keys)
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_multi_item_stream(case):
    rng = np.random.default_rng(7300 + case)
    shape = _shape(rng)
    pr = _params(shape)
    pool = []
    for _ in range(3):
        g = _galois(rng, pr.n)
        pool.append(_key(pr, rng, g) + (g,))
    n_items = int(rng.integers(1, 25))
    max_batch = int(rng.choice([1, 2, 3, 8]))
    announce(f"random multi case {case}: {shape} items={n_items} max_batch={max_batch}")
    items, want = [], []
    for _ in range(n_items):
        level = int(rng.integers(1, shape[1] + 1))
        kb, ka, seed, g = pool[int(rng.integers(0, 3))]
        ct = _ct(rng, pr, level)
        stored = bool(rng.integers(0, 2))
        items.append((gpu(ct), level, gpu(kb), g, None if stored else seed, gpu(ka) if stored else None, None))
        want.append(oks.keyswitch(pr, ct, level, kb, g, key_a=ka))
    ctx = _ctx(shape, max_batch)
    try:
        outs = ctx.keyswitch_multi(items)
        got = [host(o) for o in outs]
    finally:
        ctx.close()
    for i, (o, w) in enumerate(zip(got, want)):
        assert np.array_equal(o, w), (i, first_mismatch(o, w))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_mul_relin_rescale(case):
    rng = np.random.default_rng(7400 + case)
    shape = _shape(rng)
    pr = _params(shape)
    level = int(rng.integers(2, shape[1] + 1))
    batch = int(rng.choice([1, 2, 4, 5, 8, 9]))
    regen = bool(case % 2)
    announce(f"random mul_relin_rescale case {case}: {shape} level={level} batch={batch} regen={regen}")
    s = synth.ternary(rng, pr.n)
    errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
    seed = rng.bytes(32)
    kb, ka = omult.relin_keygen(pr, s, errs, seed)
    x, y = _ct(rng, pr, level, (batch,)), _ct(rng, pr, level, (batch,))
    ctx = _ctx(shape, batch)
    try:
        got = host(ctx.mul_relin_rescale(gpu(x), gpu(y), level, gpu(kb), key_seed=seed if regen else None,
                                         key_a=None if regen else gpu(ka)))
    finally:
        ctx.close()
    want = omult.mul_relin_rescale(pr, x, y, level, kb, key_a=ka)
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_bsgs(case):
    rng = np.random.default_rng(7500 + case)
    shape = _shape(rng)
    pr = _params(shape)
    level = int(rng.integers(1, shape[1] + 1))
    n1, n2 = int(rng.integers(1, 5)), int(rng.integers(1, 4))
    announce(f"random bsgs case {case}: {shape} level={level} n1={n1} n2={n2}")

    def keys(count):
        ora, dev = [], []
        for _ in range(count):
            g = _galois(rng, pr.n)
            kb, ka, seed = _key(pr, rng, g)
            stored = bool(rng.integers(0, 2))
            ora.append({"b": kb, "a": ka if stored else None, "seed": seed, "g": g})
            dev.append((gpu(kb), g, None if stored else seed, gpu(ka) if stored else None))
        return ora, dev

    ob, db = keys(n1 - 1)
    og, dg = keys(n2 - 1)
    ct = _ct(rng, pr, level)
    diags = rand_limbs(rng, [pr.primes[t] for t in pr.ext(level)], pr.n, (n2, n1))
    ctx = _ctx(shape, 16)
    try:
        got = host(ctx.linear_transform_bsgs(gpu(ct), level, gpu(diags), db, dg))
    finally:
        ctx.close()
    want = obsgs.linear_transform(pr, ct, level, diags, ob, og)
    assert np.array_equal(got, want), first_mismatch(got, want)
