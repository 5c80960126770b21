"""GPU parity on ring sizes and digit shapes beyond the five workloads, and call-level behaviour.

Ring degrees 2^13..2^15 exercise the other column-pass lengths; dnum = 1 (one
digit covering every ciphertext prime) and alpha = 1 (one prime per digit) are
the extreme digit shapes; a partial last digit appears at several levels.  Rings
2^15 and 2^16 with 31-bit primes take the column kernels' canonical butterflies
(chains whose primes all exceed 2^31 take the lazy ones).
"""
import functools

import numpy as np
import pytest

from tests.gpu_common import announce, first_mismatch, gpu, host, rand_limbs, torch
from oracle.pool import keyswitch_many

pytestmark = pytest.mark.gpu

from oracle import ks as oks  # noqa: E402
from oracle.chacha import expand_key_a  # noqa: E402
from oracle.ntt import intt, ntt  # noqa: E402
from oracle.params import Params  # noqa: E402
from rns_ckks_key_amd import synth  # noqa: E402
from rns_ckks_key_amd.api import CkksError, Context  # noqa: E402

SHAPES = [  # (log_n, L, K, dnum, bits)
    (13, 6, 3, 2, 32),
    (14, 5, 3, 2, 32),
    (15, 8, 4, 2, 32),
    (12, 4, 4, 1, 30),   # dnum = 1
    (12, 4, 1, 4, 30),   # alpha = 1
    (13, 7, 3, 3, 31),   # partial digits, 31-bit primes
    (15, 6, 3, 2, 31),   # large rings with primes below 2^31: the canonical-butterfly column kernels
    (16, 4, 2, 2, 31),
]


@functools.lru_cache(maxsize=None)
def setup(shape):
    pr = Params.make(*shape)
    ctx = Context(shape[0], shape[1], shape[2], shape[3], pr.primes, 4)
    return pr, ctx


@pytest.mark.parametrize("shape", SHAPES)
def test_ntt_other_rings(shape):
    announce(f"ntt shape {shape}")
    pr, ctx = setup(shape)
    rng = np.random.default_rng(shape[0] + shape[1])
    nl = pr.L + pr.K
    a = rand_limbs(rng, pr.primes, pr.n, (2,))
    t = gpu(a)
    ctx.ntt_fwd(t, 0)
    want = ntt(a, pr.primes, pr.psis)
    got = host(t)
    assert np.array_equal(got, want), first_mismatch(got, want)
    ctx.ntt_inv(t, 0)
    assert np.array_equal(host(t), a)
    assert nl == len(pr.primes)


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_keyswitch_other_shapes_every_level(shape, variant):
    announce(f"keyswitch shape {shape} {variant}")
    pr, ctx = setup(shape)
    rng = np.random.default_rng(7 * shape[0] + shape[3])
    g = 5
    s = synth.ternary(rng, pr.n)
    s_src = oks.rotation_source(s, g, pr)
    errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
    seed = rng.bytes(32)
    kb, ka = oks.keygen(pr, s, s_src, errs, seed)
    dkb, dka = gpu(kb), gpu(ka)
    for level in range(1, pr.L + 1):
        ct = np.stack([np.stack([rand_limbs(rng, pr.primes[:level], pr.n) for _ in range(2)]) for _ in range(2)])
        got = host(ctx.keyswitch(gpu(ct), level, dkb, g, key_seed=seed if variant == "regen" else None,
                                 key_a=dka if variant == "stored" else None))
        want = oks.keyswitch(pr, ct, level, kb, g, key_a=ka)
        assert np.array_equal(got, want), (level, first_mismatch(got, want))
    assert oks.switch_error(pr, ct[0], got[0], pr.L, s, s_src, g) < oks.noise_bound(pr, pr.L)


def test_expand_a_other_ring():
    shape = (15, 8, 4, 2, 32)
    pr, ctx = setup(shape)
    seed = bytes(range(40, 72))
    got = host(ctx.expand_a(seed))
    assert np.array_equal(got, expand_key_a(seed, pr.primes, pr.dnum, pr.n))


def test_batch_limit_and_argument_errors_on_device():
    shape = (13, 6, 3, 2, 32)
    pr, ctx = setup(shape)
    ct = torch.zeros((5, 2, 6, pr.n), dtype=torch.int32, device="cuda")
    kb = torch.zeros((2, 9, pr.n), dtype=torch.int32, device="cuda")
    with pytest.raises(CkksError) as ei:
        ctx.keyswitch(ct, 6, kb, 5, key_seed=bytes(32))  # batch 5 > max_batch 4
    assert ei.value.name == "CKKS_ERANGE"
    with pytest.raises(CkksError):
        ctx.keyswitch(ct[:2], 6, kb, 6, key_seed=bytes(32))  # even Galois element
    with pytest.raises(ValueError):
        ctx.keyswitch(ct[:2], 5, kb, 5, key_seed=bytes(32))  # shape does not match the level


def test_repeatable_and_stream_ordered():
    # same inputs -> identical bits, on the default stream and on a side stream
    shape = (14, 5, 3, 2, 32)
    pr, ctx = setup(shape)
    rng = np.random.default_rng(3)
    ct = gpu(np.stack([np.stack([rand_limbs(rng, pr.primes[:5], pr.n) for _ in range(2)]) for _ in range(3)]))
    kb = gpu(synth.uniform_key_rows(9, pr.primes, pr.dnum, pr.n))
    seed = bytes(32)
    first = host(ctx.keyswitch(ct, 5, kb, 25, key_seed=seed))
    for _ in range(3):
        assert np.array_equal(host(ctx.keyswitch(ct, 5, kb, 25, key_seed=seed)), first)
    side = torch.cuda.Stream()
    with torch.cuda.stream(side):
        out = ctx.keyswitch(ct, 5, kb, 25, key_seed=seed)
    side.synchronize()
    assert np.array_equal(host(out), first)


@pytest.mark.parametrize("shape,levels", [((14, 5, 3, 2, 32), (4,)), ((15, 8, 4, 2, 32), (8, 5, 4))])
def test_keyswitch_batch4_conversion_remainders(shape, levels):
    # batch 4 puts the conversions' last partial round of (target, column) tasks on
    # 2 or 4 lanes per task: 4 targets per workgroup (ring 2^14, level 4; ring 2^15,
    # level 4's ModDown) and 8 (ring 2^15, levels 8 and 5)
    announce(f"keyswitch shape {shape} batch 4")
    pr, ctx = setup(shape)
    rng = np.random.default_rng(11 * shape[0])
    g = 25
    s = synth.ternary(rng, pr.n)
    s_src = oks.rotation_source(s, g, pr)
    errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
    seed = rng.bytes(32)
    kb, ka = oks.keygen(pr, s, s_src, errs, seed)
    dkb = gpu(kb)
    for level in levels:
        ct = np.stack([np.stack([rand_limbs(rng, pr.primes[:level], pr.n) for _ in range(2)]) for _ in range(4)])
        got = host(ctx.keyswitch(gpu(ct), level, dkb, g, key_seed=seed))
        want = oks.keyswitch(pr, ct, level, kb, g, key_a=ka)
        assert np.array_equal(got, want), (level, first_mismatch(got, want))


@functools.lru_cache(maxsize=None)
def setup_wide():
    shape = (12, 8, 2, 8, 30)  # dnum = 8, the largest digit count: eight key tiles per workgroup
    pr = Params.make(*shape)
    return pr, Context(shape[0], shape[1], shape[2], shape[3], pr.primes, 12)


@pytest.mark.parametrize("batch", [4, 5, 8, 12])
def test_keyswitch_batches_eight_digits(batch):
    # batches of 4..7 and of 8 or more take the multi-wave inner-product kernels;
    # eight digits make the regenerated tiles span more than one pass of the workgroup
    announce(f"keyswitch dnum 8 batch {batch}")
    pr, ctx = setup_wide()
    rng = np.random.default_rng(100 + batch)
    g = 3 ** 5 % (2 * pr.n)
    s = synth.ternary(rng, pr.n)
    s_src = oks.rotation_source(s, g, pr)
    errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
    seed = rng.bytes(32)
    kb, ka = oks.keygen(pr, s, s_src, errs, seed)
    dkb, dka = gpu(kb), gpu(ka)
    for level in (pr.L, 5):
        ct = np.stack([np.stack([rand_limbs(rng, pr.primes[:level], pr.n) for _ in range(2)]) for _ in range(batch)])
        want = oks.keyswitch(pr, ct, level, kb, g, key_a=ka)
        for variant in ("regen", "stored"):
            got = host(ctx.keyswitch(gpu(ct), level, dkb, g, key_seed=seed if variant == "regen" else None,
                                     key_a=dka if variant == "stored" else None))
            assert np.array_equal(got, want), (variant, level, first_mismatch(got, want))


@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_smaller_ring_workload(variant):
    # the smaller-ring benchmark configuration: N=2^15, 20+7 primes of 32 bits, dnum 3,
    # batch 8 at level 20, g = 5; every ciphertext against the oracle
    announce(f"smaller ring batch 8 level 20 {variant}")
    shape = (15, 20, 7, 3, 32)
    pr = Params.make(*shape)
    ctx = Context(shape[0], shape[1], shape[2], shape[3], pr.primes, 8)
    rng = np.random.default_rng(8008)
    ct = np.stack([np.stack([rand_limbs(rng, pr.primes[:20], pr.n) for _ in range(2)]) for _ in range(8)])
    kb = synth.uniform_key_rows(8000, pr.primes, pr.dnum, pr.n).astype(np.uint64)
    seed = rng.bytes(32)
    ka = expand_key_a(seed, pr.primes, pr.dnum, pr.n)
    got = host(ctx.keyswitch(gpu(ct), 20, gpu(kb), 5, key_seed=seed if variant == "regen" else None,
                             key_a=gpu(ka) if variant == "stored" else None))
    wants = keyswitch_many(shape, kb, ka, [(ct[b], 20, 5) for b in range(8)])
    for b, want in enumerate(wants):
        assert np.array_equal(got[b], want), (b, first_mismatch(got[b], want))
    ctx.close()


@pytest.mark.parametrize("shape", [(15, 36, 12, 3, 32), (15, 36, 12, 3, 31), (16, 36, 12, 3, 31)])
def test_wide_conversion_workgroups_other_rings(shape):
    # batch 8 at level 36: both conversions have 36 targets x 16 columns per
    # workgroup and take 512-thread workgroups; ring 2^15 (32-bit primes: lazy
    # column butterflies; 31-bit: canonical) and ring 2^16 with 31-bit primes cover
    # the instantiations the main chain does not; every ciphertext against the oracle
    announce(f"wide conversion shape {shape} batch 8 level 36")
    pr = Params.make(*shape)
    ctx = Context(shape[0], shape[1], shape[2], shape[3], pr.primes, 8)
    rng = np.random.default_rng(3600 + shape[0] + shape[4])
    ct = np.stack([np.stack([rand_limbs(rng, pr.primes[:36], pr.n) for _ in range(2)]) for _ in range(8)])
    kb = synth.uniform_key_rows(3601, pr.primes, pr.dnum, pr.n).astype(np.uint64)
    seed = rng.bytes(32)
    ka = expand_key_a(seed, pr.primes, pr.dnum, pr.n)
    got = host(ctx.keyswitch(gpu(ct), 36, gpu(kb), 25, key_seed=seed))
    wants = keyswitch_many(shape, kb, ka, [(ct[b], 36, 25) for b in range(8)])
    for b, want in enumerate(wants):
        assert np.array_equal(got[b], want), (b, first_mismatch(got[b], want))
    ctx.close()
