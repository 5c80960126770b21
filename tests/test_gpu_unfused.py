"""GPU parity of the unfused key-switch (ckks_ctx_set_fused(ctx, 0)): ModUp, the digits' row
NTT, the inner product over all level+K primes and a standalone ModDown as separate launches.

Its outputs must equal the oracle's and the fused key-switch's bit for bit: ModDown of
P*sigma(c0) + acc is sigma(c0) + ModDown(acc) exactly (Han and Ki, 2020).
"""
import numpy as np
import pytest

from tests.gpu_common import announce, context, first_mismatch, gpu, host, params, rand_limbs
from tests.test_gpu_keyswitch import _batch8_case, _ct, oracle_key

pytestmark = pytest.mark.gpu

from oracle import ks as oks  # noqa: E402
from oracle.params import Params  # noqa: E402
from rns_ckks_key_amd import synth  # noqa: E402
from rns_ckks_key_amd.api import CkksError, Context  # noqa: E402


def _both_routes(ctx, ct, level, kb, g, kw):
    """(unfused output, fused output) of one key-switch call on the same context."""
    ctx.set_fused(False)
    try:
        unf = host(ctx.keyswitch(gpu(ct), level, kb, g, **kw))
    finally:
        ctx.set_fused(True)
    return unf, host(ctx.keyswitch(gpu(ct), level, kb, g, **kw))


@pytest.mark.parametrize("g", [5, 8191])
@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_unfused_tiny_every_level(g, variant):
    announce(f"unfused keyswitch tiny g={g} {variant}")
    pr = params("tiny")
    ctx = context("tiny", 3)
    kb, ka, seed, s, s_src = oracle_key("tiny", g)
    kw = dict(key_seed=seed) if variant == "regen" else dict(key_a=gpu(ka))
    rng = np.random.default_rng(50 + g)
    for level in (4, 3, 2, 1):
        ct = _ct(rng, pr, level, 3)
        if level == 4:
            ct[1, 1] = 0  # c1 = 0: the output is (sigma(c0), 0)
        unf, fused = _both_routes(ctx, ct, level, gpu(kb), g, kw)
        want = oks.keyswitch(pr, ct, level, kb, g, key_a=ka)
        assert np.array_equal(unf, want), (level, first_mismatch(unf, want))
        assert np.array_equal(unf, fused), (level, first_mismatch(unf, fused))


def test_unfused_in_groups_and_the_workspace_limit():
    # L = K = 4, dnum 1: a pair of 8 extended limbs per ciphertext, so a context of
    # max_batch 4 (3*4*4 words of pairs per coefficient) takes the batch of 4 in groups
    # of 2 (ModDown's row buffer bounds it too); max_batch 1 cannot hold one pair
    shape = (12, 4, 4, 1, 30)
    announce(f"unfused keyswitch in groups {shape}")
    pr = Params.make(*shape)
    rng = np.random.default_rng(4141)
    g = 25
    s = synth.ternary(rng, pr.n)
    errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
    seed = rng.bytes(32)
    kb, ka = oks.keygen(pr, s, oks.rotation_source(s, g, pr), errs, seed)
    ctx = Context(shape[0], shape[1], shape[2], shape[3], pr.primes, 4)
    for level, batch in ((4, 4), (3, 3), (1, 4)):
        ct = np.stack([np.stack([rand_limbs(rng, pr.primes[:level], pr.n) for _ in range(2)]) for _ in range(batch)])
        for kw in (dict(key_seed=seed), dict(key_a=gpu(ka))):
            unf, fused = _both_routes(ctx, ct, level, gpu(kb), g, kw)
            want = oks.keyswitch(pr, ct, level, kb, g, key_a=ka)
            assert np.array_equal(unf, want), (level, first_mismatch(unf, want))
            assert np.array_equal(unf, fused), (level, first_mismatch(unf, fused))
    small = Context(shape[0], shape[1], shape[2], shape[3], pr.primes, 1)
    small.set_fused(False)
    ct = np.stack([np.stack([rand_limbs(rng, pr.primes[:4], pr.n) for _ in range(2)])])
    with pytest.raises(CkksError) as ei:
        small.keyswitch(gpu(ct), 4, gpu(kb), g, key_seed=seed)
    assert ei.value.name == "CKKS_ERANGE"
    small.set_fused(True)
    got = host(small.keyswitch(gpu(ct), 4, gpu(kb), g, key_seed=seed))
    assert np.array_equal(got, oks.keyswitch(pr, ct, 4, kb, g, key_a=ka))


@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_unfused_boot_batch8_every_ciphertext(variant):
    # the single key-switch workload's shape through the unfused route: every ciphertext
    # against the oracle (the same cases as the fused test of that shape)
    announce(f"unfused keyswitch boot batch 8 {variant}")
    ctx = context("boot", 8)
    kb, ka, seed, s, s_src = oracle_key("boot", 5)
    ct, want = _batch8_case()
    ctx.set_fused(False)
    got = host(ctx.keyswitch(gpu(ct), 36, gpu(kb), 5, key_seed=seed if variant == "regen" else None,
                             key_a=gpu(ka) if variant == "stored" else None))
    for b in range(8):
        assert np.array_equal(got[b], want[b]), (b, first_mismatch(got[b], want[b]))


def test_unfused_boot_partial_digits_equal_fused():
    announce("unfused keyswitch boot levels 24, 13, 4")
    pr = params("boot")
    ctx = context("boot", 16)
    kb, ka, seed, s, s_src = oracle_key("boot", 5)
    rng = np.random.default_rng(2413)
    for level, batch in ((24, 16), (13, 3), (4, 2)):
        ct = _ct(rng, pr, level, batch)
        unf, fused = _both_routes(ctx, ct, level, gpu(kb), 5, dict(key_seed=seed))
        assert np.array_equal(unf, fused), (level, first_mismatch(unf, fused))
    want = oks.keyswitch(pr, ct[1], 4, kb, 5, key_a=ka)
    assert np.array_equal(unf[1], want), first_mismatch(unf[1], want)
