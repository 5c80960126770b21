"""GPU parity of the matrix-core base conversion (ckks_ctx_set_conv_mfma) on the N=2^16 chain.

ModUp and ModDown through the int8 matrix-core kernel are compared with the oracle
at full size, and at every level with batches 1, 2 and 3 (which change how the
targets are split over workgroups) bit for bit with the vector-unit kernel, itself
checked against the oracle in the other test files.  The key-switch (batch 8,
regenerated and stored a-half), the hoisted key-switch, multiply-relinearise-rescale
and the BSGS transform run through both paths and must agree bit for bit; one
key-switched ciphertext is also checked against the oracle.
"""
import functools

import numpy as np
import pytest

from tests.gpu_common import CHAINS, announce, first_mismatch, gpu, host, params, rand_limbs, torch

pytestmark = pytest.mark.gpu

from oracle import ks as oks  # noqa: E402
from oracle.chacha import expand_key_a  # noqa: E402
from oracle.rns import moddown, modup  # noqa: E402
from rns_ckks_key_amd import synth  # noqa: E402
from rns_ckks_key_amd.api import CkksError, Context  # noqa: E402


@functools.lru_cache(maxsize=None)
def mx_context() -> Context:
    log_n, L, K, dnum, bits = CHAINS["boot"]
    return Context(log_n, L, K, dnum, params("boot").primes, 8)


def both_paths(fn):
    """(vector-path result, matrix-core result) of fn(ctx), as device tensors."""
    ctx = mx_context()
    try:
        ctx.set_conv_mfma(False)
        a = fn(ctx).clone()
        ctx.set_conv_mfma(True)
        b = fn(ctx).clone()
    finally:
        ctx.set_conv_mfma(False)
    torch.cuda.synchronize()
    return a, b


def assert_same(a, b, what):
    if not torch.equal(a, b):
        ha, hb = host(a), host(b)
        pytest.fail(f"{what}: {first_mismatch(hb, ha)}")


@functools.lru_cache(maxsize=None)
def key_rows(seed_int: int):
    pr = params("boot")
    return synth.uniform_key_rows(seed_int, pr.primes, pr.dnum, pr.n).astype(np.uint64)


@pytest.mark.parametrize("level", [36, 13])
def test_modup_matrix_cores_against_oracle(level):
    announce(f"mfma modup level={level}")
    pr = params("boot")
    ctx = mx_context()
    rng = np.random.default_rng(300 + level)
    c1 = rand_limbs(rng, pr.primes[:level], pr.n, (1,))
    c1[0, 0, :5] = 0
    c1[0, level - 1, :5] = pr.primes[level - 1] - 1
    ctx.set_conv_mfma(True)
    try:
        got = host(ctx.modup(gpu(c1), level))
    finally:
        ctx.set_conv_mfma(False)
    want = modup(c1, level, pr)
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("level", [36, 5])
def test_moddown_matrix_cores_against_oracle(level):
    announce(f"mfma moddown level={level}")
    pr = params("boot")
    ctx = mx_context()
    rng = np.random.default_rng(400 + level)
    ext = [pr.primes[t] for t in pr.ext(level)]
    x = rand_limbs(rng, ext, pr.n, (2,))
    ctx.set_conv_mfma(True)
    try:
        got = host(ctx.moddown(gpu(x), level))
    finally:
        ctx.set_conv_mfma(False)
    want = moddown(x, level, pr)
    assert np.array_equal(got, want), first_mismatch(got, want)


def test_modup_moddown_every_level_both_paths_agree():
    pr = params("boot")
    rng = np.random.default_rng(77)
    for level in range(1, pr.L + 1):
        batch = 1 + level % 3
        announce(f"mfma vs vector level={level} batch={batch}")
        c1 = gpu(rand_limbs(rng, pr.primes[:level], pr.n, (batch,)))
        a, b = both_paths(lambda ctx: ctx.modup(c1, level))
        assert_same(a, b, f"modup level {level}")
        ext = [pr.primes[t] for t in pr.ext(level)]
        x = gpu(rand_limbs(rng, ext, pr.n, (batch,)))
        a, b = both_paths(lambda ctx: ctx.moddown(x, level))
        assert_same(a, b, f"moddown level {level}")


@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_keyswitch_batch8_both_paths_and_oracle(variant):
    announce(f"mfma keyswitch batch 8 {variant}")
    pr = params("boot")
    rng = np.random.default_rng(5)
    kb = key_rows(9001)
    seed = bytes(range(100, 132))
    ka = expand_key_a(seed, pr.primes, pr.dnum, pr.n)
    ct = np.stack([np.stack([rand_limbs(rng, pr.primes[:36], pr.n) for _ in range(2)]) for _ in range(8)])
    dct, dkb, dka = gpu(ct), gpu(kb), gpu(ka)
    a, b = both_paths(lambda ctx: ctx.keyswitch(dct, 36, dkb, 5, key_seed=seed if variant == "regen" else None,
                                                 key_a=dka if variant == "stored" else None))
    assert_same(a, b, "keyswitch")
    if variant == "regen":
        want = oks.keyswitch(pr, ct[6], 36, kb, 5, key_a=ka)
        got = host(b)[6]
        assert np.array_equal(got, want), first_mismatch(got, want)


def test_hoisted_multiply_and_bsgs_both_paths_agree():
    pr = params("boot")
    rng = np.random.default_rng(6)
    seeds = [bytes([k]) * 32 for k in range(3)]
    kbs = [gpu(key_rows(9100 + k)) for k in range(3)]
    announce("mfma hoisted 3 keys level 24")
    ct = gpu(np.stack([rand_limbs(rng, pr.primes[:24], pr.n) for _ in range(2)]))
    keys = [(kbs[k], pow(5, k + 1, 2 * pr.n), seeds[k], None) for k in range(3)]
    a, b = both_paths(lambda ctx: ctx.keyswitch_hoisted(ct, 24, keys))
    assert_same(a, b, "hoisted")
    announce("mfma multiply-relinearise-rescale batch 3 level 36")
    x = gpu(np.stack([np.stack([rand_limbs(rng, pr.primes[:36], pr.n) for _ in range(2)]) for _ in range(3)]))
    y = gpu(np.stack([np.stack([rand_limbs(rng, pr.primes[:36], pr.n) for _ in range(2)]) for _ in range(3)]))
    a, b = both_paths(lambda ctx: ctx.mul_relin_rescale(x, y, 36, kbs[0], key_seed=seeds[0]))
    assert_same(a, b, "mul_relin_rescale")
    announce("mfma bsgs 2x3 level 13")
    ct13 = gpu(np.stack([rand_limbs(rng, pr.primes[:13], pr.n) for _ in range(2)]))
    ext = [pr.primes[t] for t in pr.ext(13)]
    diags = gpu(rand_limbs(rng, ext, pr.n, (3, 2)))
    baby = [(kbs[1], 5, seeds[1], None)]
    giant = [(kbs[2], 25, seeds[2], None), (kbs[0], 625, seeds[0], None)]
    a, b = both_paths(lambda ctx: ctx.linear_transform_bsgs(ct13, 13, diags, baby, giant))
    assert_same(a, b, "bsgs")


def test_multi_item_both_paths_agree():
    # six items at four levels: launch sequences on several streams, matrix-core conversions in each
    pr = params("boot")
    rng = np.random.default_rng(8)
    kbs = [gpu(key_rows(9200 + k)) for k in range(2)]
    announce("mfma multi-item 6 items")
    items = []
    for i, level in enumerate((36, 24, 13, 36, 5, 24)):
        ct = gpu(np.stack([rand_limbs(rng, pr.primes[:level], pr.n) for _ in range(2)]))
        out = torch.empty((2, level, pr.n), dtype=torch.int32, device="cuda")
        items.append((ct, level, kbs[i % 2], pow(5, i + 1, 2 * pr.n), bytes([i]) * 32, None, out))

    def run(ctx):
        ctx.keyswitch_multi(items)
        return torch.cat([it[6].flatten() for it in items])

    a, b = both_paths(run)
    assert_same(a, b, "multi")


def test_matrix_cores_refused_for_other_shapes():
    announce("mfma unsupported shape")
    pr = params("tiny")
    log_n, L, K, dnum, bits = CHAINS["tiny"]
    ctx = Context(log_n, L, K, dnum, pr.primes, 2)
    with pytest.raises(CkksError) as ei:
        ctx.set_conv_mfma(True)
    assert ei.value.name == "CKKS_EUNSUPPORTED"
    ctx.close()
