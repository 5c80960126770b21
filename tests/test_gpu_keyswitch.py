"""GPU parity of ModUp, ModDown, the a-half expander, key-switch and hoisted key-switch with the oracle.

Every comparison is bit-exact on every residue, on every ciphertext of the batch.
Full-size cases run the oracle on the host's cores (oracle.pool), as it takes
several seconds per ciphertext at level 36.
"""
import functools

import numpy as np
import pytest

from tests.gpu_common import CHAINS, announce, context, first_mismatch, gpu, host, params, rand_limbs, torch
from oracle.pool import keyswitch_many

pytestmark = pytest.mark.gpu

from oracle import ks as oks  # noqa: E402
from oracle.automorph import automorph_ntt  # noqa: E402
from oracle.chacha import expand_key_a, expand_row  # noqa: E402
from oracle.rns import moddown, modup  # noqa: E402
from rns_ckks_key_amd import synth  # noqa: E402


@functools.lru_cache(maxsize=None)
def oracle_key(name: str, g: int, seed_id: int = 0):
    """(key_b, key_a, seed, s, s_src) from the oracle's keygen on seeded secrets."""
    pr = params(name)
    rng = np.random.default_rng(1234 + seed_id + 17 * g)
    s = synth.ternary(rng, pr.n)
    s_src = synth.ternary(rng, pr.n) if g == 1 else oks.rotation_source(s, g, pr)
    errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
    seed = rng.bytes(32)
    kb, ka = oks.keygen(pr, s, s_src, errs, seed)
    return kb, ka, seed, s, s_src


@pytest.mark.parametrize("name,level,batch", [("tiny", 4, 2), ("tiny", 3, 1), ("tiny", 1, 1), ("boot", 36, 1),
                                              ("boot", 13, 1), ("boot", 4, 1)])
def test_modup_bit_exact(name, level, batch):
    announce(f"modup {name} level={level} batch={batch}")
    pr = params(name)
    ctx = context(name, 4)
    rng = np.random.default_rng(level)
    c1 = rand_limbs(rng, pr.primes[:level], pr.n, (batch,))
    got = host(ctx.modup(gpu(c1), level))
    want = modup(c1, level, pr)
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("name,level,batch", [("tiny", 4, 2), ("tiny", 2, 1), ("boot", 36, 1), ("boot", 5, 2)])
def test_moddown_bit_exact(name, level, batch):
    announce(f"moddown {name} level={level} batch={batch}")
    pr = params(name)
    ctx = context(name, 4)
    rng = np.random.default_rng(100 + level)
    ext = [pr.primes[t] for t in pr.ext(level)]
    x = rand_limbs(rng, ext, pr.n, (batch,))
    got = host(ctx.moddown(gpu(x), level))
    want = moddown(x, level, pr)
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("name", ["tiny", "boot"])
def test_expand_a_matches_oracle(name):
    announce(f"expand_a {name}")
    pr = params(name)
    ctx = context(name, 4)
    seed = bytes(range(3, 35))
    got = host(ctx.expand_a(seed))
    if name == "tiny":
        want = expand_key_a(seed, pr.primes, pr.dnum, pr.n)
        assert np.array_equal(got, want), first_mismatch(got, want)
    else:
        for j, t in [(0, 0), (1, 17), (2, 35), (0, 36), (2, 47)]:
            want = expand_row(seed, j, t, pr.primes[t], pr.n)
            assert np.array_equal(got[j, t], want), (j, t, first_mismatch(got[j, t], want))


def _ct(rng, pr, level, batch):
    return np.stack([np.stack([rand_limbs(rng, pr.primes[:level], pr.n) for _ in range(2)]) for _ in range(batch)])


@pytest.mark.parametrize("g", [1, 5, 25, 8191])
@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_keyswitch_tiny_all_levels(g, variant):
    announce(f"keyswitch tiny g={g} {variant}")
    pr = params("tiny")
    ctx = context("tiny", 4)
    kb, ka, seed, s, s_src = oracle_key("tiny", g)
    dkb, dka = gpu(kb), gpu(ka)
    rng = np.random.default_rng(g)
    for level in (4, 3, 2, 1):
        ct = _ct(rng, pr, level, 3)
        if level == 4:
            ct[1, 1] = 0  # c1 = 0 in the middle ciphertext
            ct[2, :, 0] = pr.primes[0] - 1
        out = ctx.keyswitch(gpu(ct), level, dkb, g, key_seed=seed if variant == "regen" else None,
                            key_a=dka if variant == "stored" else None)
        got = host(out)
        want = oks.keyswitch(pr, ct, level, kb, g, key_a=ka)
        assert np.array_equal(got, want), (level, first_mismatch(got, want))
        if level == 4:
            assert np.array_equal(got[1, 0], automorph_ntt(ct[1, 0], g)) and not got[1, 1].any()
            err = oks.switch_error(pr, ct[0], got[0], level, s, s_src, g)
            assert err < oks.noise_bound(pr, level)


def test_keyswitch_regen_continuation_path():
    # with exactly 64 blocks per tile, every tile with a rejected word takes the continuation path
    announce("keyswitch tiny continuation")
    pr = params("tiny")
    ctx = context("tiny", 4)
    kb, ka, seed, s, s_src = oracle_key("tiny", 5)
    rng = np.random.default_rng(5)
    ct = _ct(rng, pr, 4, 4)
    ctx.set_regen_blocks(64)
    try:
        got = host(ctx.keyswitch(gpu(ct), 4, gpu(kb), 5, key_seed=seed))
        a = host(ctx.expand_a(seed))
    finally:
        ctx.set_regen_blocks(68)
    assert np.array_equal(a, ka)
    assert np.array_equal(got, oks.keyswitch(pr, ct, 4, kb, 5, key_a=ka))


def test_hoisted_tiny_equals_oracle():
    announce("hoisted tiny")
    pr = params("tiny")
    ctx = context("tiny", 2)
    keys = [oracle_key("tiny", g, 3) for g in (5, 25, 125, 1)]
    rng = np.random.default_rng(77)
    ct = _ct(rng, pr, 4, 1)[0]
    dk = [(gpu(k[0]), g, k[2], gpu(k[1]) if i % 2 else None) for i, (k, g) in enumerate(zip(keys, (5, 25, 125, 1)))]
    got = host(ctx.keyswitch_hoisted(gpu(ct), 4, dk))
    want = oks.keyswitch_hoisted(pr, ct, 4, [(k[0], k[1], g) for k, g in zip(keys, (5, 25, 125, 1))])
    assert np.array_equal(got, want), first_mismatch(got, want)


def test_hoisted_tiny_forty_keys_and_the_key_limit():
    # 40 keys cross the launch groups of 16 key groups (16 + 16 + 8); 64 is the limit
    announce("hoisted tiny 40 keys")
    pr = params("tiny")
    ctx = context("tiny", 2)
    rng = np.random.default_rng(40)
    s = synth.ternary(rng, pr.n)
    twon = 2 * pr.n
    gs = [pow(5, k, twon) if k % 7 else pow(5, k, twon) * (twon - 1) % twon for k in range(1, 41)]
    keys, dk = [], []
    for i, g in enumerate(gs):
        errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
        seed = rng.bytes(32)
        kb, ka = oks.keygen(pr, s, oks.rotation_source(s, g, pr), errs, seed)
        keys.append((kb, ka, g))
        dk.append((gpu(kb), g, seed, gpu(ka) if i % 3 == 0 else None))
    ct = _ct(rng, pr, 3, 1)[0]
    got = host(ctx.keyswitch_hoisted(gpu(ct), 3, dk))
    want = oks.keyswitch_hoisted(pr, ct, 3, keys)
    assert np.array_equal(got, want), first_mismatch(got, want)
    from rns_ckks_key_amd.api import CkksError
    with pytest.raises(CkksError) as ei:
        ctx.keyswitch_hoisted(gpu(ct), 3, dk + dk[:25])  # 65 keys
    assert ei.value.name == "CKKS_ERANGE"


def test_multi_tiny_chunks_of_sixteen_against_oracle():
    # 21 items at level 3 (one ModUp batch of 16, then 5) and 3 at level 2, five keys,
    # stored and regenerated mixed: every output against the oracle
    announce("multi tiny 24 items")
    pr = params("tiny")
    ctx = context("tiny", 16)
    rng = np.random.default_rng(24)
    keys = [oracle_key("tiny", g, 7) for g in (5, 25, 1, 8191, 125)]
    gals = (5, 25, 1, 8191, 125)
    items, want = [], []
    for i in range(24):
        k = i % 5
        kb, ka, seed = keys[k][0], keys[k][1], keys[k][2]
        level = 3 if i < 21 else 2
        ct = _ct(rng, pr, level, 1)[0]
        stored = i % 4 == 0
        items.append((gpu(ct), level, gpu(kb), gals[k], None if stored else seed, gpu(ka) if stored else None, None))
        want.append(oks.keyswitch(pr, ct, level, kb, gals[k], key_a=ka))
    outs = ctx.keyswitch_multi(items)
    for i, (o, w) in enumerate(zip(outs, want)):
        got = host(o)
        assert np.array_equal(got, w), (i, first_mismatch(got, w))


def test_multi_concurrent_sequences_share_a_small_workspace():
    # max_batch 3: 30 items at levels 4, 3, 2, 1 in an interleaved order make launch
    # sequences of 1 to 3 items that run on four streams and take the three workspace
    # items in turn, so most sequences wait for one on another stream.  Every output
    # against the oracle; then the same call on a side torch stream, twice in a row.
    announce("multi concurrent sequences max_batch 3")
    pr = params("tiny")
    ctx = context("tiny", 3)
    rng = np.random.default_rng(31)
    gals = (5, 25, 1, 8191, 125)
    keys = [oracle_key("tiny", g, 9) for g in gals]
    levels = [4, 3, 4, 2, 1, 4, 3, 3, 2, 4, 1, 1, 4, 3, 2, 2, 4, 4, 3, 1, 2, 3, 4, 4, 1, 2, 3, 4, 3, 2]
    items, want = [], []
    for i, level in enumerate(levels):
        k = (3 * i) % 5
        kb, ka, seed = keys[k][0], keys[k][1], keys[k][2]
        ct = _ct(rng, pr, level, 1)[0]
        stored = i % 4 == 1
        items.append((gpu(ct), level, gpu(kb), gals[k], None if stored else seed, gpu(ka) if stored else None, None))
        want.append(oks.keyswitch(pr, ct, level, kb, gals[k], key_a=ka))
    outs = ctx.keyswitch_multi(items)
    for i, (o, w) in enumerate(zip(outs, want)):
        got = host(o)
        assert np.array_equal(got, w), (i, levels[i], first_mismatch(got, w))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        outs2 = [torch.full_like(o, -1) for o in outs]
        items2 = [it[:6] + (o,) for it, o in zip(items, outs2)]
        ctx.keyswitch_multi(items2)
        ctx.keyswitch_multi(items2)
        same = [bool(torch.equal(a, b)) for a, b in zip(outs, outs2)]
    torch.cuda.synchronize()
    assert all(same), [i for i, v in enumerate(same) if not v]
    # max_batch 1: one item per launch sequence, all on the caller's stream in one workspace item
    outs1 = context("tiny", 1).keyswitch_multi([it[:6] + (None,) for it in items])
    same = [bool(torch.equal(a, b)) for a, b in zip(outs, outs1)]
    assert all(same), [i for i, v in enumerate(same) if not v]


@functools.lru_cache(maxsize=None)
def _batch8_case():
    """The batch-8, level-36, g = 5 case and the oracle's output for every ciphertext of it."""
    pr = params("boot")
    kb, ka, seed, s, s_src = oracle_key("boot", 5)
    rng = np.random.default_rng(2)
    ct = _ct(rng, pr, 36, 8)
    want = np.stack(keyswitch_many(CHAINS["boot"], kb, ka, [(ct[b], 36, 5) for b in range(8)]))
    return ct, want


@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_keyswitch_boot_batch8_every_ciphertext(variant):
    # the single key-switch workload's launch shape: batch 8 at level 36, g = 5.  Every
    # ciphertext (each is one wave of the eight-wave inner-product kernels) against the oracle.
    announce(f"keyswitch boot batch 8 {variant}")
    pr = params("boot")
    ctx = context("boot", 8)
    kb, ka, seed, s, s_src = oracle_key("boot", 5)
    ct, want = _batch8_case()
    out = ctx.keyswitch(gpu(ct), 36, gpu(kb), 5, key_seed=seed if variant == "regen" else None,
                        key_a=gpu(ka) if variant == "stored" else None)
    got = host(out)
    for b in range(8):
        assert np.array_equal(got[b], want[b]), (b, first_mismatch(got[b], want[b]))
    assert oks.switch_error(pr, ct[3], got[3], 36, s, s_src, 5) < oks.noise_bound(pr, 36)


@functools.lru_cache(maxsize=None)
def _batch37_case():
    pr = params("boot")
    kb, ka, seed, s, s_src = oracle_key("boot", 25)
    rng = np.random.default_rng(37)
    ct = _ct(rng, pr, 36, 37)
    want = keyswitch_many(CHAINS["boot"], kb, ka, [(ct[b], 36, 25) for b in range(37)])
    return ct, dict(enumerate(want))


@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_keyswitch_boot_batch37_ragged(variant):
    # a batch of 37 at level 36 (each wave of the eight-wave kernels loops over four or
    # five ciphertexts): every ciphertext against the oracle, and the whole batch
    # bit-identical to calls on slices of 8, 8, 8, 8 and 5
    announce(f"keyswitch boot batch 37 {variant}")
    ctx = context("boot", 37)
    kb, ka, seed, s, s_src = oracle_key("boot", 25)
    ct, want = _batch37_case()
    dct, dkb = gpu(ct), gpu(kb)
    kw = dict(key_seed=seed) if variant == "regen" else dict(key_a=gpu(ka))
    out = ctx.keyswitch(dct, 36, dkb, 25, **kw)
    for lo, hi in ((0, 8), (8, 16), (16, 24), (24, 32), (32, 37)):
        part = ctx.keyswitch(dct[lo:hi].contiguous(), 36, dkb, 25, **kw)
        if not torch.equal(part, out[lo:hi]):
            a, b = host(out[lo:hi]), host(part)
            pytest.fail(f"slice {lo}:{hi}: {first_mismatch(a, b)}")
    got = host(out)
    for b, w in want.items():
        assert np.array_equal(got[b], w), (b, first_mismatch(got[b], w))


def test_keyswitch_boot_partial_digit_level():
    announce("keyswitch boot level 13 and 4")
    pr = params("boot")
    ctx = context("boot", 8)
    kb, ka, seed, s, s_src = oracle_key("boot", 5)
    rng = np.random.default_rng(3)
    for level in (13, 4):
        ct = _ct(rng, pr, level, 2)
        got = host(ctx.keyswitch(gpu(ct), level, gpu(kb), 5, key_seed=seed))
        want = oks.keyswitch(pr, ct, level, kb, 5, key_a=ka)
        assert np.array_equal(got, want), (level, first_mismatch(got, want))


def test_hoisted_boot_two_keys():
    announce("hoisted boot 2 keys")
    pr = params("boot")
    ctx = context("boot", 8)
    k5 = oracle_key("boot", 5)
    k25 = oracle_key("boot", 25)
    rng = np.random.default_rng(4)
    ct = _ct(rng, pr, 36, 1)[0]
    got = host(ctx.keyswitch_hoisted(gpu(ct), 36, [(gpu(k5[0]), 5, k5[2], None), (gpu(k25[0]), 25, k25[2], None)]))
    want = oks.keyswitch_hoisted(pr, ct, 36, [(k5[0], k5[1], 5), (k25[0], k25[1], 25)])
    assert np.array_equal(got, want), first_mismatch(got, want)
