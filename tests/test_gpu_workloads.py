"""GPU parity on the shapes of the level sweep, the hoisted 16-key stage and the mixed decode stream.

Each run executes the whole workload on the GPU in the launch configuration the
benchmark times, and every output is compared bit-exactly with the oracle (run
on the host's cores by tests/oracle_jobs.py).  Key b-halves are uniform residues
(the same distribution as a real b-half): the bits of the output do not depend
on whether the key is a valid encryption.
"""
import functools
import hashlib
import json
import os

import numpy as np
import pytest

from tests.gpu_common import CHAINS, announce, context, first_mismatch, gpu, host, params
from tests.oracle_jobs import switch_all

pytestmark = pytest.mark.gpu

from oracle import ks as oks  # noqa: E402
from oracle.chacha import expand_key_a  # noqa: E402
from oracle.ntt import intt, ntt, ntt_definition  # noqa: E402
from oracle.params import Params  # noqa: E402
from rns_ckks_key_amd import synth  # noqa: E402


@functools.lru_cache(maxsize=None)
def key_rows(seed_int: int):
    pr = params("boot")
    return synth.uniform_key_rows(seed_int, pr.primes, pr.dnum, pr.n).astype(np.uint64)


@functools.lru_cache(maxsize=None)
def key_a(seed: bytes):
    pr = params("boot")
    return expand_key_a(seed, pr.primes, pr.dnum, pr.n)


@functools.lru_cache(maxsize=None)
def _sweep_oracle():
    # all 64 ciphertexts of the sweep (16 at each level) under workload 2's key
    pr = params("boot")
    d = synth.draw(3, pr.primes)
    seed = d.keys[0].seed
    jobs = [(ct, lvl, 5, 3003, seed) for ct, lvl in zip(d.cts, d.levels)]
    return switch_all(CHAINS["boot"], jobs)


@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_level_sweep_batch16(variant):
    # workload 3: batch 16 at levels 36, 24, 12, 4 under workload 2's key, with the a-half
    # regenerated or stored; every ciphertext of every level against the oracle
    pr = params("boot")
    ctx = context("boot", 16)
    d = synth.draw(3, pr.primes)
    seed = d.keys[0].seed
    dkb = gpu(key_rows(3003))
    dka = gpu(key_a(seed)) if variant == "stored" else None
    announce(f"level sweep oracle (64 switches) {variant}")
    want = _sweep_oracle()
    for li, level in enumerate(synth.WORKLOADS[3].levels):
        announce(f"level sweep level={level} {variant}")
        cts = np.stack(d.cts[16 * li:16 * li + 16])
        got = host(ctx.keyswitch(gpu(cts), level, dkb, 5, key_seed=seed if dka is None else None, key_a=dka))
        for b in range(16):
            w = want[16 * li + b]
            assert np.array_equal(got[b], w), (level, b, first_mismatch(got[b], w))


@functools.lru_cache(maxsize=None)
def _hoist_oracle():
    # the ciphertext under each of the 16 keys
    pr = params("boot")
    d = synth.draw(4, pr.primes)
    jobs = [(d.cts[0], 36, kd.galois, 4000 + k, kd.seed) for k, kd in enumerate(d.keys)]
    return switch_all(CHAINS["boot"], jobs)


@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_hoisted_sixteen_keys(variant):
    # workload 4: one ciphertext at level 36, 16 keys g = 5^k with their own seeds (or their
    # stored a-halves), one hoisted call; every key's output against the oracle
    announce(f"hoisted 16 keys {variant}")
    pr = params("boot")
    ctx = context("boot", 16)
    d = synth.draw(4, pr.primes)
    ct = d.cts[0]
    keys = []
    for k, kd in enumerate(d.keys):
        ka = gpu(key_a(kd.seed)) if variant == "stored" else None
        keys.append((gpu(key_rows(4000 + k)), kd.galois, kd.seed if ka is None else None, ka))
    got = host(ctx.keyswitch_hoisted(gpu(ct), 36, keys))
    announce(f"hoisted oracle (16 switches) {variant}")
    for k, want in enumerate(_hoist_oracle()):
        assert np.array_equal(got[k], want), (k, first_mismatch(got[k], want))


@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_tiny_workload_exact_draw(variant):
    # workload 1 exactly as drawn: N = 2^12, 4 + 2 primes below 2^30, dnum 2, the
    # relinearisation-style key (s' -> s, g = 1) from the oracle's keygen on the drawn
    # secrets, errors and seed; one key-switch, and the forward and inverse NTT of the
    # ciphertext (every limb against the oracle, limb 0 also against the O(N^2) definition)
    announce(f"workload 1 exact draw {variant}")
    wl = synth.WORKLOADS[1]
    pr = Params.make(wl.log_n, wl.L, wl.K, wl.dnum, wl.bits)
    ctx = context("tiny", 1)
    assert ctx.primes == pr.primes
    d = synth.draw(1, pr.primes)
    kd = d.keys[0]
    kb, ka = oks.keygen(pr, d.s, d.s_prime, kd.errors, kd.seed)
    ct = d.cts[0].astype(np.uint64)
    got = host(ctx.keyswitch(gpu(ct[None]), 4, gpu(kb), 1, key_seed=kd.seed if variant == "regen" else None,
                             key_a=gpu(ka) if variant == "stored" else None))[0]
    want = oks.keyswitch(pr, ct, 4, kb, 1, seed=kd.seed)
    assert np.array_equal(got, want), first_mismatch(got, want)
    assert oks.switch_error(pr, ct, got, 4, d.s, d.s_prime, 1) < oks.noise_bound(pr, 4)
    # and the stored expected value (written from the oracle by tests/golden/make_golden.py)
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "oracle_golden.json")) as f:
        golden = json.load(f)["workload1"]
    assert hashlib.sha256(np.ascontiguousarray(got, dtype="<u4").tobytes()).hexdigest() == golden["sha256_keyswitch_out"]
    # standalone NTT of the ciphertext [2][4][N]: its residues read as coefficients (a batch of
    # two items of limbs q_0..q_3), forward then inverse in place, and the inverse on its own
    qs, ps = pr.primes[:4], pr.psis[:4]
    t = gpu(ct)
    ctx.ntt_fwd(t, 0)
    fwd = host(t)
    want_f = ntt(ct, qs, ps)
    assert np.array_equal(fwd, want_f), first_mismatch(fwd, want_f)
    assert np.array_equal(fwd[0, 0], ntt_definition(ct[0, 0], qs[0], ps[0]))
    ctx.ntt_inv(t, 0)
    assert np.array_equal(host(t), ct)
    t2 = gpu(ct)
    ctx.ntt_inv(t2, 0)
    want_i = intt(ct, qs, ps)
    assert np.array_equal(host(t2), want_i), first_mismatch(host(t2), want_i)


@functools.lru_cache(maxsize=None)
def _mixed_oracle():
    # each of the 64 ciphertexts under its key
    pr = params("boot")
    d = synth.draw(5, pr.primes)
    wl = synth.WORKLOADS[5]
    jobs = [(ct, d.levels[i], wl.galois[d.key_index[i]], 5000 + d.key_index[i], d.keys[d.key_index[i]].seed)
            for i, ct in enumerate(d.cts)]
    return switch_all(CHAINS["boot"], jobs)


def test_mixed_stream_sixty_four():
    # workload 5: 64 ciphertexts, levels 8..36, each under one of 33 keys; one call per
    # ciphertext; every output against the oracle
    announce("mixed stream 64")
    pr = params("boot")
    ctx = context("boot", 16)
    d = synth.draw(5, pr.primes)
    wl = synth.WORKLOADS[5]
    dkb = {}
    outs = []
    for i, ct in enumerate(d.cts):
        k = d.key_index[i]
        if k not in dkb:
            dkb[k] = gpu(key_rows(5000 + k))
        lvl = d.levels[i]
        outs.append(ctx.keyswitch(gpu(ct[None]), lvl, dkb[k], wl.galois[k], key_seed=d.keys[k].seed))
    announce("mixed stream oracle (64 switches)")
    for i, want in enumerate(_mixed_oracle()):
        got = host(outs[i])[0]
        assert np.array_equal(got, want), (i, d.levels[i], d.key_index[i], first_mismatch(got, want))


def test_multi_item_equals_single_calls():
    # ckks_keyswitch_multi over the mixed stream (levels repeat, keys differ, stored and regenerated mixed)
    # is bit-identical to one ckks_keyswitch call per item, and every item equals the oracle
    announce("multi-item stream")
    pr = params("boot")
    ctx = context("boot", 16)
    d = synth.draw(5, pr.primes)
    wl = synth.WORKLOADS[5]
    dkb, dka, items = {}, {}, []
    for i, ct in enumerate(d.cts):
        k = d.key_index[i]
        if k not in dkb:
            dkb[k] = gpu(key_rows(5000 + k))
        stored = (i % 3 == 1)
        if stored and k not in dka:
            dka[k] = ctx.expand_a(d.keys[k].seed)
        items.append((gpu(ct), d.levels[i], dkb[k], wl.galois[k], None if stored else d.keys[k].seed,
                      dka[k] if stored else None, None))
    outs = ctx.keyswitch_multi(items)
    for i in range(len(items)):
        ct, lvl, kb, g, seed, ka, _ = items[i]
        single = ctx.keyswitch(ct[None], lvl, kb, g, key_seed=seed, key_a=ka)
        a, b = host(outs[i]), host(single)[0]
        assert np.array_equal(a, b), (i, lvl, first_mismatch(a, b))
    for i, want in enumerate(_mixed_oracle()):
        assert np.array_equal(host(outs[i]), want), (i, first_mismatch(host(outs[i]), want))
