"""Seeded random key-switch configurations against the oracle, every ciphertext bit for bit.

Each case draws a chain shape (ring 2^12 or 2^13, 2..8 ciphertext primes, dnum, a
special part at least one digit wide, 30- to 32-bit primes), a level, a batch size
that selects each inner-product kernel shape (1..3: one wave, 4..7: four, 8+: eight,
looping over the batch above 8), a Galois element (1, a relinearisation-style key, in
about one case of eight), the stored or regenerated a-half, and the fused or unfused
route (whose context of max_batch = batch often makes it run in groups).
"""
import functools

import numpy as np
import pytest

from tests.gpu_common import announce, first_mismatch, gpu, host, rand_limbs

pytestmark = pytest.mark.gpu

from oracle import ks as oks  # noqa: E402
from oracle.params import Params  # noqa: E402
from rns_ckks_key_amd import synth  # noqa: E402
from rns_ckks_key_amd.api import CkksError, Context  # noqa: E402

N_CASES = 64


def _draw(case: int) -> dict:
    rng = np.random.default_rng(90210 + case)
    log_n = int(rng.choice([12, 13]))
    L = int(rng.integers(2, 9))
    dnum = int(rng.integers(1, L + 1))
    alpha = -(-L // dnum)
    K = alpha + int(rng.integers(0, 3))
    bits = int(rng.choice([30, 31, 32]))
    level = int(rng.integers(1, L + 1))
    batch = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 9, 12, 16, 17]))
    g = 1 if rng.integers(0, 8) == 0 else int(rng.integers(0, 1 << log_n)) * 2 + 1
    return dict(shape=(log_n, L, K, dnum, bits), level=level, batch=batch, g=g,
                regen=bool(case % 2), fused=bool((case // 2) % 2), seed=90210 + case)


@functools.lru_cache(maxsize=None)
def _params(shape):
    return Params.make(*shape)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_configuration_against_oracle(case):
    d = _draw(case)
    announce(f"random keyswitch case {case}: {d}")
    pr = _params(d["shape"])
    log_n, L, K, dnum, bits = d["shape"]
    rng = np.random.default_rng(d["seed"])
    s = synth.ternary(rng, pr.n)
    s_src = synth.ternary(rng, pr.n) if d["g"] == 1 else oks.rotation_source(s, d["g"], pr)
    errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
    seed = rng.bytes(32)
    kb, ka = oks.keygen(pr, s, s_src, errs, seed)
    level, batch = d["level"], d["batch"]
    ct = np.stack([np.stack([rand_limbs(rng, pr.primes[:level], pr.n) for _ in range(2)]) for _ in range(batch)])
    def run(max_batch):
        ctx = Context(log_n, L, K, dnum, pr.primes, max_batch)
        try:
            ctx.set_fused(d["fused"])
            return host(ctx.keyswitch(gpu(ct), level, gpu(kb), d["g"], key_seed=seed if d["regen"] else None,
                                      key_a=None if d["regen"] else gpu(ka)))
        finally:
            ctx.close()
    try:
        got = run(batch)
    except CkksError as e:  # the unfused route refuses a workspace too small for one group
        assert not d["fused"] and e.name == "CKKS_ERANGE", (d, e)
        got = run(4 * batch)
    want = oks.keyswitch(pr, ct, level, kb, d["g"], key_a=ka)
    assert np.array_equal(got, want), (d, first_mismatch(got, want))
    assert oks.switch_error(pr, ct[0], got[0], level, s, s_src, d["g"]) < oks.noise_bound(pr, level)
