"""The oracle pool (spawned worker processes) returns what the oracle returns in this process."""
import numpy as np

from oracle import ks as oks
from oracle.params import Params
from rns_ckks_key_amd import synth
from oracle.pool import keyswitch_many


def test_pool_equals_direct_oracle_calls():
    chain = (12, 4, 2, 2, 30)
    pr = Params.make(*chain)
    rng = np.random.default_rng(55)
    seeds = [rng.bytes(32) for _ in range(2)]
    kbs = [synth.uniform_key_rows(60 + i, pr.primes, pr.dnum, pr.n) for i in range(2)]
    from oracle.chacha import expand_key_a
    kas = [expand_key_a(sd, pr.primes, pr.dnum, pr.n) for sd in seeds]
    cts = [np.stack([synth.residues(rng, pr.primes[:lv], pr.n) for _ in range(2)]) for lv in (4, 3, 1)]
    jobs = [(cts[0], 4, 5, 0), (cts[1], 3, 25, 1), (cts[2], 1, 1, 0)]
    got = keyswitch_many(chain, kbs, kas, jobs, max_workers=2)
    for (ct, lv, g, k), out in zip(jobs, got):
        want = oks.keyswitch(pr, ct.astype(np.uint64), lv, kbs[k].astype(np.uint64), g, key_a=kas[k])
        assert np.array_equal(out, want)
    one = keyswitch_many(chain, kbs[1], kas[1], [(cts[0], 4, 125)])
    assert np.array_equal(one[0], oks.keyswitch(pr, cts[0].astype(np.uint64), 4, kbs[1].astype(np.uint64), 125,
                                                key_a=kas[1]))
