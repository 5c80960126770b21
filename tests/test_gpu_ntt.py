"""GPU parity of the standalone NTT/INTT (ckks_ntt_fwd / ckks_ntt_inv) with the oracle: bit-exact."""
import numpy as np
import pytest

from tests.gpu_common import announce, context, first_mismatch, gpu, host, params, rand_limbs

pytestmark = pytest.mark.gpu

from oracle.ntt import intt, ntt  # noqa: E402


@pytest.mark.parametrize("name,first,nl,batch", [("tiny", 0, 6, 2), ("tiny", 2, 3, 1), ("boot", 0, 4, 2),
                                                 ("boot", 34, 4, 1), ("boot", 44, 4, 1)])
def test_ntt_forward_inverse_bit_exact(name, first, nl, batch):
    announce(f"ntt {name} first={first} limbs={nl} batch={batch}")
    pr = params(name)
    ctx = context(name, 4)
    qs, ps = pr.primes[first:first + nl], pr.psis[first:first + nl]
    rng = np.random.default_rng(first * 7 + nl)
    a = rand_limbs(rng, qs, pr.n, (batch,))
    a[0, 0, :] = 0
    a[0, 0, 5] = 1                    # single nonzero coefficient
    a[-1, -1, :] = qs[-1] - 1         # all q-1
    t = gpu(a)
    ctx.ntt_fwd(t, first)
    want = ntt(a, qs, ps)
    got = host(t)
    assert np.array_equal(got, want), first_mismatch(got, want)
    ctx.ntt_inv(t, first)
    got = host(t)
    assert np.array_equal(got, a), first_mismatch(got, a)
    # inverse alone on NTT-domain input
    t2 = gpu(want)
    ctx.ntt_inv(t2, first)
    assert np.array_equal(host(t2), intt(want, qs, ps))


def test_ntt_full_ciphertext_batch_of_eight():
    # the shape of a batch of 8 ciphertexts at level 36: [8][72][N] over q_0..q_35 twice
    announce("ntt boot 8x2x36")
    pr = params("boot")
    ctx = context("boot", 8)
    rng = np.random.default_rng(99)
    a = rand_limbs(rng, pr.primes[:36], pr.n, (16,))
    t = gpu(a)
    ctx.ntt_fwd(t, 0)
    got = host(t)
    want = ntt(a, pr.primes[:36], pr.psis[:36])  # every limb of every item
    assert np.array_equal(got, want), first_mismatch(got, want)
    ctx.ntt_inv(t, 0)
    assert np.array_equal(host(t), a)
