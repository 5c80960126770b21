"""GPU parity of rescale and multiply-relinearise-rescale with the oracle (bit-exact).

Covers every level of the N=2^12 chain, batches that take each inner-product
kernel shape (1, 5 and 8 ciphertexts), regenerated and stored key halves, the
multiply-by-one identity, the decryption of an encrypted product, the
bootstrapping-scale configuration (batch 8 at level 36, every product against
the oracle, run on the host's cores by tests/oracle_jobs.py) and the argument
errors.
"""
import functools

import numpy as np
import pytest

from tests.gpu_common import CHAINS, announce, context, first_mismatch, gpu, host, params, rand_limbs, torch
from tests.oracle_jobs import mul_relin_rescale_all

pytestmark = pytest.mark.gpu

from oracle import ks as oks  # noqa: E402
from oracle import mult as omult  # noqa: E402
from oracle.ntt import ntt  # noqa: E402
from rns_ckks_key_amd import synth  # noqa: E402
from rns_ckks_key_amd.api import CkksError  # noqa: E402


@functools.lru_cache(maxsize=None)
def relin_key(name: str):
    pr = params(name)
    rng = np.random.default_rng(777)
    s = synth.ternary(rng, pr.n)
    errs = [synth.gaussian(rng, pr.n) for _ in range(pr.dnum)]
    seed = rng.bytes(32)
    kb, ka = omult.relin_keygen(pr, s, errs, seed)
    return kb, ka, seed, s


def _ct(rng, pr, level, batch):
    return np.stack([np.stack([rand_limbs(rng, pr.primes[:level], pr.n) for _ in range(2)]) for _ in range(batch)])


@pytest.mark.parametrize("name,level,batch", [("tiny", 4, 3), ("tiny", 3, 1), ("tiny", 2, 2), ("boot", 36, 2),
                                              ("boot", 13, 1), ("boot", 2, 1)])
def test_rescale_bit_exact(name, level, batch):
    announce(f"rescale {name} level={level} batch={batch}")
    pr = params(name)
    ctx = context(name, 8)
    rng = np.random.default_rng(50 + level)
    ct = _ct(rng, pr, level, batch)
    if name == "tiny":
        ct[0, 0, 0] = 0
        ct[0, 1, level - 1] = pr.primes[level - 1] - 1
    got = host(ctx.rescale(gpu(ct), level))
    want = omult.rescale(pr, ct, level)
    assert np.array_equal(got, want), first_mismatch(got, want)


@pytest.mark.parametrize("batch", [1, 5, 8])
@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_mul_relin_rescale_tiny_all_levels(batch, variant):
    announce(f"mul_relin_rescale tiny batch={batch} {variant}")
    pr = params("tiny")
    ctx = context("tiny", 8)
    kb, ka, seed, s = relin_key("tiny")
    dkb, dka = gpu(kb), gpu(ka)
    rng = np.random.default_rng(batch)
    for level in (4, 3, 2):
        x, y = _ct(rng, pr, level, batch), _ct(rng, pr, level, batch)
        got = host(ctx.mul_relin_rescale(gpu(x), gpu(y), level, dkb, key_seed=seed if variant == "regen" else None,
                                         key_a=dka if variant == "stored" else None))
        want = omult.mul_relin_rescale(pr, x, y, level, kb, key_a=ka)
        assert np.array_equal(got, want), (level, first_mismatch(got, want))


def test_mul_by_one_is_rescale_and_product_decrypts():
    announce("mul_relin_rescale tiny identities")
    pr = params("tiny")
    ctx = context("tiny", 8)
    kb, ka, seed, s = relin_key("tiny")
    rng = np.random.default_rng(9)
    level = 4
    x = _ct(rng, pr, level, 2)
    one = np.zeros_like(x)
    one[:, 0] = 1
    got = host(ctx.mul_relin_rescale(gpu(x), gpu(one), level, gpu(kb), key_seed=seed))
    assert np.array_equal(got, host(ctx.rescale(gpu(x), level)))
    # encrypted messages: the result decrypts to m_x*m_y / q_3 within the switch and rounding error
    q = np.array(pr.primes[:level], dtype=np.uint64).reshape((-1, 1))
    sh = oks.to_ntt_all(s, pr, list(range(level)))
    ms = [rng.integers(-(1 << 40), 1 << 40, pr.n, dtype=np.int64) for _ in range(2)]
    cts = []
    for m in ms:
        a = rand_limbs(rng, pr.primes[:level], pr.n)
        mh = ntt(np.stack([np.mod(m, qi).astype(np.uint64) for qi in pr.primes[:level]]), pr.primes[:level],
                 pr.psis[:level])
        cts.append(np.stack([(mh + q - a * sh % q) % q, a])[None])
    out = host(ctx.mul_relin_rescale(gpu(cts[0]), gpu(cts[1]), level, gpu(kb), key_seed=seed))[0]
    # m_x*m_y (|coefficients| < 2^93 < Q_4/2), exactly, from the product of the messages' NTTs
    mxh, myh = (oks.to_ntt_all(m, pr, list(range(level))) for m in ms)
    prod_m = oks.decrypt_coeffs(pr, np.stack([mxh * myh % q, np.zeros_like(mxh)]), level, np.zeros(pr.n, np.int64))
    dec = oks.decrypt_coeffs(pr, out, level - 1, s)
    ql = pr.primes[level - 1]
    worst = max(abs(d * ql - m) for d, m in zip(dec, prod_m)) / ql
    assert worst < oks.noise_bound(pr, level) / ql + pr.n + 2, worst


@functools.lru_cache(maxsize=None)
def _batch8_oracle():
    pr = params("boot")
    kb, ka, seed, s = relin_key("boot")
    rng = np.random.default_rng(12)
    x, y = _ct(rng, pr, 36, 8), _ct(rng, pr, 36, 8)
    return mul_relin_rescale_all(CHAINS["boot"], kb, ka, [(x[b], y[b], 36) for b in range(8)])


@pytest.mark.parametrize("variant", ["regen", "stored"])
def test_mul_relin_rescale_boot_batch8(variant):
    # batch 8 at level 36 (the bootstrapping-scale chain); every product against the oracle
    announce(f"mul_relin_rescale boot batch 8 {variant}")
    pr = params("boot")
    ctx = context("boot", 8)
    kb, ka, seed, s = relin_key("boot")
    rng = np.random.default_rng(12)
    x, y = _ct(rng, pr, 36, 8), _ct(rng, pr, 36, 8)
    got = host(ctx.mul_relin_rescale(gpu(x), gpu(y), 36, gpu(kb), key_seed=seed if variant == "regen" else None,
                                     key_a=gpu(ka) if variant == "stored" else None))
    for b, want in enumerate(_batch8_oracle()):
        assert np.array_equal(got[b], want), (b, first_mismatch(got[b], want))


def test_mul_relin_rescale_boot_low_level():
    announce("mul_relin_rescale boot level 5")
    pr = params("boot")
    ctx = context("boot", 8)
    kb, ka, seed, s = relin_key("boot")
    rng = np.random.default_rng(13)
    x, y = _ct(rng, pr, 5, 4), _ct(rng, pr, 5, 4)
    got = host(ctx.mul_relin_rescale(gpu(x), gpu(y), 5, gpu(kb), key_seed=seed))
    want = omult.mul_relin_rescale(pr, x[2], y[2], 5, kb, key_a=ka)
    assert np.array_equal(got[2], want), first_mismatch(got[2], want)


def test_rescale_and_multiply_argument_errors():
    announce("rescale / mul errors")
    from rns_ckks_key_amd._lib import lib
    pr = params("tiny")
    ctx = context("tiny", 8)
    ct = torch.zeros((2, 2, 4, pr.n), dtype=torch.int32, device="cuda")
    out = torch.zeros((2, 2, 3, pr.n), dtype=torch.int32, device="cuda")
    kb = torch.zeros((pr.dnum, pr.L + pr.K, pr.n), dtype=torch.int32, device="cuda")
    seed = bytes(32)
    # level 1 has no prime to drop; level 5 is above the chain
    for level in (1, 5):
        assert lib.ckks_rescale(ctx.handle, ct.data_ptr(), level, out.data_ptr(), 2, None) == -2
        assert lib.ckks_mul_relin_rescale(ctx.handle, ct.data_ptr(), ct.data_ptr(), level, kb.data_ptr(), seed, None,
                                          out.data_ptr(), 2, None) == -2
    # out inside the input
    inside = ct.view(-1)[: 2 * 2 * 3 * pr.n].view(2, 2, 3, pr.n)
    with pytest.raises(CkksError) as ei:
        ctx.rescale(ct, 4, out=inside)
    assert ei.value.name == "CKKS_EINVAL"
    with pytest.raises(CkksError) as ei:
        ctx.mul_relin_rescale(ct, ct, 4, kb)  # neither key_a nor a seed
    assert ei.value.name == "CKKS_EINVAL"
    with pytest.raises(CkksError) as ei:
        ctx.rescale(torch.zeros((9, 2, 4, pr.n), dtype=torch.int32, device="cuda"), 4)  # batch 9 > 8
    assert ei.value.name == "CKKS_ERANGE"
    torch.cuda.synchronize()
