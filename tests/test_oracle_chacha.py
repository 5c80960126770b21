"""Pins of the oracle's ChaCha block function and its counter-mode rejection expander.

The block function is checked at 20 rounds against OpenSSL's ChaCha20 (run as a
black-box tool, whose 16-byte IV is state words 12..15: block counter then
nonce); that pins constants, key/counter/nonce placement, the quarter round and
the byte order.  No ChaCha12 vector is available here, but the 12-round output
follows from OpenSSL's 20-round output exactly: the double round P is a
permutation of the state, ChaCha_r(x) = x + P^(r/2)(x), so
ChaCha12(x) = x + P^-4(ChaCha20(x) - x), with P^-1 written out below from the
quarter round's steps undone in reverse order.
"""
import shutil
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle.chacha import chacha_blocks, expand_key_a, expand_row, keystream_bytes
from oracle.chain import chain_primes

HAVE_OPENSSL = shutil.which("openssl") is not None


def _openssl(key: bytes, counter: int, nonce, nbytes: int) -> bytes:
    iv = counter.to_bytes(4, "little") + b"".join(int(w).to_bytes(4, "little") for w in nonce)
    r = subprocess.run(["openssl", "enc", "-chacha20", "-K", key.hex(), "-iv", iv.hex()],
                       input=bytes(nbytes), capture_output=True, check=True)
    return r.stdout


@pytest.mark.skipif(not HAVE_OPENSSL, reason="openssl not on PATH")
@settings(max_examples=25, deadline=None)
@given(key=st.binary(min_size=32, max_size=32), counter=st.integers(0, 2**32 - 8),
       nonce=st.tuples(st.integers(0, 2**32 - 1), st.integers(0, 2**32 - 1), st.integers(0, 2**32 - 1)),
       nblocks=st.integers(1, 5))
def test_chacha20_matches_openssl(key, counter, nonce, nblocks):
    assert keystream_bytes(key, counter, nonce, nblocks, rounds=20) == _openssl(key, counter, nonce, 64 * nblocks)


M32 = 0xFFFFFFFF


def _inverse_double_round(s: list) -> None:
    """Undo one double round in place: the diagonal round, then the column round (its four
    quarter rounds touch disjoint words, so their order within a round does not matter)."""
    def rotr(x, r):
        return ((x >> r) | (x << (32 - r))) & M32

    def inv_quarter(a, b, c, d):
        s[b] = rotr(s[b], 7) ^ s[c]
        s[c] = (s[c] - s[d]) & M32
        s[d] = rotr(s[d], 8) ^ s[a]
        s[a] = (s[a] - s[b]) & M32
        s[b] = rotr(s[b], 12) ^ s[c]
        s[c] = (s[c] - s[d]) & M32
        s[d] = rotr(s[d], 16) ^ s[a]
        s[a] = (s[a] - s[b]) & M32

    for a, b, c, d in ((0, 5, 10, 15), (1, 6, 11, 12), (2, 7, 8, 13), (3, 4, 9, 14)):
        inv_quarter(a, b, c, d)
    for a, b, c, d in ((0, 4, 8, 12), (1, 5, 9, 13), (2, 6, 10, 14), (3, 7, 11, 15)):
        inv_quarter(a, b, c, d)


def _chacha_from_openssl20(key: bytes, counter: int, nonce, rounds: int) -> list:
    """ChaCha_rounds block derived from OpenSSL's ChaCha20 block by undoing 10 - rounds/2 double rounds."""
    x = list(np.frombuffer(b"expand 32-byte k" + key, dtype="<u4").tolist()) + [counter] + list(nonce)
    out20 = np.frombuffer(_openssl(key, counter, nonce, 64), dtype="<u4").tolist()
    s = [(o - w) & M32 for o, w in zip(out20, x)]
    for _ in range(10 - rounds // 2):
        _inverse_double_round(s)
    return [(v + w) & M32 for v, w in zip(s, x)]


@pytest.mark.skipif(not HAVE_OPENSSL, reason="openssl not on PATH")
@settings(max_examples=25, deadline=None)
@given(key=st.binary(min_size=32, max_size=32), counter=st.integers(0, 2**32 - 1),
       nonce=st.tuples(st.integers(0, 2**32 - 1), st.integers(0, 2**32 - 1), st.integers(0, 2**32 - 1)))
def test_chacha12_from_openssl_chacha20_by_inverse_rounds(key, counter, nonce):
    want = _chacha_from_openssl20(key, counter, nonce, 12)
    got = chacha_blocks(key, counter, nonce[0], nonce[1], nonce[2], rounds=12).tolist()
    assert got == want
    # the derivation is not vacuous: other round counts land elsewhere
    assert chacha_blocks(key, counter, nonce[0], nonce[1], nonce[2], rounds=8).tolist() == \
        _chacha_from_openssl20(key, counter, nonce, 8)
    assert got != chacha_blocks(key, counter, nonce[0], nonce[1], nonce[2], rounds=14).tolist()


def test_rounds_change_output_and_blocks_are_independent():
    key = bytes(range(32))
    b12 = chacha_blocks(key, np.arange(4), 1, 2, 3, rounds=12)
    b20 = chacha_blocks(key, np.arange(4), 1, 2, 3, rounds=20)
    assert b12.shape == (4, 16) and not np.array_equal(b12, b20)
    assert np.array_equal(chacha_blocks(key, 2, 1, 2, 3, rounds=12), b12[2])
    assert len(set(map(bytes, b12.astype("<u4")))) == 4


def _plain_expand(seed, j, t, q, n):
    """Rejection sampling written as a loop over the flat keystream of each tile."""
    tile = min(1024, n)
    out = []
    bound = (2**32 // q) * q
    for tau in range(n // tile):
        got, ctr = [], 0
        while len(got) < tile:
            words = np.frombuffer(keystream_bytes(seed, ctr, (j, t, tau), 1, rounds=12), dtype="<u4")
            for w in words.tolist():
                if w < bound and len(got) < tile:
                    got.append(w % q)
            ctr += 1
        out += got
    return out


@pytest.mark.parametrize("n,bits,t", [(16, 32, 0), (64, 32, 3), (2048, 32, 1), (1 << 12, 30, 5)])
def test_expander_placement_matches_plain_loop(n, bits, t):
    qs = chain_primes(n, bits, t + 1)
    seed = bytes(range(100, 132))
    assert expand_row(seed, 2, t, qs[t], n).tolist() == _plain_expand(seed, 2, t, qs[t], n)


def test_expander_rejects_high_words():
    # q in (2^31, 2^32): floor(2^32/q) = 1, so exactly the words >= q are rejected
    n = 1024
    q = chain_primes(n, 32, 200)[-1]  # smallest of the 200 (largest rejection)
    seed = b"\x07" * 32
    words = np.frombuffer(keystream_bytes(seed, 0, (0, 0, 0), 200, rounds=12), dtype="<u4").astype(np.uint64)
    acc = words[words < q][:n]
    assert np.array_equal(expand_row(seed, 0, 0, q, n), acc % q)


def test_expander_statistics_and_determinism():
    n = 1 << 16
    qs = chain_primes(n, 32, 48)
    seed = b"\x5a" * 32
    a = expand_key_a(seed, qs[-2:], 2, n)
    assert np.array_equal(a, expand_key_a(seed, qs[-2:], 2, n))
    assert not np.array_equal(a[0, 0], a[1, 0])
    for row, q in ((a[0, 0], qs[-2]), (a[1, 1], qs[-1])):
        assert row.max() < q
        # chi-square over 64 equal bins of [0, q)
        cnt = np.bincount((row * 64 // q).astype(np.int64), minlength=64)
        chi2 = ((cnt - n / 64) ** 2 / (n / 64)).sum()
        assert chi2 < 120  # 63 degrees of freedom; p ~ 3e-5
    # acceptance rate of the raw stream matches floor(2^32/q)*q/2^32
    q = qs[-1]
    words = np.frombuffer(keystream_bytes(seed, 0, (0, 47, 0), 4096, rounds=12), dtype="<u4").astype(np.uint64)
    rate = (words < (2**32 // q) * q).mean()
    assert abs(rate - (2**32 // q) * q / 2**32) < 0.002
