"""ChaCha block function and the counter-mode uniform-mod-q expander (oracle; test infrastructure only).

The method: the uniformly random half a of each key-switching key is not
stored but regenerated inside the kernels that use it by a counter-mode
ChaCha12 expander (Perseus summary on ai4snews, "Interpretation" paragraph 2).
The block function is ChaCha as Bernstein (2008) defines it, with the RFC 8439
state layout; only the round count (12) is the pages'.

The pages are silent on the stream layout and on how words become residues.
Readings adopted (one sub-stream per (digit j, absolute prime t, tile tau)):

* state words 0..3: the constant "expand 32-byte k" as little-endian words;
  4..11: the 32 seed bytes as little-endian words; 12: block counter from 0;
  13, 14, 15: j, t, tau;
* the output is the feed-forward sum of the state after the rounds;
* words are consumed in counter order and, within a block, in word order;
* a word w is accepted iff w < floor(2**32/q)*q, giving residue w mod q
  (rejection sampling, so residues are exactly uniform);
* the k-th accepted word of sub-stream (j, t, tau) is a_j[t][tau*TILE + k] with
  TILE = min(1024, N).
"""
from __future__ import annotations

import numpy as np

SIGMA = np.frombuffer(b"expand 32-byte k", dtype="<u4").astype(np.uint32)
TILE_MAX = 1024


def _rotl(x: np.ndarray, r: int) -> np.ndarray:
    return (x << np.uint32(r)) | (x >> np.uint32(32 - r))


def _quarter(s: list, a: int, b: int, c: int, d: int) -> None:
    s[a] = s[a] + s[b]; s[d] = _rotl(s[d] ^ s[a], 16)
    s[c] = s[c] + s[d]; s[b] = _rotl(s[b] ^ s[c], 12)
    s[a] = s[a] + s[b]; s[d] = _rotl(s[d] ^ s[a], 8)
    s[c] = s[c] + s[d]; s[b] = _rotl(s[b] ^ s[c], 7)


def chacha_blocks(key: bytes, counter, n13, n14, n15, rounds: int = 12) -> np.ndarray:
    """Keystream blocks for arrays of (counter, word13, word14, word15); returns [..., 16] uint32.

    `rounds` is even: rounds/2 double rounds (column round then diagonal round).
    """
    assert len(key) == 32 and rounds % 2 == 0
    kw = np.frombuffer(key, dtype="<u4").astype(np.uint32)
    counter, n13, n14, n15 = np.broadcast_arrays(*(np.asarray(v, dtype=np.uint32) for v in (counter, n13, n14, n15)))
    shape = counter.shape
    init = [np.full(shape, SIGMA[i], dtype=np.uint32) for i in range(4)]
    init += [np.full(shape, kw[i], dtype=np.uint32) for i in range(8)]
    init += [counter.astype(np.uint32), n13.astype(np.uint32), n14.astype(np.uint32), n15.astype(np.uint32)]
    s = [w.copy() for w in init]
    with np.errstate(over="ignore"):
        for _ in range(rounds // 2):
            _quarter(s, 0, 4, 8, 12); _quarter(s, 1, 5, 9, 13)
            _quarter(s, 2, 6, 10, 14); _quarter(s, 3, 7, 11, 15)
            _quarter(s, 0, 5, 10, 15); _quarter(s, 1, 6, 11, 12)
            _quarter(s, 2, 7, 8, 13); _quarter(s, 3, 4, 9, 14)
        out = [s[i] + init[i] for i in range(16)]
    return np.stack(out, axis=-1)


def keystream_bytes(key: bytes, counter0: int, nonce: tuple[int, int, int], nblocks: int, rounds: int) -> bytes:
    """Serialized keystream (little-endian words) of `nblocks` consecutive blocks."""
    ctr = np.arange(counter0, counter0 + nblocks, dtype=np.uint64).astype(np.uint32)
    blk = chacha_blocks(key, ctr, nonce[0], nonce[1], nonce[2], rounds)
    return blk.astype("<u4").tobytes()


def expand_row(seed: bytes, j: int, t: int, q: int, n: int, rounds: int = 12) -> np.ndarray:
    """a_j[t][0..N) for one (digit j, absolute prime t): TILE-sized sub-streams with rejection."""
    tile = min(TILE_MAX, n)
    ntiles = n // tile
    bound = (2**32 // q) * q
    out = np.empty(n, dtype=np.uint64)
    nblk = -(-tile // 16) + 8
    while True:
        tau = np.arange(ntiles, dtype=np.uint32)[:, None]
        ctr = np.arange(nblk, dtype=np.uint32)[None, :]
        words = chacha_blocks(seed, ctr, j, t, tau, rounds).reshape(ntiles, nblk * 16).astype(np.uint64)
        ok = words < bound
        if ok.sum(axis=1).min() >= tile:
            break
        nblk *= 2
    for k in range(ntiles):
        acc = words[k][ok[k]][:tile]
        out[k * tile:(k + 1) * tile] = acc % q
    return out


def expand_key_a(seed: bytes, primes: list[int], dnum: int, n: int, rounds: int = 12) -> np.ndarray:
    """The whole a-half [dnum][len(primes)][N], rows indexed by absolute prime index t."""
    return np.stack([np.stack([expand_row(seed, j, t, q, n, rounds) for t, q in enumerate(primes)])
                     for j in range(dnum)])
