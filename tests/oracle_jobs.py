"""Oracle key-switches of whole GPU workloads on the host's cores (test infrastructure).

A job names its key by the seeds the key is drawn from, and the worker builds the
key itself: the b-half as uniform residues from the input generator
(`rns_ckks_key_amd.synth`, the module both sides may use), the a-half with the
oracle's expander.  So no key crosses a process boundary, and a worker that
meets a key again reuses it.  Workers are spawned processes that import numpy,
the oracle and the input generator only: they never touch the GPU.
"""
from __future__ import annotations

import functools
import multiprocessing as mp
from concurrent.futures import ProcessPoolExecutor

import numpy as np


@functools.lru_cache(maxsize=None)
def _params(chain: tuple):
    from oracle.params import Params

    return Params.make(*chain)


@functools.lru_cache(maxsize=2)  # two keys of 151 MB each per worker
def _key(chain: tuple, kb_seed: int, a_seed: bytes):
    from oracle.chacha import expand_key_a
    from rns_ckks_key_amd import synth

    pr = _params(chain)
    kb = synth.uniform_key_rows(kb_seed, pr.primes, pr.dnum, pr.n).astype(np.uint64)
    return kb, expand_key_a(a_seed, pr.primes, pr.dnum, pr.n)


def _switch(job: tuple) -> np.ndarray:
    from oracle import ks

    chain, ct, level, galois, kb_seed, a_seed = job
    kb, ka = _key(chain, kb_seed, a_seed)
    return ks.keyswitch(_params(chain), ct.astype(np.uint64), level, kb, galois, key_a=ka)


def switch_all(chain: tuple, jobs: list[tuple], max_workers: int | None = None) -> list[np.ndarray]:
    """Oracle key-switch of each job (ct [2][level][N], level, galois, b-half seed, a-half seed),
    in job order.  chain = (log_n, L, K, dnum, bits) of oracle.params.Params.make."""
    from oracle.pool import workers

    n = max(1, min(len(jobs), max_workers or workers(16)))
    args = [(chain, np.ascontiguousarray(ct, dtype=np.uint32), int(level), int(g), int(kbs), bytes(a))
            for ct, level, g, kbs, a in jobs]
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn")) as ex:
        return list(ex.map(_switch, args, timeout=900.0))


_KEY: dict = {}


def _init_key(chain: tuple, kb: np.ndarray, ka: np.ndarray) -> None:
    _KEY["pr"] = _params(chain)
    _KEY["key"] = (kb.astype(np.uint64), ka.astype(np.uint64))


def _mul_relin_rescale(job: tuple) -> np.ndarray:
    from oracle import mult

    x, y, level = job
    kb, ka = _KEY["key"]
    return mult.mul_relin_rescale(_KEY["pr"], x.astype(np.uint64), y.astype(np.uint64), level, kb, key_a=ka)


def mul_relin_rescale_all(chain: tuple, kb, ka, jobs: list[tuple], max_workers: int | None = None) -> list[np.ndarray]:
    """Oracle multiply-relinearise-rescale of each job (x, y [2][level][N], level) under one
    relinearisation key (kb, ka [dnum][L+K][N]), given to each worker once; outputs in job order."""
    from oracle.pool import workers

    n = max(1, min(len(jobs), max_workers or workers(16)))
    key = (np.ascontiguousarray(kb, dtype=np.uint32), np.ascontiguousarray(ka, dtype=np.uint32))
    args = [(np.ascontiguousarray(x, dtype=np.uint32), np.ascontiguousarray(y, dtype=np.uint32), int(level))
            for x, y, level in jobs]
    with ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"), initializer=_init_key,
                             initargs=(chain, *key)) as ex:
        return list(ex.map(_mul_relin_rescale, args, timeout=900.0))
