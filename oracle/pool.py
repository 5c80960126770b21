"""The oracle's key-switch on several host cores at once (test infrastructure only:
used by tests/ and by the benchmark's CPU baseline).

Workers are spawned processes that import numpy and the oracle only: they never
touch the GPU, whatever the parent process has initialised.  The keys go to each
worker once, through the pool initializer; each job is one ciphertext.
"""
from __future__ import annotations

import multiprocessing as mp
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np

_STATE: dict = {}
START_TIMEOUT_S = 120.0   # a worker that has not started by then has failed


def _init(chain: tuple, keys: list) -> None:
    from oracle.params import Params

    _STATE["pr"] = Params.make(*chain)
    _STATE["keys"] = [(kb.astype(np.uint64), ka.astype(np.uint64)) for kb, ka in keys]


def _keyswitch(job: tuple) -> np.ndarray:
    from oracle import ks as oks

    ct, level, g, k = job
    kb, ka = _STATE["keys"][k]
    return oks.keyswitch(_STATE["pr"], ct.astype(np.uint64), level, kb, g, key_a=ka)


def workers(limit: int = 8) -> int:
    """Worker count: the host cores this process may use, at most `limit` (16 is a GPU machine's share)."""
    return max(1, min(limit, len(os.sched_getaffinity(0))))


def _nap(seconds: float) -> int:
    import time

    time.sleep(seconds)
    return os.getpid()


def start_pool(chain: tuple, key_b, key_a, max_workers: int) -> ProcessPoolExecutor:
    """A started pool of `max_workers` spawned workers holding the keys (see keyswitch_many)."""
    keys = list(zip(key_b, key_a)) if isinstance(key_b, (list, tuple)) else [(key_b, key_a)]
    keys32 = [(np.ascontiguousarray(kb, dtype=np.uint32), np.ascontiguousarray(ka, dtype=np.uint32))
              for kb, ka in keys]
    ex = ProcessPoolExecutor(max_workers=max_workers, mp_context=mp.get_context("spawn"), initializer=_init,
                             initargs=(chain, keys32))
    # one short nap per worker: returns once every worker has started and holds the keys
    try:
        list(ex.map(_nap, [0.5] * max_workers, timeout=START_TIMEOUT_S))
    except BaseException:
        ex.shutdown(wait=False, cancel_futures=True)
        raise
    return ex


def run_jobs(ex: ProcessPoolExecutor, jobs: list[tuple], timeout: float = 600.0) -> list[np.ndarray]:
    """Oracle key-switch of each (ct, level, galois[, key index]) on a started pool, in job order."""
    jobs = [j if len(j) == 4 else tuple(j) + (0,) for j in jobs]
    return list(ex.map(_keyswitch, [(np.ascontiguousarray(c, dtype=np.uint32), lv, g, k) for c, lv, g, k in jobs],
                       timeout=timeout))


def keyswitch_many(chain: tuple, key_b, key_a, jobs: list[tuple], max_workers: int | None = None) -> list[np.ndarray]:
    """Oracle key-switch of each job, in job order.

    chain = (log_n, L, K, dnum, bits) of oracle.params.Params.make.  Either key_b and
    key_a are one key's halves and a job is (ct [2][l][N], level, galois), or they
    are equal-length lists of keys and a job is (ct, level, galois, key index)."""
    keys = list(zip(key_b, key_a)) if isinstance(key_b, (list, tuple)) else [(key_b, key_a)]
    jobs = [j if len(j) == 4 else tuple(j) + (0,) for j in jobs]
    n = min(len(jobs), max_workers or workers())
    ctx = mp.get_context("spawn")
    keys32 = [(np.ascontiguousarray(kb, dtype=np.uint32), np.ascontiguousarray(ka, dtype=np.uint32))
              for kb, ka in keys]
    with ProcessPoolExecutor(max_workers=n, mp_context=ctx, initializer=_init, initargs=(chain, keys32)) as ex:
        return list(ex.map(_keyswitch, [(np.ascontiguousarray(c, dtype=np.uint32), lv, g, k) for c, lv, g, k in jobs],
                           timeout=600.0))
