"""The oracle over every request of a batch, in a pool of worker processes.

Full-size parity compares every request, which takes the float64 oracle
minutes in one process.  Here the host copies of the inputs go into shared
memory once, and spawned worker processes (numpy and the oracle only: they
never touch the GPU) each run the oracle over a chunk of requests.  Results
are merged back in request order.
"""

from __future__ import annotations

import multiprocessing as mp
import os
from multiprocessing import shared_memory

import numpy as np

from . import verify as oracle


def default_workers() -> int:
    """Worker count: the host cores this process may use, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


_ATTACHED: dict = {}


def _attach(spec):
    name, shape, dtype = spec
    if name not in _ATTACHED:
        shm = shared_memory.SharedMemory(name=name)
        _ATTACHED[name] = (shm, np.ndarray(shape, dtype=np.dtype(dtype), buffer=shm.buf))
    return _ATTACHED[name][1]


def _wide(a: np.ndarray) -> np.ndarray:
    """float64 copy of logits held as bfloat16 bit patterns (int16) or float32."""
    if a.dtype == np.int16:
        return oracle.bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def _job(args):
    kind, specs, params, lo, hi = args
    A = {k: _attach(s)[lo:hi] for k, s in specs.items()}
    T, top_k, top_p = params.get("T", 1.0), params.get("top_k", 0), params.get("top_p", 1.0)
    if kind == "sample":
        o = oracle.verify_sample(_wide(A["logits"]), A["q"], A["ids"], A["u_accept"], A["u_resample"], T, top_k,
                                 top_p, beta=params.get("beta", 1.0))
    elif kind == "sample_draft_logits":
        o = oracle.verify_sample_draft_logits(_wide(A["logits"]), _wide(A["draft_logits"]), A["ids"], A["u_accept"],
                                              A["u_resample"], T, top_k, top_p)
    elif kind == "greedy":
        o = oracle.verify_greedy(_wide(A["logits"]), A["ids"])
    elif kind == "stats":
        o = oracle.accept_stats(_wide(A["logits"]), A["q"], A["ids"], T, top_k, top_p, with_boundary=True)
    elif kind == "stats_draft_logits":
        o = oracle.accept_stats_draft_logits(_wide(A["logits"]), _wide(A["draft_logits"]), A["ids"], T, top_k,
                                             top_p, with_boundary=True)
    else:
        raise ValueError(kind)
    return lo, o


def make_pool(workers: int | None = None):
    """A pool of oracle workers (spawned: fresh interpreters that import
    numpy and the oracle only), for several ``run`` calls."""
    return mp.get_context("spawn").Pool(workers or default_workers())


def run(kind: str, arrays: dict, params: dict, B: int, workers: int | None = None, pool=None, repeat: int = 1):
    """The oracle call `kind` over requests 0..B-1 of `arrays` (host numpy
    arrays, first axis = request), split over `workers` processes (or the
    processes of `pool`, from ``make_pool``).  Returns what the oracle call
    returns for the whole batch.  ``repeat`` > 1 runs the whole batch that
    many times (for timing; the results of the first run are returned)."""
    own = pool is None
    if own:
        workers = workers or default_workers()
    else:
        workers = pool._processes
    shms, specs = [], {}
    try:
        for k, a in arrays.items():
            a = np.ascontiguousarray(a)
            shm = shared_memory.SharedMemory(create=True, size=max(1, a.nbytes))
            shms.append(shm)
            np.ndarray(a.shape, dtype=a.dtype, buffer=shm.buf)[...] = a
            specs[k] = (shm.name, a.shape, a.dtype.str)
        chunk = max(1, -(-B // (workers * 4)))
        jobs = [(kind, specs, params, lo, min(lo + chunk, B)) for lo in range(0, B, chunk)]
        nj = len(jobs)
        jobs = jobs * max(1, int(repeat))
        if own:
            with make_pool(workers) as p:
                parts = list(p.imap(_job, jobs))[:nj]
        else:
            parts = list(pool.imap(_job, jobs))[:nj]
    finally:
        for shm in shms:
            shm.close()
            shm.unlink()
    outs = [o for _, o in parts]
    if isinstance(outs[0], dict):
        return {k: np.concatenate([o[k] for o in outs]) for k in outs[0]}
    return tuple(np.concatenate([o[i] for o in outs]) for i in range(len(outs[0])))
