"""Oracle results for the full-size parity cases, computed in CPU worker processes.

The oracle needs seconds per (sequence, kv head) at 32k tokens and more at 131k, so the full-size tests
compare many pairs only if that work runs in parallel and early.  The workers are started when the test
session is configured, before any test touches the GPU, so that the test process never starts a process
after it has initialised the GPU; they import only the seeded input generators and the oracle (no torch,
no library).  After collection the jobs of the selected tests are submitted and run while the other tests
use the GPU; a test then waits for its results.  Without a pool (a CPU-only session, or a test run on its
own with the pool switched off) a job runs in the test process.
"""
from __future__ import annotations

import multiprocessing as mp
import os
import time
from concurrent.futures import ProcessPoolExecutor
from typing import Dict, Optional

import numpy as np

_POOL: Optional[ProcessPoolExecutor] = None
_FUTURES: Dict[str, object] = {}


def n_workers() -> int:
    """Worker count: the cores this process may use, less four for the test process, at most 8."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(8, n - 4))


def _ready() -> int:
    import oracle  # noqa: F401  (the imports a job needs, done once per worker)
    import synth  # noqa: F401
    # the workers yield to the test process (which runs its own oracle work with a full BLAS pool) and use one
    # BLAS thread each
    os.nice(10)
    from threadpoolctl import threadpool_limits
    threadpool_limits(limits=1)
    time.sleep(0.5)  # busy while the other workers start, so that every submission starts a process of its own
    return os.getpid()


def start() -> None:
    """Start every worker now (a spawn pool starts a process per submission while none is idle)."""
    global _POOL
    if _POOL is not None:
        return
    n = n_workers()
    _POOL = ProcessPoolExecutor(max_workers=n, mp_context=mp.get_context("spawn"))
    pids = {f.result() for f in [_POOL.submit(_ready) for _ in range(n)]}
    assert len(pids) == n, f"oracle pool: {len(pids)} of {n} workers started"


def stop() -> None:
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=False, cancel_futures=True)
        _POOL = None


def submit(jobs: Dict[str, dict]) -> None:
    if _POOL is None:
        return
    for key, spec in jobs.items():
        if key not in _FUTURES:
            _FUTURES[key] = _POOL.submit(pair_job, spec)


def result(key: str, spec: dict, timeout: float = 1200.0) -> dict:
    fut = _FUTURES.get(key)
    if fut is None:
        return pair_job(spec)
    return fut.result(timeout=timeout)


# ------------------------------------------------------------------------------------------------ jobs


def job(workload: str, lens, b: int, heads, overrides: Optional[dict] = None, groups: Optional[dict] = None,
        tokens: Optional[dict] = None) -> dict:
    """One sequence of a seeded workload: the oracle output of the given kv heads, the quantized state of
    sampled groups (grouped schemes: {head: [group, ...]}) or tokens (INT4 per token: {head: [token, ...]}),
    and the band of those heads."""
    return {"workload": workload, "overrides": dict(overrides or {}), "lens": [int(t) for t in lens], "b": int(b),
            "heads": [int(h) for h in heads], "groups": {int(k): [int(g) for g in v] for k, v in (groups or {}).items()},
            "tokens": {int(k): [int(t) for t in v] for k, v in (tokens or {}).items()}}


def pair_job(spec: dict) -> dict:
    import oracle as O
    import synth
    from kvq_cases import GROUPED, rotations, source_of

    wl = synth.scaled(synth.WORKLOADS[spec["workload"]], batch=len(spec["lens"]), **spec["overrides"])
    rk, rv = rotations(wl)
    q = synth.queries(wl)
    b = spec["b"]
    T = spec["lens"][b]
    gq = wl.n_q_heads // wl.n_kv_heads
    res = {}
    if T == 0:
        return {h: {"out": np.zeros((gq, 128))} for h in spec["heads"]}
    k, v = source_of(wl, b, T)
    for h in spec["heads"]:
        qh = q[b, h * gq:(h + 1) * gq]
        r = {}
        if wl.scheme in GROUPED:
            o, st = O.decode_int2(qh, k[:, h], v[:, h], T, wl.n_sink, wl.n_recent, wl.clip_k, wl.clip_v, rk, rv,
                                  axis=GROUPED[wl.scheme])
            gs = spec["groups"].get(h, [])
            r["groups"] = {int(g): {key: st[key][int(g)] for key in ("k_codes", "v_codes", "k_s16", "k_z16",
                                                                      "v_s16", "v_z16")} for g in gs}
            if gs:
                r["band"] = (st["band_pos"], st["band_k"], st["band_v"])
        else:
            o, st = O.decode_int4(qh, k[:, h], v[:, h], T, rk.astype(np.int8),
                                  None if rv is None else rv.astype(np.int8), block=wl.hadamard_block)
            ts = np.asarray(spec["tokens"].get(h, []), dtype=np.int64)
            r["tokens"] = ts
            r["state"] = {key: st[key][ts] for key in ("k_codes", "v_codes", "k_s16", "k_z16", "v_s16", "v_z16")}
        r["out"] = o
        res[h] = r
    return res
