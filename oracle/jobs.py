"""Parallel oracle row jobs (test infrastructure).

The oracle itself stays single-threaded; independent query rows run in
separate spawned processes, each regenerating the workload's inputs on the
host (keys are generated once per process and cached).
"""
from __future__ import annotations

import os
from concurrent.futures import ProcessPoolExecutor
import multiprocessing as mp

import numpy as np

_keys_cache: dict = {}


def _workload(name: str, k: int | None):
    from dsa_inputs import configs
    wl = configs.WORKLOADS[name]
    return wl if k is None else wl.with_k(k)


def _prefill_keys(wl, n: int) -> np.ndarray:
    from dsa_inputs import configs
    key = (wl.name, 0)
    have = _keys_cache.get(key)
    if have is None or have.shape[0] < n:
        _keys_cache.clear()
        have = configs.k_idx_bytes(wl, 0, np.arange(wl.N))
        _keys_cache[key] = have
    return have


def prefill_job(args):
    """args = (workload name, row t, k or None) -> oracle chain dict."""
    import oracle
    name, t, k = args
    wl = _workload(name, k)
    keys = _prefill_keys(wl, t + 1)
    return oracle.prefill_row(wl, int(t), keys)


def indexer_row_job(args):
    """args = (prefill workload name, row t) -> the oracle's index scores of row t
    over keys 0..t (float64 [t + 1])."""
    import oracle
    from dsa_inputs import configs
    name, t = args
    wl = _workload(name, None)
    keys = _prefill_keys(wl, t + 1)
    return oracle.indexer_row(configs.q_idx_bytes(wl, [t])[0], configs.w_f32(wl, [t])[0], keys[: t + 1])


def decode_indexer_row_job(args):
    """args = (decode workload name, sequence b) -> the oracle's index scores of
    the decode query of sequence b over its ctx_len[b] keys."""
    import oracle
    from dsa_inputs import configs
    name, b = args
    wl = _workload(name, None)
    n = int(configs.ctx_lens(wl)[b])
    keys = configs.k_idx_bytes(wl, int(b), np.arange(n))
    return oracle.indexer_row(configs.q_idx_bytes(wl, [b])[0], configs.w_f32(wl, [b])[0], keys)


def timed_prefill_row_job(args):
    """args = (prefill workload name, row t) -> (n_t, seconds spent in the
    oracle's indexer, top-k and attention for row t).  Input generation (the
    row's query values and the selected latent rows) is outside the timing."""
    import time

    import oracle
    from dsa_inputs import configs
    name, t = args
    wl = _workload(name, None)
    keys = _prefill_keys(wl, t + 1)
    q_i, w, q = configs.q_idx_bytes(wl, [t])[0], configs.w_f32(wl, [t])[0], configs.q_bf16(wl, [t])[0]
    t0 = time.perf_counter()
    scores = oracle.indexer_row(q_i, w, keys[: t + 1])
    idx = oracle.topk_row(scores, wl.k)
    t1 = time.perf_counter()
    kv = oracle.gather_kv(wl, 0, idx)
    t2 = time.perf_counter()
    oracle.sparse_mla_row(q, kv, wl.scale, wl.D_v)
    t3 = time.perf_counter()
    return min(t + 1, wl.N), (t1 - t0) + (t3 - t2)


def decode_job(args):
    """args = (workload name, sequence b, k or None) -> oracle chain dict."""
    import oracle
    name, b, k = args
    wl = _workload(name, k)
    return oracle.decode_row(wl, int(b))


def dense_kl_job(args):
    """args = (workload name, row t) -> oracle dense warm-up loss dict."""
    import oracle
    name, t = args
    wl = _workload(name, None)
    keys = _prefill_keys(wl, t + 1)
    return oracle.dense_kl_row(wl, int(t), keys)


def paged_prefill_job(args):
    """args = (workload name, sequence b, position, k or None) -> oracle chain dict."""
    import oracle
    from dsa_inputs import configs
    name, b, pos, k = args
    wl = _workload(name, k)
    key = (wl.name, int(b))
    keys = _keys_cache.get(key)
    if keys is None:
        _keys_cache.clear()
        keys = configs.k_idx_bytes(wl, int(b), np.arange(int(configs.ctx_lens(wl)[b])))
        _keys_cache[key] = keys
    return oracle.paged_prefill_row(wl, int(b), int(pos), keys)


def default_procs() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def run(fn, jobs, procs: int | None = None):
    procs = procs or default_procs()
    if procs == 1 or len(jobs) == 1:
        return [fn(j) for j in jobs]
    ctx = mp.get_context("spawn")
    with ProcessPoolExecutor(max_workers=min(procs, len(jobs)), mp_context=ctx) as ex:
        return list(ex.map(fn, jobs, chunksize=max(1, len(jobs) // (4 * procs))))
