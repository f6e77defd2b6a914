"""Process-pool drivers of the CPU oracle.

TEST INFRASTRUCTURE ONLY, like ``hils_oracle``: the tests and the benchmark's
CPU-baseline leg use it; nothing in the product path may.  It adds no
arithmetic: every worker calls the unchanged ``ref_forward`` / ``ref_backward``
on a block of query positions of one (batch, KV head) group, and the caller
sums the per-block gradient contributions (disjoint query sets, so the sum is
the oracle's own sum over queries, in another order).

Workers are started with the "spawn" method and import only numpy and the
oracle, so they never touch a GPU, and each runs its linear algebra on one
thread (the pool is the parallelism).
"""
import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np


def _init_worker():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:   # threadpoolctl is optional; the variables above still apply
        pass


def default_workers():
    """Host cores to use: all of them, capped at 16 (the host share of one GPU)."""
    return max(1, min(os.cpu_count() or 1, 16))


def make_pool(workers=None):
    ctx = multiprocessing.get_context("spawn")
    return ProcessPoolExecutor(max_workers=workers or default_workers(), mp_context=ctx,
                               initializer=_init_worker)


def _group(arr, b, hs):
    return None if arr is None else arr[b:b + 1, hs]


class _OneGroup:
    """A [1, 1, L, d] stand-in for one group's K or V: ``x[0, 0]`` returns the
    group's rows (a numpy view, or a lazily regenerated cache that is never
    materialised whole), which is all the oracle reads."""

    def __init__(self, rows):
        self.rows = rows
        self.shape = (1, 1) + tuple(rows.shape)

    def __getitem__(self, key):
        if key != (0, 0):
            raise IndexError("one group only")
        return self.rows


class _QueryRows:
    """A [1, G, Lq, d] stand-in for one group's query-side rows (q, q_ret or dO)
    that holds only the rows of the queries a job computes: ``x[0, 0:G, i]`` is
    query i's [G, d] rows, which is all the oracle reads."""

    def __init__(self, group_rows, queries):
        self.shape = (1,) + tuple(group_rows.shape)
        self.rows = {int(i): np.array(group_rows[:, int(i)]) for i in queries}

    def __getitem__(self, key):
        b, hs, i = key
        if b != 0 or hs != slice(0, self.shape[1]):
            raise IndexError("one group only")
        return self.rows[int(i)]


def _fwd_job(args):
    from .hils_oracle import ref_forward
    q, k, v, lmk, bias, q_ret, qs, kw = args
    return ref_forward(q, k, v, lmk, bias, queries=qs, q_ret=q_ret, **kw)


def _bwd_job(args):
    from .hils_oracle import ref_backward
    q, k, v, lmk, bias, dout, q_ret, qs, forced, kw = args
    return ref_backward(q, k, v, lmk, bias, dout, queries=qs, forced_idx=forced, q_ret=q_ret, **kw)


def _blocks(queries, nblocks):
    queries = np.asarray(queries)
    n = max(1, min(nblocks, len(queries)))
    return [blk for blk in np.array_split(queries, n) if len(blk)]


def _job_inputs(host, b, g, queries, with_dout=False):
    """Pickle-sized inputs of one job: the group's rows of the job's queries, its
    K, V (views or lazy), landmarks and bias."""
    G = host["q"].shape[1] // host["k"].shape[1]
    hs = slice(g * G, (g + 1) * G)
    rows = lambda name: (None if host.get(name) is None
                         else _QueryRows(host[name][b, hs], queries))
    out = dict(q=rows("q"), q_ret=rows("q_ret"),
               k=_OneGroup(host["k"][b, g]), v=_OneGroup(host["v"][b, g]),
               lmk=host["lmk"][b:b + 1, g:g + 1],
               bias=None if host.get("bias") is None else host["bias"][b:b + 1, g:g + 1])
    if with_dout:
        out["dout"] = rows("dout")
    return out


def forward_tasks(pool, host, tasks, timeout=900, **kw):
    """ref_forward for each task (b, g, queries) of ``tasks``, in the pool.
    Returns, per task, out [G, nq, d], idx [nq, K], lse [G, nq]."""
    jobs = []
    for b, g, qs in tasks:
        x = _job_inputs(host, b, g, qs)
        jobs.append((x["q"], x["k"], x["v"], x["lmk"], x["bias"], x["q_ret"], np.asarray(qs), kw))
    return [(r[0][0], r[1][0, 0], r[2][0]) for r in pool.map(_fwd_job, jobs, timeout=timeout)]


def group_forward(pool, host, b, g, queries, nblocks, timeout=900, **kw):
    """ref_forward of the queries of group (b, g), split over the pool.
    Returns out [G, nq, d], idx [nq, K], lse [G, nq]."""
    res = forward_tasks(pool, host, [(b, g, blk) for blk in _blocks(queries, nblocks)],
                        timeout=timeout, **kw)
    return (np.concatenate([r[0] for r in res], axis=1), np.concatenate([r[1] for r in res], axis=0),
            np.concatenate([r[2] for r in res], axis=1))


def group_backward(pool, host, b, g, queries, forced_idx, nblocks, timeout=900, **kw):
    """ref_backward of the queries of group (b, g) with the selection ``forced_idx``
    ([nq, K], -1 padded, rows in the order of ``queries``), split over the pool.
    Returns (dq, dk, dv, dlmk, dbias[, dq_ret]) for the group alone: dq [G, Lq, d]
    (rows outside ``queries`` zero), dk, dv [Lkv, d], dlmk [NCcap, d], dbias [NCcap]."""
    queries = np.asarray(queries)
    pos = {int(i): n for n, i in enumerate(queries)}
    jobs = []
    for blk in _blocks(queries, nblocks):
        x = _job_inputs(host, b, g, blk, with_dout=True)
        forced = np.asarray(forced_idx)[[pos[int(i)] for i in blk]][None, None]
        jobs.append((x["q"], x["k"], x["v"], x["lmk"], x["bias"], x["dout"], x["q_ret"], blk,
                     forced, kw))
    total = None
    for r in pool.map(_bwd_job, jobs, timeout=timeout):
        parts = [r[0][0], r[1][0, 0], r[2][0, 0], r[3][0, 0], r[4][0, 0]]
        if len(r) > 5:
            parts.append(r[5][0])
        total = parts if total is None else [a + p for a, p in zip(total, parts)]
    return tuple(total)


def _noop(x):
    return x


def warm_up(pool, workers):
    """Start every worker (and its imports) before anything is timed."""
    list(pool.map(_noop, range(4 * workers), timeout=300))
    from . import hils_oracle  # noqa: F401  (the parent imports it too, for symmetry)
