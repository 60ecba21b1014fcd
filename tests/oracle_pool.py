"""Parallel evaluation of the CPU oracle, one (sequence, q head) per task.

Test infrastructure: the full-size parity tests compare every output element of a
workload with the oracle, which evaluates one N x N score matrix per (sequence, q head)
in float64.  Those evaluations are independent, so they run in a pool of CPU worker
processes; each worker calls ``oracle.rope_attention`` unchanged on its head and returns
only the error of the GPU's rows against it.  The workers import numpy and the oracle
only (never torch or the HIP library) and use one BLAS thread each.
"""

import multiprocessing as mp
import os

import numpy as np

import oracle as orc

_BLAS_ENV = ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS")


def head_error(task):
    """Oracle attention of one (sequence, q head) against the GPU's rows of it.

    task: (q [L, D], k [L, D], v [L, D], cos [L, D], sin [L, D], scale, causal, pairing,
    got_o [L, D], got_lse [L] or None), every array holding the exact values both sides
    consumed (inputs and tables as stored, outputs as returned).
    Returns (max |got_o - ref_o|, max |got_lse - ref_lse| or 0, finite).
    """
    q, k, v, cos, sin, scale, causal, pairing, got_o, got_lse = task
    L = q.shape[0]
    ref_o, ref_lse = orc.rope_attention(q[:, None], k[:, None], v[:, None], cos, sin, [L], scale, causal,
                                        pairing=pairing)
    got_o = np.asarray(got_o, dtype=np.float64)
    finite = bool(np.all(np.isfinite(got_o)))
    err_o = float(np.abs(got_o - ref_o[:, 0]).max()) if L else 0.0
    err_l = 0.0
    if got_lse is not None and L:
        err_l = float(np.abs(np.asarray(got_lse, dtype=np.float64) - ref_lse[0]).max())
    return err_o, err_l, finite


def workers_for(seq_len: int) -> int:
    """Pool size: the CPUs this process may use (at most 16), bounded by the memory that
    one N x N float64 evaluation needs (about five N^2 arrays live at its peak)."""
    cpus = min(16, len(os.sched_getaffinity(0)))
    per_task = 5 * 8 * float(seq_len) ** 2 + 256e6
    try:
        with open("/proc/meminfo") as fh:
            avail = next(int(ln.split()[1]) * 1024 for ln in fh if ln.startswith("MemAvailable"))
    except (OSError, StopIteration, ValueError):
        avail = 16e9
    return max(1, min(cpus, int(0.6 * avail / per_task)))


def map_heads(tasks, seq_len: int):
    """Run head_error over an iterable of tasks in a spawned worker pool; results in task
    order.  Tasks are drawn from the iterable as workers take them, so a generator keeps
    only a few of them in memory."""
    n = workers_for(seq_len)
    saved = {k: os.environ.get(k) for k in _BLAS_ENV}
    for k in _BLAS_ENV:
        os.environ[k] = "1"
    try:
        pool = mp.get_context("spawn").Pool(n)
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    try:
        return list(pool.imap(head_error, tasks, chunksize=1))
    finally:
        pool.close()
        pool.join()
