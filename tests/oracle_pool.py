"""Oracle work on full-size layers spread over worker processes (test
infrastructure).

The full-size layers route hundreds of distinct experts whose fp32 weights
come from the GPU generator; quantizing and evaluating each with the float64
oracle takes a second or two, so the parity tests hand one expert per job to
a pool of spawned workers.  Workers import NumPy and the oracle only (never
torch or the GPU runtime); every job carries the expert's fp32 weights and the
activation rows routed to it, and returns the oracle's outputs for them.
"""
import concurrent.futures as cf
import multiprocessing as mp
import os

import numpy as np


def expert_job(job):
    """job = (fmt_gate_up, wg [F, H], wu [F, H], fmt_down, wd_rows [C, H's F],
    X [m, H]): the oracle's expert FFN on the rows X with the gate/up
    weights quantized whole and the down weights quantized on the sampled
    output rows only (quantization runs along the reduction axis, so a
    subset of rows quantizes exactly as in the whole matrix).  Returns
    (o [m, C], bound [m, C])."""
    from oracle import formats as fm
    from oracle import moe
    fgu, wg, wu, fd, wd_rows, X = job
    F, H = wg.shape
    X = np.asarray(X, dtype=np.float64)
    g, _ = moe.gemv(fgu, fm.quantize(fgu, wg), F, H, X)
    u, _ = moe.gemv(fgu, fm.quantize(fgu, wu), F, H, X)
    h = moe.silu(g) * u
    return moe.gemv(fd, fm.quantize(fd, wd_rows), wd_rows.shape[0], F, h)


def workers():
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def run(fn, jobs, inflight=None):
    """Results of fn over the job iterator, in job order, with at most
    `inflight` jobs submitted at a time (jobs hold large weight arrays)."""
    n = workers()
    inflight = inflight or 2 * n
    out = {}
    with cf.ProcessPoolExecutor(n, mp_context=mp.get_context("spawn")) as ex:
        pending = {}
        it = iter(enumerate(jobs))
        done_all = False
        while not done_all or pending:
            while not done_all and len(pending) < inflight:
                try:
                    i, job = next(it)
                except StopIteration:
                    done_all = True
                    break
                pending[ex.submit(fn, job)] = i
            if not pending:
                break
            finished, _ = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
            for f in finished:
                out[pending.pop(f)] = f.result()
    return [out[i] for i in range(len(out))]
