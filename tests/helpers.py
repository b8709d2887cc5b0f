"""Shared test helpers: weight preparation on both sides and the tolerance check.

The GPU side quantizes fp32 weights with the library's mx_quantize; the oracle
side quantizes the same fp32 weights with oracle.mx.  Neither side ever sees
the other's codes as input; tests compare them.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os
import sys

import numpy as np
import torch

from block_scaled_precision_amd import inputs as gen

# y tolerance: max|gpu - ref| <= 2e-2 * max|ref| and ||gpu - ref|| / ||ref|| <= 1e-2
MAX_REL = 2e-2
RMS_REL = 1e-2


def y_error(gpu_y: np.ndarray, ref_y: np.ndarray):
    d = gpu_y.astype(np.float64) - ref_y
    max_rel = np.max(np.abs(d)) / max(np.max(np.abs(ref_y)), 1e-300)
    rms_rel = np.linalg.norm(d) / max(np.linalg.norm(ref_y), 1e-300)
    return float(max_rel), float(rms_rel)


def assert_y_close(gpu_y, ref_y, what=""):
    mr, rr = y_error(gpu_y, ref_y)
    assert mr <= MAX_REL and rr <= RMS_REL, f"{what}: max_rel={mr:.3e} rms_rel={rr:.3e}"
    return mr, rr


def print_flush(*a):
    print(*a, flush=True)


# ------------------------------------------------------------ GPU side ----

def gpu_weights(w: gen.Workload, seed: int = 0, experts=None, device="cuda", fp32_on="cpu"):
    """Quantize every expert's fp32 weights with the library (mx_quantize).

    fp32 weights are drawn on `fp32_on` ("cpu" for small workloads so the
    oracle can receive the identical tensors; "cuda" for full-size runs).
    Returns MoeWeights with [E, ...] packed tensors on the GPU.
    """
    from block_scaled_precision_amd import moe_mx as m
    E = w.E if experts is None else experts
    bits = m.FORMAT_BITS[w.wfmt]
    w1 = torch.empty((E, 2 * w.I, w.H * bits // 8), dtype=torch.uint8, device=device)
    s1 = torch.empty((E, 2 * w.I, w.H // 32), dtype=torch.uint8, device=device)
    w2 = torch.empty((E, w.H, w.I * bits // 8), dtype=torch.uint8, device=device)
    s2 = torch.empty((E, w.H, w.I // 32), dtype=torch.uint8, device=device)
    for e in range(E):
        a = gen.expert_w1(w, e, seed, device=fp32_on).to(device)
        m.mx_quantize(a, w.wfmt, codes=w1[e], scales=s1[e])
        b = gen.expert_w2(w, e, seed, device=fp32_on).to(device)
        m.mx_quantize(b, w.wfmt, codes=w2[e], scales=s2[e])
    mw = m.MoeWeights(w1, s1, w2, s2, w.wfmt)
    if w.I_shared:
        a = gen.shared_w1(w, seed, device=fp32_on).to(device)
        b = gen.shared_w2(w, seed, device=fp32_on).to(device)
        mw.ws1, mw.ws1_scale = m.mx_quantize(a, w.wfmt)
        mw.ws2, mw.ws2_scale = m.mx_quantize(b, w.wfmt)
    return mw


# --------------------------------------------------------- oracle side ----

from tests.oracle_jobs import ExpertArrays, partial_job, quantize_job  # noqa: E402

_POOL = None


def pool_workers() -> int:
    """Pool size: the CPUs this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def pool() -> cf.ProcessPoolExecutor:
    """One process pool for the oracle jobs, started with "spawn": its workers
    are fresh interpreters that import only numpy and the oracle, so nothing
    is forked from a process that has initialised HIP."""
    global _POOL
    if _POOL is None:
        _POOL = cf.ProcessPoolExecutor(max_workers=pool_workers(), mp_context=mp.get_context("spawn"))
    return _POOL


def shutdown_pool():
    global _POOL
    if _POOL is not None:
        _POOL.shutdown(wait=True, cancel_futures=True)
        _POOL = None


def _bounded_map(fn, jobs, in_flight):
    """fn over the jobs in the pool, keeping at most `in_flight` submitted
    (each job may carry a large array); results in job order."""
    ex = pool()
    out = [None] * len(jobs)
    pending = {}
    it = iter(enumerate(jobs))
    for i, job in it:
        pending[ex.submit(fn, job)] = i
        if len(pending) >= in_flight:
            done, _ = cf.wait(pending, return_when=cf.FIRST_COMPLETED)
            for f in done:
                out[pending.pop(f)] = f.result()
    for f in cf.as_completed(list(pending)):
        out[pending.pop(f)] = f.result()
    return out


def oracle_weights(w: gen.Workload, seed: int = 0, experts=None, fp32_on="cpu", cache=None):
    """Quantize the fp32 weights of the listed experts with the oracle.

    Returns dict expert -> (w1, s1, w2, s2) numpy arrays, plus "shared" when
    the workload has a shared expert.  `cache` (a dict) keeps results across
    calls for workloads with the same weight shapes and seed.
    """
    ids = list(range(w.E)) if experts is None else list(experts)
    if w.I_shared:
        ids.append("shared")
    cache = {} if cache is None else cache
    key = lambda e: (w.H, w.I, w.E, w.I_shared, w.wfmt, seed, e)  # noqa: E731
    todo = [e for e in ids if key(e) not in cache]

    def mats(e):
        if e == "shared":
            return (gen.shared_w1(w, seed, device=fp32_on).cpu().numpy(),
                    gen.shared_w2(w, seed, device=fp32_on).cpu().numpy())
        return (gen.expert_w1(w, e, seed, device=fp32_on).cpu().numpy(),
                gen.expert_w2(w, e, seed, device=fp32_on).cpu().numpy())

    values = sum(3 * (w.I_shared if e == "shared" else w.I) * w.H for e in todo)
    if values <= 4_000_000:
        for e in todo:
            a, b = mats(e)
            cache[key(e)] = quantize_job((a, w.wfmt)) + quantize_job((b, w.wfmt))
    else:
        # fp32 matrices are drawn lazily, a bounded number in flight
        ex = pool()
        limit = 2 * pool_workers()
        pending = {}
        res = {e: [None, None] for e in todo}

        finished = [0]

        def drain(block):
            done, _ = cf.wait(pending, return_when=cf.FIRST_COMPLETED if block else cf.ALL_COMPLETED)
            for f in done:
                e, part = pending.pop(f)
                res[e][part] = f.result()
                finished[0] += 1
                if finished[0] % 64 == 0:  # progress on stderr: bench.py's stdout is one JSON line
                    print(f"  oracle quantized {finished[0]} of {2 * len(todo)} weight matrices",
                          file=sys.stderr, flush=True)

        for e in todo:
            for part, m in enumerate(mats(e)):
                pending[ex.submit(quantize_job, (m, w.wfmt))] = (e, part)
                if len(pending) >= limit:
                    drain(True)
        while pending:
            drain(False)
        for e, (q1, q2) in res.items():
            cache[key(e)] = q1 + q2
    return {e: cache[key(e)] for e in ids}


def oracle_rows(w: gen.Workload, x_rows: torch.Tensor, ids: np.ndarray, wts: np.ndarray, seed: int = 0,
                fp32_on="cpu", cache=None, shared_weight: float = 1.0) -> np.ndarray:
    """Oracle layer output (float64) for the given token rows, computed as one
    job per expert shard (and one for the shared expert) in the pool and
    summed in the oracle's own order.  x_rows [n, H] bf16; ids / wts [n, k]:
    the oracle's routing of those tokens."""
    experts = sorted(set(int(e) for e in np.asarray(ids).ravel()))
    ow = oracle_weights(w, seed, experts, fp32_on=fp32_on, cache=cache)
    xs = x_rows.to(torch.float64).cpu().numpy()
    jobs = [(e, ow[e], None, 1.0, xs, ids, wts, w.E, w.k, w.wfmt, w.act) for e in experts]
    if w.I_shared:
        jobs.append((-1, None, ow["shared"], shared_weight, xs, ids, wts, w.E, w.k, w.wfmt, w.act))
    parts = _bounded_map(partial_job, jobs, 2 * pool_workers())
    y = np.zeros((xs.shape[0], w.H), dtype=np.float64)
    for _, part in parts:  # ascending expert, then the shared expert
        y += part
    return y


def oracle_arrays(ow: dict, E: int):
    """(w1, s1, w2, s2) indexable by expert, from oracle_weights()."""
    routed = {e: v for e, v in ow.items() if e != "shared"}
    return tuple(ExpertArrays({e: v[i] for e, v in routed.items()}, E) for i in range(4))
