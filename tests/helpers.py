"""Shared test helpers: weight preparation on both sides and the tolerance check.

The GPU side quantizes fp32 weights with the library's mx_quantize; the oracle
side quantizes the same fp32 weights with oracle.mx.  Neither side ever sees
the other's codes as input; tests compare them.
"""
from __future__ import annotations

import concurrent.futures as cf
import multiprocessing as mp
import os

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

def _oracle_quantize(arr: np.ndarray, fmt: str):
    from oracle import moe as om
    return om.quantize_weight(arr.astype(np.float64), fmt)


def oracle_weights(w: gen.Workload, seed: int = 0, experts=None, fp32_on="cpu", workers=None):
    """Quantize the fp32 weights of the listed experts with the oracle.

    Returns dict expert -> (w1, s1, w2, s2) numpy arrays, plus "shared" when
    the workload has a shared expert.
    """
    ids = list(range(w.E)) if experts is None else list(experts)
    jobs = []
    for e in ids:
        jobs.append((e, "w1", gen.expert_w1(w, e, seed, device=fp32_on).cpu().numpy()))
        jobs.append((e, "w2", gen.expert_w2(w, e, seed, device=fp32_on).cpu().numpy()))
    if w.I_shared:
        jobs.append(("shared", "w1", gen.shared_w1(w, seed, device=fp32_on).cpu().numpy()))
        jobs.append(("shared", "w2", gen.shared_w2(w, seed, device=fp32_on).cpu().numpy()))
    big = sum(j[2].size for j in jobs) > 4_000_000
    res = {}
    if big:
        nw = workers or min(8, os.cpu_count() or 1, len(jobs))
        # fork: the workers only run numpy and never touch the GPU
        with cf.ProcessPoolExecutor(max_workers=nw, mp_context=mp.get_context("fork")) as ex:
            outs = list(ex.map(_oracle_quantize, [j[2] for j in jobs], [w.wfmt] * len(jobs)))
    else:
        outs = [_oracle_quantize(j[2], w.wfmt) for j in jobs]
    for (e, kind, _), (p, s) in zip(jobs, outs):
        res.setdefault(e, {})[kind] = (p, s)
    return {e: (d["w1"][0], d["w1"][1], d["w2"][0], d["w2"][1]) for e, d in res.items()}


class ExpertArrays:
    """Indexable stand-in for an [E, ...] array holding only some experts;
    indexing a missing expert raises KeyError."""

    def __init__(self, per_expert: dict, E: int):
        self._d = per_expert
        some = next(iter(per_expert.values()))
        self.shape = (E,) + some.shape

    def __getitem__(self, e):
        return self._d[int(e)]


def oracle_arrays(ow: dict, E: int):
    """(w1, s1, w2, s2) indexable by expert, from oracle_weights()."""
    routed = {e: v for e, v in ow.items() if e != "shared"}
    return tuple(ExpertArrays({e: v[i] for e, v in routed.items()}, E) for i in range(4))
