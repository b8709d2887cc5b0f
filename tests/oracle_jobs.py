"""Oracle work cut into independent jobs for a process pool (test
infrastructure; imports only numpy and the oracle, so a pool worker started
with the "spawn" method never loads torch or touches the GPU).

* ``quantize_job``: one fp32 weight matrix -> the oracle's packed MX codes and
  E8M0 scales.
* ``partial_job``: the layer output of one expert's shard (local_offset = e,
  local_count = 1) on a set of token rows, or of the shared expert alone
  (local_count = 0).  The oracle's layer output is the sum of these shard
  outputs taken in ascending expert order and then the shared expert, which
  is the order its own loop adds them in (the shard-sum pin in
  tests/test_oracle_moe.py ties the two).
"""
from __future__ import annotations

import numpy as np

from oracle import moe as om


class ExpertArrays:
    """Indexable stand-in for an [E, ...] array holding only some experts;
    indexing a missing expert raises KeyError."""

    def __init__(self, per_expert: dict, E: int):
        self._d = per_expert
        some = next(iter(per_expert.values()))
        self.shape = (E,) + some.shape

    def __getitem__(self, e):
        return self._d[int(e)]


def quantize_job(args):
    """(fp32 matrix [N, K], fmt) -> (packed codes, scale codes)."""
    w, fmt = args
    return om.quantize_weight(np.asarray(w, dtype=np.float64), fmt)


class _Unused:
    """Stands in for an [E, ...] weight array that is never indexed (a shard
    with no local expert); moe_forward reads only its shape."""

    def __init__(self, E: int):
        self.shape = (E, 2, 1)

    def __getitem__(self, e):
        raise KeyError(e)


def partial_job(args):
    """One shard's output rows.

    args = (e, packed (w1, s1, w2, s2) of expert e or None, shared (ws1, ws1s,
    ws2, ws2s) or None, shared_weight, x rows [n, H] (exact bf16 values as
    float64), ids [n, k], weights [n, k], E, k, wfmt, act).  e = -1 computes
    the shared expert alone.  Returns (e, y rows [n, H] float64)."""
    e, packed, shared, shared_weight, x, ids, w, E, k, wfmt, act = args
    if e >= 0:
        arrs = tuple(ExpertArrays({e: a}, E) for a in packed)
        off, cnt, sh = e, 1, None
    else:
        arrs = (_Unused(E),) * 4
        off, cnt, sh = 0, 0, shared
    r = om.moe_forward(x, None, *arrs, k=k, wfmt=wfmt, act=act, topk_ids=ids, topk_w=w, shared=sh,
                       shared_weight=shared_weight, local_offset=off, local_count=cnt)
    return e, r["y"]
