"""Softmax/top-k routing and the permutation of assignments by expert -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources.
* "mxfp6-sm120" page, table of paths: the routed MoE path begins with routing;
  section "Execution model": the grouped path uses indirect routing (rows are
  gathered per expert through an index list).
* "TokenSpeed SiTU" page, section "Supported contract": top-k expert ids are
  global ids; routing may be supplied precomputed; each rank keeps only the
  experts of its contiguous shard [local_offset, local_offset + local_count).
* "fusedtok" page, determinism notes: selection ties resolve to the earliest
  index.

Readings (where the pages are silent):
* top-k is taken on the fp32 logits (softmax is monotone, so this is the same
  set as top-k of the probabilities), larger logit first, equal logits ->
  lower expert id first;
* the routing weights are the softmax over all E logits renormalised over the k
  chosen experts, which equals exp(l_j - l_max) / sum_selected exp(l_i - l_max);
* within one expert's segment, assignments are ordered by ascending token.
"""
from __future__ import annotations

import numpy as np


def topk_route(logits: np.ndarray, k: int):
    """logits [T, E] float32 -> (ids [T, k] int32, weights [T, k] float64).

    For each token: order experts by (logit descending, id ascending), keep
    the first k in that order, then weight them by a softmax over the chosen
    logits computed in float64.
    """
    logits = np.asarray(logits, dtype=np.float32)
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError("need 1 <= k <= E")
    if np.any(np.isnan(logits)):
        raise ValueError("NaN logits")
    ids = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    expert = np.arange(E)
    for t in range(T):
        row = logits[t].astype(np.float64)
        order = np.lexsort((expert, -row))   # primary: -logit ascending, then id
        sel = order[:k]
        ids[t] = sel
        ls = row[sel]
        top = ls.max()
        if not np.isfinite(top):
            raise ValueError("token with no finite logit among its top-k")
        ex = np.exp(ls - top)
        w[t] = ex / ex.sum()
    return ids, w


def permute(ids: np.ndarray, num_experts: int, local_offset: int = 0, local_count: int | None = None):
    """Counting sort of the assignments a = t*k + j by expert.

    Returns (counts [L], offsets [L+1], sorted_assign [offsets[L]]) over the
    local experts e in [local_offset, local_offset + L), L = local_count
    (default: all experts).  offsets is the exclusive prefix sum of counts and
    sorted_assign[offsets[i]:offsets[i+1]] lists, in ascending assignment id
    (= ascending token), the assignments routed to expert local_offset + i.
    Assignments to experts outside the shard are dropped.
    """
    if local_count is None:
        local_count = num_experts
    flat = np.asarray(ids, dtype=np.int64).ravel()
    counts = np.zeros(local_count, dtype=np.int64)
    lists = [[] for _ in range(local_count)]
    for a, e in enumerate(flat):
        i = e - local_offset
        if 0 <= i < local_count:
            counts[i] += 1
            lists[i].append(a)
    offsets = np.zeros(local_count + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_assign = np.array([a for lst in lists for a in lst], dtype=np.int64)
    return counts.astype(np.int32), offsets.astype(np.int32), sorted_assign.astype(np.int32)
