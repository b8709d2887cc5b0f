"""Forward pass of the routed MX mixture-of-experts layer -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

The dataflow and its quantization points follow the pages:

* "mxfp6-sm120" page, table of paths, "Routed MoE" row: routing, W1,
  SiLU-and-mul, intermediate quantization, W2, shared-expert combine and the
  routed/shared reduction.
* "mxfp6-sm120" page, section "Execution model" (figure): bf16 activations are
  dynamically quantized to E4M3 with one UE8M0 scale per 32 K values; the
  weight is packed MX (E3M2 there) with one UE8M0 scale per 32 K values; the
  products accumulate in FP32 and the output is FP16/BF16.
* "TokenSpeed SiTU" page, section "Activation precision (w4a16 vs w4a8)":
  bf16 activations times MXFP4 weights (w4a16), or MXFP8 activations times
  MXFP4 weights (w4a8) where the FC1 fp8 output is dequantized to bf16 before
  FC2; weights stay MXFP4 either way.
* "TokenSpeed SiTU" page, section "Supported contract": precomputed top-k may
  be passed in; experts outside the local shard are skipped and the output is
  then a partial sum.

Readings of points the pages leave open:
* the gated activation is SiLU(gate) * up, with W1 rows [0, I) the gate and
  rows [I, 2I) the up projection;
* w4a16: h is rounded once to bf16 (round half to even) before FC2;
  MXFP8 modes: h is MX-quantized to E4M3 per 32 along I and decoded, which is
  exactly representable in bf16, so "dequantize to bf16" adds no rounding;
* the routing weight multiplies the FC2 output (not h), the shared expert is
  added with its own weight (1.0) and the whole sum is rounded once to bf16 by
  the caller of this function (the oracle returns float64).
All arithmetic here is float64 over exactly decoded MX values.
"""
from __future__ import annotations

import numpy as np

from . import mx
from .routing import permute, topk_route

_WFMT = {"e2m1", "e3m2"}


def silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + exp(-g)), float64."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


# SwiGLU-OAI constants (the gpt-oss gated activation): the gate is clipped
# from above and the up projection on both sides at this limit, and the
# sigmoid takes the gate scaled by this slope.
OAI_LIMIT = 7.0
OAI_ALPHA = 1.702


def gated(g: np.ndarray, u: np.ndarray, act_fn: str = "silu") -> np.ndarray:
    """The gated activation of FC1's two halves, float64 ("b12x" page, "What's
    in here", MoE: SiLU, ReLU2 and SwiGLU-OAI activations):
      silu        SiLU(g) * u
      relu2       max(g, 0)**2 * u
      swiglu_oai  (clip(u, -L, L) + 1) * g' / (1 + exp(-alpha g')),
                  g' = min(g, L), L = 7, alpha = 1.702."""
    if act_fn == "silu":
        return silu(g) * u
    if act_fn == "relu2":
        r = np.maximum(g, 0.0)
        return r * r * u
    if act_fn == "swiglu_oai":
        gc = np.minimum(g, OAI_LIMIT)
        uc = np.clip(u, -OAI_LIMIT, OAI_LIMIT)
        with np.errstate(over="ignore"):
            return (uc + 1.0) * (gc / (1.0 + np.exp(-OAI_ALPHA * gc)))
    raise ValueError(act_fn)


def decode_weight(packed: np.ndarray, scales: np.ndarray, fmt: str, k: int) -> np.ndarray:
    """One expert's packed weight [N, k*bits/8] + scales [N, k/32] -> float64 [N, k]."""
    codes = mx.unpack(packed, fmt, k)
    return mx.dequantize(codes, scales, fmt)


def quantize_weight(w: np.ndarray, fmt: str):
    """float weights [..., N, K] -> (packed bytes, scale codes), quantized along K."""
    codes, scales = mx.quantize(np.asarray(w, dtype=np.float64), fmt)
    return mx.pack(codes, fmt), scales


def activations(x: np.ndarray, act: str) -> np.ndarray:
    """What FC1 multiplies: the bf16 values of x (w4a16), or x MX-quantized to
    E4M3 per 32 along H and decoded (MXFP8 activations)."""
    if act == "bf16":
        return np.asarray(x, dtype=np.float64)
    if act == "mxfp8":
        codes, scales = mx.quantize(x, "e4m3")
        return mx.dequantize(codes, scales, "e4m3")
    raise ValueError(act)


def intermediate(h: np.ndarray, act: str) -> np.ndarray:
    """The FC2 input made from h = SiLU(g)*u: bf16-rounded (w4a16) or MXFP8
    quantized along I and decoded (MXFP8 modes)."""
    if act == "bf16":
        return mx.round_to_bf16(h)
    if act == "mxfp8":
        codes, scales = mx.quantize(h, "e4m3")
        return mx.dequantize(codes, scales, "e4m3")
    raise ValueError(act)


def expert_hidden(a: np.ndarray, w1: np.ndarray, act_fn: str = "silu") -> np.ndarray:
    """a [M, H] float64, decoded w1 [2I, H] -> h = act(gate, up) [M, I] (FC1
    and the gated activation, before the intermediate rounding)."""
    I = w1.shape[0] // 2
    z = a @ w1.T                      # FC1, K = H
    g, u = z[:, :I], z[:, I:]
    return gated(g, u, act_fn)


def expert_ffn(a: np.ndarray, w1: np.ndarray, w2: np.ndarray, act: str, act_fn: str = "silu") -> np.ndarray:
    """a [M, H] float64, decoded w1 [2I, H], decoded w2 [H, I] -> o [M, H]."""
    ht = intermediate(expert_hidden(a, w1, act_fn), act)
    return ht @ w2.T                  # FC2, K = I


def moe_forward(x, logits, w1, w1_scale, w2, w2_scale, *, k, wfmt, act,
                topk_ids=None, topk_w=None,
                shared=None, shared_weight=1.0,
                local_offset=0, local_count=None, tokens=None, intermediates=False, act_fn="silu"):
    """Full layer output in float64.

    x [T, H] exact bf16 values (float64); logits [T, E] float32 (or None when
    topk_ids / topk_w are given); w1 [E, 2I, H*b/8] uint8 + w1_scale [E, 2I, H/32];
    w2 [E, H, I*b/8] + w2_scale [E, H, I/32]; wfmt "e2m1" | "e3m2";
    act "bf16" | "mxfp8"; shared = (ws1, ws1_scale, ws2, ws2_scale) or None;
    act_fn the gated activation of every expert ("silu", "relu2", "swiglu_oai").
    ``tokens`` restricts the computation to a subset of token rows (each
    token's output depends only on its own row); the result then has one row
    per listed token.

    Returns dict(y, ids, w, counts, offsets, sorted_assign) where the routing
    entries cover the computed tokens.  With ``intermediates`` it also holds
    "intermediates": assignment id t*k + j (t indexing the computed tokens) ->
    the FC2 input of that assignment: (E4M3 codes [I], E8M0 scales [I/32]) for
    MXFP8 activations, or the bf16-rounded values [I] (float64) for bf16.
    """
    if wfmt not in _WFMT:
        raise ValueError(wfmt)
    x = np.asarray(x, dtype=np.float64)
    T, H = x.shape
    E = w1.shape[0]
    I = w1.shape[1] // 2
    if local_count is None:
        local_count = E
    rows = np.arange(T) if tokens is None else np.asarray(tokens, dtype=np.int64)

    if topk_ids is None:
        ids, w = topk_route(np.asarray(logits)[rows], k)
    else:
        ids = np.asarray(topk_ids, dtype=np.int32)[rows]
        w = np.asarray(topk_w, dtype=np.float64)[rows]
    counts, offsets, sorted_assign = permute(ids, E, local_offset, local_count)

    a = activations(x[rows], act)
    y = np.zeros((rows.size, H), dtype=np.float64)
    inter = {}
    for i in range(local_count):
        seg = sorted_assign[offsets[i]:offsets[i + 1]]
        if seg.size == 0:
            continue
        e = local_offset + i
        t_loc, slot = seg // k, seg % k
        d1 = decode_weight(w1[e], w1_scale[e], wfmt, H)
        d2 = decode_weight(w2[e], w2_scale[e], wfmt, I)
        if intermediates:
            h = expert_hidden(a[t_loc], d1, act_fn)
            if act == "mxfp8":
                codes, scales = mx.quantize(h, "e4m3")
                for r, asg in enumerate(seg):
                    inter[int(asg)] = (codes[r], scales[r])
            else:
                for r, asg in enumerate(seg):
                    inter[int(asg)] = intermediate(h[r:r + 1], act)[0]
        o = expert_ffn(a[t_loc], d1, d2, act, act_fn)
        y[t_loc] += w[t_loc, slot][:, None] * o   # a token meets an expert at most once
    if shared is not None:
        ws1, ws1_scale, ws2, ws2_scale = shared
        Is = ws1.shape[0] // 2
        d1 = decode_weight(ws1, ws1_scale, wfmt, H)
        d2 = decode_weight(ws2, ws2_scale, wfmt, Is)
        y += shared_weight * expert_ffn(a, d1, d2, act, act_fn)
    out = dict(y=y, ids=ids, w=w, counts=counts, offsets=offsets, sorted_assign=sorted_assign)
    if intermediates:
        out["intermediates"] = inter
    return out
