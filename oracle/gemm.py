"""Dense MX GEMM with bf16 output -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources.
* "mxfp6-sm120" page, table of paths, "Dense" row: a shape-aware W6A8 GEMM
  for linear, attention and MLP projections.
* Same page, section "Execution model" (figure): FP16/BF16 activations are
  quantized dynamically to E4M3 with one UE8M0 scale per 32 K values; the
  weight is packed MX with one UE8M0 scale per 32 K values; the block-scaled
  products accumulate in FP32 and the output is FP16/BF16.
* Same page, section "Dense GEMM and MoE layer": the dense outputs were
  compared exactly against a matmul of the decoded operands.
* Same page, section "Validated scope", "Dense GEMM" row: M > 0, N % 8 == 0,
  K % 128 == 0.

Readings (the plainest ones): C[m, n] = alpha * sum_k A'[m, k] * W'[n, k],
where W' is the decoded MX weight [N, K] and A' is either the bf16 values of
A (bf16 activations: the W4A16 form of the layer's own FC GEMMs) or A
quantized to MXFP8 along K and decoded (the W4A8 / W6A8 form); A may also be
given already quantized (E4M3 codes + E8M0 scales).  The result is float64;
the device returns one bf16 rounding (round half to even) of its fp32
accumulation, so wherever that accumulation is exact the two agree bit for
bit after rounding this result to bf16.
"""
from __future__ import annotations

import numpy as np

from . import mx
from .moe import activations, decode_weight


def mx_gemm(a, w_packed, w_scale, *, wfmt: str, act: str, alpha: float = 1.0, a_scale=None) -> np.ndarray:
    """a [M, K] exact bf16 values (float64), or E4M3 codes (uint8) when
    ``a_scale`` [M, K/32] is given; w_packed [N, K*bits/8] + w_scale [N, K/32]
    in ``wfmt`` ("e2m1" | "e3m2"); act "bf16" | "mxfp8".  Returns C [M, N]
    float64."""
    if a_scale is not None:
        if act != "mxfp8":
            raise ValueError("pre-quantized activations are MXFP8")
        A = mx.dequantize(np.asarray(a, dtype=np.uint8), a_scale, "e4m3")
    else:
        A = activations(np.asarray(a, dtype=np.float64), act)
    K = A.shape[1]
    W = decode_weight(w_packed, w_scale, wfmt, K)
    return alpha * (A @ W.T)
