"""Pins for the oracle's dense MX GEMM (CPU only): exact rational arithmetic
from the raw codes and the hand-typed OCP element tables, integer inputs whose
result is a plain integer matmul, power-of-two alpha, K-splits, and the
pre-quantized activation form."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import gemm as og
from oracle import moe as om
from oracle import mx


def _table(golden_dir, name):
    """code -> value from a hand-typed table (tests/golden/<fmt>_values.txt)."""
    vals = {}
    for line in open(f"{golden_dir}/{name}_values.txt"):
        line = line.split("#")[0].strip()
        if line:
            c, v = line.split()
            vals[int(c, 0)] = Fraction(v)
    return vals


def _bf16(rng, shape, scale=1.0):
    x = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32)).to(torch.bfloat16)
    return x.to(torch.float64).numpy()


@pytest.mark.parametrize("wfmt", ["e2m1", "e3m2"])
@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_exact_rational_from_codes(golden_dir, wfmt, act):
    rng = np.random.default_rng(11)
    M, N, K = 2, 3, 64
    a = _bf16(rng, (M, K))
    p, s = om.quantize_weight(rng.standard_normal((N, K)) * 0.3, wfmt)
    c = og.mx_gemm(a, p, s, wfmt=wfmt, act=act)
    wt = _table(golden_dir, wfmt)
    wc = mx.unpack(p, wfmt, K)
    if act == "mxfp8":
        ac, asc = mx.quantize(a, "e4m3")
        e4 = {int(code): Fraction(float(v)) for code, v in
              enumerate(torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().tolist())
              if np.isfinite(v)}
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                w = wt[int(wc[n, k])] * Fraction(2) ** (int(s[n, k // 32]) - 127)
                if act == "mxfp8":
                    av = e4[int(ac[m, k])] * Fraction(2) ** (int(asc[m, k // 32]) - 127)
                else:
                    av = Fraction(float(a[m, k]))
                acc += av * w
            assert float(acc) == c[m, n]


@pytest.mark.parametrize("wfmt", ["e2m1", "e3m2"])
@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
def test_integer_inputs_give_the_integer_matmul(wfmt, act):
    """A of integers in [-8, 8] (exact in bf16 and, after its block scale, in
    E4M3) and weights quantized with scale code 127 (value = element value):
    C is the plain matmul of A with the decoded element values."""
    rng = np.random.default_rng(12)
    M, N, K = 5, 16, 256
    a = rng.integers(-8, 9, size=(M, K)).astype(np.float64)
    a[:, ::32] = 8.0  # every block holds an 8: scale 2**-5 for E4M3
    table = mx.decode_table(wfmt)
    nfin = table.size if wfmt != "e4m3" else 255
    codes = rng.integers(0, nfin, size=(N, K)).astype(np.uint8)
    p = mx.pack(codes, wfmt)
    s = np.full((N, K // 32), 127, np.uint8)
    c = og.mx_gemm(a, p, s, wfmt=wfmt, act=act)
    w = table[codes]
    # values are multiples of 1/16: the products and sums are exact integers after scaling
    ref = (np.rint(a * 16).astype(np.int64) @ np.rint(w * 16).astype(np.int64).T) / 256.0
    assert np.array_equal(c, ref)


def test_alpha_and_k_split():
    rng = np.random.default_rng(13)
    M, N, K = 7, 24, 256
    a = _bf16(rng, (M, K))
    p, s = om.quantize_weight(rng.standard_normal((N, K)) * 0.02, "e2m1")
    for act in ("bf16", "mxfp8"):
        c = og.mx_gemm(a, p, s, wfmt="e2m1", act=act)
        assert np.array_equal(og.mx_gemm(a, p, s, wfmt="e2m1", act=act, alpha=0.25), c * 0.25)
        # blocks of 32 along K are independent: splitting K at 128 adds up
        c1 = og.mx_gemm(a[:, :128], p[:, :64], s[:, :4], wfmt="e2m1", act=act)
        c2 = og.mx_gemm(a[:, 128:], p[:, 64:], s[:, 4:], wfmt="e2m1", act=act)
        assert np.allclose(c1 + c2, c, rtol=1e-13, atol=1e-15)
        assert np.abs(c).max() > 0


def test_prequantized_activations_and_the_layer_fc1():
    """Codes + scales of A give the same C as A with act="mxfp8"; and the gate
    half of the layer's FC1 (E = 1, dense) is this GEMM."""
    rng = np.random.default_rng(14)
    M, N, K = 4, 32, 128
    a = _bf16(rng, (M, K))
    p, s = om.quantize_weight(rng.standard_normal((N, K)) * 0.02, "e3m2")
    ac, asc = mx.quantize(a, "e4m3")
    assert np.array_equal(og.mx_gemm(ac, p, s, wfmt="e3m2", act="mxfp8", a_scale=asc),
                          og.mx_gemm(a, p, s, wfmt="e3m2", act="mxfp8"))
    with pytest.raises(ValueError):
        og.mx_gemm(ac, p, s, wfmt="e3m2", act="bf16", a_scale=asc)
    d1 = om.decode_weight(p, s, "e3m2", K)
    z = om.activations(a, "mxfp8") @ d1.T
    assert np.array_equal(og.mx_gemm(a, p, s, wfmt="e3m2", act="mxfp8"), z)
