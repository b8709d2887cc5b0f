"""mx_gemm (dense MX GEMM, bf16 output) on the GPU against the oracle.

* Exact cases: A of small integers and weights whose codes are random bytes
  with scale code 127.  Every product and partial sum is then a multiple of
  1/16 well inside fp32's 24 bits, so the device's fp32 accumulation is
  exact and its one bf16 rounding equals the oracle's exact result rounded
  to bf16: the outputs must agree bit for bit (the mxfp6-sm120 page, "Dense
  GEMM and MoE layer", compares its dense outputs exactly against a decoded
  matmul).  One case per kernel family the dispatch can take, plus N not a
  multiple of 64 (masked columns) and pre-quantized activations.
* Random cases: N(0,1) activations and N(0,0.02) weights quantized by each
  side's own quantizer, within the layer's output bar.
"""
import numpy as np
import pytest
import torch

from block_scaled_precision_amd import inputs as gen
from oracle import gemm as og
from oracle import moe as om
from oracle import mx
from tests.conftest import has_gpu
from tests.helpers import assert_y_close, print_flush

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

BITS = {"e2m1": 4, "e3m2": 6}
# (M, N, K, fmt, act): the kernel each takes on 256 CUs
EXACT = [
    (300, 512, 1024, "e2m1", "mxfp8"),   # wide (192-row tiles, 256-row N-blocks)
    (300, 256, 512, "e3m2", "mxfp8"),    # tiled
    (200, 384, 512, "e2m1", "mxfp8"),    # tiled (N not a multiple of 256)
    (10, 200, 384, "e2m1", "mxfp8"),     # stream, M < 16, N % 64 != 0
    (40, 136, 256, "e3m2", "mxfp8"),     # stream, K not a multiple of 512
    (100, 512, 512, "e2m1", "bf16"),     # mid-M (64-row tiles)
    (130, 256, 1024, "e2m1", "bf16"),    # mid-M (128-row tiles)
    (8, 256, 1024, "e2m1", "bf16"),      # small-M, K split in 2 (partials summed after)
    (5, 256, 2048, "e2m1", "bf16"),      # small-M, K split in 4
    (17, 256, 1536, "e2m1", "bf16"),     # small-M, two M-tiles, K split in 3
    (16, 512, 7168, "e2m1", "bf16"),     # small-M, K split in 14 (the decode K)
    (5, 72, 128, "e3m2", "bf16"),        # stream, E3M2 x bf16
    (1, 8, 128, "e2m1", "bf16"),         # one row, one 8-column block
]


def _exact_inputs(M, N, K, fmt, seed):
    a = gen.small_integers((M, K), seed, 20)
    w = gen.random_bytes((N, K * BITS[fmt] // 8), seed, 21)
    s = torch.full((N, K // 32), 127, dtype=torch.uint8)
    return a, w, s


@pytest.mark.parametrize("M,N,K,fmt,act", EXACT)
def test_exact_gemm_is_bit_identical(M, N, K, fmt, act):
    from block_scaled_precision_amd import moe_mx as m
    a, w, s = _exact_inputs(M, N, K, fmt, 0)
    print_flush(f"mx_gemm exact M={M} N={N} K={K} {fmt}/{act}")
    for alpha in (1.0, -0.5):
        c = m.mx_gemm(a.cuda(), w.cuda(), s.cuda(), fmt, act, alpha=alpha)
        torch.cuda.synchronize()
        ref = mx.round_to_bf16(og.mx_gemm(a.double().numpy(), w.numpy(), s.numpy(), wfmt=fmt, act=act, alpha=alpha))
        got = c.float().cpu().numpy().astype(np.float64)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, f"{bad.size} of {got.size} differ, first at {np.unravel_index(bad[0], got.shape)}"
        assert np.abs(ref).max() > 0


def test_prequantized_activations():
    from block_scaled_precision_amd import moe_mx as m
    M, N, K = 64, 256, 512
    a, w, s = _exact_inputs(M, N, K, "e3m2", 1)
    codes, scales = m.mx_quantize(a.cuda(), "e4m3")
    oc, osc = mx.quantize(a.double().numpy(), "e4m3")
    assert np.array_equal(codes.cpu().numpy(), oc) and np.array_equal(scales.cpu().numpy(), osc)
    c = m.mx_gemm(codes, w.cuda(), s.cuda(), "e3m2", "mxfp8", a_scale=scales)
    c2 = m.mx_gemm(a.cuda(), w.cuda(), s.cuda(), "e3m2", "mxfp8")
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), c2.view(torch.int16))
    ref = mx.round_to_bf16(og.mx_gemm(oc, w.numpy(), s.numpy(), wfmt="e3m2", act="mxfp8", a_scale=osc))
    assert np.array_equal(c.float().cpu().numpy().astype(np.float64), ref)


RANDOM = [
    (2048, 1024, 5120, "e3m2", "mxfp8"),  # the shared expert's FC1 shape at reduced N
    (512, 1024, 2048, "e2m1", "mxfp8"),
    (96, 512, 1024, "e2m1", "bf16"),
    (7, 1000, 256, "e2m1", "mxfp8"),
    (3, 64, 384, "e3m2", "bf16"),
    (8, 1024, 3584, "e2m1", "bf16"),     # small-M with a K split
]


@pytest.mark.parametrize("M,N,K,fmt,act", RANDOM)
def test_random_gemm_within_bar(M, N, K, fmt, act):
    from block_scaled_precision_amd import moe_mx as m
    a = gen.normal((M, K), 0, 22).to(torch.bfloat16)
    wf = gen.normal((N, K), 0, 23, std=0.02)
    wq, sq = m.mx_quantize(wf.cuda(), fmt)
    op, osc = om.quantize_weight(wf.double().numpy(), fmt)
    assert np.array_equal(wq.cpu().numpy(), op) and np.array_equal(sq.cpu().numpy(), osc)
    print_flush(f"mx_gemm random M={M} N={N} K={K} {fmt}/{act}")
    c = m.mx_gemm(a.cuda(), wq, sq, fmt, act)
    torch.cuda.synchronize()
    ref = og.mx_gemm(a.double().numpy(), op, osc, wfmt=fmt, act=act)
    assert_y_close(c.float().cpu().numpy(), ref, f"mx_gemm {M}x{N}x{K} {fmt}/{act}")


def test_zero_rows_and_repeat():
    from block_scaled_precision_amd import moe_mx as m
    a, w, s = _exact_inputs(0, 64, 256, "e2m1", 2)
    c = m.mx_gemm(a.cuda(), w.cuda(), s.cuda(), "e2m1", "mxfp8")
    assert c.shape == (0, 64)
    a, w, s = _exact_inputs(33, 320, 1024, "e2m1", 3)
    c1 = m.mx_gemm(a.cuda(), w.cuda(), s.cuda(), "e2m1", "mxfp8")
    c2 = m.mx_gemm(a.cuda(), w.cuda(), s.cuda(), "e2m1", "mxfp8")
    torch.cuda.synchronize()
    assert torch.equal(c1.view(torch.int16), c2.view(torch.int16))


@pytest.mark.parametrize("M,N,K", [(8, 256, 1024), (17, 256, 1536), (8, 1024, 3584)])
def test_k_split_matches_unsplit(M, N, K):
    """With a workspace for the partial sums the few-row bf16 GEMM splits K;
    given none it runs unsplit.  Exact inputs give identical bits either way,
    random inputs agree within fp32 summation order (and with the oracle)."""
    import ctypes
    from block_scaled_precision_amd import moe_mx as m
    L = m.lib()
    need = m.mx_gemm_workspace_bytes(M, N, K, "bf16", "e2m1")
    assert need >= 2 * M * N * 4, "this shape is expected to split K"

    def run(a, w, s, ws):
        c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        st = L.mx_gemm(ctypes.c_void_p(a.data_ptr()), None, M, N, K, 0, ctypes.c_void_p(w.data_ptr()),
                       ctypes.c_void_p(s.data_ptr()), 1, ctypes.c_float(1.0), ctypes.c_void_p(c.data_ptr()),
                       ctypes.c_void_p(ws.data_ptr()) if ws is not None else None,
                       ws.numel() if ws is not None else 0, None)
        assert st == 0, m.status_str(st) if hasattr(m, "status_str") else st
        return c

    print_flush(f"mx_gemm K split vs unsplit M={M} N={N} K={K}")
    a, w, s = (t.cuda() for t in _exact_inputs(M, N, K, "e2m1", 4))
    ws = torch.empty((need,), dtype=torch.uint8, device="cuda")
    c_split, c_plain = run(a, w, s, ws), run(a, w, s, None)
    torch.cuda.synchronize()
    assert torch.equal(c_split.view(torch.int16), c_plain.view(torch.int16))
    a = gen.normal((M, K), 0, 24).to(torch.bfloat16).cuda()
    wq, sq = m.mx_quantize(gen.normal((N, K), 0, 25, std=0.02).cuda(), "e2m1")
    c_split, c_plain = run(a, wq, sq, ws), run(a, wq, sq, None)
    torch.cuda.synchronize()
    d = (c_split.float() - c_plain.float()).abs().max().item()
    assert d <= 2e-2 * c_plain.float().abs().max().item()
    ref = og.mx_gemm(a.double().cpu().numpy(), wq.cpu().numpy(), sq.cpu().numpy(), wfmt="e2m1", act="bf16")
    assert_y_close(c_split.float().cpu().numpy(), ref, f"split {M}x{N}x{K}")


def _draw_exact(n, seed=20261204):
    """Seeded random dense problems with exact inputs: any M, N a multiple of
    8 and K of 128 (K <= 4096 keeps every E3M2 partial sum, a multiple of
    1/16, inside fp32's 24 bits), either format and activation mode."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        M = int(rng.choice([1, 2, 7, 16, 17, 31, 33, 64, 100, 191, 193, 300, 600]))
        N = 8 * int(rng.integers(1, 129))
        K = 128 * int(rng.integers(1, 33))
        fmt = str(rng.choice(["e2m1", "e3m2"]))
        act = str(rng.choice(["bf16", "mxfp8"]))
        cases.append(pytest.param(M, N, K, fmt, act, id=f"{i}_{M}x{N}x{K}_{fmt}_{act}"))
    return cases


@pytest.mark.parametrize("M,N,K,fmt,act", _draw_exact(32))
def test_random_exact_gemm_is_bit_identical(M, N, K, fmt, act):
    """Randomly drawn shapes, so that the dispatch meets sizes nobody picked
    for it; exact inputs, so the output must equal the oracle bit for bit."""
    from block_scaled_precision_amd import moe_mx as m
    a, w, s = _exact_inputs(M, N, K, fmt, 5)
    print_flush(f"mx_gemm random exact M={M} N={N} K={K} {fmt}/{act}")
    c = m.mx_gemm(a.cuda(), w.cuda(), s.cuda(), fmt, act)
    torch.cuda.synchronize()
    ref = mx.round_to_bf16(og.mx_gemm(a.double().numpy(), w.numpy(), s.numpy(), wfmt=fmt, act=act))
    got = c.float().cpu().numpy().astype(np.float64)
    bad = np.flatnonzero(got != ref)
    assert bad.size == 0, f"{bad.size} of {got.size} differ, first at {np.unravel_index(bad[0], got.shape)}"
