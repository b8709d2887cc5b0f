"""mx_quantize on the GPU against the oracle quantizer: bit-exact codes and scales."""
import numpy as np
import pytest
import torch

from oracle import mx
from tests.conftest import has_gpu
from tests.helpers import print_flush

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not has_gpu(), reason="needs a GPU")]

FMTS = ["e2m1", "e3m2", "e4m3"]


def _gpu_quant(x_cpu: torch.Tensor, fmt: str):
    from block_scaled_precision_amd import moe_mx as m
    codes, scales = m.mx_quantize(x_cpu.cuda(), fmt)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), scales.cpu().numpy()


def _oracle_quant(x_cpu: torch.Tensor, fmt: str):
    c, s = mx.quantize(x_cpu.to(torch.float64).numpy(), fmt)
    return mx.pack(c, fmt), s


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_random_matrix(fmt, dtype):
    g = torch.Generator().manual_seed(1)
    # rows with very different magnitudes, ragged number of 32-blocks
    x = torch.randn((37, 32 * 13), generator=g) * torch.exp2(torch.randint(-30, 30, (37, 1), generator=g).float())
    x = x * torch.exp2(torch.randint(-8, 8, (37, 32 * 13), generator=g).float())
    x = x.to(dtype)
    print_flush(f"mx_quantize random {fmt} {dtype}")
    gc, gs = _gpu_quant(x, fmt)
    oc, os_ = _oracle_quant(x, fmt)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


@pytest.mark.parametrize("fmt", FMTS)
def test_exhaustive_bf16(fmt):
    """Every finite bf16 pattern, in blocks whose maximum sits 0..6 binades
    above the block's other elements."""
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    vals = bits[torch.isfinite(bits.float())]
    n = vals.numel() - vals.numel() % 31
    v = vals[:n].reshape(-1, 31)
    for up in (0, 1, 3, 6):
        amax = v.float().abs().amax(1)
        ex = torch.frexp(torch.where(amax == 0, torch.ones_like(amax), amax)).exponent
        anchor = torch.ldexp(torch.ones_like(amax), (ex - 1 + up).clamp(max=127).float())
        anchor = torch.where(amax == 0, torch.ones_like(amax), anchor).to(torch.bfloat16)
        blocks = torch.cat([v, anchor[:, None]], 1).contiguous()
        print_flush(f"mx_quantize exhaustive bf16 {fmt} up={up}")
        gc, gs = _gpu_quant(blocks, fmt)
        oc, os_ = _oracle_quant(blocks, fmt)
        assert np.array_equal(gs, os_)
        assert np.array_equal(gc, oc)


@pytest.mark.parametrize("fmt", FMTS)
def test_special_blocks(fmt):
    rows = []
    z = torch.zeros(32)
    rows.append(z.clone())
    nz = torch.zeros(32)
    nz[3] = -0.0
    nz[7] = -0.0
    rows.append(nz)
    rows.append(torch.full((32,), 2.0 ** -140))      # tiny: scale clamps to code 0
    rows.append(torch.full((32,), -(2.0 ** 120)))    # large
    t = torch.zeros(32)
    t[:8] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 7.0])
    rows.append(t)                                   # E2M1 ties at scale 1
    sub = torch.full((32,), 2.0 ** -130)
    sub[0] = 2.0 ** -126 * 1.5                       # fp32 subnormals and a normal max
    rows.append(sub)
    x = torch.stack(rows).float()
    print_flush(f"mx_quantize special {fmt}")
    gc, gs = _gpu_quant(x, fmt)
    oc, os_ = _oracle_quant(x, fmt)
    assert np.array_equal(gs, os_)
    assert np.array_equal(gc, oc)


def test_strided_source_and_empty():
    from block_scaled_precision_amd import moe_mx as m
    g = torch.Generator().manual_seed(2)
    big = torch.randn((20, 200), generator=g).to(torch.bfloat16)
    view = big[:, 4:4 + 160]                         # row stride 200, rows start 8 bytes off 16
    print_flush("mx_quantize strided")
    gc, gs = m.mx_quantize(big.cuda()[:, 4:4 + 160], "e2m1")
    torch.cuda.synchronize()
    oc, os_ = _oracle_quant(view.contiguous(), "e2m1")
    assert np.array_equal(gs.cpu().numpy(), os_)
    assert np.array_equal(gc.cpu().numpy(), oc)
    c, s = m.mx_quantize(torch.empty((0, 64), dtype=torch.bfloat16, device="cuda"), "e4m3")
    assert c.shape == (0, 64) and s.shape == (0, 2)


def test_weight_tensor_of_tiny_layer():
    from block_scaled_precision_amd import inputs as gen
    w = gen.WORKLOADS["tiny_w4a16"]
    for e in range(w.E):
        a = gen.expert_w1(w, e)
        gc, gs = _gpu_quant(a, "e2m1")
        oc, os_ = _oracle_quant(a, "e2m1")
        assert np.array_equal(gs, os_) and np.array_equal(gc, oc)


def _draw(n, seed=20261206):
    """Seeded random shapes: 1-3000 rows, any multiple of 32 columns up to
    5120, a row stride of the columns or wider, either source type, every
    format."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        rows = int(rng.choice([1, 2, 5, 31, 64, 100, 257, 1000, 3000]))
        cols = 32 * int(rng.integers(1, 161))
        pad = int(rng.choice([0, 0, 8, 32, 96]))
        fmt = str(rng.choice(FMTS))
        dtype = str(rng.choice(["bf16", "fp32"]))
        cases.append(pytest.param(rows, cols, pad, fmt, dtype, i, id=f"{i}_{rows}x{cols}+{pad}_{fmt}_{dtype}"))
    return cases


@pytest.mark.parametrize("rows,cols,pad,fmt,dtype,i", _draw(32))
def test_random_shapes(rows, cols, pad, fmt, dtype, i):
    from block_scaled_precision_amd import moe_mx as m
    g = torch.Generator().manual_seed(2000 + i)
    td = torch.bfloat16 if dtype == "bf16" else torch.float32
    big = (torch.randn((rows, cols + pad), generator=g)
           * torch.exp2(torch.randint(-20, 20, (rows, 1), generator=g).float())).to(td)
    print_flush(f"mx_quantize random {rows}x{cols} (row stride {cols + pad}) {fmt} {dtype}")
    gc, gs = m.mx_quantize(big.cuda()[:, :cols], fmt)
    torch.cuda.synchronize()
    oc, os_ = _oracle_quant(big[:, :cols].contiguous(), fmt)
    assert np.array_equal(gs.cpu().numpy(), os_)
    assert np.array_equal(gc.cpu().numpy(), oc)
