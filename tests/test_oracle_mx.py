"""Pins for the oracle's MX codecs, quantizer and packing (CPU only).

Each check ties ``oracle.mx`` to something outside it: hand-typed tables in
tests/golden, torch's own float8 codecs, a brute-force nearest-value search,
or an algebraic property of the block quantizer.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import mx


def _read_pairs(path):
    out = []
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            a, b = line.split()[:2]
            out.append((a, b))
    return out


@pytest.mark.parametrize("fmt,fname", [("e2m1", "e2m1_values.txt"), ("e3m2", "e3m2_values.txt")])
def test_decode_matches_hand_table(golden_dir, fmt, fname):
    table = mx.decode_table(fmt)
    pairs = _read_pairs(os.path.join(golden_dir, fname))
    assert len(pairs) == table.size
    for code, val in pairs:
        v = float(val)
        got = table[int(code)]
        assert got == v and math.copysign(1, got) == math.copysign(1, v), (fmt, code, got, v)


def test_e3m2_range_and_count():
    t = mx.decode_table("e3m2")
    assert np.nanmax(t) == 28.0
    assert np.min(t[t > 0]) == 0.0625
    assert np.unique(np.abs(t)).size == 32


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = mx.decode_table("e4m3")
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))
    assert np.nanmax(got) == 448.0 and np.isnan(got[0x7F]) and np.isnan(got[0xFF])


def test_e8m0_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = mx.decode_e8m0(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_emax():
    assert (mx.emax("e2m1"), mx.emax("e3m2"), mx.emax("e4m3")) == (2, 4, 8)


@pytest.mark.parametrize("fmt,fname,amax", [("e2m1", "e2m1_ties.txt", 7.0), ("e3m2", "e3m2_ties.txt", 28.0)])
def test_ties_and_saturation(golden_dir, fmt, fname, amax):
    pairs = _read_pairs(os.path.join(golden_dir, fname))
    vals = np.array([float(a) for a, _ in pairs])
    want = np.array([int(b) for _, b in pairs])
    block = np.zeros(32)
    block[:vals.size] = vals
    assert np.max(np.abs(block)) == amax
    codes, scale = mx.quantize(block[None], fmt)
    assert scale[0, 0] == 127
    assert np.array_equal(codes[0, :vals.size], want)


def _brute_block(v, fmt):
    """Brute force: search the exponent, then scan every code for the nearest."""
    table = mx.decode_table(fmt)
    bits = mx.bits_per_code(fmt)
    emax = {"e2m1": 2, "e3m2": 4, "e4m3": 8}[fmt]
    amax = max(abs(float(x)) for x in v)
    if amax == 0:
        s = -127
    else:
        e = -200
        while not (2.0 ** e <= amax < 2.0 ** (e + 1)):
            e += 1
        s = min(max(e - emax, -127), 127)
    codes = []
    sign_bit = 1 << (bits - 1)
    for x in v:
        q = float(x) * 2.0 ** (-s)
        best, best_d = None, None
        for c in range(sign_bit):           # magnitudes only
            t = table[c]
            if np.isnan(t):
                continue
            d = abs(abs(q) - t)
            if best is None or d < best_d or (d == best_d and c % 2 == 0):
                best, best_d = c, d
        codes.append(best | (sign_bit if math.copysign(1, x) < 0 else 0))
    return np.array(codes, dtype=np.uint8), s + 127


@pytest.mark.parametrize("fmt", ["e2m1", "e3m2", "e4m3"])
def test_quantizer_vs_bruteforce_random_blocks(fmt):
    rng = np.random.default_rng(7)
    blocks = []
    for i in range(60):
        spread = rng.uniform(0, 12)
        b = rng.standard_normal(32) * np.exp2(rng.uniform(-spread, spread, 32))
        b = b.astype(np.float32).astype(np.float64) * 2.0 ** rng.integers(-40, 40)
        if i % 10 == 0:
            b[rng.integers(0, 32, 8)] = 0.0
        if i % 17 == 0:
            b[:] = 0.0
            b[3] = -0.0
        blocks.append(b)
    v = np.stack(blocks)
    codes, scales = mx.quantize(v, fmt)
    for i, b in enumerate(blocks):
        bc, bs = _brute_block(b, fmt)
        assert scales[i, 0] == bs, (i, scales[i, 0], bs)
        assert np.array_equal(codes[i], bc), (i, codes[i], bc)


@pytest.mark.parametrize("fmt", ["e2m1", "e3m2", "e4m3"])
def test_quantizer_exhaustive_bf16(fmt):
    """Every finite bf16 pattern, quantized inside blocks whose maximum sits
    0..6 binades above it, against a vectorised nearest search over the table."""
    bits = np.arange(65536, dtype=np.uint32)
    with np.errstate(invalid="ignore"):
        vals = mx.bf16_bits_to_f64(bits)
    vals = vals[np.isfinite(vals)]
    table = mx.decode_table(fmt)
    mags = np.where(np.isnan(table[: 1 << (mx.bits_per_code(fmt) - 1)]), np.inf,
                    table[: 1 << (mx.bits_per_code(fmt) - 1)])
    emax = {"e2m1": 2, "e3m2": 4, "e4m3": 8}[fmt]
    for up in (0, 1, 3, 6):
        v = vals.copy()
        n = v.size - v.size % 31
        v = v[:n].reshape(-1, 31)
        # anchor: a power of two `up` binades above each block's largest element
        amax_in = np.max(np.abs(v), axis=1)
        _, ex = np.frexp(np.where(amax_in == 0, 1.0, amax_in))
        anchor = np.ldexp(1.0, np.minimum(ex - 1 + up, 127))
        anchor = np.where(amax_in == 0, 1.0, anchor)
        blocks = np.concatenate([v, anchor[:, None]], axis=1)
        codes, scales = mx.quantize(blocks, fmt)
        # expected, by exhaustive nearest search over magnitudes (ties -> even code)
        amax = np.max(np.abs(blocks), axis=1)
        e = np.floor(np.log2(amax)).astype(np.int64)       # amax are exact powers/bf16 -> log2 exact enough
        e = np.where(np.ldexp(1.0, e) > amax, e - 1, e)
        e = np.where(np.ldexp(1.0, e + 1) <= amax, e + 1, e)
        s = np.clip(e - emax, -127, 127)
        assert np.array_equal(scales[:, 0].astype(np.int64), s + 127)
        q = np.abs(np.ldexp(blocks, -s[:, None]))
        d = np.abs(q[..., None] - mags[None, None, :])
        best = np.argmin(d, axis=-1)             # lowest code among equals
        dmin = np.take_along_axis(d, best[..., None], -1)[..., 0]
        nxt = np.minimum(best + 1, mags.size - 1)
        tie = (np.take_along_axis(d, nxt[..., None], -1)[..., 0] == dmin) & (nxt != best)
        best = np.where(tie & (best % 2 == 1), nxt, best)
        sign = np.signbit(blocks).astype(np.int64) << (mx.bits_per_code(fmt) - 1)
        assert np.array_equal(codes.astype(np.int64), best | sign)


def test_e4m3_encode_matches_torch_in_range():
    """Inside the E4M3 range the element rounding is IEEE-style round half to
    even; torch's float32 -> float8_e4m3fn cast is an independent encoder."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((2000, 32)) * np.exp2(rng.uniform(-6, 6, (2000, 32)))).astype(np.float32)
    codes, scales = mx.quantize(x.astype(np.float64), "e4m3")
    q = np.ldexp(x.astype(np.float64), -(scales.astype(np.int64) - 127).repeat(32, axis=1))
    inside = np.abs(q) < 464          # below 448 + half an ulp: no clamp involved
    assert inside.mean() > 0.9
    ref = torch.from_numpy(q.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(codes[inside], ref[inside])
    assert np.all(codes[~inside] & 0x7F == 0x7E)   # beyond it: saturate to 448


@pytest.mark.parametrize("fmt", ["e2m1", "e3m2", "e4m3"])
def test_round_trip_and_scale_equivariance(fmt):
    table = mx.decode_table(fmt)
    finite = np.nonzero(~np.isnan(table))[0]
    # every code, placed in a block with the largest magnitude present
    top = np.nanargmax(table)
    for s in (-20, 0, 7):
        blk = np.zeros((finite.size, 32))
        blk[:, 0] = table[finite]
        blk[:, 1] = table[top]
        blk *= 2.0 ** s
        codes, scales = mx.quantize(blk, fmt)
        assert np.all(scales == 127 + s)
        # -0 and +0 keep their sign bit
        assert np.array_equal(codes[:, 0], finite)
    rng = np.random.default_rng(11)
    x = rng.standard_normal((50, 64)).astype(np.float32).astype(np.float64)
    c0, s0 = mx.quantize(x, fmt)
    for n in (-9, 1, 13):
        c1, s1 = mx.quantize(np.ldexp(x, n), fmt)
        assert np.array_equal(c0, c1)
        assert np.array_equal(s1.astype(int), s0.astype(int) + n)


def test_zero_and_tiny_blocks():
    z = np.zeros((1, 32))
    z[0, 5] = -0.0
    c, s = mx.quantize(z, "e2m1")
    assert s[0, 0] == 0 and c[0, 5] == 8 and c[0, 0] == 0
    tiny = np.full((1, 32), 2.0 ** -135)
    tiny[0, 1] = 2.0 ** -140
    c, s = mx.quantize(tiny, "e4m3")
    assert s[0, 0] == 0                      # clamped to 2**-127
    d = mx.dequantize(c, s, "e4m3")[0]
    assert d[0] == 2.0 ** -135               # 2**-8 is an E4M3 subnormal (2 * 2**-9)
    assert d[1] == 0.0                       # 2**-13 is below half the smallest subnormal


def test_fp6_packing_golden(golden_dir):
    for line in open(os.path.join(golden_dir, "fp6_pack.txt")):
        line = line.split("#")[0].strip()
        if not line:
            continue
        f = line.split()
        codes = np.array([int(v) for v in f[:4]], dtype=np.uint8)
        want = np.array([int(v, 16) for v in f[4:]], dtype=np.uint8)
        assert np.array_equal(mx.pack(codes, "e3m2"), want)
        assert np.array_equal(mx.unpack(want, "e3m2", 4), codes)


def test_fp4_packing_and_round_trips():
    assert np.array_equal(mx.pack(np.array([1, 2, 15, 0], np.uint8), "e2m1"), np.array([0x21, 0x0F], np.uint8))
    rng = np.random.default_rng(5)
    for fmt, top in (("e2m1", 16), ("e3m2", 64), ("e4m3", 256)):
        c = rng.integers(0, top, (7, 96)).astype(np.uint8)
        p = mx.pack(c, fmt)
        assert p.shape[-1] == 96 * mx.bits_per_code(fmt) // 8
        assert np.array_equal(mx.unpack(p, fmt, 96), c)


def test_round_to_bf16_matches_torch():
    rng = np.random.default_rng(9)
    x = np.concatenate([
        (rng.standard_normal(20000) * np.exp2(rng.uniform(-140, 120, 20000))),
        # exact midpoints between neighbouring bf16 values (ties)
        (np.arange(1, 2000) * 2 + 1) * 2.0 ** -9,
        -(np.arange(1, 2000) * 2 + 1) * 2.0 ** -140,
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = mx.round_to_bf16(x.astype(np.float64))
    assert np.array_equal(ref, got)
