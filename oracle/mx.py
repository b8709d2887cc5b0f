"""OCP microscaling (MX) codecs, block quantizer and packing -- oracle.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources.  The pages name the formats but do not print their bit layouts:

* "TokenSpeed SiTU" page, section "Supported contract": MXFP4 weights
  (``MxE2m1``) and MXFP8 activations with a block-scale tensor; the wheel
  description names the ``MxE4m3_MxE2m1MxE4m3`` family.
* "mxfp6-sm120" page, section "Execution model" (figure): dynamic E4M3
  activation quantization with one UE8M0 scale per 32 K values; packed MXFP6
  E3M2 weights with one UE8M0 scale per 32 K values; four E3M2 values occupy
  three bytes.

The bit fields below are the plain reading of those names under the OCP
Microscaling Formats v1.0 specification: sign | exponent | mantissa with the
usual subnormals, E2M1 bias 1, E3M2 bias 3, E4M3 bias 7 (the OCP E4M3 variant:
no infinities, S.1111.111 is NaN, largest finite 448), and E8M0 an unsigned
biased exponent 2**(c-127) with c = 255 NaN.

Block quantization follows the OCP rule for converting a block of 32 values:
shared exponent = floor(log2(max|v|)) - emax(element format), clamped to the
E8M0 range; each element is v / 2**shared rounded to the nearest representable
element value, ties to the even code, clamped to the largest finite magnitude.
"""
from __future__ import annotations

import numpy as np

BLOCK = 32  # elements that share one E8M0 scale

# exponent bits, mantissa bits, bias, storage bits
_FIELDS = {
    "e2m1": (2, 1, 1, 4),
    "e3m2": (3, 2, 3, 6),
    "e4m3": (4, 3, 7, 8),
}


def _decode_code(fmt: str, code: int) -> float:
    """Value of one element code, read from its sign/exponent/mantissa fields."""
    ebits, mbits, bias, bits = _FIELDS[fmt]
    sign = -1.0 if (code >> (ebits + mbits)) & 1 else 1.0
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    if fmt == "e4m3" and e == (1 << ebits) - 1 and m == (1 << mbits) - 1:
        return float("nan")
    if e == 0:  # subnormal: 0.m * 2**(1-bias)
        return sign * (m / (1 << mbits)) * 2.0 ** (1 - bias)
    return sign * (1.0 + m / (1 << mbits)) * 2.0 ** (e - bias)


def decode_table(fmt: str) -> np.ndarray:
    """float64 value of every code 0 .. 2**bits-1 (NaN where the code is NaN)."""
    bits = _FIELDS[fmt][3]
    return np.array([_decode_code(fmt, c) for c in range(1 << bits)], dtype=np.float64)


def emax(fmt: str) -> int:
    """Exponent of the largest finite magnitude: E2M1 -> 2, E3M2 -> 4, E4M3 -> 8."""
    t = decode_table(fmt)
    top = np.nanmax(np.abs(t))
    return int(np.floor(np.log2(top)))


def decode_e8m0(codes: np.ndarray) -> np.ndarray:
    """E8M0 scale codes -> float64 2**(c-127); code 255 -> NaN."""
    c = np.asarray(codes).astype(np.int64)
    out = np.ldexp(1.0, c - 127).astype(np.float64)
    return np.where(c == 255, np.nan, out)


def decode(codes: np.ndarray, fmt: str) -> np.ndarray:
    """Element codes (one per uint8) -> float64 values."""
    return decode_table(fmt)[np.asarray(codes).astype(np.int64)]


def _positive_magnitudes(fmt: str) -> np.ndarray:
    """Finite non-negative magnitudes indexed by their (sign-clear) code."""
    ebits, mbits, _, _ = _FIELDS[fmt]
    n = 1 << (ebits + mbits)
    t = decode_table(fmt)[:n]
    finite = ~np.isnan(t)
    return t[finite]  # codes 0 .. n-1 (e4m3 drops 0x7F)


def _nearest_code(mag: np.ndarray, fmt: str) -> np.ndarray:
    """Code of the representable magnitude nearest to each |q|; ties -> even code;
    magnitudes above the largest finite one saturate to it."""
    table = _positive_magnitudes(fmt)
    n = table.size
    hi = np.searchsorted(table, mag, side="left")          # first table[hi] >= mag
    sat = hi >= n
    hi = np.minimum(hi, n - 1)
    lo = np.maximum(hi - 1, 0)
    exact = table[hi] == mag
    d_lo = mag - table[lo]
    d_hi = table[hi] - mag
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi)
    code = np.where(exact, hi, code)
    code = np.where(sat, n - 1, code)
    return code.astype(np.uint8)


def quantize(v: np.ndarray, fmt: str):
    """Block-quantize the last axis of ``v`` (length a multiple of 32).

    ``v`` holds exact values (bf16 or fp32 inputs widened to float64).
    Returns (codes uint8 [..., n], scale codes uint8 [..., n/32]).

    Per 32-element block:
      1. amax = max |v|;
      2. amax == 0 -> scale code 0 and element codes +-0 (sign kept);
      3. e = floor(log2 amax), read exactly from the binary exponent;
      4. s = clamp(e - emax, -127, 127), scale code s + 127;
      5. q = v * 2**-s (exact);
      6. element code = nearest magnitude to |q| (ties to even code, saturating),
         with the sign bit of v.
    """
    v = np.asarray(v, dtype=np.float64)
    if v.shape[-1] % BLOCK:
        raise ValueError("last axis must be a multiple of 32")
    if not np.all(np.isfinite(v)):
        raise ValueError("quantize: inputs must be finite")
    ebits, mbits, _, _ = _FIELDS[fmt]
    blocks = v.reshape(v.shape[:-1] + (v.shape[-1] // BLOCK, BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    _, ex = np.frexp(amax)            # amax = f * 2**ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1       # floor(log2 amax) for amax > 0
    s = np.clip(e - emax(fmt), -127, 127)
    s = np.where(amax == 0, -127, s)
    scale_codes = (s + 127).astype(np.uint8)
    q = np.ldexp(blocks, -s[..., None])
    mag_code = _nearest_code(np.abs(q), fmt)
    sign = np.signbit(blocks).astype(np.uint8) << (ebits + mbits)
    codes = (mag_code | sign).astype(np.uint8)
    return codes.reshape(v.shape), scale_codes


def dequantize(codes: np.ndarray, scale_codes: np.ndarray, fmt: str) -> np.ndarray:
    """Element codes [..., n] and scale codes [..., n/32] -> float64 values."""
    vals = decode(codes, fmt)
    blocks = vals.reshape(vals.shape[:-1] + (vals.shape[-1] // BLOCK, BLOCK))
    scale = decode_e8m0(scale_codes)[..., None]
    return (blocks * scale).reshape(vals.shape)


# ---------------------------------------------------------------- packing ---
# Canonical byte layout of codes along the contraction axis (the library ABI):
#   E2M1: two codes per byte, element 2j in bits 0-3, element 2j+1 in bits 4-7;
#   E3M2: four codes in three bytes, element 4j+i in bits 6i..6i+5 of the
#         little-endian 24-bit word (the "four values in three bytes" packing);
#   E4M3: one code per byte.

def bits_per_code(fmt: str) -> int:
    return _FIELDS[fmt][3]


def pack(codes: np.ndarray, fmt: str) -> np.ndarray:
    c = np.asarray(codes).astype(np.uint32)
    if fmt == "e4m3":
        return c.astype(np.uint8)
    if fmt == "e2m1":
        if c.shape[-1] % 2:
            raise ValueError("odd length")
        lo = c[..., 0::2] & 0xF
        hi = c[..., 1::2] & 0xF
        return (lo | (hi << 4)).astype(np.uint8)
    if fmt == "e3m2":
        if c.shape[-1] % 4:
            raise ValueError("length not a multiple of 4")
        g = c.reshape(c.shape[:-1] + (c.shape[-1] // 4, 4)) & 0x3F
        word = g[..., 0] | (g[..., 1] << 6) | (g[..., 2] << 12) | (g[..., 3] << 18)
        b = np.stack([word & 0xFF, (word >> 8) & 0xFF, (word >> 16) & 0xFF], axis=-1)
        return b.reshape(c.shape[:-1] + (c.shape[-1] // 4 * 3,)).astype(np.uint8)
    raise ValueError(fmt)


def unpack(packed: np.ndarray, fmt: str, n: int) -> np.ndarray:
    """Inverse of ``pack``: bytes [..., n*bits/8] -> codes uint8 [..., n]."""
    p = np.asarray(packed).astype(np.uint32)
    if fmt == "e4m3":
        return p.astype(np.uint8)[..., :n]
    if fmt == "e2m1":
        out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
        out[..., 0::2] = p & 0xF
        out[..., 1::2] = p >> 4
        return out[..., :n]
    if fmt == "e3m2":
        g = p.reshape(p.shape[:-1] + (p.shape[-1] // 3, 3))
        word = g[..., 0] | (g[..., 1] << 8) | (g[..., 2] << 16)
        c = np.stack([(word >> (6 * i)) & 0x3F for i in range(4)], axis=-1)
        return c.reshape(p.shape[:-1] + (p.shape[-1] // 3 * 4,)).astype(np.uint8)[..., :n]
    raise ValueError(fmt)


# ------------------------------------------------------------------ bf16 ----

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64 values (exact)."""
    u = (np.asarray(bits).astype(np.uint32) << 16).astype(np.uint32)
    return u.view(np.float32).astype(np.float64)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (round half to even), returned as float64.

    bfloat16 keeps 8 significant bits with the float32 exponent range; below
    2**-126 the grid spacing is fixed at 2**-133 (subnormals).  Finite inputs only.
    """
    x = np.asarray(x, dtype=np.float64)
    _, ex = np.frexp(x)                       # |x| in [2**(ex-1), 2**ex)
    quantum_exp = np.maximum(ex.astype(np.int64) - 8, -133)
    quantum_exp = np.where(x == 0, -133, quantum_exp)
    return np.ldexp(np.rint(np.ldexp(x, -quantum_exp)), quantum_exp)
