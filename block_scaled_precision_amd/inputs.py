"""Seeded synthetic inputs for the routed MX mixture-of-experts layer.

This module only draws random numbers and shapes them; it holds none of the
layer's arithmetic (no quantization, routing or GEMM).  Both the HIP path and
the CPU oracle receive the tensors it returns.

Recipe (the pages' real weights, records and request sets are not available,
so these stand in for them):
* router logits: standard normal, float32;
* x: standard normal float32, rounded to bfloat16 by torch (bf16 ~ N(0, 1));
* weights: 0.02 * standard normal, float32, drawn per expert; the caller
  quantizes them to MX codes;
* the skewed workload adds a per-expert bias 3 * r**-1.2 in float32, where r is
  a seeded random ranking 1..E, and forces the last two experts to -inf.

Every tensor comes from its own ``torch.Generator`` seeded from
(seed, tensor id, expert); on CPU that is torch's Mersenne twister, on a GPU
torch's Philox.  The two devices give different (each deterministic) streams,
so a test draws once and hands the same tensor to both sides.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

# tensor ids for seeding
LOGITS, X, W1, W2, SW1, SW2, RANKING = range(7)


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    wfmt: str            # "e2m1" (MXFP4) | "e3m2" (MXFP6)
    act: str             # "bf16" (w4a16) | "mxfp8" (w4a8 / w6a8)
    I_shared: int = 0
    skew: bool = False
    note: str = field(default="", compare=False)


WORKLOADS = {
    "tiny_w4a16": Workload("tiny_w4a16", 16, 256, 512, 8, 2, "e2m1", "bf16",
                           note="tiny MXFP4 layer, bf16 activations"),
    "decode_w4a16": Workload("decode_w4a16", 64, 7168, 2048, 384, 8, "e2m1", "bf16",
                             note="decode batch of 64 tokens over 384 resident MXFP4 experts"),
    "prefill_w4a8": Workload("prefill_w4a8", 8192, 7168, 2048, 384, 8, "e2m1", "mxfp8",
                             note="prefill batch of 8192 tokens, MXFP8 activations x MXFP4 weights"),
    "skew_w4a16": Workload("skew_w4a16", 4096, 4096, 1536, 128, 8, "e2m1", "bf16", skew=True,
                           note="skewed router (bias 3*r^-1.2, two dead experts), MXFP4"),
    "w6a8_shared": Workload("w6a8_shared", 2048, 5120, 1536, 256, 8, "e3m2", "mxfp8", I_shared=4096,
                            note="MXFP6 E3M2 weights, MXFP8 activations, one shared expert I=4096"),
}


def seed_of(seed: int, tensor: int, index: int = 0) -> int:
    """Deterministic 63-bit seed for (seed, tensor id, expert index)."""
    h = 0x9E3779B97F4A7C15
    for v in (seed, tensor, index):
        h ^= (v + 0x632BE59BD9B4E019 + ((h << 6) & 0xFFFFFFFFFFFFFFFF) + (h >> 2)) & 0xFFFFFFFFFFFFFFFF
        h &= 0xFFFFFFFFFFFFFFFF
    return h & 0x7FFFFFFFFFFFFFFF


def normal(shape, seed: int, tensor: int, index: int = 0, device="cpu", std: float = 1.0) -> torch.Tensor:
    g = torch.Generator(device=device)
    g.manual_seed(seed_of(seed, tensor, index))
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    return t * std if std != 1.0 else t


def router_logits(w: Workload, seed: int = 0, device="cpu", T: int | None = None) -> torch.Tensor:
    T = w.T if T is None else T
    logits = normal((T, w.E), seed, LOGITS, device=device)
    if w.skew:
        g = torch.Generator(device="cpu")
        g.manual_seed(seed_of(seed, RANKING))
        r = (torch.randperm(w.E, generator=g) + 1).to(torch.float32)
        bias = (3.0 * r.to(torch.float64) ** -1.2).to(torch.float32)
        bias[w.E - 2:] = float("-inf")
        logits = logits + bias.to(device)
    return logits


def hidden_states(w: Workload, seed: int = 0, device="cpu", T: int | None = None) -> torch.Tensor:
    T = w.T if T is None else T
    return normal((T, w.H), seed, X, device=device).to(torch.bfloat16)


def expert_w1(w: Workload, e: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """float32 [2I, H]: rows [0, I) gate, [I, 2I) up."""
    return normal((2 * w.I, w.H), seed, W1, e, device=device, std=0.02)


def expert_w2(w: Workload, e: int, seed: int = 0, device="cpu") -> torch.Tensor:
    """float32 [H, I]."""
    return normal((w.H, w.I), seed, W2, e, device=device, std=0.02)


def shared_w1(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    return normal((2 * w.I_shared, w.H), seed, SW1, device=device, std=0.02)


def shared_w2(w: Workload, seed: int = 0, device="cpu") -> torch.Tensor:
    return normal((w.H, w.I_shared), seed, SW2, device=device, std=0.02)


def random_bytes(shape, seed: int, tensor: int, index: int = 0) -> torch.Tensor:
    """Uniform random bytes (uint8, CPU).  Read as packed E2M1 or E3M2 codes
    every field is a finite element code, so they serve as weights whose codes
    are drawn directly."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_of(seed, tensor, index))
    return torch.randint(0, 256, shape, generator=g, dtype=torch.uint8)


def small_integers(shape, seed: int, tensor: int, lo: int = -8, hi: int = 8) -> torch.Tensor:
    """Integers uniform in [lo, hi] as bf16 (exact), CPU."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed_of(seed, tensor))
    return torch.randint(lo, hi + 1, shape, generator=g).to(torch.bfloat16)


def scaled(w: Workload, **changes) -> Workload:
    """Same workload with some sizes replaced (for small parity cases)."""
    d = dict(w.__dict__)
    d.update(changes)
    return Workload(**d)
