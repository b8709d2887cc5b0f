"""Pins for the oracle's layer forward (CPU only).

The layer is tied to plain dense computations it must reduce to (a gated MLP
written with torch in float64), to exact rational arithmetic, and to
invariants: identical experts make the output independent of routing,
x = 0 gives y = 0, scaling W2 by 2**n scales y by 2**n, relabelling experts
changes nothing, shard outputs add up to the full output.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch
import scipy.special

from oracle import moe as om
from oracle import mx

H, I, E, T = 64, 96, 4, 9


def _weights(rng, E, I, H, fmt, std=0.02):
    w1 = (rng.standard_normal((E, 2 * I, H)) * std).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * std).astype(np.float32)
    p1, s1 = om.quantize_weight(w1, fmt)
    p2, s2 = om.quantize_weight(w2, fmt)
    return p1, s1, p2, s2


def _x(rng, T, H, scale=1.0):
    x = torch.from_numpy((rng.standard_normal((T, H)) * scale).astype(np.float32)).to(torch.bfloat16)
    return x.to(torch.float64).numpy()


def _dense_mlp(a, d1, d2, act):
    """Textbook gated MLP in torch float64: (silu(a Wg^T) * (a Wu^T)) W2^T,
    with the intermediate passed through the pinned bf16 / MXFP8 rounding."""
    a = torch.from_numpy(a)
    wg = torch.from_numpy(d1[: d1.shape[0] // 2])
    wu = torch.from_numpy(d1[d1.shape[0] // 2:])
    h = torch.nn.functional.silu(a @ wg.T) * (a @ wu.T)
    h = h.numpy()
    if act == "bf16":
        h = mx.round_to_bf16(h)
    else:
        c, s = mx.quantize(h, "e4m3")
        h = mx.dequantize(c, s, "e4m3")
    return (torch.from_numpy(h) @ torch.from_numpy(d2).T).numpy()


def _act_input(x, act):
    if act == "bf16":
        return x
    c, s = mx.quantize(x, "e4m3")
    return mx.dequantize(c, s, "e4m3")


@pytest.mark.parametrize("fmt,act", [("e2m1", "bf16"), ("e2m1", "mxfp8"), ("e3m2", "mxfp8")])
def test_identical_experts_reduce_to_dense_mlp(fmt, act):
    rng = np.random.default_rng(0)
    p1, s1, p2, s2 = _weights(rng, 1, I, H, fmt)
    P1, S1, P2, S2 = (np.repeat(a, E, axis=0) for a in (p1, s1, p2, s2))
    x = _x(rng, T, H)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    y = om.moe_forward(x, lg, P1, S1, P2, S2, k=3, wfmt=fmt, act=act)["y"]
    d1 = om.decode_weight(p1[0], s1[0], fmt, H)
    d2 = om.decode_weight(p2[0], s2[0], fmt, I)
    ref = _dense_mlp(_act_input(x, act), d1, d2, act)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)


def test_two_experts_weighting_per_slot():
    """E = 2, k = 2: y = w_a * MLP_a + w_b * MLP_b with w = softmax of the two
    logits (scipy); k = 1: y = MLP of the arg-max expert."""
    rng = np.random.default_rng(1)
    p1, s1, p2, s2 = _weights(rng, 2, I, H, "e2m1")
    x = _x(rng, T, H)
    lg = rng.standard_normal((T, 2)).astype(np.float32)
    dense = [_dense_mlp(x, om.decode_weight(p1[e], s1[e], "e2m1", H),
                        om.decode_weight(p2[e], s2[e], "e2m1", I), "bf16") for e in range(2)]
    y2 = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e2m1", act="bf16")["y"]
    p = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(y2, p[:, :1] * dense[0] + p[:, 1:] * dense[1], rtol=1e-12, atol=1e-14)
    y1 = om.moe_forward(x, lg, p1, s1, p2, s2, k=1, wfmt="e2m1", act="bf16")["y"]
    arg = np.where(lg[:, 1] > lg[:, 0], 1, 0)
    assert np.allclose(y1, np.where(arg[:, None] == 1, dense[1], dense[0]), rtol=1e-12, atol=1e-14)


def test_fc1_exact_rational():
    """FC1 of decoded MX values is a sum of dyadic rationals: compare the
    float64 product with exact Fraction arithmetic from the raw codes."""
    rng = np.random.default_rng(2)
    Hs, Is = 64, 32
    p1, s1, _, _ = _weights(rng, 1, Is, Hs, "e2m1", std=1.0)
    x = _x(rng, 3, Hs)
    codes = mx.unpack(p1[0], "e2m1", Hs)
    vals = {0: 0, 1: Fraction(1, 2), 2: 1, 3: Fraction(3, 2), 4: 2, 5: 3, 6: 4, 7: 6}
    d1 = om.decode_weight(p1[0], s1[0], "e2m1", Hs)
    z = x @ d1.T
    for t in range(3):
        for n in range(0, 2 * Is, 5):
            acc = Fraction(0)
            for kk in range(Hs):
                c = int(codes[n, kk])
                v = vals[c & 7] * (-1 if c & 8 else 1)
                sc = Fraction(2) ** (int(s1[0, n, kk // 32]) - 127)
                acc += Fraction(float(x[t, kk])) * v * sc
            assert float(acc) == z[t, n]


def test_zero_input_and_w2_power_of_two_scaling():
    rng = np.random.default_rng(3)
    p1, s1, p2, s2 = _weights(rng, E, I, H, "e2m1")
    lg = rng.standard_normal((T, E)).astype(np.float32)
    y0 = om.moe_forward(np.zeros((T, H)), lg, p1, s1, p2, s2, k=2, wfmt="e2m1", act="bf16")["y"]
    assert np.all(y0 == 0)
    x = _x(rng, T, H)
    y = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e2m1", act="bf16")["y"]
    y5 = om.moe_forward(x, lg, p1, s1, p2, (s2.astype(np.int64) + 5).astype(np.uint8),
                        k=2, wfmt="e2m1", act="bf16")["y"]
    assert np.array_equal(y5, y * 32.0)


def test_expert_relabelling_invariance():
    rng = np.random.default_rng(4)
    p1, s1, p2, s2 = _weights(rng, E, I, H, "e3m2")
    x = _x(rng, T, H)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    y = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e3m2", act="mxfp8")["y"]
    perm = rng.permutation(E)
    yp = om.moe_forward(x, lg[:, perm], p1[perm], s1[perm], p2[perm], s2[perm],
                        k=2, wfmt="e3m2", act="mxfp8")["y"]
    assert np.allclose(y, yp, rtol=1e-13, atol=1e-15)


def test_shared_expert_adds_dense_mlp():
    rng = np.random.default_rng(5)
    p1, s1, p2, s2 = _weights(rng, E, I, H, "e3m2")
    q1, r1, q2, r2 = _weights(rng, 1, 2 * I, H, "e3m2")
    x = _x(rng, T, H)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    base = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e3m2", act="mxfp8")["y"]
    both = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e3m2", act="mxfp8",
                          shared=(q1[0], r1[0], q2[0], r2[0]))["y"]
    dense = _dense_mlp(_act_input(x, "mxfp8"), om.decode_weight(q1[0], r1[0], "e3m2", H),
                       om.decode_weight(q2[0], r2[0], "e3m2", 2 * I), "mxfp8")
    assert np.allclose(both - base, dense, rtol=1e-10, atol=1e-13)


@pytest.mark.parametrize("sw", [0.375, -2.0, 0.0])
def test_shared_weight_scales_the_shared_expert(sw):
    """The shared expert enters y as shared_weight * dense MLP: the difference
    from the routed-only layer is that multiple of the textbook MLP (exact for
    a power-of-two weight, since scaling by 2**n commutes with every rounding
    after FC2), and weight 0 leaves the routed output unchanged."""
    rng = np.random.default_rng(8)
    p1, s1, p2, s2 = _weights(rng, E, I, H, "e2m1")
    q1, r1, q2, r2 = _weights(rng, 1, I, H, "e2m1")
    x = _x(rng, T, H)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    shared = (q1[0], r1[0], q2[0], r2[0])
    base = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e2m1", act="bf16")["y"]
    got = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e2m1", act="bf16", shared=shared,
                         shared_weight=sw)["y"]
    dense = _dense_mlp(x, om.decode_weight(q1[0], r1[0], "e2m1", H),
                       om.decode_weight(q2[0], r2[0], "e2m1", I), "bf16")
    assert np.allclose(got - base, sw * dense, rtol=1e-10, atol=1e-13)
    if sw == 0.0:
        assert np.array_equal(got, base)
    else:
        # the shared term is a nonzero multiple of the dense MLP, with sw's sign
        one = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e2m1", act="bf16", shared=shared)["y"]
        assert np.allclose(got - base, sw * (one - base), rtol=1e-10, atol=1e-13)
        assert np.abs(dense).max() > 0


def test_intermediates_match_the_dataflow():
    """The optional intermediates are the FC2 inputs of each assignment: E4M3
    codes + E8M0 scales of SiLU(gate)*up per 32 along I (MXFP8), or its bf16
    values; feeding them through decoded W2 reproduces the expert outputs."""
    rng = np.random.default_rng(9)
    p1, s1, p2, s2 = _weights(rng, E, I, H, "e2m1")
    x = _x(rng, T, H)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    for act in ("mxfp8", "bf16"):
        out = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e2m1", act=act, intermediates=True)
        inter = out["intermediates"]
        assert sorted(inter) == list(range(T * 2))
        y = np.zeros_like(out["y"])
        for a, v in inter.items():
            t, j = divmod(a, 2)
            e = int(out["ids"][t, j])
            if act == "mxfp8":
                codes, scales = v
                assert codes.dtype == np.uint8 and codes.shape == (I,) and scales.shape == (I // 32,)
                h = mx.dequantize(codes, scales, "e4m3")
            else:
                h = v
                assert np.array_equal(h, mx.round_to_bf16(h))
            d2 = om.decode_weight(p2[e], s2[e], "e2m1", I)
            d1 = om.decode_weight(p1[e], s1[e], "e2m1", H)
            ref_h = _dense_mlp(_act_input(x[t:t + 1], act), d1, np.eye(I), act)[0]
            assert np.array_equal(h, ref_h)
            y[t] += out["w"][t, j] * (h @ d2.T)
        assert np.allclose(y, out["y"], rtol=1e-12, atol=1e-15)


def test_token_subset_and_precomputed_topk():
    rng = np.random.default_rng(6)
    p1, s1, p2, s2 = _weights(rng, E, I, H, "e2m1")
    x = _x(rng, T, H)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    full = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e2m1", act="bf16")
    sub = om.moe_forward(x, lg, p1, s1, p2, s2, k=2, wfmt="e2m1", act="bf16", tokens=[7, 2])
    assert np.array_equal(sub["y"], full["y"][[7, 2]])
    given = om.moe_forward(x, None, p1, s1, p2, s2, k=2, wfmt="e2m1", act="bf16",
                           topk_ids=full["ids"], topk_w=full["w"])
    assert np.array_equal(given["y"], full["y"])


def test_expert_shards_sum_to_full_output():
    rng = np.random.default_rng(7)
    p1, s1, p2, s2 = _weights(rng, 8, I, H, "e2m1")
    x = _x(rng, T, H)
    lg = rng.standard_normal((T, 8)).astype(np.float32)
    full = om.moe_forward(x, lg, p1, s1, p2, s2, k=3, wfmt="e2m1", act="bf16")["y"]
    parts = sum(om.moe_forward(x, lg, p1, s1, p2, s2, k=3, wfmt="e2m1", act="bf16",
                               local_offset=2 * r, local_count=2)["y"] for r in range(4))
    assert np.allclose(parts, full, rtol=1e-13, atol=1e-15)


def test_silu_closed_forms():
    g = np.array([0.0, 50.0, -50.0, 1.0, -800.0])
    s = om.silu(g)
    assert s[0] == 0.0 and abs(s[1] - 50.0) < 1e-15 * 50 and abs(s[2]) < 1e-19
    assert abs(s[3] - 1.0 / (1.0 + np.exp(-1.0))) < 1e-16 and s[4] == 0.0


def test_gated_activation_closed_forms():
    """Values worked by hand at points where each form is elementary."""
    g = np.array([0.0, 2.0, -3.0, 1.0, 7.0, 10.0, -0.5])
    u = np.array([5.0, 3.0, 4.0, -10.0, 0.0, 2.0, 9.0])
    # SiLU: g / (1 + e^-g) * u
    s = om.gated(g, u, "silu")
    assert s[0] == 0.0 and abs(s[1] - 2.0 / (1 + np.exp(-2.0)) * 3.0) < 1e-15
    # ReLU2: relu(g)^2 * u -> 0, 12, 0, -10, 0, 200, 0
    r = om.gated(g, u, "relu2")
    assert np.array_equal(r, np.array([0.0, 12.0, 0.0, -10.0, 0.0, 200.0, 0.0]))
    # SwiGLU-OAI: gate clipped above at 7, up clipped to [-7, 7], (u + 1) * g sigmoid(1.702 g)
    o = om.gated(g, u, "swiglu_oai")
    sig = lambda z: 1.0 / (1.0 + np.exp(-z))  # noqa: E731
    assert o[0] == 0.0                                   # g = 0
    assert abs(o[1] - 4.0 * 2.0 * sig(3.404)) < 1e-14    # (3 + 1) * 2 * sig(1.702 * 2)
    assert abs(o[3] - (-6.0) * 1.0 * sig(1.702)) < 1e-14  # up clipped to -7: (-7 + 1)
    assert abs(o[4] - 1.0 * 7.0 * sig(11.914)) < 1e-14   # (0 + 1) * 7 * sig(1.702 * 7)
    assert o[5] == 3.0 * 7.0 * sig(11.914)               # gate clipped from 10 to 7
    assert o[6] < 0 and abs(o[6] - 8.0 * -0.5 * sig(-0.851)) < 1e-14   # up 9 clipped to 7
    # the gate is clipped from above only: g = -10 stays -10
    assert om.gated(np.array([-10.0]), np.array([1.0]), "swiglu_oai")[0] == 2.0 * -10.0 * sig(-17.02)
    with pytest.raises(ValueError):
        om.gated(g, u, "gelu")


@pytest.mark.parametrize("act_fn", ["relu2", "swiglu_oai"])
def test_activation_variant_reaches_every_expert(act_fn):
    """The chosen activation replaces SiLU in every routed and shared expert:
    with identical experts the layer is the dense MLP with that activation."""
    rng = np.random.default_rng(15)
    p1, s1, p2, s2 = _weights(rng, 1, I, H, "e2m1", std=0.1)
    P1, S1, P2, S2 = (np.repeat(a, E, axis=0) for a in (p1, s1, p2, s2))
    x = _x(rng, T, H)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    d1 = om.decode_weight(p1[0], s1[0], "e2m1", H)
    d2 = om.decode_weight(p2[0], s2[0], "e2m1", I)
    z = x @ d1.T
    h = mx.round_to_bf16(om.gated(z[:, :I], z[:, I:], act_fn))
    ref = h @ d2.T
    y = om.moe_forward(x, lg, P1, S1, P2, S2, k=2, wfmt="e2m1", act="bf16", act_fn=act_fn)["y"]
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-14)
    ys = om.moe_forward(x, lg, P1, S1, P2, S2, k=2, wfmt="e2m1", act="bf16", act_fn=act_fn,
                        shared=(p1[0], s1[0], p2[0], s2[0]), shared_weight=0.5)["y"]
    assert np.allclose(ys, 1.5 * ref, rtol=1e-12, atol=1e-14)
    silu = om.moe_forward(x, lg, P1, S1, P2, S2, k=2, wfmt="e2m1", act="bf16")["y"]
    assert not np.allclose(silu, y)
