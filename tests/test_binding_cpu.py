"""The Python binding checks every tensor against the problem before the C ABI
sees a pointer: dtype, exact shape, contiguity and the device.  These run on
the CPU with CPU tensors, so a call that passes every shape check stops at the
device check; nothing reaches the library's compute entry points."""
import pytest
import torch

from block_scaled_precision_amd import moe_mx as m

T, H, I, E, K = 16, 256, 512, 8, 2


def _weights(fmt="e2m1", L=E, Is=0):
    b = m.FORMAT_BITS[fmt]
    u8 = torch.uint8
    w = m.MoeWeights(torch.zeros((L, 2 * I, H * b // 8), dtype=u8), torch.zeros((L, 2 * I, H // 32), dtype=u8),
                     torch.zeros((L, H, I * b // 8), dtype=u8), torch.zeros((L, H, I // 32), dtype=u8), fmt)
    if Is:
        w.ws1 = torch.zeros((2 * Is, H * b // 8), dtype=u8)
        w.ws1_scale = torch.zeros((2 * Is, H // 32), dtype=u8)
        w.ws2 = torch.zeros((H, Is * b // 8), dtype=u8)
        w.ws2_scale = torch.zeros((H, Is // 32), dtype=u8)
    return w


def _call(**kw):
    fmt = kw.pop("fmt", "e2m1")
    Is = kw.pop("Is", 0)
    L = kw.pop("L", 0)
    prob = kw.pop("prob", None) or m.make_problem(T, H, I, E, K, fmt, "bf16", I_shared=Is,
                                                  local_offset=0, local_count=L)
    args = dict(x=torch.zeros((T, H), dtype=torch.bfloat16), weights=_weights(fmt, L or E, Is),
                router_logits=torch.zeros((T, E), dtype=torch.float32))
    args.update(kw)
    return m.moe_fused(prob, **args)


def test_valid_shapes_stop_at_the_device_check():
    with pytest.raises(ValueError, match="GPU"):
        _call()
    with pytest.raises(ValueError, match="GPU"):
        _call(fmt="e3m2", Is=256)
    with pytest.raises(ValueError, match="GPU"):
        _call(L=4, weights=_weights(L=4))


@pytest.mark.parametrize("change,msg", [
    (dict(router_logits=torch.zeros((T, E), dtype=torch.bfloat16)), "router_logits: dtype"),
    (dict(router_logits=torch.zeros((T, E + 1), dtype=torch.float32)), "router_logits: shape"),
    (dict(router_logits=torch.zeros((E, T), dtype=torch.float32).t()), "router_logits: must be contiguous"),
    (dict(x=torch.zeros((T, H), dtype=torch.float32)), "x: dtype"),
    (dict(x=torch.zeros((T + 1, H), dtype=torch.bfloat16)), "x: shape"),
    (dict(x=torch.zeros((H, T), dtype=torch.bfloat16).t()), "x: must be contiguous"),
    (dict(y=torch.zeros((T, H - 32), dtype=torch.bfloat16)), "y: shape"),
    (dict(y=torch.zeros((T, 2 * H), dtype=torch.bfloat16)[:, ::2]), "y: must be contiguous"),
    (dict(y=torch.zeros((T, H), dtype=torch.float16)), "y: dtype"),
    (dict(router_logits=None), "router_logits or a precomputed"),
    (dict(topk_ids_in=torch.zeros((T, K), dtype=torch.int32)), "go together"),
    (dict(topk_ids_in=torch.zeros((T, K), dtype=torch.int64), topk_w_in=torch.zeros((T, K))), "topk_ids_in: dtype"),
    (dict(topk_ids_in=torch.zeros((T, K + 1), dtype=torch.int32), topk_w_in=torch.zeros((T, K))),
     "topk_ids_in: shape"),
    (dict(topk_ids_out=torch.zeros((T, K), dtype=torch.int64)), "topk_ids_out: dtype"),
    (dict(topk_w_out=torch.zeros((T, K + 1))), "topk_w_out: shape"),
    (dict(workspace=torch.zeros(16, dtype=torch.uint8)), "workspace: 16 bytes"),
    (dict(workspace=torch.zeros(1 << 24, dtype=torch.int32)), "workspace: expected"),
])
def test_bad_tensor_is_rejected(change, msg):
    with pytest.raises(ValueError, match=msg):
        _call(**change)


@pytest.mark.parametrize("part,bad_shape", [
    ("w1", (E - 1, 2 * I, H // 2)), ("w1", (E, 2 * I, H)), ("w1_scale", (E, 2 * I, H // 16)),
    ("w2", (E, H, I)), ("w2_scale", (E, I, H // 32)),
])
def test_bad_weight_shape_is_rejected(part, bad_shape):
    w = _weights()
    setattr(w, part, torch.zeros(bad_shape, dtype=torch.uint8))
    with pytest.raises(ValueError, match=f"{part}: shape"):
        _call(weights=w)


def test_weight_dtype_format_and_shared_checks():
    w = _weights()
    w.w2 = w.w2.to(torch.int8)
    with pytest.raises(ValueError, match="w2: dtype"):
        _call(weights=w)
    with pytest.raises(ValueError, match="weights are e2m1"):
        _call(prob=m.make_problem(T, H, I, E, K, "e3m2", "bf16"))
    w = _weights(Is=256)
    w.ws2 = torch.zeros((H, 256), dtype=torch.uint8)
    with pytest.raises(ValueError, match="ws2: shape"):
        _call(Is=256, weights=w)
    with pytest.raises(ValueError, match="ws1: expected a tensor"):
        _call(Is=256, weights=_weights())
    # a shard holds L experts: full-E weights are the wrong shape
    with pytest.raises(ValueError, match="w1: shape"):
        _call(L=4, weights=_weights(L=E))


def test_route_and_quantize_checks():
    with pytest.raises(ValueError, match="logits: dtype"):
        m.moe_route(torch.zeros((T, E), dtype=torch.bfloat16), K)
    with pytest.raises(ValueError, match="outside"):
        m.moe_route(torch.zeros((T, E)), E + 1)
    with pytest.raises(ValueError, match="GPU"):
        m.moe_route(torch.zeros((T, E)), K)
    with pytest.raises(ValueError, match="dtype"):
        m.mx_quantize(torch.zeros((4, 64), dtype=torch.float16), "e2m1")
    with pytest.raises(ValueError, match="multiple of 32"):
        m.mx_quantize(torch.zeros((4, 48)), "e2m1")
    with pytest.raises(ValueError, match="codes: shape"):
        m.mx_quantize(torch.zeros((4, 64)), "e3m2", codes=torch.zeros((4, 32), dtype=torch.uint8))
    with pytest.raises(ValueError, match="scales: dtype"):
        m.mx_quantize(torch.zeros((4, 64)), "e2m1", scales=torch.zeros((4, 2), dtype=torch.int8))
    with pytest.raises(ValueError, match="contiguous"):
        m.mx_quantize(torch.zeros((64, 4)).t(), "e2m1")
    with pytest.raises(ValueError, match="unknown MX format"):
        m.mx_quantize(torch.zeros((4, 64)), "e5m2")
    with pytest.raises(ValueError, match="GPU"):
        m.mx_quantize(torch.zeros((4, 64)), "e2m1")
