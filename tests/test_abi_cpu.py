"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before any device work (no GPU needed)."""
import ctypes
import os
import re

import pytest

from tests.conftest import ROOT, has_gpu

HEADER = os.path.join(ROOT, "include", "moe_mx.h")

# These calls pass fake (never dereferenced) device pointers that validation
# must reject on the host; they are kept off machines with a GPU.
pytestmark = pytest.mark.skipif(has_gpu(), reason="host-only checks with fake device pointers")


def _lib():
    from block_scaled_precision_amd import moe_mx as m
    if not os.path.exists(m.LIB_PATH):
        from block_scaled_precision_amd import build
        build.build()
    return m, m.lib()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\*?\s+\**(\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol():
    m, L = _lib()
    names = _declared_functions()
    assert set(names) == set(m.EXPORTS), names
    for n in names:
        assert getattr(L, n) is not None


def test_status_strings_and_version():
    m, L = _lib()
    for s in range(6):
        assert m.status_str(s)
    assert m.status_str(99) == "unknown status"
    assert L.moe_mx_version().decode().count(".") == 2


def _problem(m, **kw):
    d = dict(T=16, H=256, I=512, E=8, k=2, fmt="e2m1", act="bf16")
    d.update(kw)
    return m.make_problem(d["T"], d["H"], d["I"], d["E"], d["k"], d["fmt"], d["act"],
                          I_shared=d.get("I_shared", 0), local_offset=d.get("off", 0),
                          local_count=d.get("cnt", 0))


def _tensors(m, **kw):
    fake = 1 << 20  # aligned, never dereferenced: validation fails first
    base = dict(x=fake, router_logits=fake, w1=fake, w1_scale=fake, w2=fake, w2_scale=fake, y=fake)
    base.update(kw)
    return m.MoeTensors(**base)


@pytest.mark.parametrize("change,status", [
    (dict(T=-1), 1), (dict(H=0), 1), (dict(H=100), 1), (dict(I=48), 1),
    (dict(E=0), 1), (dict(E=1025), 1), (dict(k=0), 1), (dict(k=9), 1),
    (dict(off=4, cnt=8), 1), (dict(off=-1), 1), (dict(I_shared=-32), 1),
    (dict(H=160), 2), (dict(I=96), 2), (dict(I_shared=64), 2), (dict(I_shared=48), 1),
    (dict(fmt="e4m3"), 2),
])
def test_invalid_problems_rejected_on_host(change, status):
    m, L = _lib()
    p = _problem(m, **change)
    t = _tensors(m, ws1=1 << 20, ws1_scale=1 << 20, ws2=1 << 20, ws2_scale=1 << 20)
    assert L.moe_fused(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(1 << 20), 1 << 40, None) == status


@pytest.mark.parametrize("tkw,status", [
    (dict(x=None), 1), (dict(y=None), 1), (dict(w2_scale=None), 1),
    (dict(router_logits=None), 1),                                   # no routing source
    (dict(router_logits=None, topk_ids_in=1 << 20), 1),              # ids without weights
    (dict(x=(1 << 20) + 4), 1),                                      # misaligned
])
def test_invalid_tensors_rejected_on_host(tkw, status):
    m, L = _lib()
    p = _problem(m)
    t = _tensors(m, **tkw)
    assert L.moe_fused(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(1 << 20), 1 << 40, None) == status


def test_flags_and_activation_validation():
    m, L = _lib()
    t = _tensors(m)
    for fields, status in [(dict(flags=2), 1), (dict(act_fn=3), 1),
                           (dict(flags=1, T=9), 2), (dict(flags=1, act="mxfp8"), 2), (dict(flags=1), 2)]:
        p = _problem(m, T=fields.pop("T", 16), act=fields.pop("act", "bf16"))
        for k_, v in fields.items():
            setattr(p, k_, v)
        # (flags=1 with H = 256: not a multiple of 512 -> unsupported)
        assert L.moe_fused(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(1 << 20), 1 << 40, None) == status
    p = _problem(m, T=4, H=1024)
    p.flags = 1
    assert L.moe_fused(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(1 << 20), 1 << 40, None) == 4


def test_workspace_checks():
    m, L = _lib()
    p = _problem(m)
    need = m.moe_fused_workspace_bytes(p)
    assert need > 0
    t = _tensors(m)
    assert L.moe_fused(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(1 << 20), need - 1, None) == 3
    assert L.moe_fused(ctypes.byref(p), ctypes.byref(t), None, need, None) == 3
    # monotone in T, and larger for MXFP8 activations (x codes, h codes + scales)
    assert m.moe_fused_workspace_bytes(_problem(m, T=64)) > need
    assert m.moe_fused_workspace_bytes(_problem(m, act="mxfp8")) != need
    assert L.moe_route_workspace_bytes(0, 8, 2) > 0
    assert L.moe_route_workspace_bytes(1000, 64, 8) > L.moe_route_workspace_bytes(10, 64, 8)


def test_zero_tokens_is_ok_without_device():
    m, L = _lib()
    p = _problem(m, T=0)
    t = m.MoeTensors()
    assert L.moe_fused(ctypes.byref(p), ctypes.byref(t), None, 0, None) == 0


def test_quantize_and_route_validation():
    m, L = _lib()
    vp = ctypes.c_void_p
    a = vp(1 << 20)
    assert L.mx_quantize(a, 0, 4, 48, 48, 1, a, a, None) == 1            # cols % 32
    assert L.mx_quantize(a, 0, 4, 64, 32, 1, a, a, None) == 1            # ld < cols
    assert L.mx_quantize(a, 7, 4, 64, 64, 1, a, a, None) == 1            # bad dtype
    assert L.mx_quantize(a, 0, 4, 64, 64, 9, a, a, None) == 1            # bad format
    assert L.mx_quantize(a, 0, 4, 64, 64, 1, vp((1 << 20) + 8), a, None) == 1  # misaligned codes
    assert L.mx_quantize(None, 0, 0, 64, 64, 1, None, None, None) == 0   # empty
    assert L.moe_route(a, 4, 8, 9, a, a, a, a, a, 1 << 30, None) == 1    # k > E
    assert L.moe_route(a, 4, 2000, 2, a, a, a, a, a, 1 << 30, None) == 1 # E > 1024
    assert L.moe_route(a, 4, 8, 2, a, a, a, a, a, 0, None) == 3          # no workspace


def test_valid_call_without_gfx950_fails_closed():
    m, L = _lib()
    a = ctypes.c_void_p(1 << 20)
    assert L.mx_quantize(a, 0, 4, 64, 64, 1, a, a, None) == 4
    p = _problem(m)
    t = _tensors(m)
    assert L.moe_fused(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(1 << 20), 1 << 40, None) == 4


def test_gemm_validation():
    m, L = _lib()
    vp = ctypes.c_void_p
    a = vp(1 << 20)
    f = ctypes.c_float(1.0)
    # (a, a_scale, M, N, K, act, w, w_scale, fmt, alpha, c, ws, ws_bytes, stream)
    call = lambda *args: L.mx_gemm(*args)  # noqa: E731
    assert call(a, None, 4, 64, 100, 0, a, a, 1, f, a, None, 0, None) == 1        # K % 32
    assert call(a, None, -1, 64, 128, 0, a, a, 1, f, a, None, 0, None) == 1       # M < 0
    assert call(a, None, 4, 0, 128, 0, a, a, 1, f, a, None, 0, None) == 1         # N = 0
    assert call(a, None, 4, 64, 128, 5, a, a, 1, f, a, None, 0, None) == 1        # bad act
    assert call(a, None, 4, 64, 128, 0, a, a, 9, f, a, None, 0, None) == 1        # bad format
    assert call(a, a, 4, 64, 128, 0, a, a, 1, f, a, None, 0, None) == 1           # scales with bf16
    assert call(None, None, 4, 64, 128, 0, a, a, 1, f, a, None, 0, None) == 1     # null A
    assert call(vp((1 << 20) + 2), None, 4, 64, 128, 0, a, a, 1, f, a, None, 0, None) == 1  # misaligned
    assert call(a, None, 4, 60, 128, 0, a, a, 1, f, a, None, 0, None) == 2        # N % 8
    assert call(a, None, 4, 64, 96, 0, a, a, 1, f, a, None, 0, None) == 2         # K % 128
    assert call(a, None, 4, 64, 128, 0, a, a, 3, f, a, None, 0, None) == 2        # E4M3 weights
    assert call(a, None, 4, 64, 128, 1, a, a, 1, f, a, None, 0, None) == 3        # no workspace
    need = L.mx_gemm_workspace_bytes(4, 64, 128, 1, 1)
    assert need >= 4 * 128 + 4 * 4 and L.mx_gemm_workspace_bytes(4, 64, 128, 0, 1) == 0
    # bf16 x E2M1 with few rows: room for a K split's fp32 partial sums (a whole
    # number of 256-K stages per range, at least two); none when the rows or
    # column blocks already fill the workgroups, or for E3M2 weights
    split = L.mx_gemm_workspace_bytes(8, 4096, 7168, 0, 1)
    assert split >= 7 * 8 * 4096 * 4 and split % 256 == 0
    assert L.mx_gemm_workspace_bytes(8, 4096, 7168, 0, 2) == 0
    assert L.mx_gemm_workspace_bytes(64, 4096, 7168, 0, 1) == 0
    assert L.mx_gemm_workspace_bytes(8, 65536, 7168, 0, 1) == 0
    assert L.mx_gemm_workspace_bytes(8, 4096, 256, 0, 1) == 0
    assert call(a, None, 4, 64, 128, 1, a, a, 1, f, a, vp(1 << 20), need - 1, None) == 3
    assert call(a, a, 4, 64, 128, 1, a, a, 1, f, a, None, 0, None) == 4          # pre-quantized: no workspace
    assert call(None, None, 0, 64, 128, 0, None, None, 1, f, None, None, 0, None) == 0  # M = 0
    assert call(a, None, 4, 64, 128, 0, a, a, 2, f, a, None, 0, None) == 4        # valid: no gfx950 here
