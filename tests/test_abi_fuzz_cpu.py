"""Host-side validation of every entry point under random arguments: any sizes,
formats, activations, flags and shard ranges give one of the status codes
(never a crash), and a problem that validates reaches the architecture check,
which fails closed on a machine without a GPU, so nothing is launched.
Workspace-size queries return 0 or a size large enough for the problem's own
outputs, never a value wrapped around by overflow."""
import ctypes

import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

from tests.conftest import has_gpu

# fake (never dereferenced) device pointers: kept off machines with a GPU
pytestmark = pytest.mark.skipif(has_gpu(), reason="host-only checks with fake device pointers")

STATUS = {0, 1, 2, 3, 4, 5}
ARCH = 4
FAKE = 1 << 20
HUGE_WS = 1 << 62

# sizes: small, typical, boundary and out-of-range values
SIZE = st.one_of(st.integers(-4, 70), st.sampled_from(
    [96, 127, 128, 255, 256, 512, 1000, 1024, 1025, 1536, 2048, 4096, 7168, 8192, 65536,
     2 ** 20, 2 ** 31 - 1, -(2 ** 31)]))
SETTINGS = dict(max_examples=250, deadline=None, derandomize=True,
                suppress_health_check=[HealthCheck.too_slow])


def _lib():
    from tests.test_abi_cpu import _lib as load
    return load()


def _tensors(m):
    return m.MoeTensors(x=FAKE, router_logits=FAKE, w1=FAKE, w1_scale=FAKE, w2=FAKE, w2_scale=FAKE,
                        ws1=FAKE, ws1_scale=FAKE, ws2=FAKE, ws2_scale=FAKE, y=FAKE)


@settings(**SETTINGS)
@given(T=SIZE, H=SIZE, I=SIZE, E=SIZE, k=SIZE, fmt=st.integers(-1, 4), act=st.integers(-1, 2), Is=SIZE,
       off=SIZE, cnt=SIZE, fn=st.integers(-1, 3), flags=st.integers(0, 5),
       sw=st.sampled_from([1.0, 0.0, -2.0, float("nan")]))
def test_moe_fused_any_problem(T, H, I, E, k, fmt, act, Is, off, cnt, fn, flags, sw):
    m, L = _lib()
    p = m.MoeProblem(T=T, H=H, I=I, E=E, k=k, w_fmt=fmt, act=act, I_shared=Is, shared_weight=sw,
                     local_expert_offset=off, local_num_experts=cnt, act_fn=fn, flags=flags)
    t = _tensors(m)
    need = L.moe_fused_workspace_bytes(ctypes.byref(p))
    status = L.moe_fused(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(FAKE), HUGE_WS, None)
    assert status in STATUS
    if status == ARCH:
        # it validated: the workspace holds at least the routing and y-sized staging
        assert need >= max(T, 0) * max(k, 0) * 4
    for part in range(4):
        L.moe_fused_workspace_offset(ctypes.byref(p), part)
    assert L.moe_fused_noalloc(ctypes.byref(p), ctypes.byref(t), None) in STATUS


@settings(**SETTINGS)
@given(M=SIZE, N=SIZE, K=SIZE, act=st.integers(-1, 2), fmt=st.integers(-1, 4),
       scaled=st.booleans(), alpha=st.sampled_from([1.0, -0.5, 0.0]))
def test_mx_gemm_any_shape(M, N, K, act, fmt, scaled, alpha):
    m, L = _lib()
    need = L.mx_gemm_workspace_bytes(M, N, K, act, fmt)
    status = L.mx_gemm(FAKE, FAKE if scaled else None, M, N, K, act, FAKE, FAKE, fmt, alpha, FAKE, FAKE,
                       HUGE_WS, None)
    assert status in STATUS
    if status == ARCH and act == 1 and not scaled:
        assert need >= M * K  # room for the quantized activations


@settings(**SETTINGS)
@given(rows=SIZE, cols=SIZE, ld=SIZE, src=st.integers(-1, 2), fmt=st.integers(-1, 4))
def test_mx_quantize_any_shape(rows, cols, ld, src, fmt):
    m, L = _lib()
    assert L.mx_quantize(FAKE, src, rows, cols, ld, fmt, FAKE, FAKE, None) in STATUS


@settings(**SETTINGS)
@given(T=SIZE, E=SIZE, k=SIZE)
def test_moe_route_any_shape(T, E, k):
    m, L = _lib()
    need = L.moe_route_workspace_bytes(T, E, k)
    status = L.moe_route(FAKE, T, E, k, FAKE, FAKE, FAKE, FAKE, FAKE, HUGE_WS, None)
    assert status in STATUS
    if status == ARCH:
        assert need < HUGE_WS


@st.composite
def near_valid_problem(draw):
    """A layer problem that mostly validates and is supported (H, I and
    I_shared multiples of 128, a local expert range inside E), with one field
    then moved to a boundary or out of range in half of the draws."""
    E = draw(st.integers(1, 1024))
    d = dict(T=draw(st.integers(0, 300)), H=128 * draw(st.integers(1, 64)), I=128 * draw(st.integers(1, 24)),
             E=E, k=draw(st.integers(1, min(E, 64))), w_fmt=draw(st.sampled_from([1, 2])),
             act=draw(st.sampled_from([0, 1])), I_shared=128 * draw(st.integers(0, 16)),
             local_expert_offset=0, local_num_experts=0, act_fn=draw(st.integers(0, 2)),
             flags=draw(st.sampled_from([0, 0, 0, 1])))
    off = draw(st.integers(0, E - 1))
    d["local_expert_offset"], d["local_num_experts"] = off, draw(st.integers(0, E - off))
    if draw(st.booleans()):
        field = draw(st.sampled_from(sorted(d)))
        d[field] = draw(st.sampled_from([-1, 0, 1, 3, 33, 1025, 2 ** 31 - 1]))
    return d


@settings(**SETTINGS)
@given(d=near_valid_problem())
def test_moe_fused_near_valid_problem(d):
    m, L = _lib()
    p = m.MoeProblem(shared_weight=1.0, **d)
    t = _tensors(m)
    need = L.moe_fused_workspace_bytes(ctypes.byref(p))
    status = L.moe_fused(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(FAKE), HUGE_WS, None)
    assert status in STATUS
    if status == ARCH:
        assert 0 < need < HUGE_WS and need >= d["T"] * d["k"] * 4
        # too little workspace is caught before the architecture check
        if need > 1:
            assert L.moe_fused(ctypes.byref(p), ctypes.byref(t), ctypes.c_void_p(FAKE), need - 1, None) == 3
    assert L.moe_fused_noalloc(ctypes.byref(p), ctypes.byref(t), None) in STATUS


def test_near_valid_strategy_reaches_the_architecture_check():
    """The strategy above is only useful if many draws validate."""
    m, L = _lib()
    seen = []

    @settings(max_examples=200, deadline=None, derandomize=True)
    @given(d=near_valid_problem())
    def collect(d):
        p = m.MoeProblem(shared_weight=1.0, **d)
        seen.append(L.moe_fused(ctypes.byref(p), ctypes.byref(_tensors(m)), ctypes.c_void_p(FAKE), HUGE_WS, None))

    collect()
    assert seen.count(ARCH) >= len(seen) // 4, {s: seen.count(s) for s in set(seen)}


@settings(**SETTINGS)
@given(M=st.integers(0, 300), N=st.integers(1, 512).map(lambda n: 8 * n), K=st.integers(1, 64).map(lambda k: 128 * k),
       act=st.sampled_from([0, 1]), fmt=st.sampled_from([1, 2]), scaled=st.booleans())
def test_mx_gemm_near_valid_shape(M, N, K, act, fmt, scaled):
    m, L = _lib()
    a_scale = FAKE if (scaled and act == 1) else None
    need = L.mx_gemm_workspace_bytes(M, N, K, act, fmt)
    status = L.mx_gemm(FAKE, a_scale, M, N, K, act, FAKE, FAKE, fmt, 1.0, FAKE, FAKE, HUGE_WS, None)
    assert status == (0 if M == 0 else ARCH)
    if M > 0 and act == 1 and a_scale is None:
        # quantizing A needs the workspace: one byte short is an error
        assert L.mx_gemm(FAKE, None, M, N, K, act, FAKE, FAKE, fmt, 1.0, FAKE, FAKE, need - 1, None) == 3
    if M > 0 and act == 0:
        # the K split's workspace is optional: none at all still validates
        assert L.mx_gemm(FAKE, None, M, N, K, act, FAKE, FAKE, fmt, 1.0, FAKE, None, 0, None) == ARCH
