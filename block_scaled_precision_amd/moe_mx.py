"""ctypes binding of libmoe_mx.so (the C ABI declared in include/moe_mx.h).

Argument marshalling only: tensors are torch device tensors used as plain
device memory, streams are torch's current HIP stream, and every step of the
layer runs in the library's HIP kernels.  There is no fallback: if the library
is not built, or the device is not gfx950, calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mx.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_ARCH, MOE_ERR_HIP = range(6)
MX_FORMATS = {"e2m1": 1, "e3m2": 2, "e4m3": 3}
FORMAT_BITS = {"e2m1": 4, "e3m2": 6, "e4m3": 8}
SRC_DTYPES = {torch.bfloat16: 0, torch.float32: 1}
ACTS = {"bf16": 0, "mxfp8": 1}
ACT_FNS = {"silu": 0, "relu2": 1, "swiglu_oai": 2}

# Every symbol include/moe_mx.h declares.
EXPORTS = ("mx_quantize", "moe_route_workspace_bytes", "moe_route", "mx_gemm_workspace_bytes", "mx_gemm",
           "moe_fused_workspace_bytes", "moe_fused", "moe_fused_workspace_offset", "moe_fused_noalloc",
           "moe_status_str", "moe_mx_version")
NOALLOC_SCRATCH_BYTES = 32 << 20  # MOE_NOALLOC_SCRATCH_BYTES


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


class MoeProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("w_fmt", ctypes.c_int),
                ("act", ctypes.c_int), ("I_shared", ctypes.c_int32), ("shared_weight", ctypes.c_float),
                ("local_expert_offset", ctypes.c_int32), ("local_num_experts", ctypes.c_int32),
                ("act_fn", ctypes.c_int), ("flags", ctypes.c_uint32)]


MOE_NUM_STAGES = 7
STAGES = ("route", "permute", "quant_x", "fc1", "fc2", "shared", "finalize")


class MoeTensors(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "x", "router_logits", "topk_ids_in", "topk_w_in", "w1", "w1_scale", "w2", "w2_scale",
        "ws1", "ws1_scale", "ws2", "ws2_scale", "y", "topk_ids_out", "topk_w_out", "stage_events")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmoe_mx.so (built in-tree by block_scaled_precision_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python -m block_scaled_precision_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        L.mx_quantize.argtypes = [vp, ctypes.c_int, i64, i64, i64, ctypes.c_int, vp, vp, vp]
        L.mx_quantize.restype = ctypes.c_int
        L.moe_route_workspace_bytes.argtypes = [i32, i32, i32]
        L.moe_route_workspace_bytes.restype = sz
        L.moe_route.argtypes = [vp, i32, i32, i32, vp, vp, vp, vp, vp, sz, vp]
        L.moe_route.restype = ctypes.c_int
        L.moe_fused_workspace_bytes.argtypes = [ctypes.POINTER(MoeProblem)]
        L.moe_fused_workspace_bytes.restype = sz
        L.moe_fused.argtypes = [ctypes.POINTER(MoeProblem), ctypes.POINTER(MoeTensors), vp, sz, vp]
        L.moe_fused.restype = ctypes.c_int
        L.mx_gemm_workspace_bytes.argtypes = [i64, i64, i64, ctypes.c_int, ctypes.c_int]
        L.mx_gemm_workspace_bytes.restype = sz
        L.mx_gemm.argtypes = [vp, vp, i64, i64, i64, ctypes.c_int, vp, vp, ctypes.c_int, ctypes.c_float, vp, vp,
                              sz, vp]
        L.mx_gemm.restype = ctypes.c_int
        L.moe_fused_noalloc.argtypes = [ctypes.POINTER(MoeProblem), ctypes.POINTER(MoeTensors), vp]
        L.moe_fused_noalloc.restype = ctypes.c_int
        L.moe_fused_workspace_offset.argtypes = [ctypes.POINTER(MoeProblem), ctypes.c_int]
        L.moe_fused_workspace_offset.restype = sz
        L.moe_status_str.argtypes = [ctypes.c_int]
        L.moe_status_str.restype = ctypes.c_char_p
        L.moe_mx_version.argtypes = []
        L.moe_mx_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().moe_status_str(status).decode()


def _check(status: int, what: str):
    if status != MOE_OK:
        raise MoeError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must live on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"tensors on different devices ({dev} and {t.device})")


def _require(t, name: str, dtype, shape):
    """The C ABI sees only a pointer: check what it will read or write."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name}: expected a tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")


def _require_workspace(ws, need: int):
    if ws.dtype != torch.uint8 or ws.dim() != 1 or not ws.is_contiguous():
        raise ValueError("workspace: expected a contiguous 1-D uint8 tensor")
    if ws.numel() < need:
        raise ValueError(f"workspace: {ws.numel()} bytes, need {need}")


# ------------------------------------------------------------ mx_quantize --

def mx_quantize(src: torch.Tensor, fmt: str, codes: torch.Tensor | None = None,
                scales: torch.Tensor | None = None, stream=None):
    """Block-quantize the last axis of a bf16/fp32 matrix [rows, cols] (or a
    batch [..., rows, cols], flattened) to MX codes + E8M0 scales."""
    if fmt not in MX_FORMATS:
        raise ValueError(f"unknown MX format {fmt!r}")
    if src.dtype not in SRC_DTYPES:
        raise ValueError(f"src: dtype {src.dtype}, expected bfloat16 or float32")
    if src.dim() < 1:
        raise ValueError("src: needs at least one axis")
    cols = src.shape[-1]
    if cols % 32 or cols == 0:
        raise ValueError(f"src: last axis {cols} is not a positive multiple of 32")
    rows = src.numel() // cols
    if src.is_contiguous():
        src2, ld = src.reshape(rows, cols), cols
    elif src.dim() == 2 and src.stride(-1) == 1 and src.stride(0) >= cols:
        src2, ld = src, src.stride(0)        # rows with a stride
    else:
        raise ValueError("src: must be contiguous, or 2-D with contiguous rows")
    nbytes = cols * FORMAT_BITS[fmt] // 8
    dev = src.device
    if codes is None:
        codes = torch.empty(src.shape[:-1] + (nbytes,), dtype=torch.uint8, device=dev)
    if scales is None:
        scales = torch.empty(src.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=dev)
    _require(codes, "codes", torch.uint8, src.shape[:-1] + (nbytes,))
    _require(scales, "scales", torch.uint8, src.shape[:-1] + (cols // 32,))
    _dev(src, codes, scales)
    _check(lib().mx_quantize(_ptr(src2), SRC_DTYPES[src.dtype], rows, cols, ld, MX_FORMATS[fmt],
                             _ptr(codes), _ptr(scales), _stream(stream)), "mx_quantize")
    return codes, scales


# ---------------------------------------------------------------- route --

def moe_route_workspace_bytes(T: int, E: int, k: int) -> int:
    return lib().moe_route_workspace_bytes(T, E, k)


def moe_route(logits: torch.Tensor, k: int, workspace: torch.Tensor | None = None, stream=None):
    """-> (topk_ids [T,k] int32, topk_w [T,k] fp32, expert_offsets [E+1] int32,
    sorted_assign [T*k] int32)."""
    if logits.dim() != 2:
        raise ValueError("logits: expected [T, E]")
    T, E = logits.shape
    _require(logits, "logits", torch.float32, (T, E))
    if not 1 <= k <= E:
        raise ValueError(f"k = {k} outside [1, E = {E}]")
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    sa = torch.empty((T * k,), dtype=torch.int32, device=dev)
    need = moe_route_workspace_bytes(T, E, k)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _require_workspace(workspace, need)
    _dev(logits, workspace)
    _check(lib().moe_route(_ptr(logits), T, E, k, _ptr(ids), _ptr(w), _ptr(off), _ptr(sa),
                           _ptr(workspace), workspace.numel(), _stream(stream)), "moe_route")
    return ids, w, off, sa


# ---------------------------------------------------------------- gemm ---

def mx_gemm_workspace_bytes(M: int, N: int, K: int, act: str, w_fmt: str) -> int:
    return lib().mx_gemm_workspace_bytes(M, N, K, ACTS[act], MX_FORMATS[w_fmt])


def mx_gemm(a: torch.Tensor, w: torch.Tensor, w_scale: torch.Tensor, fmt: str, act: str = "mxfp8",
            a_scale: torch.Tensor | None = None, alpha: float = 1.0, c: torch.Tensor | None = None,
            workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """C [M, N] bf16 = alpha * A W^T over MX weights w [N, K*b/8] + w_scale
    [N, K/32].  a: [M, K] bf16 (act "bf16", or "mxfp8" quantized on the
    device), or E4M3 codes [M, K] uint8 with a_scale [M, K/32] (act "mxfp8")."""
    if fmt not in ("e2m1", "e3m2"):
        raise ValueError(f"weight format {fmt!r} is not e2m1 or e3m2")
    if act not in ACTS:
        raise ValueError(f"unknown activation precision {act!r}")
    if a.dim() != 2 or w.dim() != 2:
        raise ValueError("a and w must be 2-D")
    M, K = a.shape
    N = w.shape[0]
    b = FORMAT_BITS[fmt]
    if a_scale is None:
        _require(a, "a", torch.bfloat16, (M, K))
    else:
        if act != "mxfp8":
            raise ValueError("a_scale goes with act='mxfp8'")
        _require(a, "a", torch.uint8, (M, K))
        _require(a_scale, "a_scale", torch.uint8, (M, K // 32))
    _require(w, "w", torch.uint8, (N, K * b // 8))
    _require(w_scale, "w_scale", torch.uint8, (N, K // 32))
    if c is None:
        c = torch.empty((M, N), dtype=torch.bfloat16, device=a.device)
    _require(c, "c", torch.bfloat16, (M, N))
    # MXFP8 from bf16: the quantized A; bf16 with few rows: the K split's partial sums
    need = mx_gemm_workspace_bytes(M, N, K, act, fmt) if a_scale is None else 0
    if workspace is None and need:
        workspace = torch.empty((need,), dtype=torch.uint8, device=a.device)
    if workspace is not None:
        _require_workspace(workspace, need)
    _dev(a, a_scale, w, w_scale, c, workspace)
    _check(lib().mx_gemm(_ptr(a), _ptr(a_scale), M, N, K, ACTS[act], _ptr(w), _ptr(w_scale), MX_FORMATS[fmt],
                         alpha, _ptr(c), _ptr(workspace), 0 if workspace is None else workspace.numel(),
                         _stream(stream)), "mx_gemm")
    return c


# ---------------------------------------------------------------- fused --

@dataclass
class MoeWeights:
    """Packed MX weights of the local experts (canonical layout, device tensors)."""
    w1: torch.Tensor          # [L, 2I, H*b/8] uint8
    w1_scale: torch.Tensor    # [L, 2I, H/32] uint8
    w2: torch.Tensor          # [L, H, I*b/8] uint8
    w2_scale: torch.Tensor    # [L, H, I/32] uint8
    fmt: str                  # "e2m1" | "e3m2"
    ws1: torch.Tensor | None = None
    ws1_scale: torch.Tensor | None = None
    ws2: torch.Tensor | None = None
    ws2_scale: torch.Tensor | None = None


FLAG_FUSED_SMALL_BATCH = 1  # MOE_FLAG_FUSED_SMALL_BATCH


def make_problem(T, H, I, E, k, fmt, act, I_shared=0, shared_weight=1.0, local_offset=0, local_count=0,
                 act_fn="silu", fused_small_batch=False):
    return MoeProblem(T, H, I, E, k, MX_FORMATS[fmt], ACTS[act], I_shared, shared_weight,
                      local_offset, local_count, ACT_FNS[act_fn],
                      FLAG_FUSED_SMALL_BATCH if fused_small_batch else 0)


def moe_fused_workspace_bytes(problem: MoeProblem) -> int:
    return lib().moe_fused_workspace_bytes(ctypes.byref(problem))


WS_PARTS = {"expert_offsets": 0, "sorted_assign": 1, "h": 2, "h_scale": 3}


def moe_fused_workspace_offset(problem: MoeProblem, part: str):
    """Byte offset of an intermediate of moe_fused in its workspace, or None."""
    off = lib().moe_fused_workspace_offset(ctypes.byref(problem), WS_PARTS[part])
    return None if off == ctypes.c_size_t(-1).value else off


_FMT_NAMES = {v: k for k, v in MX_FORMATS.items()}


def check_fused_args(problem: MoeProblem, x, weights, router_logits=None, topk_ids_in=None,
                     topk_w_in=None, y=None, workspace=None, topk_ids_out=None, topk_w_out=None):
    """Every tensor of a moe_fused call against the problem: dtype, exact shape,
    contiguity, one GPU.  Raises ValueError before anything reaches the ABI."""
    p = problem
    T, H, I, E, k, Is = p.T, p.H, p.I, p.E, p.k, p.I_shared
    if p.w_fmt not in _FMT_NAMES or _FMT_NAMES[p.w_fmt] not in ("e2m1", "e3m2"):
        raise ValueError(f"problem: weight format code {p.w_fmt} is not e2m1 or e3m2")
    if weights.fmt != _FMT_NAMES[p.w_fmt]:
        raise ValueError(f"weights are {weights.fmt}, the problem says {_FMT_NAMES[p.w_fmt]}")
    if min(T, H, I, E, k, Is) < 0 or H == 0 or I == 0 or E == 0 or k == 0:
        raise ValueError("problem: negative or zero size")
    if H % 32 or I % 32 or Is % 32:
        raise ValueError("problem: H, I and I_shared must be multiples of 32")
    L = p.local_num_experts or E
    b = FORMAT_BITS[weights.fmt]
    _require(x, "x", torch.bfloat16, (T, H))
    _require(y, "y", torch.bfloat16, (T, H))
    if (topk_ids_in is None) != (topk_w_in is None):
        raise ValueError("topk_ids_in and topk_w_in go together")
    if topk_ids_in is None:
        if router_logits is None:
            raise ValueError("need router_logits or a precomputed top-k")
        _require(router_logits, "router_logits", torch.float32, (T, E))
    else:
        _require(topk_ids_in, "topk_ids_in", torch.int32, (T, k))
        _require(topk_w_in, "topk_w_in", torch.float32, (T, k))
        if router_logits is not None:
            _require(router_logits, "router_logits", torch.float32, (T, E))
    _require(weights.w1, "w1", torch.uint8, (L, 2 * I, H * b // 8))
    _require(weights.w1_scale, "w1_scale", torch.uint8, (L, 2 * I, H // 32))
    _require(weights.w2, "w2", torch.uint8, (L, H, I * b // 8))
    _require(weights.w2_scale, "w2_scale", torch.uint8, (L, H, I // 32))
    shared = (weights.ws1, weights.ws1_scale, weights.ws2, weights.ws2_scale)
    if Is > 0:
        _require(weights.ws1, "ws1", torch.uint8, (2 * Is, H * b // 8))
        _require(weights.ws1_scale, "ws1_scale", torch.uint8, (2 * Is, H // 32))
        _require(weights.ws2, "ws2", torch.uint8, (H, Is * b // 8))
        _require(weights.ws2_scale, "ws2_scale", torch.uint8, (H, Is // 32))
    else:
        shared = ()
    if topk_ids_out is not None:
        _require(topk_ids_out, "topk_ids_out", torch.int32, (T, k))
    if topk_w_out is not None:
        _require(topk_w_out, "topk_w_out", torch.float32, (T, k))
    if workspace is not None:
        _require_workspace(workspace, moe_fused_workspace_bytes(p))
    _dev(x, y, router_logits, topk_ids_in, topk_w_in, weights.w1, weights.w1_scale, weights.w2,
         weights.w2_scale, *shared, topk_ids_out, topk_w_out, workspace)


def moe_fused(problem: MoeProblem, x: torch.Tensor, weights: MoeWeights, router_logits=None,
              topk_ids_in=None, topk_w_in=None, y=None, workspace=None, topk_ids_out=None,
              topk_w_out=None, stream=None, stage_events=None):
    """Run the whole layer; returns y [T, H] bf16.

    stage_events: optional ctypes array of MOE_NUM_STAGES + 1 hipEvent_t
    handles (see HipEvents) recorded at the stage boundaries."""
    if y is None:
        y = torch.empty((problem.T, problem.H), dtype=torch.bfloat16, device=x.device)
    need = moe_fused_workspace_bytes(problem)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
    check_fused_args(problem, x, weights, router_logits, topk_ids_in, topk_w_in, y, workspace,
                     topk_ids_out, topk_w_out)
    t = MoeTensors(*(None if v is None else v.data_ptr() for v in (
        x, router_logits, topk_ids_in, topk_w_in, weights.w1, weights.w1_scale, weights.w2,
        weights.w2_scale, weights.ws1, weights.ws1_scale, weights.ws2, weights.ws2_scale, y,
        topk_ids_out, topk_w_out)), None)
    if stage_events is not None:
        t.stage_events = ctypes.cast(stage_events, ctypes.c_void_p)
    _check(lib().moe_fused(ctypes.byref(problem), ctypes.byref(t), _ptr(workspace), workspace.numel(),
                           _stream(stream)), "moe_fused")
    return y


class FusedCall:
    """moe_fused with its arguments checked and marshalled once, for loops
    that call the layer many times on the same buffers (their contents may
    change between calls): each call then costs the host only the C call
    itself.  The stream is the current one at each call unless one is given.
    Calling returns y."""

    def __init__(self, problem: MoeProblem, x: torch.Tensor, weights: MoeWeights, router_logits=None,
                 topk_ids_in=None, topk_w_in=None, y=None, workspace=None, topk_ids_out=None,
                 topk_w_out=None, stream=None):
        if y is None:
            y = torch.empty((problem.T, problem.H), dtype=torch.bfloat16, device=x.device)
        need = moe_fused_workspace_bytes(problem)
        if workspace is None:
            workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=x.device)
        check_fused_args(problem, x, weights, router_logits, topk_ids_in, topk_w_in, y, workspace,
                         topk_ids_out, topk_w_out)
        self.y = y
        # the tensors stay referenced for as long as the call can run
        self._keep = (problem, x, weights, router_logits, topk_ids_in, topk_w_in, workspace, topk_ids_out,
                      topk_w_out)
        self._t = MoeTensors(*(None if v is None else v.data_ptr() for v in (
            x, router_logits, topk_ids_in, topk_w_in, weights.w1, weights.w1_scale, weights.w2,
            weights.w2_scale, weights.ws1, weights.ws1_scale, weights.ws2, weights.ws2_scale, y,
            topk_ids_out, topk_w_out)), None)
        self._p = ctypes.byref(problem)
        self._tp = ctypes.byref(self._t)
        self._ws = _ptr(workspace)
        self._wsn = workspace.numel()
        self._stream = None if stream is None else _stream(stream)
        self._fn = lib().moe_fused

    def __call__(self, stage_events=None):
        self._t.stage_events = None if stage_events is None else ctypes.cast(stage_events, ctypes.c_void_p)
        st = self._stream if self._stream is not None else _stream(None)
        status = self._fn(self._p, self._tp, self._ws, self._wsn, st)
        if status != MOE_OK:
            raise MoeError(status, "moe_fused")
        return self.y


def moe_fused_noalloc(problem: MoeProblem, x: torch.Tensor, weights: MoeWeights, y: torch.Tensor,
                      router_logits=None, topk_ids_in=None, topk_w_in=None, topk_ids_out=None,
                      topk_w_out=None, stream=None):
    """The whole layer into the caller's y, with the library's static scratch
    as workspace: nothing is allocated (y must be given)."""
    if problem.T > 0:
        check_fused_args(problem, x, weights, router_logits, topk_ids_in, topk_w_in, y, None,
                         topk_ids_out, topk_w_out)
    t = MoeTensors(*(None if v is None else v.data_ptr() for v in (
        x, router_logits, topk_ids_in, topk_w_in, weights.w1, weights.w1_scale, weights.w2,
        weights.w2_scale, weights.ws1, weights.ws1_scale, weights.ws2, weights.ws2_scale, y,
        topk_ids_out, topk_w_out)), None)
    _check(lib().moe_fused_noalloc(ctypes.byref(problem), ctypes.byref(t), _stream(stream)), "moe_fused_noalloc")
    return y


# ------------------------------------------------------------ HIP events --

class HipEvents:
    """A set of HIP events created with the HIP runtime that torch loaded (the
    library links the same one), for timing work on a given stream."""

    def __init__(self, n: int):
        self._hip = ctypes.CDLL("libamdhip64.so.7")
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                   ctypes.c_void_p]
        self.handles = (ctypes.c_void_p * n)()
        for i in range(n):
            r = self._hip.hipEventCreate(ctypes.byref(self.handles, i * ctypes.sizeof(ctypes.c_void_p)))
            if r != 0:
                raise RuntimeError(f"hipEventCreate failed ({r})")

    def record(self, i: int, stream=None):
        r = self._hip.hipEventRecord(ctypes.c_void_p(self.handles[i]), _stream(stream))
        if r != 0:
            raise RuntimeError(f"hipEventRecord failed ({r})")

    def elapsed_ms(self, i: int, j: int) -> float:
        ms = ctypes.c_float()
        r = self._hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.handles[i]),
                                          ctypes.c_void_p(self.handles[j]))
        if r != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({r})")
        return ms.value

    def __del__(self):
        try:
            for h in self.handles:
                if h:
                    self._hip.hipEventDestroy(ctypes.c_void_p(h))
        except Exception:
            pass
