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

# Every symbol include/moe_mx.h declares.
EXPORTS = ("mx_quantize", "moe_route_workspace_bytes", "moe_route", "moe_fused_workspace_bytes",
           "moe_fused", "moe_status_str", "moe_mx_version")


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} (status {status})")


class MoeProblem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("k", ctypes.c_int32), ("w_fmt", ctypes.c_int),
                ("act", ctypes.c_int), ("I_shared", ctypes.c_int32), ("shared_weight", ctypes.c_float),
                ("local_expert_offset", ctypes.c_int32), ("local_num_experts", ctypes.c_int32)]


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
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("tensors must live on the GPU")


# ------------------------------------------------------------ mx_quantize --

def mx_quantize(src: torch.Tensor, fmt: str, codes: torch.Tensor | None = None,
                scales: torch.Tensor | None = None, stream=None):
    """Block-quantize the last axis of a bf16/fp32 matrix [rows, cols] (or a
    batch [..., rows, cols], flattened) to MX codes + E8M0 scales."""
    _dev(src)
    cols = src.shape[-1]
    rows = src.numel() // cols if cols else 0
    if src.stride(-1) != 1:
        raise ValueError("last axis must be contiguous")
    src2 = src.reshape(rows, cols) if src.is_contiguous() else src
    ld = src2.stride(0) if src2.dim() == 2 else cols
    nbytes = cols * FORMAT_BITS[fmt] // 8
    if codes is None:
        codes = torch.empty(src.shape[:-1] + (nbytes,), dtype=torch.uint8, device=src.device)
    if scales is None:
        scales = torch.empty(src.shape[:-1] + (cols // 32,), dtype=torch.uint8, device=src.device)
    _check(lib().mx_quantize(_ptr(src2), SRC_DTYPES[src.dtype], rows, cols, ld, MX_FORMATS[fmt],
                             _ptr(codes), _ptr(scales), _stream(stream)), "mx_quantize")
    return codes, scales


# ---------------------------------------------------------------- route --

def moe_route_workspace_bytes(T: int, E: int, k: int) -> int:
    return lib().moe_route_workspace_bytes(T, E, k)


def moe_route(logits: torch.Tensor, k: int, workspace: torch.Tensor | None = None, stream=None):
    """-> (topk_ids [T,k] int32, topk_w [T,k] fp32, expert_offsets [E+1] int32,
    sorted_assign [T*k] int32)."""
    _dev(logits)
    T, E = logits.shape
    dev = logits.device
    ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    off = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    sa = torch.empty((T * k,), dtype=torch.int32, device=dev)
    need = moe_route_workspace_bytes(T, E, k)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    _check(lib().moe_route(_ptr(logits.contiguous()), T, E, k, _ptr(ids), _ptr(w), _ptr(off), _ptr(sa),
                           _ptr(workspace), workspace.numel(), _stream(stream)), "moe_route")
    return ids, w, off, sa


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


def make_problem(T, H, I, E, k, fmt, act, I_shared=0, shared_weight=1.0, local_offset=0, local_count=0):
    return MoeProblem(T, H, I, E, k, MX_FORMATS[fmt], ACTS[act], I_shared, shared_weight,
                      local_offset, local_count)


def moe_fused_workspace_bytes(problem: MoeProblem) -> int:
    return lib().moe_fused_workspace_bytes(ctypes.byref(problem))


def moe_fused(problem: MoeProblem, x: torch.Tensor, weights: MoeWeights, router_logits=None,
              topk_ids_in=None, topk_w_in=None, y=None, workspace=None, topk_ids_out=None,
              topk_w_out=None, stream=None, stage_events=None):
    """Run the whole layer; returns y [T, H] bf16.

    stage_events: optional ctypes array of MOE_NUM_STAGES + 1 hipEvent_t
    handles (see HipEvents) recorded at the stage boundaries."""
    _dev(x, router_logits, topk_ids_in, topk_w_in, weights.w1, weights.w2)
    if y is None:
        y = torch.empty((problem.T, problem.H), dtype=torch.bfloat16, device=x.device)
    if workspace is None:
        workspace = torch.empty((max(moe_fused_workspace_bytes(problem), 1),), dtype=torch.uint8,
                                device=x.device)
    t = MoeTensors(*(None if v is None else v.data_ptr() for v in (
        x, router_logits, topk_ids_in, topk_w_in, weights.w1, weights.w1_scale, weights.w2,
        weights.w2_scale, weights.ws1, weights.ws1_scale, weights.ws2, weights.ws2_scale, y,
        topk_ids_out, topk_w_out)), None)
    if stage_events is not None:
        t.stage_events = ctypes.cast(stage_events, ctypes.c_void_p)
    _check(lib().moe_fused(ctypes.byref(problem), ctypes.byref(t), _ptr(workspace), workspace.numel(),
                           _stream(stream)), "moe_fused")
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
