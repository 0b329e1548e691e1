"""ctypes binding of libnvfp4moe.so (include/nvfp4moe.h).

Argument marshalling only: torch tensors supply device memory and the current HIP stream, and
every step of the computation runs in the library's HIP kernels. There is no fallback. If the
library is missing, or a tensor is not on the GPU, the call raises.
"""
from __future__ import annotations

import ctypes as C
import os
import re

import torch  # loads torch's HIP runtime first; the library binds to that same runtime (same SONAME)

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libnvfp4moe.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "nvfp4moe.h")

NVFP4_OK = 0
STATUS_NAMES = {0: "NVFP4_OK", 1: "NVFP4_ERR_NULL", 2: "NVFP4_ERR_SHAPE", 3: "NVFP4_ERR_ALIGN",
                4: "NVFP4_ERR_WORKSPACE", 5: "NVFP4_ERR_UNSUPPORTED", 6: "NVFP4_ERR_LAUNCH"}


class NVFP4Error(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {msg} ({status})")
        self.status = status


class nvfp4_weights(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("scales", C.c_void_p), ("global_scale", C.c_void_p),
                ("groups", C.c_int32), ("rows", C.c_int32), ("k", C.c_int32)]


class fp8_channel_weights(C.Structure):
    _fields_ = [("codes", C.c_void_p), ("channel_scale", C.c_void_p), ("rows", C.c_int32), ("k", C.c_int32)]


_LIB = None
_vp, _i32, _sz = C.c_void_p, C.c_int32, C.c_size_t
_SIGS = {
    "nvfp4_abi_version": (C.c_int, []),
    "nvfp4_status_str": (C.c_char_p, [C.c_int]),
    "nvfp4_moe_plan_bytes": (_sz, [_i32, _i32, _i32]),
    "nvfp4_moe_plan": (C.c_int, [_vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "nvfp4_moe_route": (C.c_int, [_vp, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_moe_w13_swiglu": (C.c_int, [_vp, _i32, _i32, _i32, _vp, C.POINTER(nvfp4_weights), _i32, _vp, _vp]),
    "nvfp4_moe_w2_workspace_bytes": (_sz, [_i32, _i32, _i32]),
    "nvfp4_moe_w2_reduce": (C.c_int, [_vp, _i32, _i32, _i32, _vp, C.POINTER(nvfp4_weights), _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_linear": (C.c_int, [_vp, _i32, C.POINTER(nvfp4_weights), _vp, _vp]),
    "nvfp4_moe_shared_expert": (C.c_int, [_vp, _i32, C.POINTER(nvfp4_weights), _i32, C.POINTER(nvfp4_weights), _vp,
                                          _vp, _vp, _vp, _vp]),
    "nvfp4_moe_w2_reduce_shared": (C.c_int, [_vp, _i32, _i32, _i32, _vp, C.POINTER(nvfp4_weights), _vp, _vp, _vp,
                                             _vp, _vp, _sz, _vp]),
    "nvfp4_moe_w13_swiglu_with_shared": (C.c_int, [_vp, _i32, _i32, _i32, _vp, C.POINTER(nvfp4_weights), _i32, _vp,
                                                   C.POINTER(nvfp4_weights), _vp, _vp, _vp, _vp]),
    "nvfp4_moe_plan_w13_swiglu_with_shared": (C.c_int, [_vp, _i32, _i32, _i32, _vp, _sz, _vp,
                                                        C.POINTER(nvfp4_weights), _i32, _vp, C.POINTER(nvfp4_weights),
                                                        _vp, _vp, _vp, _vp]),
    "nvfp4_moe_w2_reduce_with_shared": (C.c_int, [_vp, _i32, _i32, _i32, _vp, C.POINTER(nvfp4_weights), _vp, _vp,
                                                  C.POINTER(nvfp4_weights), _vp, _vp, _vp, _vp, _sz, _vp]),
    "nvfp4_linear_swiglu": (C.c_int, [_vp, _i32, C.POINTER(nvfp4_weights), _i32, _vp, _vp]),
    "nvfp4_linear_ws_bytes": (C.c_size_t, [_i32, _i32, _i32]),
    "nvfp4_linear_ws": (C.c_int, [_vp, _i32, C.POINTER(nvfp4_weights), _vp, _vp, C.c_size_t, _vp]),
    "nvfp4_linear_swiglu_ws": (C.c_int, [_vp, _i32, C.POINTER(nvfp4_weights), _i32, _vp, _vp, C.c_size_t, _vp]),
    "nvfp4_moe_plan_w13_swiglu": (C.c_int, [_vp, _i32, _i32, _i32, _vp, _sz, _vp, C.POINTER(nvfp4_weights), _i32, _vp,
                                            _vp]),
    "nvfp4_linear_fp8": (C.c_int, [_vp, _i32, C.POINTER(fp8_channel_weights), _vp, _vp]),
    "nvfp4_moe_layer_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "nvfp4_moe_layer_noalloc": (C.c_int, [_vp, _i32, _i32, _i32, _vp, C.POINTER(nvfp4_weights), _i32,
                                          C.POINTER(nvfp4_weights), _vp, _vp, _vp]),
    "nvfp4_moe_layer": (C.c_int, [_vp, _i32, _i32, _i32, _vp, C.POINTER(nvfp4_weights), _i32,
                                  C.POINTER(nvfp4_weights), _vp, _vp, _vp, _sz, _vp]),
}


def lib() -> C.CDLL:
    """The loaded library. Raises if it has not been built (python gemm_nvfp4_amd/build.py)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python gemm_nvfp4_amd/build.py` "
                               "(or __graft_entry__.build()); there is no fallback path")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        if L.nvfp4_abi_version() != 1:
            raise RuntimeError(f"libnvfp4moe ABI version {L.nvfp4_abi_version()} != 1")
        _LIB = L
    return _LIB


def header_functions() -> list[str]:
    """Names of the functions declared in include/nvfp4moe.h."""
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(nvfp4_\w+)\s*\(", txt, flags=re.M)))


def _check(fn: str, status: int):
    if status != NVFP4_OK:
        raise NVFP4Error(fn, status, lib().nvfp4_status_str(status).decode())


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (the library has no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


_RAW_STREAM = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device_index: int | None = None) -> int:
    """The HIP stream handle: the given torch stream's, else the current stream of the device
    (device_index, or the current device), read without building a stream object when torch
    offers that."""
    if stream is not None:
        return stream.cuda_stream
    if _RAW_STREAM is not None:
        return _RAW_STREAM(torch.cuda.current_device() if device_index is None else device_index)
    return torch.cuda.current_stream().cuda_stream


def _shape(t: torch.Tensor, name: str, shape: tuple):
    """Raise unless t has exactly this shape (the library reads and writes by these sizes)."""
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows(t: torch.Tensor, name: str, min_rows: int, cols: int):
    """Raise unless t is [>= min_rows, cols] (bucket-order buffers may be longer than needed)."""
    if t.dim() != 2 or t.shape[1] != cols or t.shape[0] < min_rows:
        raise ValueError(f"{name} must have shape [>= {min_rows}, {cols}], got {tuple(t.shape)}")


def _bytes(t: torch.Tensor, name: str, need: int):
    if t.numel() * t.element_size() < need:
        raise ValueError(f"{name} holds {t.numel() * t.element_size()} bytes, {need} needed")


def _plan_ok(plan: torch.Tensor, M: int, topk: int, E: int):
    """The W13/W2 calls take no plan size: check here that the buffer is large enough."""
    _bytes(plan, "plan", nvfp4_moe_plan_bytes(M, topk, E))


class NVFP4Tensor:
    """Device storage of an NVFP4 weight: codes uint8 [G,N,K/2], scales uint8 [G,N,K/16], global
    float32 [G]."""

    def __init__(self, codes: torch.Tensor, scales: torch.Tensor, global_scale: torch.Tensor):
        if codes.dim() != 3 or scales.dim() != 3 or global_scale.dim() != 1:
            raise ValueError("codes/scales must be [G,N,K/2]/[G,N,K/16], global_scale [G]")
        self.codes, self.scales, self.global_scale = codes, scales, global_scale
        self.groups, self.rows, self.k = codes.shape[0], codes.shape[1], codes.shape[2] * 2
        if tuple(scales.shape) != (self.groups, self.rows, self.k // 16) or global_scale.shape[0] != self.groups:
            raise ValueError("inconsistent NVFP4 tensor shapes")

    @classmethod
    def from_numpy(cls, w, device="cuda"):
        codes, scales, gs = w
        return cls(torch.from_numpy(codes).to(device), torch.from_numpy(scales).to(device),
                   torch.from_numpy(gs).to(device))

    def desc(self) -> nvfp4_weights:
        """The C descriptor; built once and reused while codes, scales and global_scale are the same
        tensor objects (their storage must not be reallocated in place)."""
        c = self.__dict__.get("_desc")
        if c is not None and c[0] is self.codes and c[1] is self.scales and c[2] is self.global_scale:
            return c[3]
        d = nvfp4_weights(_dev(self.codes, "codes", torch.uint8), _dev(self.scales, "scales", torch.uint8),
                          _dev(self.global_scale, "global_scale", torch.float32), self.groups, self.rows, self.k)
        self._desc = (self.codes, self.scales, self.global_scale, d)
        return d


def nvfp4_abi_version() -> int:
    return lib().nvfp4_abi_version()


def nvfp4_status_str(status: int) -> str:
    return lib().nvfp4_status_str(int(status)).decode()


def nvfp4_moe_plan_bytes(M: int, topk: int, E: int) -> int:
    return int(lib().nvfp4_moe_plan_bytes(M, topk, E))


def nvfp4_moe_plan(topk_ids: torch.Tensor, E: int, plan: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Build the routing plan of int32 ids [M, topk]; returns the plan buffer (int32 device tensor)."""
    M, topk = topk_ids.shape
    nbytes = nvfp4_moe_plan_bytes(M, topk, E)
    if plan is None:
        plan = torch.empty(max(nbytes, 4) // 4, dtype=torch.int32, device=topk_ids.device)
    _check("nvfp4_moe_plan", lib().nvfp4_moe_plan(_dev(topk_ids, "topk_ids", torch.int32), M, topk, E,
                                                  _dev(plan, "plan", torch.int32), plan.numel() * 4, _stream(stream)))
    return plan


def nvfp4_moe_route(logits: torch.Tensor, topk: int, ids: torch.Tensor | None = None,
                    weights: torch.Tensor | None = None, plan: torch.Tensor | None = None, stream=None):
    """Top-k routing of fp32 logits [M, E] fused with the plan. Returns (ids int32 [M, topk],
    weights fp32 [M, topk], plan)."""
    M, E = logits.shape
    dev = logits.device
    if ids is None:
        ids = torch.empty((M, topk), dtype=torch.int32, device=dev)
    if weights is None:
        weights = torch.empty((M, topk), dtype=torch.float32, device=dev)
    if plan is None:
        plan = torch.empty(max(nvfp4_moe_plan_bytes(M, topk, E), 4) // 4, dtype=torch.int32, device=dev)
    _check("nvfp4_moe_route", lib().nvfp4_moe_route(
        _dev(logits, "logits", torch.float32), M, E, topk, _dev(ids, "ids", torch.int32),
        _dev(weights, "weights", torch.float32), _dev(plan, "plan", torch.int32), plan.numel() * 4, _stream(stream)))
    return ids, weights, plan


def nvfp4_moe_w13_swiglu(plan: torch.Tensor, M: int, topk: int, E: int, x: torch.Tensor, w13: NVFP4Tensor,
                         layout: int = 0, h: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Grouped W13 + SwiGLU. Returns h fp16 [M*topk, I] in bucket order (rows >= n_valid untouched)."""
    I = w13.rows // 2
    _shape(x, "x", (M, w13.k))
    _plan_ok(plan, M, topk, E)
    if h is None:
        h = torch.empty((M * topk, I), dtype=torch.float16, device=x.device)
    _rows(h, "h", M * topk, I)
    d = w13.desc()
    _check("nvfp4_moe_w13_swiglu", lib().nvfp4_moe_w13_swiglu(
        _dev(plan, "plan", torch.int32), M, topk, E, _dev(x, "x", torch.float16), C.byref(d), layout,
        _dev(h, "h", torch.float16), _stream(stream)))
    return h


def nvfp4_moe_plan_w13_swiglu(topk_ids: torch.Tensor, E: int, x: torch.Tensor, w13: NVFP4Tensor, layout: int = 0,
                              plan: torch.Tensor | None = None, h: torch.Tensor | None = None, stream=None):
    """nvfp4_moe_plan followed by nvfp4_moe_w13_swiglu, one launch for small batches. Returns (plan, h)."""
    M, topk = topk_ids.shape
    I = w13.rows // 2
    _shape(x, "x", (M, w13.k))
    if plan is None:
        plan = torch.empty(max(nvfp4_moe_plan_bytes(M, topk, E), 4) // 4, dtype=torch.int32, device=x.device)
    if h is None:
        h = torch.empty((M * topk, I), dtype=torch.float16, device=x.device)
    _rows(h, "h", M * topk, I)
    d = w13.desc()
    _check("nvfp4_moe_plan_w13_swiglu", lib().nvfp4_moe_plan_w13_swiglu(
        _dev(topk_ids, "topk_ids", torch.int32), M, topk, E, _dev(plan, "plan", torch.int32), plan.numel() * 4,
        _dev(x, "x", torch.float16), C.byref(d), layout, _dev(h, "h", torch.float16), _stream(stream)))
    return plan, h


def nvfp4_moe_w2_workspace_bytes(M: int, topk: int, K: int) -> int:
    return int(lib().nvfp4_moe_w2_workspace_bytes(M, topk, K))


def nvfp4_moe_w2_reduce(plan: torch.Tensor, M: int, topk: int, E: int, h: torch.Tensor, w2: NVFP4Tensor,
                        topk_weights: torch.Tensor, out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Grouped W2 + slot-ordered top-k weighted reduction. Returns out fp16 [M, K]."""
    K = w2.rows
    _plan_ok(plan, M, topk, E)
    _rows(h, "h", M * topk, w2.k)
    _shape(topk_weights, "topk_weights", (M, topk))
    if out is None:
        out = torch.empty((M, K), dtype=torch.float16, device=h.device)
    _shape(out, "out", (M, K))
    if ws is None:
        ws = torch.empty(max(nvfp4_moe_w2_workspace_bytes(M, topk, K), 4), dtype=torch.uint8, device=h.device)
    d = w2.desc()
    _check("nvfp4_moe_w2_reduce", lib().nvfp4_moe_w2_reduce(
        _dev(plan, "plan", torch.int32), M, topk, E, _dev(h, "h", torch.float16), C.byref(d),
        _dev(topk_weights, "topk_weights", torch.float32), _dev(out, "out", torch.float16),
        _dev(ws, "ws", ws.dtype), ws.numel() * ws.element_size(), _stream(stream)))
    return out


def nvfp4_moe_shared_expert(x: torch.Tensor, w13: NVFP4Tensor, w2: NVFP4Tensor, gate: torch.Tensor, layout: int = 0,
                            h: torch.Tensor | None = None, shared_y: torch.Tensor | None = None,
                            shared_sigma: torch.Tensor | None = None, stream=None):
    """Shared expert on fp16 x [M, K]: returns (shared_y FP32 [M, K], shared_sigma FP32 [M], h fp16 [M, I])."""
    M, K = x.shape
    I = w13.rows // 2
    dev = x.device
    _shape(gate, "gate", (K,))
    h = torch.empty((M, I), dtype=torch.float16, device=dev) if h is None else h
    shared_y = torch.empty((M, K), dtype=torch.float32, device=dev) if shared_y is None else shared_y
    shared_sigma = torch.empty((M,), dtype=torch.float32, device=dev) if shared_sigma is None else shared_sigma
    _shape(h, "h", (M, I))
    _shape(shared_y, "shared_y", (M, K))
    _shape(shared_sigma, "shared_sigma", (M,))
    d13, d2 = w13.desc(), w2.desc()
    _check("nvfp4_moe_shared_expert", lib().nvfp4_moe_shared_expert(
        _dev(x, "x", torch.float16), M, C.byref(d13), layout, C.byref(d2), _dev(gate, "gate", torch.float16),
        _dev(h, "h", torch.float16), _dev(shared_y, "shared_y", torch.float32),
        _dev(shared_sigma, "shared_sigma", torch.float32), _stream(stream)))
    return shared_y, shared_sigma, h


def nvfp4_moe_w2_reduce_shared(plan: torch.Tensor, M: int, topk: int, E: int, h: torch.Tensor, w2: NVFP4Tensor,
                               topk_weights: torch.Tensor, shared_y: torch.Tensor, shared_sigma: torch.Tensor,
                               out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                               stream=None) -> torch.Tensor:
    """Grouped W2 + slot-order reduction with the shared expert added last. Returns out fp16 [M, K]."""
    K = w2.rows
    dev = h.device
    _plan_ok(plan, M, topk, E)
    _rows(h, "h", M * topk, w2.k)
    _shape(topk_weights, "topk_weights", (M, topk))
    _shape(shared_y, "shared_y", (M, K))
    _shape(shared_sigma, "shared_sigma", (M,))
    out = torch.empty((M, K), dtype=torch.float16, device=dev) if out is None else out
    _shape(out, "out", (M, K))
    if ws is None:
        ws = torch.empty(max(nvfp4_moe_w2_workspace_bytes(M, topk, K), 256), dtype=torch.uint8, device=dev)
    d = w2.desc()
    _check("nvfp4_moe_w2_reduce_shared", lib().nvfp4_moe_w2_reduce_shared(
        _dev(plan, "plan", torch.int32), M, topk, E, _dev(h, "h", torch.float16), C.byref(d),
        _dev(topk_weights, "topk_weights", torch.float32), _dev(shared_y, "shared_y", torch.float32),
        _dev(shared_sigma, "shared_sigma", torch.float32), _dev(out, "out", torch.float16), ws.data_ptr(), ws.numel(),
        _stream(stream)))
    return out


def nvfp4_linear(x: torch.Tensor, w: NVFP4Tensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Dense NVFP4 projection y = x W^T. x fp16 [M, K]; returns fp16 [M, N]."""
    M = x.shape[0]
    _shape(x, "x", (M, w.k))
    if y is None:
        y = torch.empty((M, w.rows), dtype=torch.float16, device=x.device)
    _shape(y, "y", (M, w.rows))
    d = w.desc()
    _check("nvfp4_linear", lib().nvfp4_linear(_dev(x, "x", torch.float16), M, C.byref(d),
                                              _dev(y, "y", torch.float16), _stream(stream)))
    return y


class FP8ChannelTensor:
    """Device storage of a channel-FP8 weight: E4M3FN bytes uint8 [N, K] and float32 scales [N]."""

    def __init__(self, codes: torch.Tensor, channel_scale: torch.Tensor):
        if codes.dim() != 2 or channel_scale.dim() != 1 or channel_scale.shape[0] != codes.shape[0]:
            raise ValueError("codes must be [N, K] and channel_scale [N]")
        self.codes, self.channel_scale = codes, channel_scale
        self.rows, self.k = codes.shape

    @classmethod
    def from_numpy(cls, w, device="cuda"):
        codes, scale = w
        return cls(torch.from_numpy(codes).to(device), torch.from_numpy(scale).to(device))

    def desc(self) -> fp8_channel_weights:
        return fp8_channel_weights(_dev(self.codes, "codes", torch.uint8),
                                   _dev(self.channel_scale, "channel_scale", torch.float32), self.rows, self.k)


def nvfp4_linear_fp8(x: torch.Tensor, w: FP8ChannelTensor, y: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Channel-FP8 dense projection y = fp16(s * (x @ e4m3(W)^T)) of fp16 x [M, K]; returns y [M, N]."""
    M = x.shape[0]
    _shape(x, "x", (M, w.k))
    if y is None:
        y = torch.empty((M, w.rows), dtype=torch.float16, device=x.device)
    _shape(y, "y", (M, w.rows))
    d = w.desc()
    _check("nvfp4_linear_fp8", lib().nvfp4_linear_fp8(_dev(x, "x", torch.float16), M, C.byref(d),
                                                      _dev(y, "y", torch.float16), _stream(stream)))
    return y


def nvfp4_linear_swiglu(x: torch.Tensor, w13: NVFP4Tensor, layout: int = 0, h: torch.Tensor | None = None,
                        stream=None) -> torch.Tensor:
    """Gated dense projection h = fp16(silu(x Wg^T) * (x Wu^T)) of fp16 x [M, K]; returns h [M, I]."""
    M = x.shape[0]
    I = w13.rows // 2
    _shape(x, "x", (M, w13.k))
    if h is None:
        h = torch.empty((M, I), dtype=torch.float16, device=x.device)
    _shape(h, "h", (M, I))
    d = w13.desc()
    _check("nvfp4_linear_swiglu", lib().nvfp4_linear_swiglu(_dev(x, "x", torch.float16), M, C.byref(d), layout,
                                                            _dev(h, "h", torch.float16), _stream(stream)))
    return h


def nvfp4_linear_ws_bytes(M: int, N: int, K: int) -> int:
    return int(lib().nvfp4_linear_ws_bytes(M, N, K))


def _split_ws(ws, M, w, dev):
    need = nvfp4_linear_ws_bytes(M, w.rows, w.k)
    if ws is None:
        return torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    if ws.numel() * ws.element_size() < need:
        raise ValueError(f"ws holds {ws.numel() * ws.element_size()} bytes, the call needs {need}")
    return ws


def nvfp4_linear_ws(x: torch.Tensor, w: NVFP4Tensor, y: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                    stream=None) -> torch.Tensor:
    """Split-K form of nvfp4_linear (bitwise the same y); ws: nvfp4_linear_ws_bytes(M, N, K) bytes."""
    M = x.shape[0]
    _shape(x, "x", (M, w.k))
    if y is None:
        y = torch.empty((M, w.rows), dtype=torch.float16, device=x.device)
    _shape(y, "y", (M, w.rows))
    ws = _split_ws(ws, M, w, x.device)
    d = w.desc()
    _check("nvfp4_linear_ws", lib().nvfp4_linear_ws(_dev(x, "x", torch.float16), M, C.byref(d),
                                                    _dev(y, "y", torch.float16), ws.data_ptr(),
                                                    ws.numel() * ws.element_size(), _stream(stream)))
    return y


def nvfp4_linear_swiglu_ws(x: torch.Tensor, w13: NVFP4Tensor, layout: int = 0, h: torch.Tensor | None = None,
                           ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Split-K form of nvfp4_linear_swiglu (bitwise the same h); ws: nvfp4_linear_ws_bytes(M, 2I, K) bytes."""
    M = x.shape[0]
    I = w13.rows // 2
    _shape(x, "x", (M, w13.k))
    if h is None:
        h = torch.empty((M, I), dtype=torch.float16, device=x.device)
    _shape(h, "h", (M, I))
    ws = _split_ws(ws, M, w13, x.device)
    d = w13.desc()
    _check("nvfp4_linear_swiglu_ws", lib().nvfp4_linear_swiglu_ws(
        _dev(x, "x", torch.float16), M, C.byref(d), layout, _dev(h, "h", torch.float16), ws.data_ptr(),
        ws.numel() * ws.element_size(), _stream(stream)))
    return h


def nvfp4_moe_layer_workspace_bytes(M: int, topk: int, E: int, K: int, I: int) -> int:
    return int(lib().nvfp4_moe_layer_workspace_bytes(M, topk, E, K, I))


def layer_h_pair_order(M: int, topk: int, E: int) -> bool:
    """Whether nvfp4_moe_layer leaves h in pair order (row p = t*topk + k) instead of bucket order:
    the pair-major small-batch path of nvfp4moe.h (4*M*topk <= E, M*topk <= 256, E <= 1024)."""
    P = M * topk
    return 4 * P <= E and P <= 256 and E <= 1024


def layer_workspace_parts(M: int, topk: int, E: int, I: int) -> tuple[int, int]:
    """Byte offsets of h and of the W2 workspace inside the layer workspace (the plan is at 0)."""
    h_off = nvfp4_moe_plan_bytes(M, topk, E)
    return h_off, h_off + (M * topk * I * 2 + 255) // 256 * 256


def nvfp4_moe_layer(topk_ids: torch.Tensor, E: int, x: torch.Tensor, w13: NVFP4Tensor, w2: NVFP4Tensor,
                    topk_weights: torch.Tensor, layout: int = 0, out: torch.Tensor | None = None,
                    ws: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """The whole MoE layer (plan, W13 + SwiGLU, W2 + slot-order reduction) in one library call.
    Returns out fp16 [M, K]; ws (uint8) then holds the plan, h and the W2 workspace."""
    M, topk = topk_ids.shape
    K, I = w13.k, w13.rows // 2
    _shape(x, "x", (M, K))
    _shape(topk_weights, "topk_weights", (M, topk))
    if out is None:
        out = torch.empty((M, K), dtype=torch.float16, device=x.device)
    _shape(out, "out", (M, K))
    need = nvfp4_moe_layer_workspace_bytes(M, topk, E, K, I)
    if ws is None:
        ws = torch.empty(max(need, 256), dtype=torch.uint8, device=x.device)
    _bytes(ws, "ws", need)
    d13, d2 = w13.desc(), w2.desc()
    _check("nvfp4_moe_layer", lib().nvfp4_moe_layer(
        _dev(topk_ids, "topk_ids", torch.int32), M, topk, E, _dev(x, "x", torch.float16), C.byref(d13), layout,
        C.byref(d2), _dev(topk_weights, "topk_weights", torch.float32), _dev(out, "out", torch.float16),
        _dev(ws, "ws", torch.uint8), ws.numel(), _stream(stream)))
    return out


NOALLOC_SCRATCH_BYTES = 8 << 20  # NVFP4_NOALLOC_SCRATCH_BYTES of nvfp4moe.h


def nvfp4_moe_layer_noalloc(topk_ids: torch.Tensor, E: int, x: torch.Tensor, w13: NVFP4Tensor, w2: NVFP4Tensor,
                            topk_weights: torch.Tensor, out: torch.Tensor, layout: int = 0, stream=None) -> torch.Tensor:
    """nvfp4_moe_layer with the library's static device scratch array as its workspace: the call
    allocates nothing (out is the caller's). Calls that overlap on one GPU race."""
    M, topk = topk_ids.shape
    K = w13.k
    _shape(x, "x", (M, K))
    _shape(topk_weights, "topk_weights", (M, topk))
    _shape(out, "out", (M, K))
    d13, d2 = w13.desc(), w2.desc()
    _check("nvfp4_moe_layer_noalloc", lib().nvfp4_moe_layer_noalloc(
        _dev(topk_ids, "topk_ids", torch.int32), M, topk, E, _dev(x, "x", torch.float16), C.byref(d13), layout,
        C.byref(d2), _dev(topk_weights, "topk_weights", torch.float32), _dev(out, "out", torch.float16),
        _stream(stream)))
    return out


class MoELayer:
    """One MoE layer call (nvfp4_moe_layer: plan + W13+SwiGLU, then W2+reduce) with its buffers
    allocated once, so the call can be replayed (or captured in a HIP graph) without allocation.
    plan, h and ws are views into the one layer workspace (h in pair order where layer_h_pair_order
    holds, else in bucket order)."""

    def __init__(self, M: int, topk: int, w13: NVFP4Tensor, w2: NVFP4Tensor, layout: int = 0, device="cuda"):
        self.M, self.topk, self.E = M, topk, w13.groups
        self.K, self.I = w13.k, w13.rows // 2
        if w2.groups != self.E or w2.rows != self.K or w2.k != self.I:
            raise ValueError("w2 must be [E, K, I] for w13 [E, 2I, K]")
        self.w13, self.w2, self.layout = w13, w2, layout
        need = nvfp4_moe_layer_workspace_bytes(M, topk, self.E, self.K, self.I)
        self.workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=device)
        h_off, w2_off = layer_workspace_parts(M, topk, self.E, self.I)
        self.plan = self.workspace[:h_off].view(torch.int32)
        self.h = self.workspace[h_off:h_off + M * topk * self.I * 2].view(torch.float16).view(M * topk, self.I)
        self.ws = self.workspace[w2_off:]
        self.out = torch.empty((M, self.K), dtype=torch.float16, device=device)
        self._fast = None

    def _same(self, w: NVFP4Tensor, ref: NVFP4Tensor, name: str):
        if (w.groups, w.rows, w.k) != (ref.groups, ref.rows, ref.k):
            raise ValueError(f"{name} override must have the layer's shape {(ref.groups, ref.rows, ref.k)}")

    def __call__(self, x, topk_ids, topk_weights, w13: NVFP4Tensor | None = None, w2: NVFP4Tensor | None = None,
                 stream=None):
        # The same checks as nvfp4_moe_layer, with the fixed arguments (descriptors of the layer's
        # weights, workspace and output pointers, the C function) resolved once: an eager call
        # spends little host time before its first launch.
        if w13 is not None and w13 is not self.w13:
            self._same(w13, self.w13, "w13")
        if w2 is not None and w2 is not self.w2:
            self._same(w2, self.w2, "w2")
        f = self._fast
        if f is None:
            f = self._fast = (lib().nvfp4_moe_layer, self.out.data_ptr(), self.workspace.data_ptr(),
                              self.workspace.numel(), self.out.device.index)
        args = ((topk_ids, "topk_ids", (self.M, self.topk), torch.int32), (x, "x", (self.M, self.K), torch.float16),
                (topk_weights, "topk_weights", (self.M, self.topk), torch.float32))
        for t, name, shape, _ in args:  # every shape before any device check, as nvfp4_moe_layer
            if t.shape != shape:
                _shape(t, name, shape)
        for t, name, _, dtype in args:
            _dev(t, name, dtype)
        d13 = (w13 or self.w13).desc()
        d2 = (w2 or self.w2).desc()
        _check("nvfp4_moe_layer", f[0](topk_ids.data_ptr(), self.M, self.topk, self.E, x.data_ptr(), C.byref(d13),
                                       self.layout, C.byref(d2), topk_weights.data_ptr(), f[1], f[2], f[3],
                                       _stream(stream, f[4])))
        return self.out


def plan_fields(plan: torch.Tensor, M: int, topk: int, E: int) -> dict:
    """Slice a plan buffer (copied to the host) into its documented arrays (layout of nvfp4moe.h)."""
    p = plan.cpu().numpy()
    P = M * topk
    A = min(E, P)
    T = A + (P + 15) // 16
    o = 16
    f = {}
    for name, n in (("counts", E), ("offsets", E + 1), ("active", A), ("tile_expert", T), ("tile_row0", T),
                    ("tile_base", T), ("tile_rows", T), ("tile_pair", T * 16), ("sorted_pair", P), ("pos_of_pair", P),
                    ("pair_expert", P)):
        f[name] = p[o:o + n]
        o += n
    f["tile_pair"] = f["tile_pair"].reshape(T, 16)
    nv, na, nb, nt = (int(v) for v in p[0:4])
    f.update(n_valid=nv, n_active=na, n_bad=nb, n_tiles=nt, hdr=p[:16])
    f["sorted_pair"] = f["sorted_pair"][:nv]
    f["active"] = f["active"][:na]
    f["tile_expert"] = f["tile_expert"][:nt]
    f["tile_row0"] = f["tile_row0"][:nt]
    f["tile_base"] = f["tile_base"][:nt]
    f["tile_rows"] = f["tile_rows"][:nt]
    f["tile_pair"] = f["tile_pair"][:nt]
    return f


def nvfp4_moe_w13_swiglu_with_shared(plan: torch.Tensor, M: int, topk: int, E: int, x: torch.Tensor,
                                     w13: NVFP4Tensor, shared_w13: NVFP4Tensor, gate: torch.Tensor, layout: int = 0,
                                     h: torch.Tensor | None = None, shared_h: torch.Tensor | None = None,
                                     shared_sigma: torch.Tensor | None = None, stream=None):
    """Grouped W13 + SwiGLU with the shared expert's gate/up and its gate in the same launch.
    Returns (h fp16 [M*topk, I] in bucket order, shared_h fp16 [M, Is], shared_sigma FP32 [M])."""
    I, Is = w13.rows // 2, shared_w13.rows // 2
    dev = x.device
    _shape(x, "x", (M, w13.k))
    _shape(gate, "gate", (w13.k,))
    _plan_ok(plan, M, topk, E)
    h = torch.empty((M * topk, I), dtype=torch.float16, device=dev) if h is None else h
    shared_h = torch.empty((M, Is), dtype=torch.float16, device=dev) if shared_h is None else shared_h
    shared_sigma = torch.empty((M,), dtype=torch.float32, device=dev) if shared_sigma is None else shared_sigma
    _rows(h, "h", M * topk, I)
    _shape(shared_h, "shared_h", (M, Is))
    _shape(shared_sigma, "shared_sigma", (M,))
    d, ds = w13.desc(), shared_w13.desc()
    _check("nvfp4_moe_w13_swiglu_with_shared", lib().nvfp4_moe_w13_swiglu_with_shared(
        _dev(plan, "plan", torch.int32), M, topk, E, _dev(x, "x", torch.float16), C.byref(d), layout,
        _dev(h, "h", torch.float16), C.byref(ds), _dev(gate, "gate", torch.float16),
        _dev(shared_h, "shared_h", torch.float16), _dev(shared_sigma, "shared_sigma", torch.float32),
        _stream(stream)))
    return h, shared_h, shared_sigma


def nvfp4_moe_plan_w13_swiglu_with_shared(topk_ids: torch.Tensor, E: int, x: torch.Tensor, w13: NVFP4Tensor,
                                          shared_w13: NVFP4Tensor, gate: torch.Tensor, layout: int = 0,
                                          plan: torch.Tensor | None = None, h: torch.Tensor | None = None,
                                          shared_h: torch.Tensor | None = None,
                                          shared_sigma: torch.Tensor | None = None, stream=None):
    """nvfp4_moe_plan followed by nvfp4_moe_w13_swiglu_with_shared (one launch for small batches).
    Returns (plan, h, shared_h, shared_sigma)."""
    M, topk = topk_ids.shape
    I, Is = w13.rows // 2, shared_w13.rows // 2
    dev = x.device
    _shape(x, "x", (M, w13.k))
    _shape(gate, "gate", (w13.k,))
    if plan is None:
        plan = torch.empty(max(nvfp4_moe_plan_bytes(M, topk, E), 4) // 4, dtype=torch.int32, device=dev)
    h = torch.empty((M * topk, I), dtype=torch.float16, device=dev) if h is None else h
    shared_h = torch.empty((M, Is), dtype=torch.float16, device=dev) if shared_h is None else shared_h
    shared_sigma = torch.empty((M,), dtype=torch.float32, device=dev) if shared_sigma is None else shared_sigma
    _rows(h, "h", M * topk, I)
    _shape(shared_h, "shared_h", (M, Is))
    _shape(shared_sigma, "shared_sigma", (M,))
    d, ds = w13.desc(), shared_w13.desc()
    _check("nvfp4_moe_plan_w13_swiglu_with_shared", lib().nvfp4_moe_plan_w13_swiglu_with_shared(
        _dev(topk_ids, "topk_ids", torch.int32), M, topk, E, _dev(plan, "plan", torch.int32), plan.numel() * 4,
        _dev(x, "x", torch.float16), C.byref(d), layout, _dev(h, "h", torch.float16), C.byref(ds),
        _dev(gate, "gate", torch.float16), _dev(shared_h, "shared_h", torch.float16),
        _dev(shared_sigma, "shared_sigma", torch.float32), _stream(stream)))
    return plan, h, shared_h, shared_sigma


def nvfp4_moe_w2_reduce_with_shared(plan: torch.Tensor, M: int, topk: int, E: int, h: torch.Tensor, w2: NVFP4Tensor,
                                    topk_weights: torch.Tensor, shared_h: torch.Tensor, shared_w2: NVFP4Tensor,
                                    shared_sigma: torch.Tensor, shared_y: torch.Tensor | None = None,
                                    out: torch.Tensor | None = None, ws: torch.Tensor | None = None,
                                    stream=None) -> torch.Tensor:
    """Grouped W2 + slot-order reduction with the shared expert's down projection in the same launch
    and its term added last. Returns out fp16 [M, K]."""
    K = w2.rows
    dev = h.device
    _plan_ok(plan, M, topk, E)
    _rows(h, "h", M * topk, w2.k)
    _shape(topk_weights, "topk_weights", (M, topk))
    _shape(shared_h, "shared_h", (M, shared_w2.k))
    _shape(shared_sigma, "shared_sigma", (M,))
    out = torch.empty((M, K), dtype=torch.float16, device=dev) if out is None else out
    shared_y = torch.empty((M, K), dtype=torch.float32, device=dev) if shared_y is None else shared_y
    _shape(out, "out", (M, K))
    _shape(shared_y, "shared_y", (M, K))
    if ws is None:
        ws = torch.empty(max(nvfp4_moe_w2_workspace_bytes(M, topk, K), 256), dtype=torch.uint8, device=dev)
    d, ds = w2.desc(), shared_w2.desc()
    _check("nvfp4_moe_w2_reduce_with_shared", lib().nvfp4_moe_w2_reduce_with_shared(
        _dev(plan, "plan", torch.int32), M, topk, E, _dev(h, "h", torch.float16), C.byref(d),
        _dev(topk_weights, "topk_weights", torch.float32), _dev(shared_h, "shared_h", torch.float16), C.byref(ds),
        _dev(shared_sigma, "shared_sigma", torch.float32), _dev(shared_y, "shared_y", torch.float32),
        _dev(out, "out", torch.float16), ws.data_ptr(), ws.numel(), _stream(stream)))
    return out
