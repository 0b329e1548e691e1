"""ctypes wrapper for the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The HIP product path never does, and it shares no code with oracle.c.

All functions take numpy arrays in the storage formats of ``synth.inputs``. fp16 activations are
passed as their bit patterns, and results come back as float64. Each wrapper names the oracle.c
function it calls; the page citations are in that file.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_i64, _i32, _dbl, _vp = C.c_int64, C.c_int32, C.c_double, C.c_void_p


def lib():
    """Load liboracle.so, building it first if it is not there. NVFP4_ORACLE_LIB names another build
    of oracle.c to load instead (the sanitizer build of oracle/build.py, for the sanitizer test)."""
    global _LIB
    if _LIB is None:
        path = os.environ.get("NVFP4_ORACLE_LIB") or os.path.join(HERE, "liboracle.so")
        if not os.path.exists(path):
            from . import build as _b  # noqa: WPS433
            _b.build()
        L = C.CDLL(path)
        L.orc_e2m1.restype = _dbl
        L.orc_e2m1.argtypes = [C.c_int]
        L.orc_e4m3.restype = _dbl
        L.orc_e4m3.argtypes = [C.c_int]
        L.orc_half.restype = _dbl
        L.orc_half.argtypes = [C.c_uint16]
        L.orc_silu.restype = _dbl
        L.orc_silu.argtypes = [_dbl]
        L.orc_to_half.restype = C.c_uint16
        L.orc_to_half.argtypes = [_dbl]
        L.orc_dequant.restype = None
        L.orc_dequant.argtypes = [_vp, _vp, _vp, _i64, _i64, _i64, _vp]
        L.orc_linear.restype = None
        L.orc_linear.argtypes = [_vp, _i64, _i64, _vp, _vp, _vp, _i64, _vp, C.c_int]
        L.orc_plan.restype = None
        L.orc_plan.argtypes = [_vp, _i64, _i64, _i64, _i64] + [_vp] * 8
        L.orc_moe_token.restype = None
        L.orc_moe_token.argtypes = ([_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i32,
                                     _vp, _vp, _vp, _vp, _i64, _vp, _vp, C.c_int])
        L.orc_moe_grouped.restype = None
        L.orc_moe_grouped.argtypes = ([_vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp, _i32,
                                       _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, C.c_int])
        L.orc_gated_mlp.restype = None
        L.orc_gated_mlp.argtypes = ([_vp, _i64, _i64, _i64, _vp, _vp, _vp, _i32, _vp, _vp, _vp, _i64,
                                     _vp, _vp, C.c_int])
        L.orc_linear_fp8.restype = None
        L.orc_linear_fp8.argtypes = [_vp, _i64, _i64, _vp, _vp, _i64, _vp, C.c_int]
        L.orc_shared_gate.restype = None
        L.orc_shared_gate.argtypes = [_vp, _i64, _i64, _vp, _vp]
        L.orc_route.restype = None
        L.orc_route.argtypes = [_vp, _i64, _i64, _i64, _vp, _vp]
        L.orc_w2_reduce.restype = None
        L.orc_w2_reduce.argtypes = ([_vp, _vp, _i64, _i64, _i64, _i64, _i64, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _vp, C.c_int])
        _LIB = L
    return _LIB


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


def _threads(n):
    """Oracle threads: the argument, else OMP_NUM_THREADS, else the host's core count."""
    if n:
        return int(n)
    env = os.environ.get("OMP_NUM_THREADS", "")
    return int(env) if env.isdigit() and int(env) > 0 else (os.cpu_count() or 1)


def e2m1(code: int) -> float:
    return lib().orc_e2m1(int(code))


def e4m3(byte: int) -> float:
    return lib().orc_e4m3(int(byte))


def half(bits: int) -> float:
    return lib().orc_half(int(bits) & 0xFFFF)


def silu(g: float) -> float:
    return lib().orc_silu(float(g))


def to_half(v: float) -> int:
    return int(lib().orc_to_half(float(v)))


def dequant(codes, scales, gscale) -> np.ndarray:
    """orc_dequant: W[g,n,k] = e2m1 * e4m3 * global, as float64 [G,N,K]."""
    G, N, K2 = codes.shape
    out = np.empty((G, N, 2 * K2), dtype=np.float64)
    lib().orc_dequant(_p(np.ascontiguousarray(codes)), _p(np.ascontiguousarray(scales)),
                      _p(np.ascontiguousarray(gscale, dtype=np.float32)), G, N, 2 * K2, _p(out))
    return out


def linear(x16: np.ndarray, w, nthreads=None) -> np.ndarray:
    """orc_linear: y = x @ dq(W)^T in float64. x16 fp16 [M,K]; w = (codes, scales, gscale)."""
    codes, scales, gs = w
    M, K = x16.shape
    N = codes.shape[1]
    y = np.empty((M, N), dtype=np.float64)
    xb = np.ascontiguousarray(x16).view(np.uint16)
    lib().orc_linear(_p(xb), M, K, _p(np.ascontiguousarray(codes)), _p(np.ascontiguousarray(scales)),
                     _p(np.ascontiguousarray(gs, dtype=np.float32)), N, _p(y), _threads(nthreads))
    return y


def plan(ids: np.ndarray, E: int, BM: int = 16) -> dict:
    """orc_plan: stable counting sort of (token, slot) pairs by expert."""
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M, topk = ids.shape
    P = M * topk
    A = min(E, P)
    T = A + (P + BM - 1) // BM
    counts = np.zeros(E, np.int32)
    offsets = np.zeros(E + 1, np.int32)
    sorted_pair = np.full(max(P, 1), -7, np.int32)
    pos = np.full(max(P, 1), -7, np.int32)
    active = np.full(max(A, 1), -7, np.int32)
    te = np.full(max(T, 1), -7, np.int32)
    tr = np.full(max(T, 1), -7, np.int32)
    summ = np.zeros(4, np.int32)
    lib().orc_plan(_p(ids), M, topk, E, BM, _p(counts), _p(offsets), _p(sorted_pair), _p(pos), _p(active),
                   _p(te), _p(tr), _p(summ))
    nv, na, nb, nt = (int(v) for v in summ)
    return {"counts": counts, "offsets": offsets, "sorted_pair": sorted_pair[:nv], "pos_of_pair": pos[:P],
            "active": active[:na], "tile_expert": te[:nt], "tile_row0": tr[:nt],
            "n_valid": nv, "n_active": na, "n_bad": nb, "n_tiles": nt}


def _moe_weights(case):
    (c13, s13, g13), (c2, s2, g2) = case["w13"], case["w2"]
    return [np.ascontiguousarray(a) for a in (c13, s13, g13, c2, s2, g2)]


def moe_token(case: dict, tokens=None, layout: int = 0, want_h: bool = False, nthreads=None):
    """orc_moe_token (per-token, per-slot loop). Returns out [len(tokens), K] and, if asked,
    h [len(tokens), topk, I] (NaN for skipped slots)."""
    sh = case["shape"]
    x = np.ascontiguousarray(case["x"]).view(np.uint16)
    ids = np.ascontiguousarray(case["ids"], dtype=np.int32)
    tw = np.ascontiguousarray(case["topk_weights"], dtype=np.float32)
    tok = np.arange(sh.m, dtype=np.int32) if tokens is None else np.ascontiguousarray(tokens, dtype=np.int32)
    out = np.empty((len(tok), sh.k), np.float64)
    h = np.empty((len(tok), sh.topk, sh.i), np.float64) if want_h else None
    c13, s13, g13, c2, s2, g2 = _moe_weights(case)
    lib().orc_moe_token(_p(x), _p(ids), _p(tw), sh.m, sh.topk, sh.e, sh.k, sh.i, _p(c13), _p(s13), _p(g13),
                        int(layout), _p(c2), _p(s2), _p(g2), _p(tok), len(tok), _p(out),
                        _p(h) if want_h else None, _threads(nthreads))
    return (out, h) if want_h else out


def moe_grouped(case: dict, pl: dict, layout: int = 0, nthreads=None):
    """orc_moe_grouped (plan-driven). Returns (h [n_valid, I] in bucket order, out [M, K])."""
    sh = case["shape"]
    x = np.ascontiguousarray(case["x"]).view(np.uint16)
    tw = np.ascontiguousarray(case["topk_weights"], dtype=np.float32)
    h = np.empty((max(pl["n_valid"], 1), sh.i), np.float64)
    out = np.empty((sh.m, sh.k), np.float64)
    sp = np.ascontiguousarray(pl["sorted_pair"], dtype=np.int32)
    if sp.size == 0:
        sp = np.zeros(1, np.int32)
    c13, s13, g13, c2, s2, g2 = _moe_weights(case)
    lib().orc_moe_grouped(_p(x), _p(tw), sh.m, sh.topk, sh.e, sh.k, sh.i, _p(c13), _p(s13), _p(g13), int(layout),
                          _p(c2), _p(s2), _p(g2), _p(pl["offsets"]), _p(sp), _p(pl["pos_of_pair"]),
                          _p(h), _p(out), _threads(nthreads))
    return h[: pl["n_valid"]], out


def w2_reduce(h16: np.ndarray, case: dict, pl: dict, nthreads=None) -> np.ndarray:
    """orc_w2_reduce: W2 and the slot-ordered weighted sum, fed a given fp16 h in bucket order."""
    sh = case["shape"]
    hb = np.ascontiguousarray(h16).view(np.uint16)
    if hb.size == 0:
        hb = np.zeros((1, sh.i), np.uint16)
    tw = np.ascontiguousarray(case["topk_weights"], dtype=np.float32)
    out = np.empty((sh.m, sh.k), np.float64)
    sp = np.ascontiguousarray(pl["sorted_pair"], dtype=np.int32)
    if sp.size == 0:
        sp = np.zeros(1, np.int32)
    _, _, _, c2, s2, g2 = _moe_weights(case)
    lib().orc_w2_reduce(_p(hb), _p(tw), sh.m, sh.topk, sh.e, sh.k, sh.i, _p(c2), _p(s2), _p(g2),
                        _p(pl["offsets"]), _p(sp), _p(pl["pos_of_pair"]), _p(out), _threads(nthreads))
    return out


def route(logits: np.ndarray, topk: int):
    """Top-k routing of fp32 logits [M, E] (oracle.c: orc_route). Returns (ids int32 [M, topk],
    weights float64 [M, topk])."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    M, E = x.shape
    ids = np.zeros((M, topk), dtype=np.int32)
    w = np.zeros((M, topk), dtype=np.float64)
    lib().orc_route(_p(x), M, E, topk, _p(ids), _p(w))
    return ids, w


def gated_mlp(x16: np.ndarray, w13, w2, layout: int = 0, nthreads=None):
    """orc_gated_mlp: h = silu(x Wg^T) * (x Wu^T) and y = h W2^T in float64. x16 fp16 [M, K];
    w13 = (codes, scales, gscale) with 2I rows; w2 = (codes, scales, gscale) [N][I]. Returns (h, y)."""
    c13, s13, g13 = w13
    c2, s2, g2 = w2
    M, K = x16.shape
    I = c13.shape[1] // 2
    N = c2.shape[1]
    h = np.empty((M, I), np.float64)
    y = np.empty((M, N), np.float64)
    xb = np.ascontiguousarray(x16).view(np.uint16)
    lib().orc_gated_mlp(_p(xb), M, K, I, _p(np.ascontiguousarray(c13)), _p(np.ascontiguousarray(s13)),
                        _p(np.ascontiguousarray(g13, dtype=np.float32)), int(layout), _p(np.ascontiguousarray(c2)),
                        _p(np.ascontiguousarray(s2)), _p(np.ascontiguousarray(g2, dtype=np.float32)), N, _p(h), _p(y),
                        _threads(nthreads))
    return h, y


def linear_fp8(x16: np.ndarray, codes: np.ndarray, chscale: np.ndarray, nthreads=None) -> np.ndarray:
    """orc_linear_fp8: y = x @ (e4m3(W) * s[:, None])^T in float64. x16 fp16 [M,K]; codes uint8 [N,K];
    chscale float32 [N]."""
    M, K = x16.shape
    N = codes.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    xb = np.ascontiguousarray(x16).view(np.uint16)
    lib().orc_linear_fp8(_p(xb), M, K, _p(np.ascontiguousarray(codes, dtype=np.uint8)),
                         _p(np.ascontiguousarray(chscale, dtype=np.float32)), N, _p(y), _threads(nthreads))
    return y


def shared_gate(x16: np.ndarray, g16: np.ndarray) -> np.ndarray:
    """orc_shared_gate: sigmoid(x @ g) per token, float64 [M]. x16 fp16 [M, K], g16 fp16 [K]."""
    M, K = x16.shape
    s = np.empty(M, np.float64)
    lib().orc_shared_gate(_p(np.ascontiguousarray(x16).view(np.uint16)), M, K,
                          _p(np.ascontiguousarray(g16, dtype=np.float16).view(np.uint16)), _p(s))
    return s


def moe_with_shared(case: dict, shared: dict, layout: int = 0, tokens=None, nthreads=None):
    """The MoE output with the shared expert added: out[t] = sum_k w[t,k] y_k[t] + sigma[t] * y_s[t]
    (routed part: orc_moe_token; shared expert: orc_gated_mlp on x with its own weights; gate:
    orc_shared_gate). ``shared`` holds w13, w2 (NVFP4 tuples), layout and g (fp16 [K]). Returns
    (out, y_s, sigma) for the selected tokens, float64."""
    x = case["x"] if tokens is None else case["x"][np.asarray(tokens)]
    out = moe_token(case, tokens=tokens, layout=layout, nthreads=nthreads)
    _, ys = gated_mlp(x, shared["w13"], shared["w2"], shared.get("layout", 0), nthreads)
    sg = shared_gate(x, shared["g"])
    return out + sg[:, None] * ys, ys, sg
