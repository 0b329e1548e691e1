"""The C ABI on the host (no GPU needed): the built library loads, exports every function that
include/nvfp4moe.h declares, and its host-side logic (version, status names, buffer sizes and the
argument checks that fail closed before anything is enqueued) behaves as the header states.

None of these calls reaches the HIP runtime: each returns before a launch.
"""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4moe.h")
# NVFP4_TEST_LIB: another build of the same library to check instead (the host-sanitizer build,
# see tests/test_sanitizers.py).
LIB = os.environ.get("NVFP4_TEST_LIB") or os.path.join(ROOT, "gemm_nvfp4_amd", "libnvfp4moe.so")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (python gemm_nvfp4_amd/build.py)")
    from gemm_nvfp4_amd import _lib
    if not os.environ.get("NVFP4_TEST_LIB"):
        return _lib.lib()
    lib = C.CDLL(LIB)
    for name, (res, args) in _lib._SIGS.items():
        getattr(lib, name).restype, getattr(lib, name).argtypes = res, args
    return lib


def declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(nvfp4_\w+)\s*\(", txt, flags=re.M)))


def test_header_declares_the_expected_entry_points():
    assert declared() == sorted([
        "nvfp4_abi_version", "nvfp4_status_str", "nvfp4_moe_plan_bytes", "nvfp4_moe_plan", "nvfp4_moe_route",
        "nvfp4_moe_w13_swiglu", "nvfp4_moe_w2_workspace_bytes", "nvfp4_moe_w2_reduce", "nvfp4_linear",
        "nvfp4_linear_swiglu", "nvfp4_linear_fp8", "nvfp4_moe_shared_expert", "nvfp4_moe_w2_reduce_shared",
        "nvfp4_moe_w13_swiglu_with_shared", "nvfp4_moe_w2_reduce_with_shared", "nvfp4_moe_plan_w13_swiglu",
        "nvfp4_moe_plan_w13_swiglu_with_shared", "nvfp4_moe_layer_workspace_bytes", "nvfp4_moe_layer",
        "nvfp4_moe_layer_noalloc", "nvfp4_linear_ws_bytes", "nvfp4_linear_ws", "nvfp4_linear_swiglu_ws"])


def test_library_exports_every_declared_function():
    raw = C.CDLL(LIB)
    for name in declared():
        assert hasattr(raw, name), name


def test_version_and_status_names(L):
    assert L.nvfp4_abi_version() == 1
    names = [L.nvfp4_status_str(k).decode() for k in range(7)]
    assert names == ["NVFP4_OK", "NVFP4_ERR_NULL", "NVFP4_ERR_SHAPE", "NVFP4_ERR_ALIGN", "NVFP4_ERR_WORKSPACE",
                     "NVFP4_ERR_UNSUPPORTED", "NVFP4_ERR_LAUNCH"]
    assert L.nvfp4_status_str(99) == b"NVFP4_ERR_UNKNOWN"


def test_buffer_sizes(L):
    assert L.nvfp4_moe_plan_bytes(16, 10, 512) % 256 == 0 and L.nvfp4_moe_plan_bytes(16, 10, 512) > 0
    assert L.nvfp4_moe_plan_bytes(16, 33, 512) == 0  # topk > 32
    assert L.nvfp4_moe_plan_bytes(-1, 10, 512) == 0
    assert L.nvfp4_moe_w2_workspace_bytes(16, 10, 2048) == 16 * 10 * 2048 * 4
    assert L.nvfp4_moe_w2_workspace_bytes(3, 1, 80) == 1024  # 960 bytes, rounded up to 256


def test_argument_checks_fail_closed(L):
    null = None
    fake = C.c_void_p(0x1000)   # never dereferenced: every call below returns before any launch
    odd = C.c_void_p(0x1001)
    # plan
    assert L.nvfp4_moe_plan(null, -1, 10, 512, null, 0, null) == 2      # ERR_SHAPE
    assert L.nvfp4_moe_plan(null, 4, 10, 8192, null, 0, null) == 5      # E > 4096: ERR_UNSUPPORTED
    assert L.nvfp4_moe_plan(null, 0, 10, 512, null, 0, null) == 0       # M = 0 is a no-op
    assert L.nvfp4_moe_plan(null, 4, 10, 512, fake, 1 << 20, null) == 1  # ERR_NULL
    assert L.nvfp4_moe_plan(odd, 4, 10, 512, fake, 1 << 20, null) == 3   # ERR_ALIGN
    assert L.nvfp4_moe_plan(fake, 4, 10, 512, fake, 16, null) == 4       # ERR_WORKSPACE
    # router
    assert L.nvfp4_moe_route(fake, 4, 8, 9, fake, fake, fake, 1 << 20, null) == 2   # topk > E
    assert L.nvfp4_moe_route(fake, 0, 8, 2, null, null, null, 0, null) == 0        # M = 0
    assert L.nvfp4_moe_route(fake, 4, 8, 2, null, fake, fake, 1 << 20, null) == 1  # ERR_NULL
    assert L.nvfp4_moe_route(odd, 4, 8, 2, fake, fake, fake, 1 << 20, null) == 3   # ERR_ALIGN
    assert L.nvfp4_moe_route(fake, 4, 8, 2, fake, fake, fake, 16, null) == 4       # ERR_WORKSPACE
    # linear: K % 128 != 0 is unsupported, M < 0 a shape error
    from gemm_nvfp4_amd._lib import nvfp4_weights
    w = nvfp4_weights(fake, fake, fake, 1, 64, 96)
    assert L.nvfp4_linear(fake, 4, C.byref(w), fake, null) == 5
    assert L.nvfp4_linear(fake, -1, C.byref(w), fake, null) == 2
    w = nvfp4_weights(None, fake, fake, 1, 64, 128)
    assert L.nvfp4_linear(fake, 4, C.byref(w), fake, null) == 1
    # gated form: odd rows, I % 16 != 0, K too long, bad layout
    assert L.nvfp4_linear_swiglu(fake, 4, C.byref(nvfp4_weights(fake, fake, fake, 1, 63, 128)), 0, fake, null) == 2
    assert L.nvfp4_linear_swiglu(fake, 4, C.byref(nvfp4_weights(fake, fake, fake, 1, 40, 128)), 0, fake, null) == 5
    assert L.nvfp4_linear_swiglu(fake, 4, C.byref(nvfp4_weights(fake, fake, fake, 1, 64, 32768)), 0, fake, null) == 5
    assert L.nvfp4_linear_swiglu(fake, 4, C.byref(nvfp4_weights(fake, fake, fake, 1, 64, 128)), 2, fake, null) == 2
    assert L.nvfp4_linear_swiglu(fake, 0, C.byref(nvfp4_weights(fake, fake, fake, 1, 64, 128)), 0, null, null) == 0
    # shared expert: w2 must be [K][I] for w13 [2I][K]; I % 128
    w13 = nvfp4_weights(fake, fake, fake, 1, 256, 256)
    assert L.nvfp4_moe_shared_expert(fake, 4, C.byref(w13), 0, C.byref(nvfp4_weights(fake, fake, fake, 1, 256, 64)),
                                     fake, fake, fake, fake, null) == 2
    assert L.nvfp4_moe_shared_expert(fake, 4, C.byref(w13), 0, C.byref(nvfp4_weights(fake, fake, fake, 1, 256, 128)),
                                     null, fake, fake, fake, null) == 1
    w13b = nvfp4_weights(fake, fake, fake, 1, 128, 256)  # I = 64: not a multiple of 128
    assert L.nvfp4_moe_shared_expert(fake, 4, C.byref(w13b), 0, C.byref(nvfp4_weights(fake, fake, fake, 1, 256, 64)),
                                     fake, fake, fake, fake, null) == 5
    assert L.nvfp4_moe_w2_reduce_shared(fake, 4, 2, 8, fake, C.byref(nvfp4_weights(fake, fake, fake, 8, 256, 128)),
                                        fake, null, fake, fake, fake, 1 << 20, null) == 1
    # shared expert inside the routed launches: shapes must agree, every pointer is required
    rw13 = nvfp4_weights(fake, fake, fake, 8, 256, 256)          # E = 8, I = 128, K = 256
    sw13 = nvfp4_weights(fake, fake, fake, 1, 256, 256)
    assert L.nvfp4_moe_w13_swiglu_with_shared(fake, 4, 2, 8, fake, C.byref(rw13), 0, fake,
                                              C.byref(nvfp4_weights(fake, fake, fake, 1, 256, 128)),
                                              fake, fake, fake, null) == 2   # shared k != K
    assert L.nvfp4_moe_w13_swiglu_with_shared(fake, 4, 2, 8, fake, C.byref(rw13), 0, fake, C.byref(sw13),
                                              null, fake, fake, null) == 1   # no gate
    assert L.nvfp4_moe_w13_swiglu_with_shared(fake, 4, 2, 8, fake, C.byref(rw13), 0, fake, C.byref(sw13),
                                              odd, fake, fake, null) == 3    # gate not 2-byte aligned
    assert L.nvfp4_moe_w13_swiglu_with_shared(null, 0, 2, 8, null, C.byref(rw13), 0, null, C.byref(sw13),
                                              null, null, null, null) == 0   # M = 0
    rw2 = nvfp4_weights(fake, fake, fake, 8, 256, 128)           # E = 8, K = 256, I = 128
    assert L.nvfp4_moe_w2_reduce_with_shared(fake, 4, 2, 8, fake, C.byref(rw2), fake, fake,
                                             C.byref(nvfp4_weights(fake, fake, fake, 1, 128, 128)), fake, fake,
                                             fake, fake, 1 << 20, null) == 2  # shared rows != K
    assert L.nvfp4_moe_w2_reduce_with_shared(fake, 4, 2, 8, fake, C.byref(rw2), fake, fake,
                                             C.byref(nvfp4_weights(fake, fake, fake, 1, 256, 64)), fake, fake,
                                             fake, fake, 1 << 20, null) == 5  # shared I % 128
    assert L.nvfp4_moe_w2_reduce_with_shared(fake, 4, 2, 8, fake, C.byref(rw2), fake, fake,
                                             C.byref(nvfp4_weights(fake, fake, fake, 1, 256, 128)), fake, null,
                                             fake, fake, 1 << 20, null) == 1  # no shared_y
    # plan + W13 in one call: the checks of both calls, before anything is enqueued
    ew13 = nvfp4_weights(fake, fake, fake, 8, 256, 256)          # E = 8, I = 128, K = 256
    assert L.nvfp4_moe_plan_w13_swiglu(fake, -1, 2, 8, fake, 1 << 20, fake, C.byref(ew13), 0, fake, null) == 2
    assert L.nvfp4_moe_plan_w13_swiglu(fake, 4, 2, 8, fake, 1 << 20, fake, C.byref(ew13), 2, fake, null) == 2  # layout
    assert L.nvfp4_moe_plan_w13_swiglu(fake, 4, 2, 9, fake, 1 << 20, fake, C.byref(ew13), 0, fake, null) == 2  # groups != E
    assert L.nvfp4_moe_plan_w13_swiglu(fake, 4, 2, 8, fake, 1 << 20, fake,
                                       C.byref(nvfp4_weights(fake, fake, fake, 8, 256, 4096)), 0, fake, null) == 5  # K > 2048
    assert L.nvfp4_moe_plan_w13_swiglu(null, 0, 2, 8, null, 0, null, C.byref(ew13), 0, null, null) == 0  # M = 0
    assert L.nvfp4_moe_plan_w13_swiglu(null, 4, 2, 8, fake, 1 << 20, fake, C.byref(ew13), 0, fake, null) == 1
    assert L.nvfp4_moe_plan_w13_swiglu(fake, 4, 2, 8, fake, 1 << 20, odd, C.byref(ew13), 0, fake, null) == 3
    assert L.nvfp4_moe_plan_w13_swiglu(fake, 4, 2, 8, fake, 16, fake, C.byref(ew13), 0, fake, null) == 4
    # plan + W13 with the shared expert in one call
    assert L.nvfp4_moe_plan_w13_swiglu_with_shared(fake, 4, 2, 8, fake, 1 << 20, fake, C.byref(rw13), 0, fake,
                                                   C.byref(nvfp4_weights(fake, fake, fake, 1, 256, 128)),
                                                   fake, fake, fake, null) == 2   # shared k != K
    assert L.nvfp4_moe_plan_w13_swiglu_with_shared(fake, 4, 2, 8, fake, 1 << 20, fake, C.byref(rw13), 0, fake,
                                                   C.byref(sw13), null, fake, fake, null) == 1   # no gate
    assert L.nvfp4_moe_plan_w13_swiglu_with_shared(odd, 4, 2, 8, fake, 1 << 20, fake, C.byref(rw13), 0, fake,
                                                   C.byref(sw13), fake, fake, fake, null) == 3   # ids unaligned
    assert L.nvfp4_moe_plan_w13_swiglu_with_shared(fake, 4, 2, 8, fake, 16, fake, C.byref(rw13), 0, fake,
                                                   C.byref(sw13), fake, fake, fake, null) == 4   # plan too small
    assert L.nvfp4_moe_plan_w13_swiglu_with_shared(null, 0, 2, 8, null, 0, null, C.byref(rw13), 0, null,
                                                   C.byref(sw13), null, null, null, null) == 0   # M = 0
    # channel-FP8 projection
    from gemm_nvfp4_amd._lib import fp8_channel_weights as f8
    assert L.nvfp4_linear_fp8(fake, 4, C.byref(f8(fake, fake, 64, 96)), fake, null) == 5     # K % 128
    assert L.nvfp4_linear_fp8(fake, 4, C.byref(f8(fake, fake, 40, 128)), fake, null) == 5    # N % 16
    assert L.nvfp4_linear_fp8(fake, 4, C.byref(f8(None, fake, 64, 128)), fake, null) == 1
    assert L.nvfp4_linear_fp8(fake, 4, C.byref(f8(odd, fake, 64, 128)), fake, null) == 3
    assert L.nvfp4_linear_fp8(fake, -1, C.byref(f8(fake, fake, 64, 128)), fake, null) == 2
    assert L.nvfp4_linear_fp8(null, 0, C.byref(f8(fake, fake, 64, 128)), null, null) == 0


def test_dense_reduction_length_admission(L):
    """The dense kernels keep one FP32 partial tile per chunk in LDS. The plain projection admits
    K <= 32768 (one weight tile per wave past 16384, so the tiles fit in 160 KiB); the gated and
    channel-FP8 forms keep two tiles per wave and admit K <= 16384. Beyond: ERR_UNSUPPORTED before
    any launch. M = 0 reaches every check without launching."""
    from gemm_nvfp4_amd._lib import nvfp4_weights, fp8_channel_weights as f8
    fake, null = C.c_void_p(0x1000), None
    for k, want in ((16384, 0), (16512, 0), (16896, 0), (32768, 0), (32896, 5), (65536, 5)):
        for rows in (64, 48):  # paired 16-row tiles, and a single one
            w = nvfp4_weights(fake, fake, fake, 1, rows, k)
            assert L.nvfp4_linear(null, 0, C.byref(w), null, null) == want, (k, rows)
    for k, want in ((16384, 0), (16896, 5), (32768, 5)):
        assert L.nvfp4_linear_swiglu(null, 0, C.byref(nvfp4_weights(fake, fake, fake, 1, 64, k)), 0, null, null) == want
        assert L.nvfp4_linear_fp8(null, 0, C.byref(f8(fake, fake, 64, k)), null, null) == want
    # shared expert: gate/up K <= 16384 (two tiles), down I <= 32768 (one tile past 16384)
    for K, I, want in ((2048, 16896, 0), (2048, 32768, 0), (2048, 32896, 5), (16896, 512, 5)):
        w13 = nvfp4_weights(fake, fake, fake, 1, 2 * I, K)
        w2 = nvfp4_weights(fake, fake, fake, 1, K, I)
        assert L.nvfp4_moe_shared_expert(null, 0, C.byref(w13), 0, C.byref(w2), null, null, null, null, null) == want


def test_layer_call_checks(L):
    from gemm_nvfp4_amd._lib import nvfp4_weights
    fake, odd, null = C.c_void_p(0x1000), C.c_void_p(0x1001), None
    E, K, I = 8, 256, 128
    w13 = nvfp4_weights(fake, fake, fake, E, 2 * I, K)
    w2 = nvfp4_weights(fake, fake, fake, E, K, I)
    need = L.nvfp4_moe_layer_workspace_bytes(4, 2, E, K, I)
    assert need == (L.nvfp4_moe_plan_bytes(4, 2, E) + (4 * 2 * I * 2 + 255) // 256 * 256
                    + L.nvfp4_moe_w2_workspace_bytes(4, 2, K))
    assert L.nvfp4_moe_layer_workspace_bytes(4, 33, E, K, I) == 0
    args = lambda ids, M, topk, E_, x, a, lay, b, tw, out, ws, wsb: L.nvfp4_moe_layer(  # noqa: E731
        ids, M, topk, E_, x, C.byref(a), lay, C.byref(b), tw, out, ws, wsb, null)
    assert args(null, 0, 2, E, null, w13, 0, w2, null, null, null, 0) == 0                # M = 0
    assert args(fake, -1, 2, E, fake, w13, 0, w2, fake, fake, fake, need) == 2            # M < 0
    assert args(fake, 4, 2, E, fake, w13, 2, w2, fake, fake, fake, need) == 2             # layout
    assert args(fake, 4, 2, E, fake, w13, 0, nvfp4_weights(fake, fake, fake, E, K, 2 * I), fake, fake, fake,
                need) == 2                                                                # w2 not [E][K][I]
    assert args(fake, 4, 2, E, fake, nvfp4_weights(fake, fake, fake, E, 2 * I, 4096), 0,
                nvfp4_weights(fake, fake, fake, E, 4096, I), fake, fake, fake, need) == 5  # K > 2048
    assert args(fake, 4, 2, E, fake, nvfp4_weights(fake, fake, fake, E, 2 * 64, K), 0,
                nvfp4_weights(fake, fake, fake, E, K, 64), fake, fake, fake, need) == 5    # I % 128
    assert args(fake, 4, 2, E, fake, w13, 0, w2, null, fake, fake, need) == 1             # no weights
    assert args(fake, 4, 2, E, fake, w13, 0, w2, fake, fake, null, need) == 1             # no workspace
    assert args(odd, 4, 2, E, fake, w13, 0, w2, fake, fake, fake, need) == 3              # ids unaligned
    assert args(fake, 4, 2, E, fake, w13, 0, w2, fake, fake, odd, need) == 3              # ws unaligned
    assert args(fake, 4, 2, E, fake, w13, 0, w2, fake, fake, fake, need - 1) == 4         # ws too small


def test_split_k_dense_workspace_and_errors(L):
    """The split-K dense calls need ceil(K/512) * M * rows FP32 partials; a missing, misaligned or
    short workspace is reported before anything is enqueued (fake device pointers are never read)."""
    from gemm_nvfp4_amd._lib import nvfp4_weights
    L.nvfp4_linear_ws_bytes.restype = C.c_size_t
    for M, N, K in ((1, 4352, 5120), (32, 4352, 5120), (45, 256, 2176), (7, 64, 128)):
        assert L.nvfp4_linear_ws_bytes(M, N, K) == -(-K // 512) * M * N * 4
    assert L.nvfp4_linear_ws_bytes(-1, 64, 128) == 0 and L.nvfp4_linear_ws_bytes(4, 0, 128) == 0
    fake, odd, null = C.c_void_p(0x1000), C.c_void_p(0x1008), None
    w = nvfp4_weights(fake, fake, fake, 1, 64, 640)
    need = L.nvfp4_linear_ws_bytes(20, 64, 640)
    assert L.nvfp4_linear_ws(fake, 20, C.byref(w), fake, null, need, null) == 1          # ERR_NULL
    assert L.nvfp4_linear_ws(fake, 20, C.byref(w), fake, odd, need, null) == 3           # ERR_ALIGN
    assert L.nvfp4_linear_ws(fake, 20, C.byref(w), fake, fake, need - 1, null) == 4      # ERR_WORKSPACE
    assert L.nvfp4_linear_ws(fake, 20, C.byref(nvfp4_weights(fake, fake, fake, 1, 64, 96)), fake, fake, need,
                             null) == 5                                                  # K % 128
    assert L.nvfp4_linear_ws(null, 0, C.byref(w), null, null, 0, null) == 0              # M = 0
    w13 = nvfp4_weights(fake, fake, fake, 1, 64, 640)
    assert L.nvfp4_linear_swiglu_ws(fake, 20, C.byref(w13), 0, fake, fake, need - 4, null) == 4
    assert L.nvfp4_linear_swiglu_ws(fake, 20, C.byref(w13), 2, fake, fake, need, null) == 2   # layout
    assert L.nvfp4_linear_swiglu_ws(fake, 20, C.byref(w13), 0, fake, null, need, null) == 1
