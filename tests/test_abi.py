"""C ABI checks that need no GPU: the library loads, exports every entry point the
header declares, and rejects bad arguments on the host before any HIP call."""
from __future__ import annotations

import ctypes
import math
import os
import re

import pytest

import mixed_precision_int8_amd as m8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "llmint8.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3

# fake, never-dereferenced device addresses (validation only looks at null/alignment)
P = 0x7f0000000000
ALIGNED = ctypes.c_void_p(P)
MISALIGNED = ctypes.c_void_p(P + 2)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(m8.library_path()):
        pytest.skip("libllmint8.so not built")
    return m8.load_library()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LLMINT8_API\s+[\w\s\*]+?\b(llmint8_\w+)\s*\(", text)))


def test_header_declares_expected_entry_points():
    names = declared_symbols()
    assert "llmint8_quantize_weight" in names and "llmint8_linear" in names
    assert set(names) == set(m8.EXPORTED_SYMBOLS)


def test_library_exports_every_declared_symbol(lib):
    for name in declared_symbols():
        assert hasattr(lib, name), name


# T = 64 takes the GEMM route (T > llmint8_gemv_max_rows(1024) = 16), which needs a
# workspace; every call below fails validation, so nothing is ever launched
def _linear(lib, X=ALIGNED, T=64, K=1024, Wq=ALIGNED, sW=ALIGNED, N=1024, thr=6.0, Y=ALIGNED,
            ws=ALIGNED, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.llmint8_workspace_bytes(max(T, 0), K, N) if T >= 0 else 0
    return lib.llmint8_linear(X, T, K, Wq, sW, N, thr, Y, ws, ws_bytes, None)


def test_linear_argument_errors(lib):
    assert _linear(lib, X=None) == INVALID
    assert _linear(lib, Y=None) == INVALID
    assert _linear(lib, Wq=None) == INVALID
    assert _linear(lib, sW=None) == INVALID
    assert _linear(lib, ws=None) == INVALID
    assert _linear(lib, T=-1) == INVALID
    assert _linear(lib, K=0) == INVALID
    assert _linear(lib, N=0) == INVALID
    assert _linear(lib, thr=float("nan")) == INVALID
    assert _linear(lib, thr=0.0) == INVALID
    assert _linear(lib, thr=-6.0) == INVALID
    assert _linear(lib, X=MISALIGNED) == INVALID
    assert _linear(lib, Y=MISALIGNED) == INVALID
    assert _linear(lib, Wq=MISALIGNED) == INVALID
    assert _linear(lib, ws=ctypes.c_void_p(P + 16)) == INVALID     # workspace needs 256-B alignment
    assert _linear(lib, K=1000) == UNSUPPORTED                      # K % 16 != 0
    assert _linear(lib, K=65536 + 16) == UNSUPPORTED
    assert _linear(lib, N=1 << 20, K=4096) == UNSUPPORTED            # N*K >= 2^31
    need = lib.llmint8_workspace_bytes(64, 1024, 1024)
    assert _linear(lib, ws_bytes=need - 1) == WORKSPACE


def test_zero_rows_is_a_noop_without_launch(lib):
    # T == 0 returns OK before any HIP call, even with no X / Y / workspace
    assert lib.llmint8_linear(None, 0, 1024, ALIGNED, ALIGNED, 1024, 6.0, None, None, 0, None) == OK
    assert lib.llmint8_linear(None, 0, 1024, ALIGNED, ALIGNED, 1024, math.inf, None, None, 0, None) == OK


def test_quantize_weight_argument_errors(lib):
    q = lib.llmint8_quantize_weight
    assert q(None, 16, 64, ALIGNED, ALIGNED, None) == INVALID
    assert q(ALIGNED, 16, 64, None, ALIGNED, None) == INVALID
    assert q(ALIGNED, 16, 64, ALIGNED, None, None) == INVALID
    assert q(ALIGNED, 0, 64, ALIGNED, ALIGNED, None) == INVALID
    assert q(ALIGNED, 16, 0, ALIGNED, ALIGNED, None) == INVALID
    assert q(ALIGNED, 16, 72, ALIGNED, ALIGNED, None) == UNSUPPORTED
    assert q(MISALIGNED, 16, 64, ALIGNED, ALIGNED, None) == INVALID


def test_debug_and_timed_argument_errors(lib):
    need = lib.llmint8_workspace_bytes_path(16, 1024, 1024, m8.LLMINT8_PATH_GEMM)
    d = lib.llmint8_linear_debug
    base = [ALIGNED, 16, 1024, ALIGNED, ALIGNED, 1024, 6.0, ALIGNED, ALIGNED, need, None]
    assert d(*base, 7, None, None, None, None, None, None) == INVALID        # unknown path
    for p in (3, 15, 21, -1):                                                  # around the tile paths
        assert d(*base, p, None, None, None, None, None, None) == INVALID
    tiles = sorted(m8.LLMINT8_PATH_GEMM_TILES.values())
    assert tiles == list(range(16, 21))
    # a forced tile is the GEMM route: 3 kernels, so 2 events are too few
    assert lib.llmint8_linear_timed(*base, tiles[-1], (ctypes.c_void_p * 4)(P, P, P, P), 2,
                                    ctypes.byref(ctypes.c_int(0))) == INVALID
    assert d(*base, m8.LLMINT8_PATH_GEMM, None, None, None, MISALIGNED, None, None) == INVALID
    big_t = lib.llmint8_gemv_max_rows(1024) + 1
    need2 = lib.llmint8_workspace_bytes(big_t, 1024, 1024)
    base2 = [ALIGNED, big_t, 1024, ALIGNED, ALIGNED, 1024, 6.0, ALIGNED, ALIGNED, need2, None]
    assert d(*base2, m8.LLMINT8_PATH_GEMV, None, None, None, None, None, None) == UNSUPPORTED
    t = lib.llmint8_linear_timed
    ev = (ctypes.c_void_p * 4)(P, P, P, P)
    nk = ctypes.c_int(0)
    assert t(*base, 0, None, 4, ctypes.byref(nk)) == INVALID
    assert t(*base, m8.LLMINT8_PATH_GEMM, ev, 2, ctypes.byref(nk)) == INVALID   # 3 kernels need 4 events


def test_gemm_tile_choice(lib):
    """The host cost model (rounds of 256 CUs x tile time): the 2048 x 11008
    layer fits one round of 352 x 256 tiles; the 4096 x 28672 layer is seven
    full rounds of 256 x 256; small outputs take 128 x 128."""
    t = lib.llmint8_gemm_tile
    tiles = m8.LLMINT8_PATH_GEMM_TILES
    assert t(2048, 11008) == tiles["352x256"]
    assert t(4096, 28672) == tiles["256x256"]
    assert t(2048, 14336) == tiles["256x256"]
    assert t(16, 1024) == tiles["128x128"]
    assert t(0, 16) == INVALID and t(16, 0) == INVALID
    assert m8.llmint8_gemm_tile(2048, 11008) == "352x256"


def test_workspace_size_is_route_aware_and_bounded(lib):
    """The fused decode route needs no workspace; the GEMM route needs the int8
    activations, small tables and the 16-bit operands of min(K, 512) outlier columns
    (more outlier columns are formed in the epilogue), never the worst case |O| = K."""
    for T, K, N in [(64, 16, 1), (17, 1024, 1024), (2048, 4096, 11008), (4096, 8192, 28672),
                    (2048, 14336, 14336)]:
        ws = lib.llmint8_workspace_bytes(T, K, N)
        cols = min((K + 31) // 32 * 32, 512)
        assert ws >= T * K + 4 * T + 4 * K + 2 * cols * (T + N)
        assert ws < T * K + 4 * T + 4 * K + 2 * cols * (T + N) + 64 * 1024
        assert lib.llmint8_workspace_bytes_path(T, K, N, m8.LLMINT8_PATH_GEMM) == ws
    for K in (1024, 4096, 8192):
        r = lib.llmint8_gemv_max_rows(K)
        assert lib.llmint8_workspace_bytes(r, K, 4096) == 0
        assert lib.llmint8_workspace_bytes(r + 1, K, 4096) > 0
        assert lib.llmint8_workspace_bytes_path(r, K, 4096, m8.LLMINT8_PATH_GEMM) > 0
        assert lib.llmint8_workspace_bytes_path(r, K, 4096, m8.LLMINT8_PATH_GEMV) == 0
        assert lib.llmint8_workspace_bytes_path(r, K, 4096, 3) == 0          # unknown path
    # at the prefill shape: well under the int8 weight (the method's memory saving)
    assert lib.llmint8_workspace_bytes(2048, 4096, 11008) < 4096 * 11008 // 2
    assert lib.llmint8_workspace_bytes(16, 1000, 16) == 0
    assert lib.llmint8_workspace_bytes(-1, 1024, 16) == 0


def test_gemv_row_limit(lib):
    assert lib.llmint8_gemv_max_rows(1024) == 16
    assert lib.llmint8_gemv_max_rows(4096) >= 8
    assert lib.llmint8_gemv_max_rows(14336) >= 2
    assert lib.llmint8_gemv_max_rows(1000) == 0
    assert lib.llmint8_gemv_max_rows(65536) < 16


def test_status_strings(lib):
    for s in (OK, INVALID, UNSUPPORTED, WORKSPACE, -4):
        assert lib.llmint8_status_string(s)
    assert m8.llmint8_status_string(-3) == "workspace too small"


def _backward(lib, dY=ALIGNED, T=16, K=1024, Wq=ALIGNED, sW=ALIGNED, N=1024, dX=ALIGNED,
              ws=None, ws_bytes=0):
    return lib.llmint8_linear_backward_input(dY, T, K, Wq, sW, N, dX, ws, ws_bytes, None)


def test_backward_argument_errors(lib):
    # every call below fails validation (the workspace is not used), so nothing is launched
    assert _backward(lib, dY=None) == INVALID
    assert _backward(lib, dX=None) == INVALID
    assert _backward(lib, Wq=None) == INVALID
    assert _backward(lib, sW=None) == INVALID
    assert _backward(lib, T=-1) == INVALID
    assert _backward(lib, dY=MISALIGNED) == INVALID
    assert _backward(lib, dX=MISALIGNED) == INVALID
    assert _backward(lib, Wq=MISALIGNED) == INVALID
    assert _backward(lib, N=1020) == UNSUPPORTED                 # N % 8 != 0
    assert _backward(lib, N=65536 + 8, K=16) == UNSUPPORTED      # N > 65536
    assert _backward(lib, K=1000) == UNSUPPORTED                 # K % 16 != 0
    assert _backward(lib, dY=None, ws=ALIGNED, ws_bytes=1 << 20) == INVALID
    # T == 0 returns OK before any HIP call
    assert lib.llmint8_linear_backward_input(None, 0, 1024, ALIGNED, ALIGNED, 1024, None, None, 0,
                                             None) == OK
    t = lib.llmint8_linear_backward_input_timed
    ev = (ctypes.c_void_p * 2)(P, P)
    nk = ctypes.c_int(0)
    args = [ALIGNED, 16, 1024, ALIGNED, ALIGNED, 1024, ALIGNED, None, 0, None]
    assert t(*args, None, 2, ctypes.byref(nk)) == INVALID
    assert t(*args, ev, 1, ctypes.byref(nk)) == INVALID           # one kernel needs 2 events
    bad = list(args)
    bad[0] = None
    assert t(*bad, ev, 2, ctypes.byref(nk)) == INVALID
    d = lib.llmint8_dequantize_weight_t
    assert d(None, ALIGNED, 64, 128, ALIGNED, None) == INVALID
    assert d(ALIGNED, ALIGNED, 64, 128, None, None) == INVALID
    assert d(ALIGNED, ALIGNED, 60, 128, ALIGNED, None) == UNSUPPORTED
    assert d(ALIGNED, ALIGNED, 64, 128, MISALIGNED, None) == INVALID


def test_backward_takes_no_workspace(lib):
    """The input gradient dequantizes the weight on the fly: no workspace at any shape."""
    for T, K, N in [(1, 16, 8), (2048, 4096, 11008), (4096, 8192, 28672)]:
        assert lib.llmint8_backward_workspace_bytes(T, K, N) == 0


def test_blockwise_argument_errors(lib):
    qb, dq = lib.llmint8_quantize_blockwise, lib.llmint8_dequantize_blockwise
    F16, F32 = m8.LLMINT8_DTYPE_F16, m8.LLMINT8_DTYPE_F32
    assert qb(ALIGNED, 7, 4096, 64, ALIGNED, ALIGNED, None) == INVALID         # unknown dtype
    assert qb(None, F16, 4096, 64, ALIGNED, ALIGNED, None) == INVALID
    assert qb(ALIGNED, F16, 4096, 64, None, ALIGNED, None) == INVALID
    assert qb(ALIGNED, F32, 4096, 64, ALIGNED, None, None) == INVALID
    assert qb(ALIGNED, F16, -16, 64, ALIGNED, ALIGNED, None) == INVALID
    assert qb(MISALIGNED, F16, 4096, 64, ALIGNED, ALIGNED, None) == INVALID
    assert qb(ALIGNED, F16, 4104, 64, ALIGNED, ALIGNED, None) == UNSUPPORTED    # n % 16 != 0
    assert qb(ALIGNED, F16, 4096, 96, ALIGNED, ALIGNED, None) == UNSUPPORTED    # not a power of two
    assert qb(ALIGNED, F16, 4096, 8192, ALIGNED, ALIGNED, None) == UNSUPPORTED  # block > 4096
    assert qb(None, F16, 0, 64, None, None, None) == OK                         # empty: no-op
    assert dq(None, ALIGNED, 4096, 64, ALIGNED, F16, None) == INVALID
    assert dq(ALIGNED, ALIGNED, 4096, 64, MISALIGNED, F32, None) == INVALID
    assert dq(ALIGNED, ALIGNED, 4096, 32, ALIGNED, F32, None) == UNSUPPORTED


def test_ex_entry_points_argument_errors(lib):
    F16, BF16, F32 = m8.LLMINT8_DTYPE_F16, m8.LLMINT8_DTYPE_BF16, m8.LLMINT8_DTYPE_F32
    need = lib.llmint8_workspace_bytes(64, 1024, 1024)
    lx = lib.llmint8_linear_ex

    def call(dtype=BF16, bias=None, X=ALIGNED, ws_bytes=need):   # GEMM route (T = 64)
        return lx(X, dtype, 64, 1024, ALIGNED, ALIGNED, 1024, 6.0, bias, ALIGNED, ALIGNED,
                  ws_bytes, None)
    assert call(dtype=F32) == INVALID                  # fp32 activations are not a forward type
    assert call(dtype=7) == INVALID
    assert call(bias=ctypes.c_void_p(P + 1)) == INVALID  # bias needs 2-byte alignment
    assert call(X=None) == INVALID
    assert call(ws_bytes=need - 1) == WORKSPACE
    assert lx(None, F16, 0, 1024, ALIGNED, ALIGNED, 1024, 6.0, None, None, None, 0, None) == OK
    d = lib.llmint8_linear_debug_ex
    base = [ALIGNED, BF16, 64, 1024, ALIGNED, ALIGNED, 1024, 6.0, ALIGNED, ALIGNED, ALIGNED, need,
            None]
    assert d(*base, 7, None, None, None, None, None, None) == INVALID
    assert d(*base, m8.LLMINT8_PATH_GEMM, None, None, None, MISALIGNED, None, None) == INVALID
    q = lib.llmint8_quantize_weight_ex
    assert q(ALIGNED, F32, 16, 64, ALIGNED, ALIGNED, None) == INVALID
    assert q(None, BF16, 16, 64, ALIGNED, ALIGNED, None) == INVALID
    assert q(ALIGNED, BF16, 16, 72, ALIGNED, ALIGNED, None) == UNSUPPORTED
    assert q(MISALIGNED, BF16, 16, 64, ALIGNED, ALIGNED, None) == INVALID
    # the codec takes fp16 or fp32, not bf16
    assert lib.llmint8_quantize_blockwise(ALIGNED, BF16, 4096, 64, ALIGNED, ALIGNED, None) == INVALID


def test_4bit_code_books_match_the_oracle(lib):
    import numpy as np
    import oracle
    for name, code in (("nf4", m8.LLMINT8_QUANT_NF4), ("fp4", m8.LLMINT8_QUANT_FP4)):
        vals = (ctypes.c_float * 16)()
        assert lib.llmint8_code_book_4bit(code, vals) == OK
        got = np.array(list(vals), np.float32)
        assert np.array_equal(got.view(np.uint32), oracle.code_book(name).view(np.uint32)), name
    assert lib.llmint8_code_book_4bit(7, (ctypes.c_float * 16)()) == INVALID
    assert lib.llmint8_code_book_4bit(0, None) == INVALID


def test_4bit_argument_errors(lib):
    F16, BF16, F32 = m8.LLMINT8_DTYPE_F16, m8.LLMINT8_DTYPE_BF16, m8.LLMINT8_DTYPE_F32
    NF4, FP4 = m8.LLMINT8_QUANT_NF4, m8.LLMINT8_QUANT_FP4
    q, d, lin = lib.llmint8_quantize_4bit, lib.llmint8_dequantize_4bit, lib.llmint8_linear_4bit
    assert q(ALIGNED, F32, 4096, 64, NF4, ALIGNED, ALIGNED, None) == INVALID     # fp32 weight
    assert q(ALIGNED, F16, 4096, 64, 5, ALIGNED, ALIGNED, None) == INVALID       # unknown type
    assert q(None, F16, 4096, 64, NF4, ALIGNED, ALIGNED, None) == INVALID
    assert q(MISALIGNED, BF16, 4096, 64, FP4, ALIGNED, ALIGNED, None) == INVALID
    assert q(ALIGNED, F16, 4104, 64, NF4, ALIGNED, ALIGNED, None) == UNSUPPORTED  # n % 16
    assert q(ALIGNED, F16, 4096, 32, NF4, ALIGNED, ALIGNED, None) == UNSUPPORTED  # block < 64
    assert q(ALIGNED, F16, 4096, 96, NF4, ALIGNED, ALIGNED, None) == UNSUPPORTED
    assert q(None, F16, 0, 64, NF4, None, None, None) == OK                        # empty: no-op
    assert d(ALIGNED, ALIGNED, 4096, 64, NF4, MISALIGNED, F16, None) == INVALID
    assert d(None, ALIGNED, 4096, 64, FP4, ALIGNED, BF16, None) == INVALID

    def call(X=ALIGNED, dtype=F16, T=4, K=4096, block=64, qt=NF4, N=4096, bias=None, Y=ALIGNED):
        return lin(X, dtype, T, K, ALIGNED, ALIGNED, block, qt, N, bias, Y, None)
    assert call(dtype=F32) == INVALID
    assert call(qt=9) == INVALID
    assert call(X=None) == INVALID
    assert call(X=MISALIGNED) == INVALID
    assert call(bias=ctypes.c_void_p(P + 1)) == INVALID
    assert call(T=-1) == INVALID
    assert call(K=4160) == UNSUPPORTED              # K % 128 != 0
    assert call(block=100) == UNSUPPORTED
    assert call(N=1 << 20, K=4096) == UNSUPPORTED   # N K >= 2^31
    assert call(T=0, X=None, Y=None) == OK          # no-op


def test_timed_ex_argument_errors(lib):
    need = lib.llmint8_workspace_bytes(64, 1024, 1024)
    t = lib.llmint8_linear_timed_ex
    ev = (ctypes.c_void_p * 4)(P, P, P, P)
    nk = ctypes.c_int(0)
    base = [ALIGNED, m8.LLMINT8_DTYPE_BF16, 64, 1024, ALIGNED, ALIGNED, 1024, 6.0, None, ALIGNED,
            ALIGNED, need, None]
    assert t(*base, 0, None, 4, ctypes.byref(nk)) == INVALID
    assert t(*base, m8.LLMINT8_PATH_GEMM, ev, 2, ctypes.byref(nk)) == INVALID   # 3 kernels, 4 events
    bad = list(base)
    bad[1] = 9
    assert t(*bad, m8.LLMINT8_PATH_GEMM, ev, 4, ctypes.byref(nk)) == INVALID   # unknown dtype
