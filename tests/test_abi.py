"""C ABI checks that need no GPU: the library loads, exports every function
include/sbl.h declares, sizes match the packed-format definition, and host
validation rejects bad arguments before anything is enqueued (no compute
call is made here; only argument errors, which return before any HIP call)."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sbl.h")
LIB = os.path.join(ROOT, "sparse_linear_layers_bitlinear_amd", "libsbl.so")


@pytest.fixture(scope="module")
def S():
    if not os.path.exists(LIB):
        pytest.fail("libsbl.so is not built (run __graft_entry__.build())")
    from sparse_linear_layers_bitlinear_amd import sbl
    return sbl


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:sbl_status|const char\*)\s+(sbl_\w+)\(", text, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ["sbl_quant_act", "sbl_quant_mask_weight", "sbl_pack", "sbl_unpack", "sbl_gemm",
              "sbl_linear_fwd", "sbl_packed_bytes", "sbl_quant_mask_weight_workspace",
              "sbl_linear_fwd_workspace", "sbl_status_string", "sbl_version",
              "sbl_quant_mask_weight_batch", "sbl_quant_mask_weight_batch_workspace",
              "sbl_rmsnorm_quant_act", "sbl_act_dequant", "sbl_linear_bwd_dx",
              "sbl_linear_bwd_dw"]:
        assert n in names


def test_library_exports_every_declared_symbol(S):
    lib = ctypes.CDLL(LIB)
    for n in declared_functions():
        assert hasattr(lib, n), n
    assert S.lib.sbl_version().decode().startswith("sbl")
    for code in range(9):
        assert S.lib.sbl_status_string(code).decode().startswith("SBL_")


def test_packed_bytes_match_format(S):
    for N, M in [(n, 4) for n in range(1, 5)] + [(n, 8) for n in range(1, 9)]:
        for O, K in [(1, M), (7, 264 - 264 % M), (4864, 896), (2560, 6912), (3, 8 * 129)]:
            if K % M:
                continue
            assert S.sbl_packed_bytes(O, K, N, M) == o.packed_bytes(O, K, N, M)


FAKE = ctypes.c_void_p(0x10000)       # aligned, never dereferenced
MIS = ctypes.c_void_p(0x10008)        # misaligned


def test_quant_act_validation(S):
    L = S.lib
    assert L.sbl_quant_act(FAKE, 7, 4, 64, 64, 1e-5, FAKE, FAKE, None) == 4          # dtype
    assert L.sbl_quant_act(FAKE, 0, 4, 64, 32, 1e-5, FAKE, FAKE, None) == 2          # ldx < K
    assert L.sbl_quant_act(FAKE, 0, -1, 64, 64, 1e-5, FAKE, FAKE, None) == 2         # T < 0
    assert L.sbl_quant_act(FAKE, 0, 4, 0, 64, 1e-5, FAKE, FAKE, None) == 2           # K = 0
    assert L.sbl_quant_act(FAKE, 0, 4, 64, 64, 0.0, FAKE, FAKE, None) == 8           # eps
    assert L.sbl_quant_act(FAKE, 0, 4, 64, 64, float("nan"), FAKE, FAKE, None) == 8
    assert L.sbl_quant_act(None, 0, 4, 64, 64, 1e-5, FAKE, FAKE, None) == 1          # null
    assert L.sbl_quant_act(MIS, 0, 4, 64, 64, 1e-5, FAKE, FAKE, None) == 5           # align
    assert L.sbl_quant_act(None, 0, 0, 64, 64, 1e-5, None, None, None) == 0          # empty


def test_weight_side_validation(S):
    L = S.lib
    ws = 1 << 20
    args = lambda N, M, O, K, eps=1e-5, w=FAKE, g=FAKE, wsb=ws, wsp=FAKE: (
        w, 1, O, K, N, M, eps, None, None, FAKE, g, None, wsp, wsb, None)
    assert L.sbl_quant_mask_weight(*args(6, 8, 4, 12)) == 2       # K % M
    assert L.sbl_quant_mask_weight(*args(5, 4, 4, 16)) == 3       # N > M
    assert L.sbl_quant_mask_weight(*args(2, 16, 4, 16)) == 3      # M not 4/8
    assert L.sbl_quant_mask_weight(*args(0, 8, 4, 16)) == 3       # N = 0
    assert L.sbl_quant_mask_weight(*args(6, 8, 0, 16)) == 2       # O = 0 (gamma undefined)
    assert L.sbl_quant_mask_weight(*args(6, 8, 4, 16, eps=-1.0)) == 8
    assert L.sbl_quant_mask_weight(*args(6, 8, 4, 16, g=None)) == 1
    assert L.sbl_quant_mask_weight(*args(6, 8, 4, 16, wsb=16)) == 6
    assert L.sbl_quant_mask_weight(*args(6, 8, 4, 16, wsp=None)) == 6
    assert L.sbl_quant_mask_weight(*args(6, 8, 4, 16, w=MIS)) == 5
    assert L.sbl_quant_mask_weight(*args(6, 8, 1 << 16, 1 << 16)) == 2   # O*K >= 2^31
    n = ctypes.c_size_t()
    assert L.sbl_quant_mask_weight_workspace(4, 16, ctypes.byref(n)) == 0 and n.value > 0
    assert L.sbl_quant_mask_weight_workspace(0, 16, ctypes.byref(n)) == 2


def test_gemm_and_linear_validation(S):
    L = S.lib
    g = lambda T=4, O=8, K=64, N=6, M=8, inc=1, y=FAKE, ydt=0, sw=FAKE: (
        FAKE, FAKE, FAKE, sw, inc, T, O, K, N, M, y, ydt, None, None)
    assert L.sbl_gemm(*g(K=60)) == 2
    assert L.sbl_gemm(*g(N=9)) == 3
    assert L.sbl_gemm(*g(ydt=3)) == 4
    assert L.sbl_gemm(*g(inc=2)) == 2
    assert L.sbl_gemm(*g(y=None)) == 1
    assert L.sbl_gemm(*g(y=MIS)) == 5
    assert L.sbl_gemm(*g(T=0)) == 0           # empty: nothing enqueued
    assert L.sbl_gemm(*g(O=0)) == 0
    assert L.sbl_gemm(*g(K=(1 << 24) + 8)) == 2
    # every operand must stay below 2^31 bytes / elements (32-bit offsets):
    # xq [T,K], packed [O, pitch], y [T,O]; T and O below 2^31
    assert L.sbl_gemm(*g(T=1 << 31)) == 2
    assert L.sbl_gemm(*g(O=1 << 31)) == 2
    assert L.sbl_gemm(*g(T=1 << 21, K=1 << 10)) == 2                       # T K = 2^31
    pitch = o.packed_row_bytes(1 << 14, 6, 8)
    assert L.sbl_gemm(*g(T=4, O=-(-(1 << 31) // pitch), K=1 << 14)) == 2  # O pitch >= 2^31
    assert L.sbl_gemm(*g(T=1 << 16, O=1 << 15, K=64)) == 2                  # T O = 2^31
    assert L.sbl_gemm(*g(T=1 << 31, O=0)) == 2                              # checked before empty
    lf = lambda w=FAKE, pre=None, ws=FAKE, wsb=1 << 30, eps=1e-5, T=4: (
        FAKE, 0, w, 1, pre, FAKE, 0, T, 8, 64, 6, 8, eps, 1e-5, FAKE, 0, ws, wsb, None)
    assert L.sbl_linear_fwd(*lf(w=FAKE, pre=FAKE)) == 1      # both weight sources
    assert L.sbl_linear_fwd(*lf(w=None, pre=None)) == 1      # neither
    assert L.sbl_linear_fwd(*lf(wsb=8)) == 6
    assert L.sbl_linear_fwd(*lf(eps=0.0)) == 8
    assert L.sbl_linear_fwd(*lf(T=0)) == 0
    assert L.sbl_linear_fwd(*lf(T=1 << 31)) == 2
    assert L.sbl_linear_fwd(*lf(T=1 << 25)) == 2                             # T K = 2^31
    n = ctypes.c_size_t()
    assert L.sbl_linear_fwd_workspace(16, 128, 256, 6, 8, 0, ctypes.byref(n)) == 0
    assert n.value >= 16 * 256 + o.packed_bytes(128, 256, 6, 8)
    n2 = ctypes.c_size_t()
    assert L.sbl_linear_fwd_workspace(16, 128, 256, 6, 8, 1, ctypes.byref(n2)) == 0
    assert n2.value < n.value


def test_noalloc_prep_validation(S):
    """The allocation-free preparation validates like the workspace entry
    point, before it looks at any device (no GPU needed for these)."""
    L = S.lib
    a = lambda wdt=1, O=8, K=64, N=6, M=8, eps=1e-5, w=FAKE, g=FAKE: (
        w, wdt, O, K, N, M, eps, None, None, None, g, None, None)
    assert L.sbl_quant_mask_weight_noalloc(*a(wdt=5)) == 4
    assert L.sbl_quant_mask_weight_noalloc(*a(K=60)) == 2
    assert L.sbl_quant_mask_weight_noalloc(*a(O=0)) == 2
    assert L.sbl_quant_mask_weight_noalloc(*a(O=1 << 20, K=1 << 11)) == 2    # O K = 2^31
    assert L.sbl_quant_mask_weight_noalloc(*a(N=0)) == 3
    assert L.sbl_quant_mask_weight_noalloc(*a(eps=0.0)) == 8
    assert L.sbl_quant_mask_weight_noalloc(*a(w=None)) == 1
    assert L.sbl_quant_mask_weight_noalloc(*a(g=None)) == 1
    assert L.sbl_quant_mask_weight_noalloc(*a(w=MIS)) == 5


def test_pack_validation(S):
    L = S.lib
    assert L.sbl_pack(FAKE, FAKE, 4, 12, 6, 8, FAKE, None) == 2
    assert L.sbl_pack(None, FAKE, 4, 16, 6, 8, FAKE, None) == 1
    assert L.sbl_unpack(FAKE, 4, 16, 6, 8, MIS, FAKE, None) == 5
    assert L.sbl_pack(FAKE, FAKE, 0, 16, 6, 8, FAKE, None) == 0


def test_weight_batch_validation(S):
    L = S.lib
    WP = S.WeightPrep
    ws = 1 << 20

    def items(*specs):
        arr = (WP * max(1, len(specs)))()
        for i, (O, K, w, g) in enumerate(specs):
            arr[i] = WP(w, O, K, None, None, FAKE, g, None)
        return arr

    ok = (64, 256, FAKE, FAKE)
    call = lambda arr, cnt, N=6, M=8, dt=1, eps=1e-5, wsp=FAKE, wsb=ws: \
        L.sbl_quant_mask_weight_batch(arr, cnt, dt, N, M, eps, wsp, wsb, None)
    assert call(None, 1) == 1                                     # no items
    assert call(items(ok), 0) == 2                                # count < 1
    assert call(items(*[ok] * 9), 9) == 2                         # count > max
    assert call(items(ok), 1, dt=5) == 4                          # dtype
    assert call(items(ok), 1, eps=0.0) == 8                       # eps
    assert call(items(ok, (64, 252, FAKE, FAKE)), 2) == 2         # second item K % M
    assert call(items(ok, (64, 256, FAKE, None)), 2) == 1         # second item gamma_sw
    assert call(items(ok, (64, 256, MIS, FAKE)), 2) == 5          # second item misaligned
    assert call(items(ok), 1, N=9) == 3                           # N:M
    assert call(items(ok, ok, ok), 3, wsb=16) == 6                # workspace size
    assert call(items(ok), 1, wsp=None) == 6
    diag = items(ok)
    diag[0].prev_mask_bits = FAKE                                 # previous mask without flips
    assert call(diag, 1) == 1
    diag = items(ok)
    diag[0].flips = FAKE                                          # flips without previous mask
    assert call(diag, 1) == 1
    diag = items(ok)
    diag[0].prev_mask_bits = FAKE                                 # flips without the new mask bits
    diag[0].flips = FAKE
    assert call(diag, 1) == 1
    diag = items(ok)
    diag[0].variant = 7                                           # unknown recipe
    assert call(diag, 1) == 8
    diag = items(ok, ok)
    diag[1].variant = 2                                           # mask-then-quant mixed in
    assert call(diag, 2) == 8
    diag = items(ok)
    diag[0].group_thr = MIS                                       # misaligned diagnostics output
    assert call(diag, 1) == 5
    n = ctypes.c_size_t()
    for cnt in range(1, 9):
        assert L.sbl_quant_mask_weight_batch_workspace(cnt, ctypes.byref(n)) == 0
        assert n.value >= cnt * 128
    single = ctypes.c_size_t()
    assert L.sbl_quant_mask_weight_workspace(64, 256, ctypes.byref(single)) == 0
    assert L.sbl_quant_mask_weight_batch_workspace(1, ctypes.byref(n)) == 0 and n.value == single.value
    assert L.sbl_quant_mask_weight_batch_workspace(0, ctypes.byref(n)) == 2
    assert L.sbl_quant_mask_weight_batch_workspace(9, ctypes.byref(n)) == 2


def test_backward_validation(S):
    """Host-side checks of the Dual-STE backward calls (no launch happens)."""
    L = S.lib
    I64 = ctypes.c_int64
    segs = lambda *r: (I64 * max(1, len(r)))(*r)
    dx = lambda dy=FAKE, ldy=256, pk=FAKE, sw=FAKE, T=32, O=256, K=128, N=6, M=8, sg=None, ns=1, \
        out=FAKE, dt=0, ld=128, acc=0: L.sbl_linear_bwd_dx(dy, ldy, pk, sw, T, O, K, N, M, sg, ns,
                                                         out, dt, ld, acc, None)
    assert dx(dt=3) == 4                                    # dtype
    assert dx(N=9) == 3                                     # N:M
    assert dx(O=252, ldy=256) == 2                          # O % 8
    assert dx(K=124) == 2                                   # K % 8
    assert dx(K=132, ld=132, M=8) == 2                      # K % 8 (and % M)
    assert dx(ldy=250) == 2                                 # ldy < O
    assert dx(ld=64) == 2                                   # lddx < K
    assert dx(ns=5) == 2                                    # too many segments
    assert dx(ns=2) == 1                                    # segments missing
    assert dx(ns=2, sg=segs(128, 120)) == 2                 # do not sum to O
    assert dx(ns=2, sg=segs(124, 132)) == 2                 # not multiples of 8
    assert dx(T=0, dy=None, pk=None, sw=None, out=None) == 0  # empty call
    assert dx(dy=None) == 1
    assert dx(sw=None) == 1
    assert dx(out=MIS) == 5
    assert dx(dy=MIS) == 5
    dw = lambda dy=FAKE, ldy=256, xt=FAKE, T=32, O=256, K=128, out=FAKE, dt=1, keep=None: \
        L.sbl_linear_bwd_dw(dy, ldy, xt, T, O, K, keep, out, dt, None)
    assert dw(dt=2) == 4
    assert dw(O=0) == 2
    assert dw(K=100) == 2
    assert dw(T=-1) == 2
    assert dw(out=None) == 1
    assert dw(xt=None) == 1
    assert dw(xt=MIS) == 5
    assert dw(keep=MIS) == 5                                # keep bits misaligned
    assert L.sbl_act_dequant(FAKE, FAKE, 4, 12, FAKE, None) == 2   # K % 8
    assert L.sbl_act_dequant(FAKE, FAKE, 0, 16, None, None) == 0   # empty
    assert L.sbl_act_dequant(FAKE, None, 4, 16, FAKE, None) == 1
    assert L.sbl_act_dequant(FAKE, FAKE, 4, 16, MIS, None) == 5

