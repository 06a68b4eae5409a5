"""The C-ABI library loads on the host, exports every symbol its header
declares, and rejects invalid arguments with the documented status before
any launch (host-side checks only: no compute call needs a GPU here)."""
import ctypes
import os
import re

import pytest

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a4_moe.h")


def _lib():
    from precision_rl_amd import build, binding
    if not os.path.exists(build.LIB):
        build.build()
    return binding.load()


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w4a4_[a-z_]+)\s*\(", text)))


def test_header_declares_the_three_calls():
    syms = declared_symbols()
    for name in ("w4a4_quantize_permute", "w4a4_grouped_expert_fwd", "w4a4_expert_bwd"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name


def test_capacity_and_workspace_sizes():
    lib = _lib()
    assert lib.w4a4_rows_capacity(16384, 8, 128, 1) == 131072
    assert lib.w4a4_rows_capacity(10, 2, 8, 16) == 20 + 8 * 15
    assert lib.w4a4_rows_capacity(10, 2, 8, 3) == -1
    assert lib.w4a4_workspace_size(1, 8192, 2048, 768, 128, 8, 1) > 0
    assert lib.w4a4_workspace_size(7, 8192, 2048, 768, 128, 8, 1) == 0


def test_invalid_arguments_rejected_before_launch():
    lib = _lib()
    from precision_rl_amd import binding as b
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.c_void_p(ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16)

    def qp(T=4, K=32, idx=p, k=2, E=8, A=1, x=p, ws=p, wsb=1024):
        return lib.w4a4_quantize_permute(x, T, K, idx, k, E, A, p, p, p, p, p, p, ws, wsb, None)

    assert qp(K=24) == -1                              # K % 16 != 0
    assert qp(A=3) == -1                               # bad row_align
    assert qp(k=9, E=8) == -1                          # k > E
    assert qp(k=9, E=16) == -2                         # k > 8 unsupported
    assert qp(x=None) == -1                            # null input
    assert qp(x=ctypes.c_void_p(p.value + 2)) == -1    # misaligned
    assert qp(ws=None) == -3                           # no workspace
    assert qp(idx=None, k=2) == -1                     # identity needs k = 1
    assert b.load().w4a4_last_error().decode()
    assert lib.w4a4_status_string(-3).decode() == "workspace missing or too small"

    def fwd(H=256, I=128, T=4, ws=p, wsb=1 << 40):
        return lib.w4a4_grouped_expert_fwd(T, H, I, 8, 2, 1, p, p, p, p, p, p, p, p, p, p, p, p, p,
                                           p, None, None, None, None, None, None, ws, wsb, None)

    assert fwd(H=250) == -1                            # not a multiple of 32
    assert fwd(H=288) == -2                            # multiple of 32 but not of 256
    assert fwd(I=96) == -2
    assert fwd(ws=None) == -3
    assert fwd(wsb=16) == -3

    def bwd(H=256, I=128, T=4):
        return lib.w4a4_expert_bwd(T, H, I, 8, 2, 1, p, p, p, p, p, p, p, p, p, p, p, p, p,
                                   None, 0, None)

    assert bwd() == -3                                 # no workspace
    assert bwd(I=100) == -1

    def qpd(T=4, K=64, G=1, wsb=1 << 20):
        return lib.w4a4_quantize_permute_domain(p, T, K, p, 2, 8, 1, G, p, p, p, p, p, p, p, wsb, None)

    assert qpd(K=48) == -2                             # grouped scales need K % 32 == 0
    assert qpd(K=8192) == -2                           # and K <= 4096
    assert qpd(G=0) == -1                              # group_rows >= 1
    assert qpd(wsb=0) == -3
    assert lib.w4a4_workspace_size(4, 4, 64, 0, 8, 2, 1) >= lib.w4a4_workspace_size(0, 4, 64, 0, 8, 2, 1)

    def lin_fwd(K=256, N=256, T=4):
        return lib.w4a4_linear_fwd(T, K, N, p, p, p, p, p, p, p, p, None)

    def lin_bwd(K=256, N=256, T=4, ws=p, wsb=1 << 20):
        return lib.w4a4_linear_bwd(T, K, N, p, p, p, p, p, p, ws, wsb, None)

    assert lin_fwd(K=128) == -2                        # K % 256
    assert lin_fwd(N=384) == -2                        # N % 256
    assert lin_fwd(T=-1) == -1
    assert lin_bwd(ws=None) == -3
    assert lib.w4a4_workspace_size(3, 0, 256, 256, 1, 1, 1) > 0
    assert lib.w4a4_workspace_size(3, 0, 128, 256, 1, 1, 1) == 0


def test_mx_calls_reject_invalid_arguments_before_launch():
    lib = _lib()
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.c_void_p(ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16)

    def mqp(T=4, K=64, idx=p, k=2, E=8, A=1, x=p, ws=p, wsb=1 << 20):
        return lib.w4a4_mx_quantize_permute(x, T, K, idx, k, E, A, p, p, p, p, p, ws, wsb, None)

    assert mqp(K=48) == -2                             # MX blocks of 32: K % 32 == 0
    assert mqp(K=24) == -1                             # not even a multiple of 16
    assert mqp(K=8192) == -2                           # K <= 4096
    assert mqp(k=9, E=8) == -1
    assert mqp(x=None) == -1
    assert mqp(ws=None) == -3
    assert mqp(idx=None, k=2) == -1

    def mfwd(H=256, I=128, T=4, ws=p, wsb=1 << 40, dc=None, ds=None):
        return lib.w4a4_mx_grouped_expert_fwd(T, H, I, 8, 2, 1, p, p, p, p, p, p, p, p, p, p,
                                              p, None, None, None, dc, ds, ws, wsb, None)

    assert mfwd(H=250) == -1
    assert mfwd(H=288) == -2
    assert mfwd(I=96) == -2
    assert mfwd(ws=None) == -3
    assert mfwd(dc=p) == -1                            # debug codes without debug scales


def test_mx8_backward_rejects_invalid_arguments_before_launch():
    lib = _lib()
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.c_void_p(ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16)

    def bwd(H=256, I=256, T=4, A=128, ws=p, wsb=1 << 40):
        return lib.w4a4_mx8_expert_bwd(T, H, I, 8, 2, A, p, p, p, p, p, p, p, p, p, p, p, p, p,
                                       ws, wsb, None)

    assert bwd(A=16) == -2                             # row blocks of 32 per expert: row_align 128
    assert bwd(I=128) == -2                            # I % 256
    assert bwd(ws=None) == -3
    assert bwd(wsb=16) == -3
    assert bwd(H=250) == -1
    assert lib.w4a4_workspace_size(5, 64, 256, 256, 8, 2, 128) > lib.w4a4_workspace_size(2, 64, 256, 256, 8, 2, 128)

    def q8(R=128, C=128, pitch=128, x=p):
        return lib.w4a4_mx8_quantize(x, R, C, p, p, p, p, pitch, None)

    assert q8(R=96) == -2                              # whole 128-row tiles
    assert q8(C=64) == -2                              # C % 128
    assert q8(pitch=64) == -1                          # pitch >= R
    assert q8(x=None) == -1


def test_shape_floor_and_row_limits_rejected_before_launch():
    """The documented shape floor: H, I multiples of 32 are valid arguments,
    but the kernels take H % 256 == 0 and I % 128 == 0 (UNSUPPORTED, with the
    reason in last_error); the padded row count must fit int32 row indices;
    the MXFP4 forward's FC2-input encoder takes I <= 4096.  All are refused
    before anything is launched."""
    lib = _lib()
    from precision_rl_amd import binding as b
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.c_void_p(ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16)

    def fwd(H=2048, I=768, T=4, A=1, E=8):
        return lib.w4a4_grouped_expert_fwd(T, H, I, E, 2, A, p, p, p, p, p, p, p, p, p, p, p, p, p,
                                           p, None, None, None, None, None, None, p, 1 << 40, None)

    assert fwd(H=288, I=160) == -2
    assert "256" in b.load().w4a4_last_error().decode()
    assert fwd(H=2048, I=160) == -2
    assert fwd(H=2049) == -1
    assert fwd(T=(1 << 30), A=128, E=1024) == -2       # T*k + E*(A-1) >= 2^31
    assert "int32" in b.load().w4a4_last_error().decode()

    def qp(T=4, k=2, E=8, A=1):
        return lib.w4a4_quantize_permute(p, T, 64, p, k, E, A, p, p, p, p, p, p, p, 1 << 30, None)

    assert qp(T=(1 << 28) - 1, k=8, E=1024, A=128) == -2   # T*k < 2^31 but the padded rows are not

    def mfwd(H=256, I=8192 - 128):
        return lib.w4a4_mx_grouped_expert_fwd(4, H, I, 8, 2, 1, p, p, p, p, p, p, p, p, p, p,
                                              p, None, None, None, None, None, p, 1 << 40, None)

    assert mfwd() == -2
    assert "4096" in b.load().w4a4_last_error().decode()


def test_check_routing_rejects_invalid_arguments_before_launch():
    lib = _lib()
    buf = ctypes.create_string_buffer(4096)
    p = ctypes.c_void_p(ctypes.addressof(buf) + (-ctypes.addressof(buf)) % 16)
    assert lib.w4a4_check_routing(p, 4, 9, 16, p, None) == -2          # k <= 8
    assert lib.w4a4_check_routing(p, 4, 0, 16, p, None) == -1
    assert lib.w4a4_check_routing(p, -1, 2, 16, p, None) == -1
    assert lib.w4a4_check_routing(p, 4, 2, 16, None, None) == -1       # no error word
    assert lib.w4a4_check_routing(None, 4, 2, 16, p, None) == -1       # no ids for T > 0
    assert lib.w4a4_check_routing(p, 4, 2, 16, ctypes.c_void_p(p.value + 4), None) == -1
