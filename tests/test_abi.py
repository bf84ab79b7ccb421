"""The C-ABI library without a GPU: it loads, exports every entry point include/dg.h
declares, and rejects bad arguments before any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    import moe_grouped_gemm_e4m3_amd as m
    if not os.path.exists(m.LIB_PATH):
        from moe_grouped_gemm_e4m3_amd import build
        build.build()
    return m.lib()


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("dg_cast_fp8_per_token", "dg_gemm_fp8_nt", "dg_grouped_gemm_contiguous",
              "dg_grouped_gemm_masked", "dg_status_string", "dg_last_error_message"):
        assert n in names


def test_library_exports_every_declared_symbol(L):
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_library_exports_only_the_c_abi(L):
    # the dynamic symbol table holds exactly the dg_* functions the header declares: no C++
    # internals or compiler-generated symbols another loaded library could bind to
    import shutil
    import subprocess
    import moe_grouped_gemm_e4m3_amd as m
    nm = shutil.which("nm") or shutil.which("llvm-nm")
    if nm is None:
        pytest.skip("no nm on PATH")
    out = subprocess.run([nm, "-D", "--defined-only", m.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines() if line.strip())
    assert exported == _declared_functions()


def test_ffn_noalloc_argument_errors(L):
    f = L.dg_moe_ffn_fp8_noalloc
    # masked G=1, M_max=15888, H=128, I=2048: 2112 bytes per row exceed the 32 MiB scratch
    assert f(2, 0, P, P, P, P, P, P, P, P, 1, 15888, 128, 2048, 0, None) == 2
    assert b"static scratch" in L.dg_last_error_message()
    assert f(1, 0, P, P, P, P, P, P, P, P, 4, 16000, 128, 2048, 0, None) == 2  # contiguous rows too
    assert f(2, 0, P, P, P, P, P, P, P, None, 4, 64, 256, 128, 0, None) == 1   # y missing
    assert f(2, 0, P, P, P, P, Q, P, P, P, 4, 64, 256, 128, 0, None) == 3      # w2 misaligned
    assert f(2, 0, P, P, P, P, P, P, P, P, 4, 64, 256, 100, 0, None) == 2      # I not a multiple of 128
    assert f(2, 0, None, None, None, None, None, None, None, None, 0, 64, 256, 128, 0, None) == 0  # empty


def test_convert_argument_errors(L):
    assert L.dg_convert_fp8_e4m3(P, 6, P, None) == 2   # not a multiple of 4
    assert L.dg_convert_fp8_e4m3(P, -4, P, None) == 1
    assert L.dg_convert_fp8_e4m3(None, 8, P, None) == 1
    assert L.dg_convert_fp8_e4m3(Q, 8, P, None) == 3
    assert L.dg_convert_fp8_e4m3(None, 0, None, None) == 0  # empty: nothing enqueued


def test_masked_cast_argument_errors(L):
    c = L.dg_cast_fp8_per_token_masked
    assert c(P, 0, 0, 4, 64, 500, P, P, P, None) == 2    # K not a multiple of 128
    assert c(P, 2, 0, 4, 64, 512, P, P, P, None) == 1    # unknown dtype
    assert c(P, 0, 7, 4, 64, 512, P, P, P, None) == 1    # unknown scale format
    assert c(P, 0, 0, -1, 64, 512, P, P, P, None) == 1
    assert c(P, 0, 0, 4, 64, 512, None, P, P, None) == 1  # masked_m null
    assert c(P, 0, 0, 4, 64, 512, Q, P, P, None) == 3
    assert c(None, 0, 0, 0, 64, 512, None, None, None, None) == 0  # G = 0: nothing enqueued


def test_status_strings(L):
    for code, name in [(0, b"DG_OK"), (1, b"DG_ERR_INVALID_ARGUMENT"), (2, b"DG_ERR_UNSUPPORTED_SHAPE"),
                       (3, b"DG_ERR_MISALIGNED"), (4, b"DG_ERR_UNSUPPORTED_DEVICE"), (5, b"DG_ERR_LAUNCH")]:
        assert L.dg_status_string(code) == name


P = 0x10000  # an aligned fake address: validation never dereferences pointers
Q = 0x10001  # misaligned


def _gemm(L, a=P, sfa=P, b=P, sfb=P, d=P, M=64, N=256, K=512):
    return L.dg_gemm_fp8_nt(a, sfa, b, sfb, d, M, N, K, None)


def test_gemm_argument_errors(L):
    assert _gemm(L, K=500) == 2
    assert _gemm(L, K=0) == 2
    assert _gemm(L, N=200) == 2
    assert _gemm(L, M=-1) == 1
    assert _gemm(L, N=-128) == 1
    assert _gemm(L, a=None) == 1
    assert _gemm(L, d=None) == 1
    assert _gemm(L, sfb=Q) == 3
    assert b"16-byte" in L.dg_last_error_message()
    assert _gemm(L, M=0) == 0          # empty: nothing to do, nothing touched
    assert _gemm(L, M=0, a=None) == 0
    assert L.dg_last_error_message() == b""


def test_gemm_without_gpu_reports_device(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert _gemm(L) == 4  # arguments valid, no gfx950 device: nothing launched
    assert L.dg_cast_fp8_per_token_masked(P, 0, 1, 4, 64, 512, P, P, P, None) == 4


def test_grouped_argument_errors(L):
    c = L.dg_grouped_gemm_contiguous
    assert c(P, P, P, P, P, P, 4, 1000, 256, 512, None) == 2   # M_total % 128
    assert c(P, P, P, P, P, P, 0, 1024, 256, 512, None) == 1   # G < 1
    assert c(P, P, P, P, None, P, 4, 1024, 256, 512, None) == 1  # m_indices null
    assert c(P, P, P, P, P, P, 4, 0, 256, 512, None) == 0
    m = L.dg_grouped_gemm_masked
    assert m(P, P, P, P, P, P, 4, 64, 256, 500, 0, None) == 2
    assert m(P, P, P, P, P, P, -1, 64, 256, 512, 0, None) == 1
    assert m(P, P, P, P, P, P, 0, 64, 256, 512, 0, None) == 0  # G = 0: empty
    assert m(P, P, P, P, None, P, 4, 64, 256, 512, 0, None) == 1
    assert m(P, P, P, P, Q, P, 4, 64, 256, 512, 0, None) == 3
    s = L.dg_gemm_fp8_scheduled
    assert s(7, 0, 0, P, P, P, P, P, P, 1, 64, 256, 512, 0, None) == 1
    assert s(0, 9, 0, P, P, P, P, P, P, 1, 64, 256, 512, 0, None) == 1
    assert s(0, 0, 5, P, P, P, P, P, P, 1, 64, 256, 512, 0, None) == 1  # unknown scale format
    u = L.dg_gemm_fp8_nt_ue8m0
    assert u(P, P, P, P, P, 64, 256, 500, None) == 2
    assert u(P, P, P, P, P, 0, 256, 512, None) == 0


def test_cast_argument_errors(L):
    t = L.dg_cast_fp8_per_token
    assert t(P, 0, 1, 64, 500, P, P, None) == 2
    assert t(P, 2, 1, 64, 512, P, P, None) == 1  # unknown dtype
    assert t(None, 0, 1, 64, 512, P, P, None) == 1
    assert t(P, 0, 1, 64, 512, Q, P, None) == 3
    assert t(P, 0, 1, 0, 512, P, P, None) == 0
    assert t(P, 0, 0, 64, 512, P, P, None) == 0   # G = 0: empty
    assert t(P, 0, -1, 64, 512, P, P, None) == 1
    assert t(P, 0, 1 << 20, 1 << 12, 512, P, P, None) == 2  # G*M >= 2^31
    b = L.dg_cast_fp8_per_block
    assert b(P, 0, 100, 512, P, P, None) == 2
    assert b(P, 1, 128, 384, P, Q, None) == 3


def test_swiglu_and_ffn_argument_errors(L):
    w = L.dg_gemm_fp8_swiglu
    #        layout fmt a  sfa b  sfb meta hq sfh G  M     I    K
    assert w(3, 0, P, P, P, P, P, P, P, 4, 1024, 256, 512, 0, None) == 1      # unknown layout
    assert w(1, 2, P, P, P, P, P, P, P, 4, 1024, 256, 512, 0, None) == 1      # unknown scale format
    assert w(1, 0, P, P, P, P, P, P, P, 4, 1024, 192, 512, 0, None) == 2      # I % 128
    assert w(1, 0, P, P, P, P, P, P, P, 4, 1000, 256, 512, 0, None) == 2      # M_total % 128
    assert w(1, 0, P, P, P, P, P, P, P, 4, 1024, 256, 500, 0, None) == 2      # K % 128
    assert w(1, 0, P, P, P, P, P, P, P, 4, 1024, 256, 128 * 257, 0, None) == 2  # K > 32768
    assert w(2, 0, P, P, P, P, P, P, P, 4, 1 << 20, 256, 1 << 13, 0, None) == 2  # rows*K >= 2^32
    assert w(1, 0, P, P, P, P, None, P, P, 4, 1024, 256, 512, 0, None) == 1   # m_indices null
    assert w(2, 0, P, P, P, P, P, None, P, 4, 64, 256, 512, 0, None) == 1     # hq null
    assert w(2, 0, P, P, P, P, P, P, Q, 4, 64, 256, 512, 0, None) == 3        # sfh misaligned
    assert w(0, 0, P, P, P, P, None, P, P, 0, 64, 256, 512, 0, None) in (0, 4)  # dense ignores meta and G
    assert w(2, 0, P, P, P, P, P, P, P, 0, 64, 256, 512, 0, None) == 0        # G = 0: empty
    assert w(1, 0, P, P, P, P, P, P, P, 4, 0, 256, 512, 0, None) == 0         # M = 0: empty
    f = L.dg_moe_ffn_fp8
    #        layout fmt x  sfx w1 s1 w2 s2 meta hq sfh y  G  M     H    I
    assert f(1, 0, P, P, P, P, P, P, P, P, P, P, 4, 1024, 384, 256, 0, None) in (0, 4)
    assert f(1, 0, P, P, P, P, P, P, P, P, P, P, 4, 1024, 300, 256, 0, None) == 2  # H % 128
    assert f(1, 0, P, P, P, P, None, P, P, P, P, P, 4, 1024, 384, 256, 0, None) == 1  # w2 null
    assert f(1, 0, P, P, P, P, P, P, P, P, P, Q, 4, 1024, 384, 256, 0, None) == 3     # y misaligned
    assert f(2, 1, P, P, P, P, P, P, P, P, P, P, 0, 64, 384, 256, 0, None) == 0       # empty


def test_swiglu_without_gpu_reports_device(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert L.dg_gemm_fp8_swiglu(1, 0, P, P, P, P, P, P, P, 4, 1024, 256, 512, 0, None) == 4
    assert L.dg_moe_ffn_fp8(2, 0, P, P, P, P, P, P, P, P, P, P, 4, 64, 384, 256, 16, None) == 4
