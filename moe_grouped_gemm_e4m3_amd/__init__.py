"""Thin Python binding over libdg.so, the C ABI declared in include/dg.h.

Argument marshalling only: every step of the path runs in the HIP kernels of libdg.so.
PyTorch supplies device memory and the current stream; FP8 tensors travel as torch.uint8
(raw OCP E4M3FN bytes) and bf16 outputs as torch.bfloat16. There is no CPU fallback:
if libdg.so is missing or fails to load, every call raises.

Every entry point takes ue8m0=False; ue8m0=True selects the power-of-two (UE8M0) scale
variants (the casts round each scale up to a power of two; the GEMMs require such scales).

Activation scales are K-block-major ([K/128, M], leading [G] for the masked layout), as
include/dg.h specifies; weight scales are [N/128, K/128].

Entry points (same names as the C ABI, without the dg_ prefix):
  cast_fp8_per_token(x)                      -> (q [M,K] uint8, sf [K/128,M] fp32)
                                                (x [G,M,K] -> q [G,M,K], sf [G,K/128,M])
  cast_fp8_per_token_masked(x, masked_m)     -> (q [G,M_max,K], sf [G,K/128,M_max]): valid rows only
  cast_fp8_per_block(w)                      -> (q [N,K] uint8, sf [N/128,K/128] fp32)
  convert_fp8_e4m3(x)                        -> q uint8: the hardware conversion of the SwiGLU epilogue
  gemm_fp8_nt(a, sfa, b, sfb)                -> d [M,N] bf16
  grouped_gemm_contiguous(a, sfa, b, sfb, m_indices)      -> d [M_total,N] bf16
  grouped_gemm_masked(a, sfa, b, sfb, masked_m, expected_m) -> d [G,M_max,N] bf16
  gemm_fp8_swiglu(layout, a, sfa, w1, sfw1, meta)         -> (hq, sfh): the FP8 SwiGLU activation
  moe_ffn_fp8(layout, x, sfx, w1, sfw1, w2, sfw2, meta)    -> (y bf16, hq, sfh): the expert FFN
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdg.so")

DG_OK = 0
STATUS_NAMES = {0: "DG_OK", 1: "DG_ERR_INVALID_ARGUMENT", 2: "DG_ERR_UNSUPPORTED_SHAPE",
                3: "DG_ERR_MISALIGNED", 4: "DG_ERR_UNSUPPORTED_DEVICE", 5: "DG_ERR_LAUNCH"}
LAYOUT_DENSE, LAYOUT_CONTIGUOUS, LAYOUT_MASKED = 0, 1, 2
SCALE_F32, SCALE_UE8M0 = 0, 1
SCHED_AUTO, SCHED_DECODE, SCHED_TILE128, SCHED_TILE256 = 0, 1, 2, 3
INPUT_F32, INPUT_BF16 = 0, 1


class DGError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, status), message))
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    """Load libdg.so (built by moe_grouped_gemm_e4m3_amd.build); raises if it is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libdg.so is not built: run `python -m moe_grouped_gemm_e4m3_amd.build` "
                              "or __graft_entry__.build()")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        for sfx in ("", "_ue8m0"):
            getattr(L, "dg_cast_fp8_per_token" + sfx).argtypes = [P, ctypes.c_int, I64, I64, I64, P, P, P]
            getattr(L, "dg_cast_fp8_per_block" + sfx).argtypes = [P, ctypes.c_int, I64, I64, P, P, P]
            getattr(L, "dg_gemm_fp8_nt" + sfx).argtypes = [P, P, P, P, P, I64, I64, I64, P]
            getattr(L, "dg_grouped_gemm_contiguous" + sfx).argtypes = [P, P, P, P, P, P, I32, I64, I64, I64, P]
            getattr(L, "dg_grouped_gemm_masked" + sfx).argtypes = [P, P, P, P, P, P, I32, I64, I64, I64, I64, P]
            for fn in ("dg_cast_fp8_per_token", "dg_cast_fp8_per_block", "dg_gemm_fp8_nt",
                       "dg_grouped_gemm_contiguous", "dg_grouped_gemm_masked"):
                getattr(L, fn + sfx).restype = ctypes.c_int
        L.dg_cast_fp8_per_token_masked.argtypes = [P, ctypes.c_int, I32, I32, I64, I64, P, P, P, P]
        L.dg_cast_fp8_per_token_masked.restype = ctypes.c_int
        L.dg_gemm_fp8_scheduled.argtypes = [I32, I32, I32, P, P, P, P, P, P, I32, I64, I64, I64, I64, P]
        L.dg_gemm_fp8_swiglu.argtypes = [I32, I32, P, P, P, P, P, P, P, I32, I64, I64, I64, I64, P]
        L.dg_moe_ffn_fp8.argtypes = [I32, I32, P, P, P, P, P, P, P, P, P, P, I32, I64, I64, I64, I64, P]
        L.dg_gemm_fp8_scheduled.restype = ctypes.c_int
        L.dg_moe_ffn_fp8_noalloc.argtypes = [I32, I32, P, P, P, P, P, P, P, P, I32, I64, I64, I64, I64, P]
        L.dg_moe_ffn_fp8_noalloc.restype = ctypes.c_int
        L.dg_convert_fp8_e4m3.argtypes = [P, I64, P, P]
        L.dg_convert_fp8_e4m3.restype = ctypes.c_int
        L.dg_reload_tuning_switches.argtypes = []
        L.dg_reload_tuning_switches.restype = None
        L.dg_status_string.argtypes = [ctypes.c_int]
        L.dg_status_string.restype = ctypes.c_char_p
        L.dg_last_error_message.argtypes = []
        L.dg_last_error_message.restype = ctypes.c_char_p
        _lib = L
    return _lib


def reload_tuning_switches() -> None:
    """Makes the library re-read its DG_* tuning switches from the environment (it reads them
    once per process otherwise)."""
    lib().dg_reload_tuning_switches()


def _check(status: int) -> None:
    if status != DG_OK:
        raise DGError(status, lib().dg_last_error_message().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device: torch.device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t: torch.Tensor, dtype: torch.dtype, name: str) -> None:
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if not t.is_cuda:
        raise TypeError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


# ---- casts ---------------------------------------------------------------------------
def cast_fp8_per_token(x: torch.Tensor, q: torch.Tensor | None = None, sf: torch.Tensor | None = None,
                       ue8m0: bool = False):
    """x [M,K] or [G,M,K] fp32/bf16 -> (q uint8 e4m3 of x's shape, sf fp32 [K/128,M] or
    [G,K/128,M]: K-block-major, the sfa layout of the GEMMs)."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _need(x, x.dtype, "x")
    if x.dim() not in (2, 3):
        raise ValueError("x must be [M,K] or [G,M,K]")
    G = x.shape[0] if x.dim() == 3 else 1
    M, K = x.shape[-2:]
    lead = tuple(x.shape[:-2])
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    sf = torch.empty(lead + (K // 128, M), dtype=torch.float32, device=x.device) if sf is None else sf
    if tuple(q.shape) != tuple(x.shape) or tuple(sf.shape) != lead + (K // 128, M):
        raise ValueError("q %s / sf %s do not match x %s" % (tuple(q.shape), tuple(sf.shape), tuple(x.shape)))
    dt = INPUT_BF16 if x.dtype == torch.bfloat16 else INPUT_F32
    fn = lib().dg_cast_fp8_per_token_ue8m0 if ue8m0 else lib().dg_cast_fp8_per_token
    _check(fn(_ptr(x), dt, G, M, K, _ptr(q), _ptr(sf), _stream(x.device)))
    return q, sf


def cast_fp8_per_token_masked(x: torch.Tensor, masked_m: torch.Tensor, q: torch.Tensor | None = None,
                              sf: torch.Tensor | None = None, ue8m0: bool = False):
    """x [G,M_max,K] fp32/bf16, masked_m [G] int32 -> (q [G,M_max,K] uint8, sf [G,K/128,M_max]):
    the per-token cast of rows m < masked_m[g] only; other rows of q and sf are not written."""
    if x.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("x must be float32 or bfloat16")
    _need(x, x.dtype, "x")
    _need(masked_m, torch.int32, "masked_m")
    if x.dim() != 3:
        raise ValueError("x must be [G,M_max,K]")
    G, M, K = x.shape
    if tuple(masked_m.shape) != (G,):
        raise ValueError("masked_m must be [G]")
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    sf = torch.empty((G, K // 128, M), dtype=torch.float32, device=x.device) if sf is None else sf
    if tuple(q.shape) != tuple(x.shape) or tuple(sf.shape) != (G, K // 128, M):
        raise ValueError("q %s / sf %s do not match x %s" % (tuple(q.shape), tuple(sf.shape), tuple(x.shape)))
    dt = INPUT_BF16 if x.dtype == torch.bfloat16 else INPUT_F32
    _check(lib().dg_cast_fp8_per_token_masked(_ptr(x), dt, SCALE_UE8M0 if ue8m0 else SCALE_F32, G, M, K,
                                              _ptr(masked_m), _ptr(q), _ptr(sf), _stream(x.device)))
    return q, sf


def cast_fp8_per_block(w: torch.Tensor, q: torch.Tensor | None = None, sf: torch.Tensor | None = None,
                       ue8m0: bool = False):
    """w [N,K] or [G,N,K] fp32/bf16 -> (q uint8 e4m3 same shape, sf [..., N/128, K/128] fp32)."""
    if w.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("w must be float32 or bfloat16")
    _need(w, w.dtype, "w")
    lead = tuple(w.shape[:-2])
    N, K = w.shape[-2:]
    rows = N
    for s in lead:
        rows *= s
    q = torch.empty(w.shape, dtype=torch.uint8, device=w.device) if q is None else q
    sf = torch.empty(lead + (N // 128, K // 128), dtype=torch.float32, device=w.device) if sf is None else sf
    dt = INPUT_BF16 if w.dtype == torch.bfloat16 else INPUT_F32
    fn = lib().dg_cast_fp8_per_block_ue8m0 if ue8m0 else lib().dg_cast_fp8_per_block
    _check(fn(_ptr(w), dt, rows, K, _ptr(q), _ptr(sf), _stream(w.device)))
    return q, sf


def convert_fp8_e4m3(x: torch.Tensor, q: torch.Tensor | None = None) -> torch.Tensor:
    """x fp32 (any shape, numel % 4 == 0, |x| <= 464) -> e4m3 codes (uint8, same shape) from
    the hardware conversion the fused SwiGLU epilogue uses."""
    _need(x, torch.float32, "x")
    q = torch.empty(x.shape, dtype=torch.uint8, device=x.device) if q is None else q
    _need(q, torch.uint8, "q")
    if q.numel() != x.numel():
        raise ValueError("q must have x's size")
    _check(lib().dg_convert_fp8_e4m3(_ptr(x), x.numel(), _ptr(q), _stream(x.device)))
    return q


# ---- GEMMs ---------------------------------------------------------------------------
def _operands(a, sfa, b, sfb):
    _need(a, torch.uint8, "a")
    _need(sfa, torch.float32, "sfa")
    _need(b, torch.uint8, "b")
    _need(sfb, torch.float32, "sfb")


def gemm_fp8_nt(a, sfa, b, sfb, d: torch.Tensor | None = None, schedule: int = SCHED_AUTO, ue8m0: bool = False):
    """a [M,K] e4m3, sfa [K/128,M], b [N,K] e4m3, sfb [N/128,K/128] -> d [M,N] bf16 = A * B^T."""
    _operands(a, sfa, b, sfb)
    M, K = a.shape
    N = b.shape[0]
    if tuple(b.shape) != (N, K) or tuple(sfa.shape) != (K // 128, M) or tuple(sfb.shape) != (N // 128, K // 128):
        raise ValueError("shape mismatch: a %s sfa %s b %s sfb %s" % (tuple(a.shape), tuple(sfa.shape),
                                                                    tuple(b.shape), tuple(sfb.shape)))
    d = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if d is None else d
    _need(d, torch.bfloat16, "d")
    if schedule == SCHED_AUTO:
        fn = lib().dg_gemm_fp8_nt_ue8m0 if ue8m0 else lib().dg_gemm_fp8_nt
        st = fn(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(d), M, N, K, _stream(a.device))
    else:
        st = lib().dg_gemm_fp8_scheduled(LAYOUT_DENSE, schedule, SCALE_UE8M0 if ue8m0 else SCALE_F32, _ptr(a),
                                         _ptr(sfa), _ptr(b), _ptr(sfb), None, _ptr(d), 1, M, N, K, 0,
                                         _stream(a.device))
    _check(st)
    return d


def grouped_gemm_contiguous(a, sfa, b, sfb, m_indices, d: torch.Tensor | None = None,
                            schedule: int = SCHED_AUTO, ue8m0: bool = False):
    """a [M_total,K], sfa [K/128,M_total], b [G,N,K], sfb [G,N/128,K/128], m_indices [M_total]
    int32 (expert id or -1) -> d [M_total,N] bf16."""
    _operands(a, sfa, b, sfb)
    _need(m_indices, torch.int32, "m_indices")
    M, K = a.shape
    G, N, _ = b.shape
    if (tuple(b.shape) != (G, N, K) or tuple(sfa.shape) != (K // 128, M)
            or tuple(sfb.shape) != (G, N // 128, K // 128) or tuple(m_indices.shape) != (M,)):
        raise ValueError("shape mismatch")
    d = torch.empty((M, N), dtype=torch.bfloat16, device=a.device) if d is None else d
    _need(d, torch.bfloat16, "d")
    if schedule == SCHED_AUTO:
        fn = lib().dg_grouped_gemm_contiguous_ue8m0 if ue8m0 else lib().dg_grouped_gemm_contiguous
        st = fn(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(m_indices), _ptr(d), G, M, N, K, _stream(a.device))
    else:
        st = lib().dg_gemm_fp8_scheduled(LAYOUT_CONTIGUOUS, schedule, SCALE_UE8M0 if ue8m0 else SCALE_F32,
                                         _ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(m_indices), _ptr(d), G, M, N,
                                         K, 0, _stream(a.device))
    _check(st)
    return d


def grouped_gemm_masked(a, sfa, b, sfb, masked_m, expected_m: int = 0, d: torch.Tensor | None = None,
                        schedule: int = SCHED_AUTO, ue8m0: bool = False):
    """a [G,M_max,K], sfa [G,K/128,M_max], b [G,N,K], sfb [G,N/128,K/128], masked_m [G] int32
    -> d [G,M_max,N] bf16 (rows >= masked_m[g] are left untouched)."""
    _operands(a, sfa, b, sfb)
    _need(masked_m, torch.int32, "masked_m")
    G, M, K = a.shape
    N = b.shape[1]
    if (tuple(b.shape) != (G, N, K) or tuple(sfa.shape) != (G, K // 128, M)
            or tuple(sfb.shape) != (G, N // 128, K // 128) or tuple(masked_m.shape) != (G,)):
        raise ValueError("shape mismatch")
    d = torch.empty((G, M, N), dtype=torch.bfloat16, device=a.device) if d is None else d
    _need(d, torch.bfloat16, "d")
    if schedule == SCHED_AUTO:
        fn = lib().dg_grouped_gemm_masked_ue8m0 if ue8m0 else lib().dg_grouped_gemm_masked
        st = fn(_ptr(a), _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(masked_m), _ptr(d), G, M, N, K, expected_m,
                _stream(a.device))
    else:
        st = lib().dg_gemm_fp8_scheduled(LAYOUT_MASKED, schedule, SCALE_UE8M0 if ue8m0 else SCALE_F32, _ptr(a),
                                         _ptr(sfa), _ptr(b), _ptr(sfb), _ptr(masked_m), _ptr(d), G, M, N, K,
                                         expected_m, _stream(a.device))
    _check(st)
    return d


# ---- expert FFN ------------------------------------------------------------------------
def _ffn_shapes(layout, a, sfa, w1, sfw1, meta):
    """Checks the gate/up operands; returns (G, M, K, I) and the hq / sfh shapes."""
    if layout == LAYOUT_MASKED:
        G, M, K = a.shape
        want_sfa = (G, K // 128, M)
    else:
        M, K = a.shape
        G = w1.shape[0] if w1.dim() == 3 else 1
        want_sfa = (K // 128, M)
    two_i = w1.shape[-2]
    I = two_i // 2
    want_w1 = (G, two_i, K) if (layout != LAYOUT_DENSE or w1.dim() == 3) else (two_i, K)
    want_s1 = want_w1[:-2] + (two_i // 128, K // 128)
    if tuple(sfa.shape) != want_sfa or tuple(w1.shape) != want_w1 or two_i % 2 or tuple(sfw1.shape) != want_s1:
        raise ValueError("shape mismatch: a %s sfa %s w1 %s sfw1 %s" % (tuple(a.shape), tuple(sfa.shape),
                                                                       tuple(w1.shape), tuple(sfw1.shape)))
    if layout == LAYOUT_CONTIGUOUS and (meta is None or tuple(meta.shape) != (M,)):
        raise ValueError("contiguous layout needs m_indices [M_total]")
    if layout == LAYOUT_MASKED and (meta is None or tuple(meta.shape) != (G,)):
        raise ValueError("masked layout needs masked_m [G]")
    if layout == LAYOUT_MASKED:
        return G, M, K, I, (G, M, I), (G, I // 128, M)
    return G, M, K, I, (M, I), (I // 128, M)


def gemm_fp8_swiglu(layout, a, sfa, w1, sfw1, meta=None, expected_m: int = 0, hq=None, sfh=None,
                    ue8m0: bool = False):
    """Gate/up GEMM with the SwiGLU + per-token FP8 cast epilogue. w1 [G,2I,K] (gate rows,
    then up rows), sfw1 [G,2I/128,K/128]; returns hq (e4m3 [rows,I]) and sfh ([I/128,rows]),
    with a leading [G] for the masked layout."""
    _operands(a, sfa, w1, sfw1)
    G, M, K, I, hq_shape, sh_shape = _ffn_shapes(layout, a, sfa, w1, sfw1, meta)
    if meta is not None:
        _need(meta, torch.int32, "meta")
    hq = torch.empty(hq_shape, dtype=torch.uint8, device=a.device) if hq is None else hq
    sfh = torch.empty(sh_shape, dtype=torch.float32, device=a.device) if sfh is None else sfh
    _need(hq, torch.uint8, "hq")
    _need(sfh, torch.float32, "sfh")
    if tuple(hq.shape) != hq_shape or tuple(sfh.shape) != sh_shape:
        raise ValueError("hq / sfh shape mismatch")
    st = lib().dg_gemm_fp8_swiglu(layout, SCALE_UE8M0 if ue8m0 else SCALE_F32, _ptr(a), _ptr(sfa), _ptr(w1),
                                  _ptr(sfw1), None if meta is None else _ptr(meta), _ptr(hq), _ptr(sfh), G, M, I, K,
                                  expected_m, _stream(a.device))
    _check(st)
    return hq, sfh


def moe_ffn_fp8(layout, x, sfx, w1, sfw1, w2, sfw2, meta=None, expected_m: int = 0, hq=None, sfh=None, y=None,
                ue8m0: bool = False):
    """Expert FFN: y = down(SwiGLU(gate/up(x))). w2 [G,H,I], sfw2 [G,H/128,I/128]. Returns
    (y bf16 [rows,H] (masked [G,M_max,H]), hq, sfh) - the last two are the workspace."""
    _operands(x, sfx, w1, sfw1)
    _need(w2, torch.uint8, "w2")
    _need(sfw2, torch.float32, "sfw2")
    G, M, H, I, hq_shape, sh_shape = _ffn_shapes(layout, x, sfx, w1, sfw1, meta)
    want_w2 = (G, H, I) if (layout != LAYOUT_DENSE or w2.dim() == 3) else (H, I)
    if tuple(w2.shape) != want_w2 or tuple(sfw2.shape) != want_w2[:-2] + (H // 128, I // 128):
        raise ValueError("shape mismatch: w2 %s sfw2 %s" % (tuple(w2.shape), tuple(sfw2.shape)))
    if meta is not None:
        _need(meta, torch.int32, "meta")
    hq = torch.empty(hq_shape, dtype=torch.uint8, device=x.device) if hq is None else hq
    sfh = torch.empty(sh_shape, dtype=torch.float32, device=x.device) if sfh is None else sfh
    y_shape = (G, M, H) if layout == LAYOUT_MASKED else (M, H)
    y = torch.empty(y_shape, dtype=torch.bfloat16, device=x.device) if y is None else y
    _need(hq, torch.uint8, "hq")
    _need(sfh, torch.float32, "sfh")
    _need(y, torch.bfloat16, "y")
    if tuple(hq.shape) != hq_shape or tuple(sfh.shape) != sh_shape or tuple(y.shape) != y_shape:
        raise ValueError("hq / sfh / y shape mismatch")
    st = lib().dg_moe_ffn_fp8(layout, SCALE_UE8M0 if ue8m0 else SCALE_F32, _ptr(x), _ptr(sfx), _ptr(w1), _ptr(sfw1),
                              _ptr(w2), _ptr(sfw2), None if meta is None else _ptr(meta), _ptr(hq), _ptr(sfh),
                              _ptr(y), G, M, H, I, expected_m, _stream(x.device))
    _check(st)
    return y, hq, sfh


def moe_ffn_fp8_noalloc(layout, x, sfx, w1, sfw1, w2, sfw2, meta=None, expected_m: int = 0, y=None,
                        ue8m0: bool = False):
    """moe_ffn_fp8 with the FP8 activation between the GEMMs held in the library's static
    device scratch (dg_moe_ffn_fp8_noalloc): no workspace argument. Returns y."""
    _operands(x, sfx, w1, sfw1)
    _need(w2, torch.uint8, "w2")
    _need(sfw2, torch.float32, "sfw2")
    G, M, H, I, _, _ = _ffn_shapes(layout, x, sfx, w1, sfw1, meta)
    want_w2 = (G, H, I) if (layout != LAYOUT_DENSE or w2.dim() == 3) else (H, I)
    if tuple(w2.shape) != want_w2 or tuple(sfw2.shape) != want_w2[:-2] + (H // 128, I // 128):
        raise ValueError("shape mismatch: w2 %s sfw2 %s" % (tuple(w2.shape), tuple(sfw2.shape)))
    if meta is not None:
        _need(meta, torch.int32, "meta")
    y_shape = (G, M, H) if layout == LAYOUT_MASKED else (M, H)
    y = torch.empty(y_shape, dtype=torch.bfloat16, device=x.device) if y is None else y
    _need(y, torch.bfloat16, "y")
    if tuple(y.shape) != y_shape:
        raise ValueError("y shape mismatch")
    st = lib().dg_moe_ffn_fp8_noalloc(layout, SCALE_UE8M0 if ue8m0 else SCALE_F32, _ptr(x), _ptr(sfx), _ptr(w1),
                                      _ptr(sfw1), _ptr(w2), _ptr(sfw2), None if meta is None else _ptr(meta),
                                      _ptr(y), G, M, H, I, expected_m, _stream(x.device))
    _check(st)
    return y
