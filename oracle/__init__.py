"""CPU oracle for the FP8 (e4m3) block-scaled GEMM path (dense, contiguous-grouped,
masked-grouped) and its per-token / per-block casts.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU-baseline
leg import this package; the product library never does. The arithmetic lives in
``dg_oracle.c`` (plain C, fp64 accumulation); this module builds it with gcc on first
use and marshals numpy arrays through ctypes.

Method source (cited by page title and section):
  * DeepGEMM article ("DeepGEMM ... FP8 and fine-grained scaling"): activations are
    scaled per 1x128 slice, weights per 128x128 block, accumulation kept in higher
    precision; normal, contiguous-layout and masked-layout grouped GEMMs.
  * DeepGEMM launch write-up, "Built for modern AI compute" / "Deployment guide":
    FP8 products over a K stretch are promoted to fp32 and accumulated.
  * DeepSeek-V3 repo review, "Innovations" 4 and "Risks" 6: one scale per 128
    elements, 128x128 weight blocks, quantisation bound 448.
  * DeepGEMM article, "swapAB and Mega MoE": the expert FFN, two grouped GEMMs with the
    SwiGLU activation between them (moe_ffn_contiguous / moe_ffn_masked compose the
    GEMM and cast oracles with an fp64 SwiGLU; readings stated beside them).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dg_oracle.c")
_LIB = os.path.join(_HERE, "libdg_oracle.so")
QBLK = 128

_CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
           "-ffp-contract=off", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile dg_oracle.c with gcc into libdg_oracle.so (when missing or stale)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _L():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I32 = ctypes.c_int32
        lib.dgo_decode_table.argtypes = [P]
        lib.dgo_decode.argtypes = [ctypes.c_uint8]
        lib.dgo_decode.restype = ctypes.c_double
        lib.dgo_enc_nearest.argtypes = [ctypes.c_float]
        lib.dgo_enc_nearest.restype = ctypes.c_uint8
        lib.dgo_enc_bits.argtypes = [ctypes.c_float]
        lib.dgo_enc_bits.restype = ctypes.c_uint8
        lib.dgo_enc_crosscheck.argtypes = [ctypes.c_uint32, ctypes.c_uint32]
        lib.dgo_enc_crosscheck.restype = I64
        lib.dgo_encode_array.argtypes = [P, I64, P]
        lib.dgo_cast_per_token.argtypes = [P, I64, I64, P, P]
        lib.dgo_cast_per_block.argtypes = [P, I64, I64, P, P]
        lib.dgo_cast_per_token_pow2.argtypes = [P, I64, I64, P, P]
        lib.dgo_cast_per_block_pow2.argtypes = [P, I64, I64, P, P]
        lib.dgo_bf16_to_f32.argtypes = [P, I64, P]
        lib.dgo_gemm.argtypes = [P, P, P, P, I64, I64, I64, P]
        lib.dgo_gemm_pairs.argtypes = [P, P, P, P, P, I32, I64, I64, P, P, I64, P]
        lib.dgo_grouped_contiguous.argtypes = [P, P, P, P, P, I32, I64, I64, I64, P]
        lib.dgo_grouped_masked.argtypes = [P, P, P, P, P, I32, I64, I64, I64, P]
        lib.dgo_block_sums.argtypes = [P, P, I64, I64, I64, P]
        lib.dgo_num_threads.restype = ctypes.c_int
        lib.dgo_set_num_threads.argtypes = [ctypes.c_int]
        _lib = lib
    return _lib


def _p(arr: np.ndarray | None):
    return None if arr is None else ctypes.c_void_p(arr.ctypes.data)


def _c(arr, dtype) -> np.ndarray:
    return np.ascontiguousarray(arr, dtype=dtype)


def num_threads() -> int:
    return int(_L().dgo_num_threads())


def set_num_threads(n: int) -> None:
    _L().dgo_set_num_threads(int(n))


# ---- e4m3 codec -------------------------------------------------------------
def decode_table() -> np.ndarray:
    out = np.empty(256, np.float64)
    _L().dgo_decode_table(_p(out))
    return out


def encode(y) -> np.ndarray:
    """fp32 -> e4m3 codes (nearest, ties to even code, saturating at +-448)."""
    y = _c(y, np.float32)
    out = np.empty(y.shape, np.uint8)
    _L().dgo_encode_array(_p(y), y.size, _p(out))
    return out


def enc_nearest(y: float) -> int:
    return int(_L().dgo_enc_nearest(ctypes.c_float(y)))


def enc_bits(y: float) -> int:
    return int(_L().dgo_enc_bits(ctypes.c_float(y)))


def enc_crosscheck(lo: int, hi: int) -> int:
    """Number of finite fp32 bit patterns in [lo, hi] where the two encoders differ."""
    return int(_L().dgo_enc_crosscheck(lo, hi))


# ---- casts --------------------------------------------------------------------
def bf16_bits_to_f32(x_bits: np.ndarray) -> np.ndarray:
    x_bits = _c(x_bits, np.uint16)
    out = np.empty(x_bits.shape, np.float32)
    _L().dgo_bf16_to_f32(_p(x_bits), x_bits.size, _p(out))
    return out


def cast_per_token(x: np.ndarray, pow2: bool = False):
    """x [M,K] fp32 -> (q [M,K] uint8 e4m3, s [M,K/128] fp32); s = amax/448 (pow2: the
    smallest power of two >= that, at least 2^-126), q = e4m3(x/s)."""
    x = _c(x, np.float32)
    M, K = x.shape
    assert K % QBLK == 0
    q = np.empty((M, K), np.uint8)
    s = np.empty((M, K // QBLK), np.float32)
    fn = _L().dgo_cast_per_token_pow2 if pow2 else _L().dgo_cast_per_token
    fn(_p(x), M, K, _p(q), _p(s))
    return q, s


def cast_per_block(w: np.ndarray, pow2: bool = False):
    """w [N,K] (or [G,N,K]) fp32 -> (q uint8 e4m3, s [N/128,K/128] fp32) per 128x128 block."""
    w = _c(w, np.float32)
    if w.ndim == 3:
        qs = [cast_per_block(w[g], pow2) for g in range(w.shape[0])]
        return np.stack([q for q, _ in qs]), np.stack([s for _, s in qs])
    N, K = w.shape
    assert N % QBLK == 0 and K % QBLK == 0
    q = np.empty((N, K), np.uint8)
    s = np.empty((N // QBLK, K // QBLK), np.float32)
    fn = _L().dgo_cast_per_block_pow2 if pow2 else _L().dgo_cast_per_block
    fn(_p(w), N, K, _p(q), _p(s))
    return q, s


# ---- GEMMs ---------------------------------------------------------------------
def gemm(a, sa, b, sb) -> np.ndarray:
    """R = dequant(a) @ dequant(b)^T in fp64; a [M,K], b [N,K] e4m3 codes."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sa = _c(sa, np.float32); sb = _c(sb, np.float32)
    M, K = a.shape
    N = b.shape[0]
    assert b.shape == (N, K) and sa.shape == (M, K // QBLK) and sb.shape == (N // QBLK, K // QBLK)
    R = np.empty((M, N), np.float64)
    _L().dgo_gemm(_p(a), _p(sa), _p(b), _p(sb), M, N, K, _p(R))
    return R


def gemm_pairs(a, sa, b, sb, rows, cols, group_of_row=None) -> np.ndarray:
    """R at selected (rows[i], cols[i]). a [Mrows,K]; b [G,N,K] or [N,K]; row m uses
    group group_of_row[m] (default 0); a row whose group is outside [0, G) gives NaN."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sa = _c(sa, np.float32); sb = _c(sb, np.float32)
    K = a.shape[-1]
    N = b.shape[-2]
    G = b.shape[0] if b.ndim == 3 else 1
    assert b.shape[-1] == K and sa.shape == (a.shape[0], K // QBLK)
    assert sb.shape[-2:] == (N // QBLK, K // QBLK) and (sb.shape[0] if sb.ndim == 3 else 1) == G
    rows = _c(rows, np.int64); cols = _c(cols, np.int64)
    assert rows.shape == cols.shape
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < a.shape[0] and cols.min() >= 0 and cols.max() < N)
    gr = None if group_of_row is None else _c(group_of_row, np.int32)
    assert gr is None or gr.shape == (a.shape[0],)
    out = np.empty(rows.shape, np.float64)
    _L().dgo_gemm_pairs(_p(a), _p(sa), _p(b), _p(sb), _p(gr), G, N, K, _p(rows), _p(cols),
                        rows.size, _p(out))
    return out


def grouped_contiguous(a, sa, b, sb, m_indices) -> np.ndarray:
    """a [M_total,K], b [G,N,K], m_indices [M_total] (expert id or -1) -> R [M_total,N]
    (NaN on padding rows)."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sa = _c(sa, np.float32); sb = _c(sb, np.float32)
    mi = _c(m_indices, np.int32)
    M_total, K = a.shape
    G, N, _ = b.shape
    R = np.empty((M_total, N), np.float64)
    _L().dgo_grouped_contiguous(_p(a), _p(sa), _p(b), _p(sb), _p(mi), G, M_total, N, K, _p(R))
    return R


def grouped_masked(a, sa, b, sb, masked_m) -> np.ndarray:
    """a [G,M_max,K], b [G,N,K], masked_m [G] -> R [G,M_max,N] (NaN on rows >= masked_m)."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    sa = _c(sa, np.float32); sb = _c(sb, np.float32)
    mm = _c(masked_m, np.int32)
    G, M_max, K = a.shape
    N = b.shape[1]
    R = np.empty((G, M_max, N), np.float64)
    _L().dgo_grouped_masked(_p(a), _p(sa), _p(b), _p(sb), _p(mm), G, M_max, N, K, _p(R))
    return R


def block_sums(a, b) -> np.ndarray:
    """The fp64 per-128-K block sums the GEMM uses: P [M,N,K/128]."""
    a = _c(a, np.uint8); b = _c(b, np.uint8)
    M, K = a.shape
    N = b.shape[0]
    P = np.empty((M, N, K // QBLK), np.float64)
    _L().dgo_block_sums(_p(a), _p(b), M, N, K, _p(P))
    return P


# ---- comparison ------------------------------------------------------------------
def compare(y, R, mask=None) -> dict:
    """The GEMM acceptance test. y: produced values (any float dtype), R: fp64 oracle.
    Over the compared set S (mask, default all finite R):
      per element  |y - R| <= 2^-7 |R| + 1e-3 rms_S(R)
      global       1 - 2 sum(yR) / sum(y^2 + R^2) <= 1e-5   (0 when the denominator is 0)
    Returns a dict with 'ok', 'worst_excess', 'n_bad', 'sim'."""
    with np.errstate(invalid="ignore"):  # unwritten rows may hold signalling-NaN patterns
        y = np.asarray(y, np.float64)
    R = np.asarray(R, np.float64)
    if mask is None:
        mask = np.isfinite(R)
    ys, Rs = y[mask], R[mask]
    if Rs.size == 0:
        return {"ok": True, "n_bad": 0, "worst_excess": 0.0, "sim": 0.0, "count": 0}
    rms = float(np.sqrt(np.mean(Rs * Rs)))
    bound = 2.0 ** -7 * np.abs(Rs) + 1e-3 * rms
    err = np.abs(ys - Rs)
    bad = ~(err <= bound)  # NaN in y counts as bad
    den = float(np.sum(ys * ys + Rs * Rs))
    sim = 0.0 if den == 0.0 else 1.0 - 2.0 * float(np.sum(ys * Rs)) / den
    ok = (not bool(bad.any())) and np.isfinite(sim) and sim <= 1e-5
    excess = err - bound
    return {"ok": bool(ok), "n_bad": int(bad.sum()), "count": int(Rs.size),
            "worst_excess": float(np.nanmax(excess)) if excess.size else 0.0,
            "sim": float(sim), "rms": rms}


# ---- MoE expert FFN: gate/up GEMM -> SwiGLU -> per-token FP8 re-cast -> down GEMM ----------
# DeepGEMM article, section "swapAB and Mega MoE": the expert FFN runs two grouped GEMMs with
# the SwiGLU activation between them. Readings (the pages give no formulas for this part):
#   * the first weight tensor is [G, 2I, H]: rows [0, I) are the gate projection, rows
#     [I, 2I) the up projection; the second is [G, H, I] (the down projection);
#   * SwiGLU(g, u) = silu(g) * u with silu(x) = x * sigmoid(x), evaluated on the fp64 GEMM
#     results (no bf16 rounding of the gate/up outputs in between);
#   * the activation h is materialised in fp32 and cast to FP8 with the per-token rule
#     (1x128 chunks along I, s = amax / 448 or its power-of-two form); the down GEMM takes
#     those bytes and scales like any other activation;
#   * rows that belong to no expert (contiguous padding, masked rows >= masked_m) are not
#     part of the result (NaN here).
def silu(x) -> np.ndarray:
    """x * sigmoid(x) = x / (1 + exp(-x)) in fp64 (exp overflow for very negative x gives -0)."""
    x = np.asarray(x, np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(gate_up) -> np.ndarray:
    """[..., 2I] -> [..., I]: silu(gate) * up, the gate being the first I columns."""
    gate_up = np.asarray(gate_up, np.float64)
    I = gate_up.shape[-1] // 2
    assert gate_up.shape[-1] == 2 * I
    return silu(gate_up[..., :I]) * gate_up[..., I:]


def _recast_rows(h: np.ndarray, valid: np.ndarray, pow2: bool):
    """Per-token cast of h [R, I] on its valid rows (others are cast as zeros and then
    marked NaN in the scales)."""
    h32 = np.where(valid[:, None], h, 0.0).astype(np.float32)
    hq, sh = cast_per_token(h32, pow2)
    sh = sh.copy()
    sh[~valid] = np.nan
    return h32, hq, sh


def moe_ffn_contiguous(xq, sx, w1q, s1, w2q, s2, m_indices, pow2: bool = False) -> dict:
    """Expert FFN in the contiguous layout. xq [M_total,H] codes with sx [M_total,H/128];
    w1q [G,2I,H] with s1 [G,2I/128,H/128]; w2q [G,H,I] with s2 [G,H/128,I/128];
    m_indices [M_total]. Returns gate_up [M_total,2I], h [M_total,I] (fp64), h32 (fp32),
    hq [M_total,I] codes and sh [M_total,I/128] (the re-cast), y [M_total,H] (fp64);
    padding rows are NaN in gate_up, h, sh and y."""
    gu = grouped_contiguous(xq, sx, w1q, s1, m_indices)
    h = swiglu(gu)
    valid = np.asarray(m_indices) >= 0
    valid &= np.asarray(m_indices) < np.asarray(w1q).shape[0]
    h32, hq, sh = _recast_rows(h, valid, pow2)
    y = grouped_contiguous(hq, np.nan_to_num(sh), w2q, s2, m_indices)
    return dict(gate_up=gu, h=h, h32=h32, hq=hq, sh=sh, y=y)


def moe_ffn_masked(xq, sx, w1q, s1, w2q, s2, masked_m, pow2: bool = False) -> dict:
    """Expert FFN in the masked layout. xq [G,M_max,H] with sx [G,M_max,H/128]; weights as
    in moe_ffn_contiguous; masked_m [G]. Outputs carry a leading [G, M_max]; rows
    r >= masked_m[g] are NaN."""
    gu = grouped_masked(xq, sx, w1q, s1, masked_m)
    h = swiglu(gu)
    G, M_max, I = h.shape
    mm = np.clip(np.asarray(masked_m, np.int64), 0, M_max)
    valid = (np.arange(M_max)[None, :] < mm[:, None]).reshape(-1)
    h32, hq, sh = _recast_rows(h.reshape(G * M_max, I), valid, pow2)
    hq = hq.reshape(G, M_max, I)
    sh = sh.reshape(G, M_max, I // QBLK)
    y = grouped_masked(hq, np.nan_to_num(sh), w2q, s2, masked_m)
    return dict(gate_up=gu, h=h, h32=h32.reshape(G, M_max, I), hq=hq, sh=sh, y=y)
