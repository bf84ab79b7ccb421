"""Acceptance checks for the fused SwiGLU re-cast and the expert FFN (test infrastructure).

The FP8 codes of h are a decision taken on the GEMM's fp32 accumulators, which differ from
the oracle's fp64 values by rounding. The checks therefore compare what is unique and
verify that the rest is a valid rounding:

  * error band of the gate/up values: |g_gpu - g| <= (nkb + 130) * 2^-24 * L, where
    L = sum_k |a_k b_k| (dequantised operands) - the bound of fp32 summation over one
    128-term block sum (128 roundings at most) and nkb promoted K-block partials;
  * band of h = silu(g) * u from first-order propagation of the g and u bands, plus
    (|g| + 16) * 2^-22 |h| for the fp32 evaluation of silu (exp and reciprocal on the
    transcendental unit, two products);
  * every chunk scale must lie between the scales the rule gives at the ends of the
    amax band; every code must lie between the codes of the ends of the h / s band
    (computed with the oracle's encoder), and nearly all codes equal the oracle's;
  * the FFN output: the GEMM bound against the oracle's y, plus the largest change that
    the allowed code and scale choices of h can make through |W2|.
Every expected value and every band comes from the oracle and its inputs only.
"""
from __future__ import annotations

import numpy as np

import oracle

DEC = oracle.decode_table()


def dequant_rows(q, s):
    """Per-token operand: codes [R,K], scales [R,K/128] (row-major, oracle layout) -> fp64."""
    return DEC[np.asarray(q)] * np.repeat(np.asarray(s, np.float64), 128, axis=-1)


def dequant_blocks(q, s):
    """Block-scaled weights: codes [N,K], scales [N/128,K/128] -> fp64."""
    s = np.asarray(s, np.float64)
    return DEC[np.asarray(q)] * np.repeat(np.repeat(s, 128, axis=0), 128, axis=1)


def abs_products(a_deq, w_deq):
    """L[m,n] = sum_k |a[m,k]| |w[n,k]|."""
    return np.abs(a_deq) @ np.abs(w_deq).T


def h_band(gu, L_gu, nkb):
    """Band of the fp32 h the kernel forms from its accumulators, around the oracle's h."""
    I = gu.shape[-1] // 2
    e = (nkb + 130) * 2.0 ** -24 * L_gu
    g, u = gu[..., :I], gu[..., I:]
    eg, eu = e[..., :I], e[..., I:]
    with np.errstate(over="ignore"):
        sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = sig * (1.0 + g * (1.0 - sig))
    h = silu * u
    return (np.abs(dsilu * u) * eg + np.abs(silu) * eu + 1.2 * eg * eu
            + (np.abs(g) + 16.0) * 2.0 ** -22 * np.abs(h))


def _f32_down(x):
    f = np.asarray(x, np.float64).astype(np.float32)
    return np.where(f.astype(np.float64) > x, np.nextafter(f, np.float32(-np.inf)), f)


def _f32_up(x):
    f = np.asarray(x, np.float64).astype(np.float32)
    return np.where(f.astype(np.float64) < x, np.nextafter(f, np.float32(np.inf)), f)


def _pow2_ceil(v):
    v = np.asarray(v, np.float32).astype(np.float64)
    m, e = np.frexp(v)
    p = np.ldexp(1.0, e - 1)
    p = np.where(p >= v, p, 2.0 * p)
    p = np.where(v == 0, 0.0, p)
    return np.maximum(p, 2.0 ** -126).astype(np.float32)


def check_recast(h, e_h, hq_gpu, sh_gpu, hq_ref, pow2, what, min_exact=0.99):
    """h, e_h [R,I] (fp64 oracle value and band), hq_gpu [R,I] codes, sh_gpu [R,I/128]
    (row-major), hq_ref [R,I] the oracle's codes. Returns (lo codes, hi codes, s_lo, s_hi)
    for the output check."""
    R, I = h.shape
    nb = I // 128
    hb = np.abs(h).reshape(R, nb, 128)
    eb = e_h.reshape(R, nb, 128)
    amax_lo = np.max(np.maximum(hb - eb, 0.0), axis=2)
    amax_hi = np.max(hb + eb, axis=2)
    if pow2:
        s_lo = _pow2_ceil(_f32_down(amax_lo / 448.0))
        s_hi = _pow2_ceil(_f32_up(amax_hi / 448.0))
    else:
        s_lo = _f32_down(amax_lo / 448.0)
        s_hi = _f32_up(amax_hi / 448.0)
    sg = np.asarray(sh_gpu, np.float32)
    bad = ~((s_lo <= sg) & (sg <= s_hi))
    assert not bad.any(), "%s: %d chunk scales outside the band, first %s: gpu %r, band [%r, %r]" % (
        what, bad.sum(), tuple(np.argwhere(bad)[0]), sg[bad][0], s_lo[bad][0], s_hi[bad][0])
    S_lo = np.repeat(s_lo.astype(np.float64), 128, axis=1)
    S_hi = np.repeat(s_hi.astype(np.float64), 128, axis=1)
    hl, hh = h - e_h, h + e_h
    with np.errstate(divide="ignore", invalid="ignore"):
        x_lo = np.where(hl >= 0, hl / S_hi, hl / S_lo)
        x_hi = np.where(hh >= 0, hh / S_lo, hh / S_hi)
    x_lo = np.nan_to_num(x_lo, nan=-np.inf)
    x_hi = np.nan_to_num(x_hi, nan=np.inf)
    c_lo = oracle.encode(_f32_down(np.clip(x_lo, -1e30, 1e30)))
    c_hi = oracle.encode(_f32_up(np.clip(x_hi, -1e30, 1e30)))
    v = DEC[np.asarray(hq_gpu)]
    ok = (DEC[c_lo] <= v) & (v <= DEC[c_hi])
    zero_chunk = np.repeat(sg == 0, 128, axis=1)
    ok = np.where(zero_chunk, (np.asarray(hq_gpu) & 0x7F) == 0, ok)
    assert ok.all(), "%s: %d codes outside their band, first at %s: gpu %#x, band [%#x, %#x], h %r" % (
        what, (~ok).sum(), tuple(np.argwhere(~ok)[0]), hq_gpu[~ok][0], c_lo[~ok][0], c_hi[~ok][0], h[~ok][0])
    exact = float(np.mean(np.asarray(hq_gpu) == np.asarray(hq_ref)))
    assert exact >= min_exact, "%s: only %.4f of the codes equal the oracle's" % (what, exact)
    return c_lo, c_hi, s_lo, s_hi


def output_allowance(c_lo, c_hi, s_lo, s_hi, hq_ref, sh_ref, w2_deq):
    """Largest change of y = hdeq @ w2^T that the allowed codes / scales of h can make:
    Delta [R,I] @ |w2_deq|^T."""
    S_lo = np.repeat(s_lo.astype(np.float64), 128, axis=1)
    S_hi = np.repeat(s_hi.astype(np.float64), 128, axis=1)
    lo, hi = DEC[c_lo], DEC[c_hi]
    v_lo = np.minimum(lo * S_lo, lo * S_hi)
    v_hi = np.maximum(hi * S_lo, hi * S_hi)
    v_ref = DEC[np.asarray(hq_ref)] * np.repeat(np.asarray(sh_ref, np.float64), 128, axis=1)
    delta = np.maximum(np.abs(v_hi - v_ref), np.abs(v_lo - v_ref))
    return delta @ np.abs(w2_deq).T


def check_output(y, y_ref, allowance, what):
    """The GEMM acceptance bound (per element and similarity) with the allowance added."""
    y = np.asarray(y, np.float64)
    rms = float(np.sqrt(np.mean(y_ref * y_ref)))
    bound = 2.0 ** -7 * np.abs(y_ref) + 1e-3 * rms + allowance
    err = np.abs(y - y_ref)
    bad = ~(err <= bound)
    assert not bad.any(), "%s: %d of %d outputs out of bound, worst excess %r" % (
        what, bad.sum(), bad.size, float(np.nanmax(err - bound)))
    den = float(np.sum(y * y + y_ref * y_ref))
    sim = 0.0 if den == 0 else 1.0 - 2.0 * float(np.sum(y * y_ref)) / den
    assert sim <= 1e-5, "%s: similarity %r" % (what, sim)
    return sim
