"""Pins for the oracle's MoE expert FFN (gate/up GEMM -> SwiGLU -> per-token FP8 re-cast
-> down GEMM), DeepGEMM article, section "swapAB and Mega MoE". CPU only.

What pins it, besides the GEMM and cast pins it builds on:
  * silu at points with closed forms (tests/golden/silu_points.txt) and the identity
    silu(x) - silu(-x) = x;
  * the whole composition against a brute-force evaluation in plain Python loops on
    tiny shapes (its own block sums, its own sigmoid, float32 scalar division);
  * exact power-of-two homogeneity in the up projection: doubling the up weights'
    block scales doubles h, the re-cast scales and y bit for bit and leaves every FP8
    code of h unchanged (doubling the gate's does not);
  * the masked and contiguous layouts give the same rows for the same tokens.
"""
from __future__ import annotations

import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "silu_points.txt")


def _golden_silu():
    pts = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            k, sign, num, den = [c.strip() for c in line.split("|")]
            lnk = math.log(int(k))
            x = lnk if sign == "+" else -lnk
            pts.append((x, x * int(num) / int(den)))
    return pts


def test_silu_golden_points():
    pts = _golden_silu()
    assert len(pts) == 9
    x = np.array([p[0] for p in pts])
    want = np.array([p[1] for p in pts])
    got = oracle.silu(x)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-300)
    assert got[0] == 0.0


def test_silu_odd_part_identity_and_limits():
    x = np.random.default_rng(5).standard_normal(4096) * 6.0
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-13)
    big = np.array([40.0, 200.0, 800.0])
    np.testing.assert_array_equal(oracle.silu(big), big)  # sigmoid rounds to 1
    assert np.all(np.abs(oracle.silu(-big)) < 1e-15) and np.all(np.isfinite(oracle.silu(-big)))


def test_swiglu_takes_the_gate_first():
    # gate = ln 3 (sigmoid 3/4), up = 2 -> 1.5 ln 3; the swapped order would give
    # silu(2) * ln 3 = ln 3 * 2 / (1 + e^-2)
    gu = np.array([[math.log(3.0), 2.0]])
    assert oracle.swiglu(gu)[0, 0] == pytest.approx(1.5 * math.log(3.0), rel=1e-15)


# ---- brute force ------------------------------------------------------------------------
def _brute_gemm_row(dec, xrow, sxrow, w, sw, n):
    """sum over 128-wide K blocks of (sx * sw) * (block sum of decoded products)."""
    K = len(xrow)
    acc = 0.0
    for kb in range(K // 128):
        p = 0.0
        for k in range(kb * 128, kb * 128 + 128):
            p += dec[xrow[k]] * dec[w[n][k]]
        acc += p * (float(sxrow[kb]) * float(sw[n // 128][kb]))
    return acc


def _brute_ffn_row(dec, xrow, sxrow, w1, s1, w2, s2, pow2):
    H = len(xrow)
    I = len(w1) // 2
    dec_l = [float(v) for v in dec]
    xr = [int(v) for v in xrow]
    w1l = [[int(v) for v in r] for r in w1]
    w2l = [[int(v) for v in r] for r in w2]
    gu = [_brute_gemm_row(dec_l, xr, sxrow, w1l, s1, n) for n in range(2 * I)]
    h = []
    for j in range(I):
        g, u = gu[j], gu[I + j]
        sig = 1.0 / (1.0 + math.exp(-g))
        h.append(g * sig * u)
    h32 = np.array(h, np.float32)
    q = np.empty(I, np.uint8)
    sh = np.empty(I // 128, np.float32)
    for c in range(I // 128):
        chunk = h32[c * 128:(c + 1) * 128]
        amax = np.float32(np.max(np.abs(chunk)))
        s = np.float32(amax / np.float32(448.0))
        if pow2:
            # smallest power of two >= s, at least 2^-126
            e = math.frexp(float(s))[1] if s > 0 else -200
            p = math.ldexp(1.0, e - 1)
            s = np.float32(p if p >= float(s) else 2.0 * p)
            s = max(s, np.float32(2.0 ** -126))
        sh[c] = s
        if s == 0:
            q[c * 128:(c + 1) * 128] = np.where(np.signbit(chunk), 0x80, 0x00)
        else:
            q[c * 128:(c + 1) * 128] = oracle.encode(chunk / s)
    ql = [int(v) for v in q]
    y = [_brute_gemm_row(dec_l, ql, sh, w2l, s2, n) for n in range(H)]
    return np.array(gu), np.array(h), q, sh, np.array(y)


def _ffn_weights(G, H, I, seed, pow2=False):
    w1 = synth.normal((G, 2 * I, H), seed, synth.TID_B, std=0.02)
    w2 = synth.normal((G, H, I), seed + 1, synth.TID_B, std=0.02)
    w1q, s1 = oracle.cast_per_block(w1, pow2)
    w2q, s2 = oracle.cast_per_block(w2, pow2)
    return w1q, s1, w2q, s2


@pytest.mark.parametrize("pow2", [False, True])
def test_ffn_contiguous_matches_brute_force(pow2):
    G, H, I = 2, 256, 256
    mi = np.array([0, 0, 1, -1, 1, 0], np.int32)
    x = synth.normal((mi.size, H), 3, synth.TID_A)
    x[mi < 0] = 0.0
    x[1, :128] *= 30.0  # one chunk with a much larger range
    xq, sx = oracle.cast_per_token(x, pow2)
    w1q, s1, w2q, s2 = _ffn_weights(G, H, I, 3, pow2)
    r = oracle.moe_ffn_contiguous(xq, sx, w1q, s1, w2q, s2, mi, pow2)
    dec = oracle.decode_table()
    for m in range(mi.size):
        if mi[m] < 0:
            assert np.all(np.isnan(r["y"][m])) and np.all(np.isnan(r["h"][m])) and np.all(np.isnan(r["sh"][m]))
            continue
        e = mi[m]
        gu, h, q, sh, y = _brute_ffn_row(dec, xq[m], sx[m], w1q[e], s1[e], w2q[e], s2[e], pow2)
        np.testing.assert_allclose(r["gate_up"][m], gu, rtol=1e-13, atol=1e-16)
        np.testing.assert_allclose(r["h"][m], h, rtol=1e-12, atol=1e-18)
        np.testing.assert_array_equal(r["sh"][m].astype(np.float32).view(np.uint32), sh.view(np.uint32))
        np.testing.assert_array_equal(r["hq"][m], q)
        np.testing.assert_allclose(r["y"][m], y, rtol=1e-12, atol=1e-16)


def test_ffn_masked_matches_brute_force():
    G, M_max, H, I = 2, 4, 128, 128
    mm = np.array([3, 1], np.int32)
    x = synth.normal((G, M_max, H), 4, synth.TID_A)
    xq, sx = oracle.cast_per_token(x.reshape(-1, H))
    xq = xq.reshape(G, M_max, H)
    sx = sx.reshape(G, M_max, H // 128)
    w1q, s1, w2q, s2 = _ffn_weights(G, H, I, 4)
    r = oracle.moe_ffn_masked(xq, sx, w1q, s1, w2q, s2, mm)
    dec = oracle.decode_table()
    for g in range(G):
        for m in range(M_max):
            if m >= mm[g]:
                assert np.all(np.isnan(r["y"][g, m])) and np.all(np.isnan(r["sh"][g, m]))
                continue
            _, h, q, sh, y = _brute_ffn_row(dec, xq[g, m], sx[g, m], w1q[g], s1[g], w2q[g], s2[g], False)
            np.testing.assert_allclose(r["h"][g, m], h, rtol=1e-12, atol=1e-18)
            np.testing.assert_array_equal(r["hq"][g, m], q)
            np.testing.assert_allclose(r["y"][g, m], y, rtol=1e-12, atol=1e-16)


@pytest.mark.parametrize("pow2", [False, True])
def test_ffn_up_projection_is_exactly_homogeneous(pow2):
    G, H, I = 2, 256, 256
    mi, _ = synth.contiguous_layout(G, 150, 7)
    x = synth.normal((mi.size, H), 7, synth.TID_A)
    x[mi < 0] = 0.0
    xq, sx = oracle.cast_per_token(x, pow2)
    w1q, s1, w2q, s2 = _ffn_weights(G, H, I, 7, pow2)
    base = oracle.moe_ffn_contiguous(xq, sx, w1q, s1, w2q, s2, mi, pow2)
    up2 = s1.copy()
    up2[:, I // 128:, :] *= 2.0
    r = oracle.moe_ffn_contiguous(xq, sx, w1q, up2, w2q, s2, mi, pow2)
    ok = mi >= 0
    np.testing.assert_array_equal(r["h"][ok], 2.0 * base["h"][ok])
    np.testing.assert_array_equal(r["hq"][ok], base["hq"][ok])
    np.testing.assert_array_equal(r["sh"][ok], 2.0 * base["sh"][ok])
    np.testing.assert_array_equal(r["y"][ok], 2.0 * base["y"][ok])
    gate2 = s1.copy()
    gate2[:, :I // 128, :] *= 2.0
    rg = oracle.moe_ffn_contiguous(xq, sx, w1q, gate2, w2q, s2, mi, pow2)
    assert not np.array_equal(rg["h"][ok], 2.0 * base["h"][ok])


def test_ffn_masked_equals_contiguous_rows():
    G, H, I = 2, 128, 256
    mi = np.array([0, 0, 0, 1, 1], np.int32)
    x = synth.normal((mi.size, H), 9, synth.TID_A)
    xq, sx = oracle.cast_per_token(x)
    w1q, s1, w2q, s2 = _ffn_weights(G, H, I, 9)
    c = oracle.moe_ffn_contiguous(xq, sx, w1q, s1, w2q, s2, mi)
    M_max = 4
    xm = np.zeros((G, M_max, H), np.uint8)
    sm = np.zeros((G, M_max, H // 128), np.float32)
    xm[0, :3], sm[0, :3] = xq[:3], sx[:3]
    xm[1, :2], sm[1, :2] = xq[3:], sx[3:]
    m = oracle.moe_ffn_masked(xm, sm, w1q, s1, w2q, s2, np.array([3, 2], np.int32))
    np.testing.assert_array_equal(m["y"][0, :3], c["y"][:3])
    np.testing.assert_array_equal(m["y"][1, :2], c["y"][3:])
    np.testing.assert_array_equal(m["hq"][1, :2], c["hq"][3:])
    assert np.all(np.isnan(m["y"][0, 3])) and np.all(np.isnan(m["y"][1, 2:]))
