"""Pins for the CPU oracle (no GPU). Each test ties the oracle to something other than
itself: the e4m3 format definition (hand-derived fixture points), an independent library
codec (torch's float8_e4m3fn), a second encoder checked on every fp32 bit pattern, exact
rational arithmetic on tiny shapes, an integer formulation of the block sums, closed forms
and invariants. A mistake such as a dropped K block, a transposed scale grid, a wrong sign
or a wrong expert makes at least one of these fail (see the *_detects_* tests)."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

QBLK = 128


# ---------------------------------------------------------------------------------
# e4m3 codec
# ---------------------------------------------------------------------------------
def test_decode_table_format_points():
    t = oracle.decode_table()
    assert t[0x7E] == 448.0  # the pages' quantisation bound is the largest finite code
    assert t[0x38] == 1.0
    assert t[0x08] == 2.0 ** -6  # smallest normal
    assert t[0x01] == 2.0 ** -9  # smallest subnormal
    assert t[0x00] == 0.0 and not np.signbit(t[0x00])
    assert t[0x80] == 0.0 and np.signbit(t[0x80])
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isnan(t).sum() == 2  # no other NaN, and no infinities
    assert np.isfinite(t[np.r_[0:0x7F, 0x80:0xFF]]).all()
    pos = t[0:0x7F]
    assert (np.diff(pos) > 0).all()  # 127 non-negative finite codes, strictly increasing
    assert np.array_equal(t[0x80:0xFF], -pos)  # sign bit negates
    assert np.all(pos * 512 == np.round(pos * 512))  # all multiples of 2^-9
    # eight equally spaced values in every binade [2^e, 2^(e+1)), e = -6..8
    for e in range(-6, 9):
        vals = pos[(pos >= 2.0 ** e) & (pos < 2.0 ** (e + 1))]
        assert len(vals) == (7 if e == 8 else 8)  # 480 would be the NaN code
        assert np.allclose(np.diff(vals), 2.0 ** (e - 3))


def test_decode_matches_torch_float8_e4m3fn():
    ours = oracle.decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))


def _golden_points(golden_dir):
    pts = []
    with open(os.path.join(golden_dir, "e4m3_points.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            val, code = line.split()[:2]
            pts.append((float(val), int(code, 16)))
    return pts


def test_golden_points_both_encoders(golden_dir):
    pts = _golden_points(golden_dir)
    assert len(pts) >= 20
    for val, code in pts:
        assert oracle.enc_nearest(val) == code, (val, hex(code))
        assert oracle.enc_bits(val) == code, (val, hex(code))
    y = np.array([v for v, _ in pts], np.float32)
    assert np.array_equal(oracle.encode(y), np.array([c for _, c in pts], np.uint8))


def test_round_trip_all_codes():
    t = oracle.decode_table()
    for b in range(256):
        if np.isnan(t[b]):
            continue
        assert oracle.enc_nearest(float(t[b])) == b
        assert oracle.enc_bits(float(t[b])) == b


@pytest.mark.slow
def test_two_encoders_agree_on_every_fp32_pattern():
    # brute force: the nearest-table encoder and the bit-arithmetic encoder on all 2^32
    # patterns (non-finite ones are outside the precondition and skipped)
    assert oracle.enc_crosscheck(0, 0xFFFFFFFF) == 0


@pytest.mark.slow
def test_encoder_matches_torch_on_all_fp32_up_to_448():
    # torch's float8_e4m3fn conversion rounds to nearest-even; up to |y| <= 448 it is the
    # same function as ours (it does not saturate beyond, so larger inputs are clamped
    # first). Every non-negative fp32 pattern up to 448, and negatives on a stride.
    hi = np.float32(448.0).view(np.uint32)
    step = 1 << 26
    for start in range(0, int(hi) + 1, step):
        u = np.arange(start, min(start + step, int(hi) + 1), dtype=np.uint32)
        for sign in (0, 1):
            uu = u if sign == 0 else (u[::7] | np.uint32(0x80000000))
            y = uu.view(np.float32)
            ref = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(oracle.encode(y), ref), start


def test_saturation_above_448():
    y = np.array([448.0, 448.00003, 463.9, 464.0, 1e4, 3.0e38, np.inf], np.float32)
    assert (oracle.encode(y) == 0x7E).all()
    assert (oracle.encode(-y) == 0xFE).all()


# ---------------------------------------------------------------------------------
# casts
# ---------------------------------------------------------------------------------
def _torch_cast_reference(x: np.ndarray, group_shape):
    """The cast written with torch library routines: amax per group, s = amax / 448 in fp32,
    q = e4m3(x / s) with saturation (clamp, then torch's nearest-even conversion)."""
    xt = torch.from_numpy(x)
    gm, gk = group_shape
    M, K = x.shape
    g = xt.reshape(M // gm, gm, K // gk, gk).abs().amax(dim=(1, 3))
    s = g / torch.tensor(448.0, dtype=torch.float32)
    sx = s.repeat_interleave(gm, 0).repeat_interleave(gk, 1)
    y = (xt / sx).clamp(-448.0, 448.0)
    q = y.to(torch.float8_e4m3fn).view(torch.uint8)
    zero = sx == 0
    q[zero] = torch.where(torch.signbit(xt[zero]), 0x80, 0x00).to(torch.uint8)
    return q.numpy(), s.numpy()


def test_cast_per_token_matches_torch_reference():
    x = synth.with_outliers(synth.normal((96, 1024), 11, 1), 11)
    x[3, 128:256] = 0.0  # an all-zero chunk
    x[4, 0:128] = -0.0
    x[5, 256:384] *= 1e-40  # fp32 subnormals: s underflows to 0 for some, subnormal for others
    x[6, 384:512] *= 1e-36
    q, s = oracle.cast_per_token(x)
    qr, sr = _torch_cast_reference(x, (1, 128))
    assert np.array_equal(q, qr)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert s[3, 1] == 0 and (q[3, 128:256] == 0).all()
    assert (q[4, 0:128] == 0x80).all()


def test_cast_per_block_matches_torch_reference():
    w = synth.normal((384, 640), 12, 2, std=0.02)
    w[128:256, 256:384] = 0.0
    q, s = oracle.cast_per_block(w)
    qr, sr = _torch_cast_reference(w, (128, 128))
    assert q.shape == (384, 640) and s.shape == (3, 5)
    assert np.array_equal(q, qr)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))


def test_cast_invariants():
    x = synth.with_outliers(synth.normal((64, 2048), 13, 1), 13)
    q, s = oracle.cast_per_token(x)
    t = oracle.decode_table()
    xc = x.reshape(64, 16, 128)
    qc = q.reshape(64, 16, 128)
    # (i) the amax element of every chunk is coded +-448
    idx = np.abs(xc).argmax(axis=2)
    amax_codes = np.take_along_axis(qc, idx[..., None], 2)[..., 0]
    assert np.isin(amax_codes, [0x7E, 0xFE]).all()
    # (ii) no NaN codes
    assert not np.isin(q, [0x7F, 0xFF]).any()
    # (iii) reconstruction error within half an e4m3 step (relative 2^-4 normal, 2^-10 abs sub)
    deq = t[qc] * s[..., None].astype(np.float64)
    y = xc / s[..., None].astype(np.float64)
    step = np.where(np.abs(y) >= 2 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y), 1e-300))) - 3), 2.0 ** -9)
    assert (np.abs(deq - xc) <= (0.5 * step + 1e-6 * np.abs(y)) * s[..., None]).all()
    # (iv) power-of-two scaling of x: identical codes, scales scaled exactly
    q2, s2 = oracle.cast_per_token(x * np.float32(2.0 ** 5))
    assert np.array_equal(q2, q) and np.array_equal(s2, s * np.float32(32.0))
    # (v) a permutation inside a chunk permutes the codes
    perm = synth.rng(13, 9).permutation(128)
    xp = xc[:, :, perm].reshape(64, 2048)
    qp, sp = oracle.cast_per_token(xp)
    assert np.array_equal(qp.reshape(64, 16, 128), qc[:, :, perm]) and np.array_equal(sp, s)


def _pow2_ceil_reference(amax: np.ndarray) -> np.ndarray:
    """The reading of power-of-two scales, computed with numpy alone: the smallest power of
    two >= fp32(amax/448), at least 2^-126."""
    v = (amax.astype(np.float32) / np.float32(448.0)).astype(np.float32)
    m, e = np.frexp(v.astype(np.float64))           # v = m * 2^e, m in [0.5, 1)
    s = np.where(m == 0.5, v.astype(np.float64), np.ldexp(1.0, e))
    s = np.where(v == 0, 0.0, s)                     # frexp(0) = (0, 0): only the floor applies
    return np.maximum(s, 2.0 ** -126).astype(np.float32)


def test_pow2_golden_points(golden_dir):
    rows = []
    for line in open(os.path.join(golden_dir, "pow2_scale_points.txt")):
        if line.startswith("#") or not line.strip():
            continue
        first, rest, s_exp, code, _ = [f.strip() for f in line.split("|")]
        rows.append((float(first), float(rest), float(s_exp), int(code, 16)))
    x = np.array([[f] + [r] * 127 for f, r, _, _ in rows], np.float32)
    q, s = oracle.cast_per_token(x, pow2=True)
    for i, (_, _, s_exp, code) in enumerate(rows):
        assert s[i, 0] == np.float32(s_exp), (i, s[i, 0], s_exp)
        assert q[i, 0] == code, (i, hex(q[i, 0]), hex(code))


def test_pow2_cast_matches_reading_and_encoder():
    # s from numpy alone; q from the (separately pinned) encoder applied to the exact x / s
    x = synth.with_outliers(synth.normal((96, 1024), 31, synth.TID_A), 31)
    x[0, :128] = 0.0
    x[1, :128] *= np.float32(1e-38)                 # s hits the 2^-126 floor
    x[2, :128] *= np.float32(1e30)
    q, s = oracle.cast_per_token(x, pow2=True)
    amax = np.abs(x.reshape(96, 8, 128)).max(axis=2)
    s_ref = _pow2_ceil_reference(amax)
    assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
    assert ((s.view(np.uint32) & 0x7FFFFF) == 0).all()      # exact powers of two
    y = (x.reshape(96, 8, 128) / s_ref[:, :, None]).astype(np.float32).reshape(96, 1024)
    assert np.array_equal(q, oracle.encode(y))
    # no code saturates: |x / s| <= 448 by construction
    assert (np.abs(oracle.decode_table()[q]) <= 448).all()
    # weights: the same rule over 128x128 blocks
    w = synth.normal((256, 384), 32, synth.TID_B, std=0.02)
    qb, sb = oracle.cast_per_block(w, pow2=True)
    bmax = np.abs(w.reshape(2, 128, 3, 128)).max(axis=(1, 3))
    assert np.array_equal(sb.view(np.uint32), _pow2_ceil_reference(bmax).view(np.uint32))


def test_pow2_cast_power_of_two_invariance_is_exact():
    # x -> 2^p x gives identical codes and s -> 2^p s exactly (no clamp or overflow in range)
    x = synth.normal((32, 512), 33, synth.TID_A)
    q0, s0 = oracle.cast_per_token(x, pow2=True)
    for p in (-20, -3, 5, 40):
        q1, s1 = oracle.cast_per_token((x * np.float32(2.0 ** p)).astype(np.float32), pow2=True)
        assert np.array_equal(q0, q1)
        assert np.array_equal(s1, (s0 * np.float32(2.0 ** p)).astype(np.float32))


def test_bf16_input_is_widened_exactly():
    x = synth.normal((8, 256), 14, 1)
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    w = oracle.bf16_bits_to_f32(bits)
    assert np.array_equal(w, torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy())


# ---------------------------------------------------------------------------------
# GEMM
# ---------------------------------------------------------------------------------
def _quantized_pair(M, N, K, seed, outliers=False):
    a, b = synth.dense_inputs(M, N, K, seed, outliers)
    qa, sa = oracle.cast_per_token(a)
    qb, sb = oracle.cast_per_block(b)
    return qa, sa, qb, sb


def _int_dec():
    """e4m3 values in units of 2^-9, computed from integer fields (another formulation)."""
    out = np.zeros(256, np.int64)
    for c in range(256):
        e, m = (c >> 3) & 15, c & 7
        v = m if e == 0 else (8 + m) << (e - 1)
        out[c] = -v if c & 0x80 else v
    return out


def test_block_sums_equal_integer_path_bitwise():
    qa, sa, qb, sb = _quantized_pair(8, 128, 512, 21)
    P = oracle.block_sums(qa, qb)
    iv = _int_dec()
    ai = iv[qa].reshape(8, 4, 128)
    bi = iv[qb].reshape(128, 4, 128)
    Pint = np.einsum("mjk,njk->mnj", ai, bi)  # int64, exact (< 2^43)
    assert np.array_equal(P, Pint.astype(np.float64) * 2.0 ** -18)


def test_gemm_exact_rational_bruteforce_tiny():
    qa, sa, qb, sb = _quantized_pair(3, 128, 256, 22)
    R = oracle.gemm(qa, sa, qb, sb)
    dec = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).tolist()
    for m in range(3):
        for n in range(0, 128, 17):
            acc = Fraction(0)
            for k in range(256):
                acc += (Fraction(dec[qa[m, k]]) * Fraction(float(sa[m, k // 128]))
                        * Fraction(dec[qb[n, k]]) * Fraction(float(sb[n // 128, k // 128])))
            assert abs(R[m, n] - float(acc)) <= 4e-16 * max(abs(float(acc)), 1e-300) + 1e-300


def _torch_dequant_first(qa, sa, qb, sb):
    A = torch.from_numpy(qa).view(torch.float8_e4m3fn).to(torch.float64)
    B = torch.from_numpy(qb).view(torch.float8_e4m3fn).to(torch.float64)
    SA = torch.from_numpy(sa).double().repeat_interleave(128, 1)
    SB = torch.from_numpy(sb).double().repeat_interleave(128, 0).repeat_interleave(128, 1)
    Ad, Bd = A * SA, B * SB
    return (Ad @ Bd.T).numpy(), (Ad.abs() @ Bd.abs().T).numpy()


def test_gemm_matches_dequantize_first_library_matmul():
    qa, sa, qb, sb = _quantized_pair(200, 384, 640, 23, outliers=True)
    R = oracle.gemm(qa, sa, qb, sb)
    Rt, absum = _torch_dequant_first(qa, sa, qb, sb)
    assert (np.abs(R - Rt) <= 1e-12 * absum).all()


def test_gemm_closed_forms():
    K, N = 512, 256
    # identity B (1.0 on the diagonal, sb = 1): R[m, n] = dequantised A[m, n]
    qa, sa, _, _ = _quantized_pair(16, N, K, 24)
    qb = np.zeros((N, K), np.uint8)
    qb[np.arange(N), np.arange(N)] = 0x38
    sb = np.ones((N // 128, K // 128), np.float32)
    R = oracle.gemm(qa, sa, qb, sb)
    t = oracle.decode_table()
    deqA = t[qa] * np.repeat(sa.astype(np.float64), 128, axis=1)
    assert np.array_equal(R, deqA[:, :N])
    # all ones with constant scales alpha, beta: R = K * alpha * beta
    alpha, beta = 0.375, 1.5
    qa1 = np.full((4, K), 0x38, np.uint8)
    qb1 = np.full((N, K), 0x38, np.uint8)
    R1 = oracle.gemm(qa1, np.full((4, K // 128), alpha, np.float32), qb1,
                     np.full((N // 128, K // 128), beta, np.float32))
    assert (R1 == K * alpha * beta).all()
    # one-hot K block: zero scales except block j -> R is that block's term alone
    qa2, sa2, qb2, sb2 = _quantized_pair(8, N, K, 25)
    for j in range(K // 128):
        sa_j = np.zeros_like(sa2)
        sa_j[:, j] = sa2[:, j]
        Rj = oracle.gemm(qa2, sa_j, qb2, sb2)
        P = oracle.block_sums(qa2, qb2)[:, :, j]
        expect = (sa2[:, j].astype(np.float64)[:, None] * sb2[np.arange(N) // 128, j][None, :]) * P
        assert np.array_equal(Rj, expect)


def test_gemm_pairs_equal_full_gemm():
    qa, sa, qb, sb = _quantized_pair(40, 256, 384, 26)
    R = oracle.gemm(qa, sa, qb, sb)
    r = synth.rng(26, 7)
    rows, cols = r.integers(0, 40, 500), r.integers(0, 256, 500)
    assert np.array_equal(oracle.gemm_pairs(qa, sa, qb, sb, rows, cols), R[rows, cols])


def _wrong_expert_stride(qb, sb):
    """The expert weights as a kernel with a halved expert stride would read them: expert g's
    slab starting g*N*K/2 bytes (and g*(N/128)*(K/128)/2 scales) into the stacked tensors."""
    G, N, K = qb.shape
    fb, fs = qb.reshape(-1), sb.reshape(-1)
    nb, ns = N * K, sb.shape[1] * sb.shape[2]
    bad_b = np.stack([fb[g * nb // 2: g * nb // 2 + nb].reshape(N, K) for g in range(G)])
    bad_s = np.stack([fs[g * ns // 2: g * ns // 2 + ns].reshape(sb.shape[1:]) for g in range(G)])
    return bad_b, bad_s


def test_gemm_pairs_grouped_equals_grouped_oracles():
    # the sampled form used by the full-size grouped parity checks, pinned against the
    # contiguous and masked oracles (themselves pinned to the dense one per expert below)
    G, N, K = 4, 256, 384
    a, b, mi = synth.contiguous_inputs(G, 300, N, K, seed=33)
    qa, sa = oracle.cast_per_token(a)
    qb, sb = oracle.cast_per_block(b.reshape(G * N, K))
    qb, sb = qb.reshape(G, N, K), sb.reshape(G, N // 128, K // 128)
    Rc = oracle.grouped_contiguous(qa, sa, qb, sb, mi)
    r = synth.rng(33, 7)
    rows, cols = r.integers(0, mi.size, 3000), r.integers(0, N, 3000)
    got = oracle.gemm_pairs(qa, sa, qb, sb, rows, cols, group_of_row=mi)
    pad = mi[rows] < 0
    assert pad.any() and (~pad).any()
    assert np.isnan(got[pad]).all()  # padding rows (-1): NaN, never a read before b
    assert np.array_equal(got[~pad], Rc[rows[~pad], cols[~pad]])
    # planted mistakes: a halved expert stride, and the expert of every row taken as 0
    bad_b, bad_s = _wrong_expert_stride(qb, sb)
    wrong = oracle.gemm_pairs(qa, sa, bad_b, bad_s, rows[~pad], cols[~pad], group_of_row=mi)
    assert not oracle.compare(wrong, Rc[rows[~pad], cols[~pad]])["ok"]
    zero = oracle.gemm_pairs(qa, sa, qb, sb, rows[~pad], cols[~pad], group_of_row=np.zeros_like(mi))
    assert not oracle.compare(zero, Rc[rows[~pad], cols[~pad]])["ok"]
    # out-of-range groups give NaN as well
    assert np.isnan(oracle.gemm_pairs(qa, sa, qb, sb, rows[:4], cols[:4],
                                      group_of_row=np.full_like(mi, G))).all()

    # masked layout: rows of [G*M_max, K] with group r // M_max
    M_max = 96
    am, bm, mm = synth.masked_inputs(G, M_max, N, K, seed=34)
    qam, sam = oracle.cast_per_token(am.reshape(G * M_max, K))
    qbm, sbm = oracle.cast_per_block(bm.reshape(G * N, K))
    qbm, sbm = qbm.reshape(G, N, K), sbm.reshape(G, N // 128, K // 128)
    full = np.full(G, M_max, np.int32)
    Rm = oracle.grouped_masked(qam.reshape(G, M_max, K), sam.reshape(G, M_max, K // 128), qbm, sbm, full)
    Rm = Rm.reshape(G * M_max, N)
    group = (np.arange(G * M_max) // M_max).astype(np.int32)
    rows, cols = r.integers(0, G * M_max, 2000), r.integers(0, N, 2000)
    got = oracle.gemm_pairs(qam, sam, qbm, sbm, rows, cols, group_of_row=group)
    assert np.array_equal(got, Rm[rows, cols])
    bad_b, bad_s = _wrong_expert_stride(qbm, sbm)
    wrong = oracle.gemm_pairs(qam, sam, bad_b, bad_s, rows, cols, group_of_row=group)
    assert not oracle.compare(wrong, Rm[rows, cols])["ok"]


# ---------------------------------------------------------------------------------
# grouped layouts
# ---------------------------------------------------------------------------------
def test_contiguous_equals_dense_per_expert():
    G, N, K = 4, 256, 384
    a, b, mi = synth.contiguous_inputs(G, 300, N, K, seed=31)
    qa, sa = oracle.cast_per_token(a)
    qb, sb = oracle.cast_per_block(b)
    R = oracle.grouped_contiguous(qa, sa, qb, sb, mi)
    assert np.isnan(R[mi < 0]).all()
    for g in range(G):
        rows = np.nonzero(mi == g)[0]
        Rd = oracle.gemm(qa[rows], sa[rows], qb[g], sb[g])
        assert np.array_equal(R[rows], Rd)
    # layout: every 128-row block holds one expert, padded with -1 at its end
    assert mi.size % 128 == 0
    for blk in mi.reshape(-1, 128):
        assert blk[0] >= 0 and set(np.unique(blk)) <= {blk[0], -1}


def test_masked_equals_dense_per_expert_and_clamps():
    G, Mm, N, K = 3, 64, 128, 256
    a, b, _ = synth.masked_inputs(G, Mm, N, K, seed=32)
    qa, sa = oracle.cast_per_token(a.reshape(G * Mm, K))
    qa, sa = qa.reshape(G, Mm, K), sa.reshape(G, Mm, K // 128)
    qb, sb = oracle.cast_per_block(b)
    full = oracle.grouped_masked(qa, sa, qb, sb, np.full(G, Mm, np.int32))
    for g in range(G):
        assert np.array_equal(full[g], oracle.gemm(qa[g], sa[g], qb[g], sb[g]))
    none = oracle.grouped_masked(qa, sa, qb, sb, np.zeros(G, np.int32))
    assert np.isnan(none).all()
    part = oracle.grouped_masked(qa, sa, qb, sb, np.array([-5, 17, 1000], np.int32))
    assert np.isnan(part[0]).all()
    assert np.array_equal(part[1, :17], full[1, :17]) and np.isnan(part[1, 17:]).all()
    assert np.array_equal(part[2], full[2])


# ---------------------------------------------------------------------------------
# the acceptance comparison, and that the pins catch planted mistakes
# ---------------------------------------------------------------------------------
def test_compare_accepts_bf16_rounding_of_the_exact_result():
    qa, sa, qb, sb = _quantized_pair(128, 256, 512, 41)
    R = oracle.gemm(qa, sa, qb, sb)
    y = torch.from_numpy(R).to(torch.float32).to(torch.bfloat16).double().numpy()
    res = oracle.compare(y, R)
    assert res["ok"], res


def test_pins_detect_planted_mistakes():
    qa, sa, qb, sb = _quantized_pair(64, 256, 512, 42)
    R = oracle.gemm(qa, sa, qb, sb)
    Rt, _ = _torch_dequant_first(qa, sa, qb, sb)
    # a dropped K block
    sa_drop = sa.copy()
    sa_drop[:, -1] = 0
    assert not oracle.compare(oracle.gemm(qa, sa_drop, qb, sb), Rt)["ok"]
    # a transposed weight-scale grid (wrong block index)
    sb_sq = np.ascontiguousarray(sb[:, :2])  # [2, 2]: square so the transpose is the same shape
    qa_s = np.ascontiguousarray(qa[:, :256])
    sa_s = np.ascontiguousarray(sa[:, :2])
    qb_s = np.ascontiguousarray(qb[:, :256])
    good = oracle.gemm(qa_s, sa_s, qb_s, sb_sq)
    bad = oracle.gemm(qa_s, sa_s, qb_s, np.ascontiguousarray(sb_sq.T * np.float32(1.7)))
    assert not oracle.compare(bad, good)["ok"]
    # a sign error on one row
    y = R.copy()
    y[5] = -y[5]
    assert not oracle.compare(y, Rt)["ok"]
    # a transposed result (operand roles swapped) on a square problem
    qa2, sa2, qb2, sb2 = _quantized_pair(128, 128, 256, 44)
    R2 = oracle.gemm(qa2, sa2, qb2, sb2)
    assert not oracle.compare(R2.T, R2)["ok"]
    # the wrong expert in a grouped call
    G, N, K = 2, 128, 256
    a, b, mi = synth.contiguous_inputs(G, 200, N, K, seed=43)
    qa, sa = oracle.cast_per_token(a)
    qb, sb = oracle.cast_per_block(b)
    R = oracle.grouped_contiguous(qa, sa, qb, sb, mi)
    wrong = np.where(mi >= 0, 1 - mi, -1).astype(np.int32)
    Rw = oracle.grouped_contiguous(qa, sa, qb, sb, wrong)
    assert not oracle.compare(Rw, R, mask=mi >= 0)["ok"]
