"""The FFN acceptance checks (tests/ffn_checks.py) on the CPU: they accept the oracle's own
results and reject planted mistakes (a code two steps off, a scale 1% off, a wrong
output). CPU only."""
import numpy as np
import pytest

import ffn_checks as fc
import oracle
import synth


def _case(pow2):
    G, H, I = 2, 256, 256
    mi = np.repeat(np.arange(G, dtype=np.int32), 40)
    x = synth.normal((mi.size, H), 11, synth.TID_A)
    w1, w2 = synth.ffn_weights(G, H, I, 11)
    xq, sx = oracle.cast_per_token(x, pow2)
    w1q, s1 = oracle.cast_per_block(w1, pow2)
    w2q, s2 = oracle.cast_per_block(w2, pow2)
    ref = oracle.moe_ffn_contiguous(xq, sx, w1q, s1, w2q, s2, mi, pow2)
    rows = np.nonzero(mi == 1)[0]
    L = fc.abs_products(fc.dequant_rows(xq[rows], sx[rows]), fc.dequant_blocks(w1q[1], s1[1]))
    e_h = fc.h_band(ref["gate_up"][rows], L, H // 128)
    sub = {k: v[rows] for k, v in ref.items()}
    return sub, e_h, fc.dequant_blocks(w2q[1], s2[1])


@pytest.mark.parametrize("pow2", [False, True])
def test_checks_accept_the_oracle(pow2):
    r, e_h, w2d = _case(pow2)
    c_lo, c_hi, s_lo, s_hi = fc.check_recast(r["h"], e_h, r["hq"], r["sh"], r["hq"], pow2, "oracle", min_exact=1.0)
    allow = fc.output_allowance(c_lo, c_hi, s_lo, s_hi, r["hq"], r["sh"], w2d)
    fc.check_output(r["y"], r["y"], allow, "oracle")
    # the band is narrow: most codes are pinned to one value (the worst-case band grows
    # with K; the GPU tests also require 99% of the codes to equal the oracle's)
    assert np.mean(c_lo == c_hi) > 0.95


@pytest.mark.parametrize("pow2", [False, True])
def test_checks_reject_planted_mistakes(pow2):
    r, e_h, w2d = _case(pow2)
    dec = fc.DEC
    # a code two steps off (towards zero keeps it inside the format)
    hq = r["hq"].copy()
    i = np.argmax(np.abs(dec[hq[3]]) * (np.abs(dec[hq[3]]) > 1))
    hq[3, i] = hq[3, i] - 2
    with pytest.raises(AssertionError):
        fc.check_recast(r["h"], e_h, hq, r["sh"], r["hq"], pow2, "planted code")
    # a chunk scale off by 1% (pow2: by a factor of two)
    sh = r["sh"].copy()
    sh[5, 1] *= 2.0 if pow2 else 1.01
    with pytest.raises(AssertionError):
        fc.check_recast(r["h"], e_h, r["hq"], sh, r["hq"], pow2, "planted scale")
    # an output 3% off
    c_lo, c_hi, s_lo, s_hi = fc.check_recast(r["h"], e_h, r["hq"], r["sh"], r["hq"], pow2, "oracle")
    allow = fc.output_allowance(c_lo, c_hi, s_lo, s_hi, r["hq"], r["sh"], w2d)
    y = r["y"].copy()
    j = np.argmax(np.abs(y[7]))
    y[7, j] *= 1.03
    with pytest.raises(AssertionError):
        fc.check_output(y, r["y"], allow, "planted output")
