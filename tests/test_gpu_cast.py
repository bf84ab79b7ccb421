"""GPU parity of the FP8 casts against the oracle: bit-exact in codes and scales."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_same_bits, assert_same_bytes, gpu_cast_blocks, gpu_cast_tokens, kmajor, say,
                     to_dev)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import moe_grouped_gemm_e4m3_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("M,K,outliers", [(128, 512, False), (64, 2048, False), (64, 1536, False),
                                          (1, 128, False), (333, 1280, True)])
def test_cast_per_token_bit_exact(dg, M, K, outliers):
    say("cast_per_token %dx%d outliers=%s" % (M, K, outliers))
    a = synth.normal((M, K), 100 + M, synth.TID_A)
    if outliers:
        a = synth.with_outliers(a, 100 + M)
    q, s = gpu_cast_tokens(dg, a)
    torch.cuda.synchronize()
    qo, so = oracle.cast_per_token(a)
    assert_same_bytes(q, qo, "q")
    assert tuple(s.shape) == (K // 128, M)
    assert_same_bits(s, kmajor(so), "s")


def test_cast_per_token_edge_chunks(dg):
    x = synth.normal((16, 1024), 7, synth.TID_A)
    x[0, 0:128] = 0.0                      # all zero: s = 0, codes +0
    x[1, 0:128] = -0.0                     # negative zeros keep the sign
    x[1, 128:256] = 0.0
    x[1, 130] = -0.0
    x[2, 0:128] *= np.float32(1e-44)       # fp32 subnormals: s underflows to 0
    x[3, 0:128] *= np.float32(1e-36)       # s is an fp32 subnormal
    x[4, 0:128] *= np.float32(1e-30)
    x[5, 0:128] = np.float32(432.0)        # ties at the top
    x[5, 0] = np.float32(448.0)
    x[6, 0:128] = np.linspace(-448, 448, 128, dtype=np.float32)
    x[7, 0:128] = np.float32(1e30)         # huge but finite
    x[7, 1] = np.float32(-3e29)
    x[8, :128] = np.float32(2.0 ** -10)    # exact power of two everywhere
    say("cast_per_token edge chunks")
    q, s = gpu_cast_tokens(dg, x)
    qo, so = oracle.cast_per_token(x)
    assert_same_bytes(q, qo, "edge q")
    assert_same_bits(s, kmajor(so), "edge s")
    assert so[0, 0] == 0 and so[2, 0] == 0 and so[3, 0] > 0


def _anchor_sweep(values: np.ndarray) -> np.ndarray:
    """Lay values out in 128-element chunks whose first element is 448, so s = 1 exactly and
    every other element is encoded as itself."""
    per = 127
    n = (values.size + per - 1) // per
    buf = np.zeros((n, 128), np.float32)
    buf[:, 0] = 448.0
    flat = np.zeros(n * per, np.float32)
    flat[:values.size] = values
    buf[:, 1:] = flat.reshape(n, per)
    return buf


def _conversion_values() -> np.ndarray:
    """fp32 patterns in [-448, 448] around every e4m3 rounding decision: for each sign,
    exponent and top-3 mantissa prefix, low 20 bits at the edges of the rounding window;
    plus the whole fp32 range below 2^-6 on a prime stride, plus every 2^-10 multiple +-1 ulp."""
    hi = np.float32(448.0).view(np.uint32)
    top = np.arange(0, (int(hi) >> 20) + 1, dtype=np.uint32) << 20
    lows = np.array([0, 1, 2, 0x3FFFF, 0x7FFFE, 0x7FFFF, 0x80000, 0x80001, 0xBFFFF, 0xFFFFE, 0xFFFFF],
                    dtype=np.uint32)
    pats = (top[:, None] | lows[None, :]).ravel()
    sub = np.arange(0, 0x3C800000, 9973, dtype=np.uint32)
    grid = (np.arange(0, 17, dtype=np.float32) * np.float32(2.0 ** -10)).view(np.uint32)
    near = np.concatenate([grid, grid + 1, np.maximum(grid, 1) - 1])
    pats = np.unique(np.concatenate([pats, sub, near]))
    pats = pats[pats <= hi]
    v = pats.view(np.float32)
    return np.concatenate([v, -v])


def test_cast_conversion_sweep(dg):
    vals = _conversion_values()
    x = _anchor_sweep(vals)
    say("cast conversion sweep (%d values)" % vals.size)
    q, s = gpu_cast_tokens(dg, x)
    qo, so = oracle.cast_per_token(x)
    assert (so == 1.0).all()
    assert_same_bytes(q, qo, "sweep q")


def test_cast_bf16_input(dg):
    x = synth.with_outliers(synth.normal((40, 768), 8, synth.TID_A), 8)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    say("cast bf16 input 40x768")
    q, s = dg.cast_fp8_per_token(xb.to("cuda:0"))
    qo, so = oracle.cast_per_token(xb.float().numpy())
    assert_same_bytes(q, qo, "bf16 q")
    assert_same_bits(s, kmajor(so), "bf16 s")
    wb = torch.from_numpy(synth.normal((256, 384), 9, synth.TID_B, 0.02)).to(torch.bfloat16)
    q2, s2 = dg.cast_fp8_per_block(wb.to("cuda:0"))
    qo2, so2 = oracle.cast_per_block(wb.float().numpy())
    assert_same_bytes(q2, qo2, "bf16 block q")
    assert_same_bits(s2, so2, "bf16 block s")


@pytest.mark.parametrize("N,K", [(128, 128), (384, 640), (7168, 2048)])
def test_cast_per_block_bit_exact(dg, N, K):
    say("cast_per_block %dx%d" % (N, K))
    w = synth.normal((N, K), 200 + N, synth.TID_B, std=0.02)
    w[:128, :128] = 0.0
    q, s = gpu_cast_blocks(dg, w)
    qo, so = oracle.cast_per_block(w)
    assert_same_bytes(q, qo, "block q")
    assert_same_bits(s, so, "block s")


@pytest.mark.parametrize("G,M,K", [(3, 40, 384), (4, 128, 512), (2, 1, 128)])
def test_cast_per_token_grouped(dg, G, M, K):
    # [G,M,K] activations: scales [G,K/128,M], the masked GEMM's sfa; codes as for [G*M,K]
    a = synth.normal((G, M, K), 400 + G * M, synth.TID_A)
    say("cast_per_token grouped %dx%dx%d" % (G, M, K))
    q, s = gpu_cast_tokens(dg, a)
    assert tuple(q.shape) == (G, M, K) and tuple(s.shape) == (G, K // 128, M)
    qo, so = oracle.cast_per_token(a.reshape(G * M, K))
    assert_same_bytes(q, qo.reshape(G, M, K), "grouped q")
    assert_same_bits(s, kmajor(so.reshape(G, M, K // 128)), "grouped s")


def test_cast_grouped_weights(dg):
    w = synth.normal((3, 256, 384), 300, synth.TID_B, std=0.02)
    say("cast_per_block grouped 3x256x384")
    q, s = dg.cast_fp8_per_block(to_dev(w))
    assert tuple(s.shape) == (3, 2, 3)
    qo, so = oracle.cast_per_block(w)
    assert_same_bytes(q, qo, "grouped block q")
    assert_same_bits(s, so, "grouped block s")


@pytest.mark.slow
def test_cast_prefill_activation_full_size(dg):
    # the largest activation of the configurations: 4096 x 18432 with outliers
    a = synth.with_outliers(synth.normal((4096, 18432), 0, synth.TID_A), 0)
    say("cast_per_token 4096x18432 full size")
    q, s = gpu_cast_tokens(dg, a)
    qo, so = oracle.cast_per_token(a)
    assert_same_bytes(q, qo, "prefill q")
    assert_same_bits(s, kmajor(so), "prefill s")
