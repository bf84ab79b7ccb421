"""GPU parity of the power-of-two (UE8M0) scale variants against the oracle: casts bit-exact,
GEMMs (the block-scaled MFMA path and the fallbacks) within the tolerance, and the exact
power-of-two invariance of the output."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_close, assert_same_bits, assert_same_bytes, bf16_values, gpu_cast_blocks,
                     gpu_cast_tokens, kmajor, quantised_dense, say, to_dev)

pytestmark = pytest.mark.gpu

SENTINEL = -1


@pytest.fixture(scope="module")
def dg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import moe_grouped_gemm_e4m3_amd as m
    m.lib()
    return m


@pytest.mark.parametrize("shape", [(96, 1024), (3, 40, 384), (1, 128)])
def test_cast_per_token_ue8m0_bit_exact(dg, shape):
    a = synth.with_outliers(synth.normal(shape, 500 + shape[-2], synth.TID_A), 500)
    a.reshape(-1, shape[-1])[0, :128] = 0.0
    a.reshape(-1, shape[-1])[-1, :128] *= np.float32(1e-39)
    say("cast per token ue8m0 %s" % (shape,))
    q, s = gpu_cast_tokens(dg, a, ue8m0=True)
    qo, so = oracle.cast_per_token(a.reshape(-1, shape[-1]), pow2=True)
    assert_same_bytes(q, qo.reshape(shape), "q")
    assert_same_bits(s, kmajor(so.reshape(shape[:-1] + (shape[-1] // 128,))), "s")


def test_cast_per_block_ue8m0_bit_exact(dg):
    w = synth.normal((2, 256, 640), 501, synth.TID_B, std=0.02)
    w[0, :128, :128] = 0.0
    say("cast per block ue8m0")
    q, s = gpu_cast_blocks(dg, w, ue8m0=True)
    qo, so = oracle.cast_per_block(w, pow2=True)
    assert_same_bytes(q, qo, "q")
    assert_same_bits(s, so, "s")


TILES = [None, "t3_256x128", "t3_128x256", "t2_256x128", "t2_128x128", "t3_256x256b"]


@pytest.mark.parametrize("M,N,K", [(512, 512, 2304), (300, 768, 1280), (77, 256, 384), (256, 256, 128)])
def test_dense_ue8m0_tile_kernels(dg, switches, M, N, K):
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, M, N, K, seed=M + 1, outliers=True, ue8m0=True)
    R = oracle.gemm(oqa, osa, oqb, osb)
    for v in TILES:
        if v:
            switches.setenv("DG_TILE", v)
        else:
            switches.delenv("DG_TILE", raising=False)
        say("dense ue8m0 tile %s M=%d N=%d K=%d" % (v, M, N, K))
        d = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=3, ue8m0=True)
        assert_close(bf16_values(d), R, "ue8m0 tile %s" % v)


# (variable, value): the LDS decode schedule's configurations and the activation-resident
# ones (which fall back to the former where the activations do not fit beside the ring)
DECODE = [(None, None), ("DG_DECODE2", "96,4,3,8"), ("DG_DECODE2", "96,1,12,6"), ("DG_DECODE2", "32,8,2,8"),
          ("DG_DECODE2", "32,1,16,2"), ("DG_DECODE2", "16,8,3,8"), ("DG_DECODE3", "2,2,3,4"),
          ("DG_DECODE3", "1,6,1,4"), ("DG_DECODE3", "2,3,2,4"), ("DG_DECODE3", "4,1,6,4"), ("DG_DECODE3", "1,8,1,3")]


@pytest.mark.parametrize("M,N,K", [(64, 1536, 1536), (37, 768, 2048), (130, 384, 1152)])
def test_dense_ue8m0_decode(dg, switches, M, N, K):
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, M, N, K, seed=M + 2, ue8m0=True)
    R = oracle.gemm(oqa, osa, oqb, osb)
    for var, v in DECODE:
        switches.delenv("DG_DECODE2", raising=False)
        switches.delenv("DG_DECODE3", raising=False)
        if var:
            switches.setenv(var, v)
        say("dense ue8m0 decode %s=%s M=%d N=%d K=%d" % (var, v, M, N, K))
        d = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=1, ue8m0=True)
        assert_close(bf16_values(d), R, "ue8m0 decode %s" % v)
    d = dg.gemm_fp8_nt(qa, sa, qb, sb, ue8m0=True)  # automatic choice
    assert_close(bf16_values(d), R, "ue8m0 auto")


@pytest.mark.parametrize("sched", [1, 2, 3])
def test_ue8m0_power_of_two_invariance_is_bitwise(dg, sched):
    # sa -> 2^p sa gives D -> 2^p D exactly, on the block-scaled MFMA path too
    (qa, sa, qb, sb), _ = quantised_dense(dg, 256, 512, 1024, seed=9, ue8m0=True)
    say("ue8m0 invariance schedule %d" % sched)
    d1 = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=sched, ue8m0=True)
    d2 = dg.gemm_fp8_nt(qa, sa * 8.0, qb, sb, schedule=sched, ue8m0=True)
    d3 = dg.gemm_fp8_nt(qa, sa, qb, sb * 0.25, schedule=sched, ue8m0=True)
    assert torch.equal((d1.float() * 8.0).view(torch.int32), d2.float().view(torch.int32))
    assert torch.equal((d1.float() * 0.25).view(torch.int32), d3.float().view(torch.int32))


def test_contiguous_ue8m0(dg, switches):
    G, N, K = 3, 512, 4352
    a, b, mi = synth.contiguous_inputs(G, 300, N, K, 23)
    qa, sa = gpu_cast_tokens(dg, a, ue8m0=True)
    qb, sb = gpu_cast_blocks(dg, b, ue8m0=True)
    oqa, osa = oracle.cast_per_token(a, pow2=True)
    oqb, osb = oracle.cast_per_block(b, pow2=True)
    assert_same_bytes(qa, oqa, "A")
    assert_same_bits(sa, kmajor(osa), "sA")
    assert_same_bits(sb, osb, "sB")
    R = oracle.grouped_contiguous(oqa, osa, oqb, osb, mi)
    valid = mi[:, None].repeat(N, 1) >= 0
    for v in ("t3_128x256", "t2_128x128"):
        switches.setenv("DG_TILE", v)
        say("contiguous ue8m0 %s" % v)
        d = dg.grouped_gemm_contiguous(qa, sa, qb, sb, to_dev(mi), ue8m0=True)
        assert_close(bf16_values(d), R, "contiguous ue8m0 %s" % v, mask=valid)


# tile: a tile kernel forced through DG_TILE, or "d3:..." the activation-resident decode
# kernel forced through DG_DECODE3 (decode schedule)
@pytest.mark.parametrize("sched,tile", [(1, None), (3, None), (3, "t3_128x256"), (2, None), (1, "d3:1,8,1,3"),
                                        (1, "d3:2,4,1,3")])
def test_masked_ue8m0_parity_and_sentinels(dg, switches, sched, tile):
    G, M_max, N, K = 5, 300, 512, 768
    mm = np.array([0, 17, 128, 257, 300], np.int32)
    a, b, _ = synth.masked_inputs(G, M_max, N, K, 24)
    qa, sa = gpu_cast_tokens(dg, a, ue8m0=True)
    qb, sb = gpu_cast_blocks(dg, b, ue8m0=True)
    oqa, osa = oracle.cast_per_token(a.reshape(-1, K), pow2=True)
    oqb, osb = oracle.cast_per_block(b, pow2=True)
    R = oracle.grouped_masked(oqa.reshape(G, M_max, K), osa.reshape(G, M_max, K // 128), oqb, osb, mm)
    if tile and tile.startswith("d3:"):
        switches.setenv("DG_DECODE3", tile[3:])
    elif tile:
        switches.setenv("DG_TILE", tile)
    d = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    say("masked ue8m0 schedule %d tile %s" % (sched, tile))
    dg.grouped_gemm_masked(qa, sa, qb, sb, to_dev(mm), d=d, schedule=sched, ue8m0=True)
    valid = np.isfinite(R)
    assert_close(bf16_values(d), R, "masked ue8m0", mask=valid)
    assert (d.view(torch.int16).cpu().numpy()[~valid] == SENTINEL).all()


@pytest.mark.slow
def test_prefill_ue8m0_full_size_sampled(dg):
    M, N, K = 4096, 36864, 7168
    say("dense ue8m0 full size %dx%dx%d" % (M, N, K))
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, M, N, K, seed=0, outliers=True, ue8m0=True)
    d = dg.gemm_fp8_nt(qa, sa, qb, sb, ue8m0=True)
    y = bf16_values(d)
    rng = synth.rng(0, 96)
    rows = rng.integers(0, M, 4096)
    cols = rng.integers(0, N, 4096)
    R = oracle.gemm_pairs(oqa, osa, oqb, osb, rows, cols)
    assert_close(y[rows, cols], R, "ue8m0 full sampled")
