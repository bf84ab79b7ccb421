"""GPU parity of the dense FP8 block-scaled GEMM against the oracle, every schedule.

Bar (stated for this method): per element |gpu - R| <= 2^-7 |R| + 1e-3 rms(R), and global
1 - 2 sum(yR) / sum(y^2 + R^2) <= 1e-5, with R the oracle's fp64 result."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_close, bf16_bits, bf16_values, quantised_dense, say, to_dev

pytestmark = pytest.mark.gpu

SCHEDULES = {"decode": 1, "tile128": 2, "tile256": 3}


@pytest.fixture(scope="module")
def dg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import moe_grouped_gemm_e4m3_amd as m
    m.lib()
    return m


def test_tiny_config(dg):
    # 128 x 256 x 512, seed 0
    say("dense tiny 128x256x512 auto")
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, 128, 256, 512, seed=0)
    d = dg.gemm_fp8_nt(qa, sa, qb, sb)
    R = oracle.gemm(oqa, osa, oqb, osb)
    assert_close(bf16_values(d), R, "tiny")


@pytest.mark.parametrize("sched", list(SCHEDULES))
@pytest.mark.parametrize("M", [1, 15, 16, 63, 64, 65, 127, 128, 200, 256, 300])
@pytest.mark.parametrize("N,K", [(128, 128), (384, 640), (256, 2304)])
def test_shape_sweep(dg, sched, M, N, K):
    say("dense sweep %s M=%d N=%d K=%d" % (sched, M, N, K))
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, M, N, K, seed=M + N + K)
    d = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=SCHEDULES[sched])
    R = oracle.gemm(oqa, osa, oqb, osb)
    assert_close(bf16_values(d), R, "sweep %s %dx%dx%d" % (sched, M, N, K))


@pytest.mark.parametrize("sched", list(SCHEDULES))
def test_long_k_fallbacks(dg, sched):
    # K = 258 blocks: beyond the 256 K blocks whose weight scales the direct-load tile kernel
    # keeps in LDS and beyond every LDS decode configuration, so each schedule runs its
    # fallback kernel; ragged M
    M, N, K = 70, 256, 258 * 128
    say("dense long K %s M=%d N=%d K=%d" % (sched, M, N, K))
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, M, N, K, seed=5)
    d = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=SCHEDULES[sched])
    R = oracle.gemm(oqa, osa, oqb, osb)
    assert_close(bf16_values(d), R, "long K %s" % sched)


@pytest.mark.parametrize("N,K", [(7168, 2048), (24576, 1536)])
def test_decode_full_size(dg, switches, N, K):
    # the decode configurations, M = 64, in full against the whole oracle result
    say("dense decode full M=64 N=%d K=%d" % (N, K))
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, 64, N, K, seed=0)
    d = dg.gemm_fp8_nt(qa, sa, qb, sb)
    R = oracle.gemm(oqa, osa, oqb, osb)
    assert_close(bf16_values(d), R, "decode %dx%d" % (N, K))
    for sched in ("decode", "tile128", "tile256"):
        d2 = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=SCHEDULES[sched])
        assert_close(bf16_values(d2), R, "decode %dx%d %s" % (N, K, sched))
    # the activation-resident decode kernel and the 64x128 tile kernel sum the K blocks in
    # the same order with the same operations: bit for bit the same output
    switches.setenv("DG_TILE", "t3_64x128")
    d3 = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=SCHEDULES["tile256"])
    switches.setenv("DG_TILE", "d3_96")
    d4 = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=SCHEDULES["tile256"])
    switches.delenv("DG_TILE")
    assert_close(bf16_values(d3), R, "decode %dx%d tile3 64x128" % (N, K))
    assert torch.equal(d3.view(torch.int16), d4.view(torch.int16))


@pytest.mark.slow
@pytest.mark.parametrize("N,K", [(7168, 18432), (36864, 7168)])
def test_prefill_full_size_sampled(dg, N, K):
    # the prefill configurations at full size: every row against 48 sampled columns, plus
    # 4096 random elements, computed one by one by the oracle
    say("dense prefill full M=4096 N=%d K=%d" % (N, K))
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, 4096, N, K, seed=0, outliers=True)
    d = dg.gemm_fp8_nt(qa, sa, qb, sb)
    y = bf16_values(d)
    r = synth.rng(0, 99)
    cols = np.sort(r.choice(N, 48, replace=False))
    rows_a = np.repeat(np.arange(4096), cols.size)
    cols_a = np.tile(cols, 4096)
    rows_b, cols_b = r.integers(0, 4096, 4096), r.integers(0, N, 4096)
    rows = np.concatenate([rows_a, rows_b])
    cols_all = np.concatenate([cols_a, cols_b])
    R = oracle.gemm_pairs(oqa, osa, oqb, osb, rows, cols_all)
    assert_close(y[rows, cols_all], R, "prefill %dx%d sampled" % (N, K))


def test_power_of_two_scale_is_bitwise(dg):
    # sa <- 2^p sa gives D <- 2^p D exactly (fp32 ops and bf16 rounding commute with exact
    # power-of-two scaling away from overflow and underflow)
    (qa, sa, qb, sb), _ = quantised_dense(dg, 200, 384, 1024, seed=5)
    for sched in SCHEDULES.values():
        say("dense power-of-two invariance schedule %d" % sched)
        d1 = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=sched)
        d2 = dg.gemm_fp8_nt(qa, sa * 8.0, qb, sb, schedule=sched)
        d3 = dg.gemm_fp8_nt(qa, sa, qb, sb * 0.25, schedule=sched)
        assert torch.equal(d2.float(), d1.float() * 8.0)
        assert torch.equal(d3.float(), d1.float() * 0.25)


def test_row_permutation_and_determinism(dg):
    (qa, sa, qb, sb), _ = quantised_dense(dg, 256, 256, 768, seed=6)
    perm = torch.from_numpy(synth.rng(6, 5).permutation(256)).to("cuda:0")
    for sched in SCHEDULES.values():
        say("dense permutation/determinism schedule %d" % sched)
        d = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=sched)
        d_again = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=sched)
        assert torch.equal(bf16_bits_t(d), bf16_bits_t(d_again))
        dp = dg.gemm_fp8_nt(qa[perm].contiguous(), sa[:, perm].contiguous(), qb, sb, schedule=sched)
        assert torch.equal(bf16_bits_t(dp), bf16_bits_t(d[perm]))


def bf16_bits_t(t):
    return t.contiguous().view(torch.int16)


def test_output_guard_bands(dg):
    # the kernels write exactly M x N bf16 values: 4 KiB guards on both sides stay intact
    M, N, K = 77, 384, 512
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, M, N, K, seed=7)
    R = oracle.gemm(oqa, osa, oqb, osb)
    guard = 2048
    for sched in SCHEDULES.values():
        say("dense guard bands schedule %d" % sched)
        buf = torch.full((guard * 2 + M * N,), -12345, dtype=torch.int16, device="cuda:0")
        d = buf[guard:guard + M * N].view(torch.bfloat16).view(M, N)
        dg.gemm_fp8_nt(qa, sa, qb, sb, d=d, schedule=sched)
        b = buf.cpu()
        assert (b[:guard] == -12345).all() and (b[guard + M * N:] == -12345).all()
        assert_close(bf16_values(d), R, "guarded %d" % sched)


def test_zero_and_extreme_scales(dg):
    M, N, K = 64, 256, 512
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, M, N, K, seed=8)
    # the scales are edited on the oracle's side ([M, K/128] and [N/128, K/128]) and the GPU
    # gets copies of them (its activation scales K-block-major)
    osa2 = osa.copy()
    osa2[:, 1] = 0.0                                   # a K block switched off
    osa2[3, :] = 0.0                                   # a whole row of zero scales
    osa2[5, :] = osa2[5, :] * np.float32(1e-20)        # tiny scales
    osb2 = osb.copy()
    osb2[1, :] = osb2[1, :] * np.float32(1e15)         # large weight scales on the second column block
    sa2 = torch.from_numpy(np.ascontiguousarray(osa2.T)).to("cuda:0")
    sb2 = torch.from_numpy(np.ascontiguousarray(osb2)).to("cuda:0")
    R = oracle.gemm(oqa, osa2, oqb, osb2)
    for sched in SCHEDULES.values():
        say("dense zero/extreme scales schedule %d" % sched)
        d = dg.gemm_fp8_nt(qa, sa2, qb, sb2, schedule=sched)
        y = bf16_values(d)
        assert (y[3] == 0).all()
        # compare per column block so the large-scale block does not swamp the rms
        assert_close(y[:, :128], R[:, :128], "extreme scales left %d" % sched)
        assert_close(y[:, 128:], R[:, 128:], "extreme scales right %d" % sched)


def test_empty_problems_launch_nothing(dg):
    a = torch.empty((0, 256), dtype=torch.uint8, device="cuda:0")
    sa = torch.empty((2, 0), dtype=torch.float32, device="cuda:0")
    b = torch.zeros((128, 256), dtype=torch.uint8, device="cuda:0")
    sb = torch.zeros((1, 2), dtype=torch.float32, device="cuda:0")
    say("dense empty M=0")
    d = dg.gemm_fp8_nt(a, sa, b, sb)
    assert tuple(d.shape) == (0, 128)


# every tile kernel, forced through DG_TILE (None = the automatic choice); they all sum the
# K blocks in the same order with the same fp32 operations, so they must agree bit for bit
TILE_VARIANTS = [None, "t2_128x128", "t2_256x128", "t3_256x128", "t3_128x256", "t3_64x128", "d3_96", "t3_256x256b"]


@pytest.mark.parametrize("M,N,K", [(300, 512, 1280), (512, 256, 2304), (77, 768, 384), (1000, 640, 640),
                                   (256, 256, 128)])
def test_tile_kernels_parity_and_agreement(dg, switches, M, N, K):
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, M, N, K, seed=M + 3)
    R = oracle.gemm(oqa, osa, oqb, osb)
    ref = None
    for v in TILE_VARIANTS:
        if v:
            switches.setenv("DG_TILE", v)
        else:
            switches.delenv("DG_TILE", raising=False)
        say("dense tile kernel %s M=%d N=%d K=%d" % (v, M, N, K))
        d = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=SCHEDULES["tile256"])
        assert_close(bf16_values(d), R, "tile %s" % v)
        bits = d.view(torch.int16).clone()
        if ref is None:
            ref = bits
        else:
            assert torch.equal(bits, ref), "tile kernel %s differs from the automatic choice" % v


# decode schedules, forced one by one: the register-fed one (DG_DECODE=v1), the LDS ones
# (DG_DECODE2="bn,kg,kpw,waves") and the activation-resident ones (DG_DECODE3="wave rows,wave columns,strips,
# slots"; where the activations do not fit beside the ring they fall back to the LDS ones);
# each against the oracle, on full and partial 64-row blocks
DECODE_VARIANTS = [("DG_DECODE", "v1"), ("DG_DECODE2", "96,4,3,8"), ("DG_DECODE2", "96,1,12,6"),
                   ("DG_DECODE2", "96,2,6,6"), ("DG_DECODE2", "32,8,2,8"), ("DG_DECODE2", "32,2,8,4"),
                   ("DG_DECODE2", "32,1,16,2"), ("DG_DECODE2", "16,8,3,8"), ("DG_DECODE2", "128,4,3,8"),
                   ("DG_DECODE3", "2,2,3,4"), ("DG_DECODE3", "2,2,3,5"), ("DG_DECODE3", "1,6,1,4"),
                   ("DG_DECODE3", "2,3,2,4"), ("DG_DECODE3", "4,1,6,4"), ("DG_DECODE3", "1,8,1,3"),
                   ("DG_DECODE3", "2,4,1,3"), ("DG_DECODE3", "1,6,1,5")]


@pytest.mark.parametrize("M,N,K", [(64, 1536, 1536), (37, 768, 2048), (1, 384, 1152), (130, 768, 1024)])
def test_decode_variants(dg, switches, M, N, K):
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = quantised_dense(dg, M, N, K, seed=M + 11)
    R = oracle.gemm(oqa, osa, oqb, osb)
    for var, val in DECODE_VARIANTS:
        for v in ("DG_DECODE", "DG_DECODE2", "DG_DECODE3"):
            switches.delenv(v, raising=False)
        switches.setenv(var, val)
        say("decode %s=%s M=%d N=%d K=%d" % (var, val, M, N, K))
        d = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=SCHEDULES["decode"])
        assert_close(bf16_values(d), R, "decode %s" % val)
