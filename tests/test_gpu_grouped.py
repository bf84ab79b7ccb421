"""GPU parity of the MoE grouped GEMMs (contiguous and masked layouts) against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import (assert_close, assert_same_bits, assert_same_bytes, bf16_values, gpu_cast_blocks,
                     gpu_cast_tokens, kmajor, oracle_cast_tokens, say, to_dev)

pytestmark = pytest.mark.gpu

SENTINEL = -1  # 0xFFFF as int16: a bf16 NaN pattern the kernels never produce from finite data


@pytest.fixture(scope="module")
def dg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import moe_grouped_gemm_e4m3_amd as m
    m.lib()
    return m


def _both_sides_contiguous(dg, G, tokens, N, K, seed):
    a, b, mi = synth.contiguous_inputs(G, tokens, N, K, seed)
    qa_d, sa_d = gpu_cast_tokens(dg, a)
    qb_d, sb_d = gpu_cast_blocks(dg, b)
    qa, sa = oracle.cast_per_token(a)
    qb, sb = oracle.cast_per_block(b)
    assert_same_bytes(qa_d, qa, "A")
    assert_same_bits(sa_d, kmajor(sa), "sA")
    assert_same_bytes(qb_d, qb, "B")
    assert_same_bits(sb_d, sb, "sB")
    return (qa_d, sa_d, qb_d, sb_d, to_dev(mi)), (qa, sa, qb, sb, mi)


def _both_sides_masked(dg, G, M_max, N, K, seed, masked_m=None):
    a, b, mm = synth.masked_inputs(G, M_max, N, K, seed)
    if masked_m is not None:
        mm = np.asarray(masked_m, np.int32)
    qa_d, sa_d = gpu_cast_tokens(dg, a)
    qb_d, sb_d = gpu_cast_blocks(dg, b)
    qa, sa = oracle_cast_tokens(a)
    qb, sb = oracle.cast_per_block(b)
    assert_same_bytes(qa_d, qa, "A")
    assert_same_bits(sa_d, kmajor(sa), "sA")
    assert_same_bytes(qb_d, qb, "B")
    assert_same_bits(sb_d, sb, "sB")
    return (qa_d, sa_d, qb_d, sb_d, to_dev(mm)), (qa, sa, qb, sb, mm)


# ---------------------------------------------------------------------------------------
# contiguous layout
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("G,tokens,N,K", [(4, 300, 256, 384), (8, 1000, 384, 640), (3, 1, 128, 128)])
def test_contiguous_parity(dg, G, tokens, N, K):
    say("contiguous G=%d tokens=%d N=%d K=%d" % (G, tokens, N, K))
    (qa, sa, qb, sb, mi), (oqa, osa, oqb, osb, omi) = _both_sides_contiguous(dg, G, tokens, N, K, seed=G + tokens)
    d = dg.grouped_gemm_contiguous(qa, sa, qb, sb, mi)
    R = oracle.grouped_contiguous(oqa, osa, oqb, osb, omi)
    assert_close(bf16_values(d), R, "contiguous", mask=omi[:, None].repeat(N, 1) >= 0)


@pytest.mark.parametrize("variant", ["t3_128x256", "t2_128x128", None, "t3_128x256b", "hybrid"])
def test_contiguous_tile_kernels(dg, switches, variant):
    # experts of 2-4 blocks of 128 rows, so the automatic (hybrid) kernel runs 256-row tiles over
    # blocks of one expert and 128-row ones where a pair straddles two experts or the end; long
    # K; each kernel checked against the oracle and against the others bit for bit
    G, N, K = 3, 512, 4352
    (qa, sa, qb, sb, mi), (oqa, osa, oqb, osb, omi) = _both_sides_contiguous(dg, G, 1000, N, K, seed=21)
    firsts = omi.reshape(-1, 128)[:, 0]
    pairs = [(firsts[i], firsts[i + 1] if i + 1 < firsts.size else -1) for i in range(0, firsts.size, 2)]
    assert any(a == b for a, b in pairs) and any(a != b for a, b in pairs)
    if variant:
        switches.setenv("DG_TILE", variant)
    else:
        switches.delenv("DG_TILE", raising=False)
    say("contiguous tile kernel %s" % variant)
    d = dg.grouped_gemm_contiguous(qa, sa, qb, sb, mi)
    R = oracle.grouped_contiguous(oqa, osa, oqb, osb, omi)
    valid = omi[:, None].repeat(N, 1) >= 0
    assert_close(bf16_values(d), R, "contiguous %s" % variant, mask=valid)
    switches.setenv("DG_TILE", "t2_128x256")
    d2 = dg.grouped_gemm_contiguous(qa, sa, qb, sb, mi)
    rows = torch.from_numpy(np.nonzero(omi >= 0)[0]).to("cuda:0")
    assert torch.equal(d[rows].view(torch.int16), d2[rows].view(torch.int16))


def test_contiguous_equals_dense_per_expert_on_gpu(dg):
    G, N, K = 4, 256, 512
    (qa, sa, qb, sb, mi), (_, _, _, _, omi) = _both_sides_contiguous(dg, G, 700, N, K, seed=3)
    say("contiguous == dense per expert")
    d = dg.grouped_gemm_contiguous(qa, sa, qb, sb, mi)
    for g in range(G):
        rows = torch.from_numpy(np.nonzero(omi == g)[0]).to("cuda:0")
        dd = dg.gemm_fp8_nt(qa[rows].contiguous(), sa[:, rows].contiguous(), qb[g], sb[g], schedule=2)
        assert torch.equal(d[rows].view(torch.int16), dd.view(torch.int16))


def test_contiguous_padding_block_untouched(dg):
    # a whole 128-row block whose first row is -1 is skipped: its output rows keep their bytes
    G, N, K = 2, 256, 256
    (qa, sa, qb, sb, mi), (oqa, osa, oqb, osb, omi) = _both_sides_contiguous(dg, G, 200, N, K, seed=4)
    omi2 = np.concatenate([omi, np.full(128, -1, np.int32)])
    qa2 = torch.cat([qa, torch.zeros((128, K), dtype=qa.dtype, device=qa.device)])
    sa2 = torch.cat([sa, torch.zeros((K // 128, 128), dtype=sa.dtype, device=sa.device)], dim=1).contiguous()
    d = torch.full((omi2.size, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    say("contiguous padding block untouched")
    dg.grouped_gemm_contiguous(qa2, sa2, qb, sb, to_dev(omi2), d=d)
    assert (d[-128:].view(torch.int16) == SENTINEL).all()
    R = oracle.grouped_contiguous(oqa, osa, oqb, osb, omi)
    assert_close(bf16_values(d[:-128]), R, "contiguous with skipped block", mask=omi[:, None].repeat(N, 1) >= 0)


@pytest.mark.slow
@pytest.mark.parametrize("N,K", [(4096, 7168), (7168, 2048)])
def test_contiguous_full_size_sampled(dg, N, K):
    # 8 experts, 8192 routed rows padded per expert to 128; all routed rows x 32 sampled
    # columns, against the oracle one element at a time
    say("contiguous full G=8 tokens=8192 N=%d K=%d" % (N, K))
    (qa, sa, qb, sb, mi), (oqa, osa, oqb, osb, omi) = _both_sides_contiguous(dg, 8, 8192, N, K, seed=0)
    d = dg.grouped_gemm_contiguous(qa, sa, qb, sb, mi)
    y = bf16_values(d)
    cols = np.sort(synth.rng(0, 98).choice(N, 32, replace=False))
    routed = np.nonzero(omi >= 0)[0]
    rows = np.repeat(routed, cols.size)
    cc = np.tile(cols, routed.size)
    R = oracle.gemm_pairs(oqa, osa, oqb, osb, rows, cc, group_of_row=omi)
    assert_close(y[rows, cc], R, "contiguous full %dx%d" % (N, K))


# ---------------------------------------------------------------------------------------
# masked layout
# ---------------------------------------------------------------------------------------
MASKED_SCHEDULES = {"auto": 0, "decode": 1, "tile128": 2, "tile256": 3}


@pytest.mark.parametrize("sched", list(MASKED_SCHEDULES))
def test_masked_parity_and_sentinels(dg, sched):
    G, M_max, N, K = 6, 200, 256, 640
    mm = [0, 1, 63, 64, 200, 130]
    (qa, sa, qb, sb, mmd), (oqa, osa, oqb, osb, omm) = _both_sides_masked(dg, G, M_max, N, K, 11, mm)
    # invalid A rows hold the NaN code: they must not leak into valid rows
    # (the oracle's copy gets the same codes, planted in its own cast, not read back)
    oqa_nan = oqa.copy()
    for g in range(G):
        qa[g, mm[g]:] = 0x7F
        oqa_nan[g, mm[g]:] = 0x7F
    d = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    say("masked %s G=%d M_max=%d N=%d K=%d" % (sched, G, M_max, N, K))
    dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, expected_m=48 if sched == "auto" else 0, d=d,
                           schedule=MASKED_SCHEDULES[sched])
    R = oracle.grouped_masked(oqa_nan, osa, oqb, osb, omm)
    valid = np.isfinite(R)
    assert_close(bf16_values(d), R, "masked %s" % sched, mask=valid)
    bits = d.view(torch.int16).cpu().numpy()
    assert (bits[~valid] == SENTINEL).all(), "rows beyond masked_m were written"


@pytest.mark.parametrize("variant", ["t3_256x256", "t3_128x256", "t2_256x128", "t3_256x256b", "t3_128x256b"])
def test_masked_tile_kernels(dg, switches, variant):
    G, M_max, N, K = 5, 300, 512, 768
    mm = [0, 17, 128, 257, 300]
    (qa, sa, qb, sb, mmd), (oqa, osa, oqb, osb, omm) = _both_sides_masked(dg, G, M_max, N, K, 22, mm)
    switches.setenv("DG_TILE", variant)
    d = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    say("masked tile kernel %s" % variant)
    dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, d=d, schedule=MASKED_SCHEDULES["tile256"])
    R = oracle.grouped_masked(oqa, osa, oqb, osb, omm)
    valid = np.isfinite(R)
    assert_close(bf16_values(d), R, "masked %s" % variant, mask=valid)
    bits = d.view(torch.int16).cpu().numpy()
    assert (bits[~valid] == SENTINEL).all(), "rows beyond masked_m were written"
    switches.delenv("DG_TILE")
    d2 = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, d=d2, schedule=MASKED_SCHEDULES["tile256"])
    assert torch.equal(d.view(torch.int16), d2.view(torch.int16))


@pytest.mark.parametrize("cfg", ["2,3,2,4", "1,6,1,4", "2,2,3,5", "1,8,1,3"])
def test_masked_activation_resident_decode(dg, switches, cfg):
    # the activation-resident decode kernel on the masked layout, forced through DG_DECODE3
    # (decode schedule): empty, partial, full and multi-row-block groups, NaN codes in the
    # invalid activation rows, sentinels beyond the valid rows
    G, M_max, N, K = 5, 130, 384, 1024
    mm = [0, 5, 64, 130, 100]
    (qa, sa, qb, sb, mmd), (oqa, osa, oqb, osb, omm) = _both_sides_masked(dg, G, M_max, N, K, 31, mm)
    # (the oracle's copy gets the same codes, planted in its own cast, not read back)
    oqa_nan = oqa.copy()
    for g in range(G):
        qa[g, mm[g]:] = 0x7F
        oqa_nan[g, mm[g]:] = 0x7F
    switches.setenv("DG_DECODE3", cfg)
    d = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    say("masked decode3 %s G=%d M_max=%d N=%d K=%d" % (cfg, G, M_max, N, K))
    dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, d=d, schedule=MASKED_SCHEDULES["decode"])
    R = oracle.grouped_masked(oqa_nan, osa, oqb, osb, omm)
    valid = np.isfinite(R)
    assert_close(bf16_values(d), R, "masked decode3 %s" % cfg, mask=valid)
    bits = d.view(torch.int16).cpu().numpy()
    assert (bits[~valid] == SENTINEL).all(), "rows beyond masked_m were written"


@pytest.mark.parametrize("K", [128, 256, 384])
def test_masked_split_issue_short_k(dg, K):
    # the masked 256x256 tiles (weights of K block kb+2 issued at the start of K block kb) with
    # 1, 2 and 3 K blocks, where the issue and wait steps run into the end of K
    G, M_max, N = 3, 300, 512
    mm = [300, 0, 257]
    (qa, sa, qb, sb, mmd), (oqa, osa, oqb, osb, omm) = _both_sides_masked(dg, G, M_max, N, K, 40 + K, mm)
    d = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    say("masked split issue G=%d M_max=%d N=%d K=%d" % (G, M_max, N, K))
    dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, d=d, schedule=MASKED_SCHEDULES["tile256"])
    R = oracle.grouped_masked(oqa, osa, oqb, osb, omm)
    valid = np.isfinite(R)
    assert_close(bf16_values(d), R, "masked split K=%d" % K, mask=valid)
    assert (d.view(torch.int16).cpu().numpy()[~valid] == SENTINEL).all(), "rows beyond masked_m were written"


@pytest.mark.parametrize("K", [128, 256, 384, 512])
def test_split_issue_three_stages_short_k(dg, switches, K):
    # the 128x256 tiles with the split issue (three stages: weights of K block kb+3 issued at
    # the start of K block kb) with 1 to 4 K blocks, on both grouped layouts
    switches.setenv("DG_TILE", "t3_128x256b")
    G, N = 3, 512
    (qa, sa, qb, sb, mi), (oqa, osa, oqb, osb, omi) = _both_sides_contiguous(dg, G, 200, N, K, seed=50 + K)
    say("contiguous split issue N=%d K=%d" % (N, K))
    d = dg.grouped_gemm_contiguous(qa, sa, qb, sb, mi)
    R = oracle.grouped_contiguous(oqa, osa, oqb, osb, omi)
    assert_close(bf16_values(d), R, "contiguous split K=%d" % K, mask=omi[:, None].repeat(N, 1) >= 0)
    mm = [100, 0, 128]
    (qa, sa, qb, sb, mmd), (oqa, osa, oqb, osb, omm) = _both_sides_masked(dg, G, 128, N, K, 60 + K, mm)
    d = torch.full((G, 128, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    say("masked split issue (three stages) N=%d K=%d" % (N, K))
    dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, d=d, schedule=MASKED_SCHEDULES["tile256"])
    R = oracle.grouped_masked(oqa, osa, oqb, osb, omm)
    valid = np.isfinite(R)
    assert_close(bf16_values(d), R, "masked split3 K=%d" % K, mask=valid)
    assert (d.view(torch.int16).cpu().numpy()[~valid] == SENTINEL).all(), "rows beyond masked_m were written"


def test_masked_clamps_out_of_range_counts(dg):
    G, M_max, N, K = 3, 64, 128, 256
    (qa, sa, qb, sb, mmd), (oqa, osa, oqb, osb, _) = _both_sides_masked(dg, G, M_max, N, K, 12, [-7, 1000, 64])
    for sched in (1, 2, 3):
        d = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
        say("masked clamp schedule %d" % sched)
        dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, d=d, schedule=sched)
        R = oracle.grouped_masked(oqa, osa, oqb, osb, np.array([-7, 1000, 64], np.int32))
        valid = np.isfinite(R)
        assert (d[0].view(torch.int16) == SENTINEL).all()
        assert_close(bf16_values(d), R, "masked clamp", mask=valid)


def test_masked_full_equals_dense(dg):
    G, M_max, N, K = 2, 128, 256, 512
    (qa, sa, qb, sb, mmd), _ = _both_sides_masked(dg, G, M_max, N, K, 13, [128, 128])
    say("masked full == dense per group")
    for sched in (1, 2, 3):
        d = dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, schedule=sched)
        for g in range(G):
            dd = dg.gemm_fp8_nt(qa[g], sa[g], qb[g], sb[g], schedule=sched)
            assert torch.equal(d[g].view(torch.int16), dd.view(torch.int16))


@pytest.mark.slow
@pytest.mark.parametrize("N,K", [(4096, 7168), (7168, 2048)])
def test_masked_full_size_sampled(dg, N, K):
    # 32 experts x 256-row buffers, valid rows ~ U{0..256}; every valid row x 24 sampled
    # columns checked one by one; every invalid row checked untouched
    G, M_max = 32, 256
    say("masked full G=32 M_max=256 N=%d K=%d" % (N, K))
    (qa, sa, qb, sb, mmd), (oqa, osa, oqb, osb, omm) = _both_sides_masked(dg, G, M_max, N, K, 0)
    for g in range(G):
        qa[g, int(omm[g]):] = 0x7F
    d = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, expected_m=int(omm.mean()), d=d)
    bits = d.view(torch.int16).cpu().numpy()
    y = bits.view(np.uint16).astype(np.uint32) << 16
    y = y.view(np.float32).astype(np.float64).reshape(G * M_max, N)
    cols = np.sort(synth.rng(0, 97).choice(N, 24, replace=False))
    valid_rows = np.concatenate([g * M_max + np.arange(int(omm[g])) for g in range(G)])
    rows = np.repeat(valid_rows, cols.size)
    cc = np.tile(cols, valid_rows.size)
    group = (np.arange(G * M_max) // M_max).astype(np.int32)
    R = oracle.gemm_pairs(oqa.reshape(G * M_max, K), osa.reshape(G * M_max, K // 128), oqb, osb, rows, cc,
                          group_of_row=group)
    assert_close(y[rows, cc], R, "masked full %dx%d" % (N, K))
    for g in range(G):
        assert (bits[g, int(omm[g]):] == SENTINEL).all()


@pytest.mark.parametrize("G", [64, 12, 65])
def test_masked_hybrid_group_order(dg, G):
    # the automatic masked kernel takes up to 64 groups in descending order of their valid rows
    # (ties by index; dealt over the XCDs in a snake when G % 8 == 0), more in index order: many
    # ties, empty, full and over-full groups
    M_max, N, K = 200, 256, 256
    mm = synth.masked_layout(G, M_max, 40 + G)
    mm[::7] = 0
    mm[1::9] = M_max
    mm[2::11] = 77
    mm[3] = 500
    (qa, sa, qb, sb, mmd), (oqa, osa, oqb, osb, omm) = _both_sides_masked(dg, G, M_max, N, K, 41, mm)
    d = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    say("masked hybrid group order G=%d" % G)
    dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, d=d)
    R = oracle.grouped_masked(oqa, osa, oqb, osb, omm)
    valid = np.isfinite(R)
    assert_close(bf16_values(d), R, "masked group order G=%d" % G, mask=valid)
    assert (d.view(torch.int16).cpu().numpy()[~valid] == SENTINEL).all()
