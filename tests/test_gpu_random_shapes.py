"""GPU parity on seeded random shapes: every layout, schedule and scale type against the oracle,
on combinations the hand-picked cases do not reach (ragged M, odd tile counts, K from one block
up, empty and out-of-range group counts, expected_m hints). The shapes come from a fixed seed
per case, so every run checks the same cases."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_close, assert_same_bits, assert_same_bytes, bf16_values, kmajor, say, to_dev

pytestmark = pytest.mark.gpu

SENTINEL = -1  # 0xFFFF as int16: a bf16 NaN pattern the kernels never produce from finite data
SCHEDULES = [0, 1, 2, 3]  # automatic, decode, 128-row tiles, 256-row tiles


@pytest.fixture(scope="module")
def dg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import moe_grouped_gemm_e4m3_amd as m
    m.lib()
    return m


def _cast_both(dg, a, b, pow2):
    """Both sides quantise on their own; the casts must agree byte for byte."""
    K = a.shape[-1]
    qa_d, sa_d = dg.cast_fp8_per_token(to_dev(a), ue8m0=pow2)
    qb_d, sb_d = dg.cast_fp8_per_block(to_dev(b), ue8m0=pow2)
    qa, sa = oracle.cast_per_token(a.reshape(-1, K), pow2=pow2)
    qa, sa = qa.reshape(a.shape), sa.reshape(*a.shape[:-1], K // 128)
    qb, sb = oracle.cast_per_block(b, pow2=pow2)
    assert_same_bytes(qa_d, qa, "A cast")
    assert_same_bits(sa_d, kmajor(sa), "A scales")
    assert_same_bytes(qb_d, qb, "B cast")
    assert_same_bits(sb_d, sb, "B scales")
    return (qa_d, sa_d, qb_d, sb_d), (qa, sa, qb, sb)


@pytest.mark.parametrize("case", range(96))
def test_random_dense(dg, case):
    r = np.random.default_rng(1000 + case)
    M, N, K = int(r.integers(1, 700)), 128 * int(r.integers(1, 9)), 128 * int(r.integers(1, 25))
    sched, pow2, outl = SCHEDULES[case % 4], bool(r.integers(0, 2)), bool(r.integers(0, 2))
    say("random dense case %d: M=%d N=%d K=%d schedule %d ue8m0=%d" % (case, M, N, K, sched, pow2))
    a, b = synth.dense_inputs(M, N, K, seed=2000 + case, outliers=outl)
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = _cast_both(dg, a, b, pow2)
    d = dg.gemm_fp8_nt(qa, sa, qb, sb, schedule=sched, ue8m0=pow2)
    assert_close(bf16_values(d), oracle.gemm(oqa, osa, oqb, osb), "random dense case %d" % case)


@pytest.mark.parametrize("case", range(48))
def test_random_contiguous(dg, case):
    r = np.random.default_rng(3000 + case)
    G, tokens = int(r.integers(1, 7)), int(r.integers(1, 900))
    N, K = 128 * int(r.integers(1, 7)), 128 * int(r.integers(1, 21))
    sched, pow2 = [0, 2, 3][case % 3], bool(r.integers(0, 2))
    say("random contiguous case %d: G=%d tokens=%d N=%d K=%d schedule %d ue8m0=%d" % (case, G, tokens, N, K, sched, pow2))
    a, b, mi = synth.contiguous_inputs(G, tokens, N, K, seed=4000 + case)
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = _cast_both(dg, a, b, pow2)
    d = dg.grouped_gemm_contiguous(qa, sa, qb, sb, to_dev(mi), schedule=sched, ue8m0=pow2)
    R = oracle.grouped_contiguous(oqa, osa, oqb, osb, mi)
    assert_close(bf16_values(d), R, "random contiguous case %d" % case, mask=mi[:, None].repeat(N, 1) >= 0)


@pytest.mark.parametrize("case", range(48))
def test_random_masked(dg, case):
    r = np.random.default_rng(5000 + case)
    G, M_max = int(r.integers(1, 7)), int(r.integers(1, 300))
    N, K = 128 * int(r.integers(1, 7)), 128 * int(r.integers(1, 21))
    # counts: uniform on [0, M_max], with some empty, full and out-of-range ones
    mm = r.integers(0, M_max + 1, size=G).astype(np.int32)
    for g in range(G):
        u = r.random()
        mm[g] = 0 if u < 0.15 else (M_max if u < 0.3 else (M_max + 50 if u < 0.4 else (-3 if u < 0.45 else mm[g])))
    sched, pow2 = SCHEDULES[case % 4], bool(r.integers(0, 2))
    expected_m = int(r.choice([0, 8, 64, M_max]))
    say("random masked case %d: G=%d M_max=%d N=%d K=%d counts %s schedule %d expected_m %d ue8m0=%d"
        % (case, G, M_max, N, K, mm.tolist(), sched, expected_m, pow2))
    a, b, _ = synth.masked_inputs(G, M_max, N, K, seed=6000 + case)
    (qa, sa, qb, sb), (oqa, osa, oqb, osb) = _cast_both(dg, a, b, pow2)
    d = torch.full((G, M_max, N), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    dg.grouped_gemm_masked(qa, sa, qb, sb, to_dev(mm), expected_m=expected_m, d=d, schedule=sched, ue8m0=pow2)
    R = oracle.grouped_masked(oqa, osa, oqb, osb, mm)
    valid = np.isfinite(R)
    assert_close(bf16_values(d), R, "random masked case %d" % case, mask=valid)
    assert (d.view(torch.int16).cpu().numpy()[~valid] == SENTINEL).all(), "rows beyond masked_m were written"
