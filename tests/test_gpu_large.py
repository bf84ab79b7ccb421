"""GPU parity where an operand reaches 2^32 bytes: the direct-load tile kernels address with
32-bit per-lane offsets and refuse such problems, and the launcher falls back to kernels that
offset from each tile's 64-bit base. Dense M*K, contiguous M_total*K, masked M_max*K and dense
N*K at or beyond 2^32 are each checked against the oracle at sampled outputs on both sides of
the 2^32-byte row, with the same tolerance as every other GEMM test.

The 4.3 GB operands are built on the device from a small seeded pool of rows, both sides
quantising the pool on their own (bit-for-bit equality asserted). Row r takes pool row
r mod P with P not dividing 2^32 / K, so a 32-bit offset that wrapped would land on a different
pool row and fail the comparison."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import assert_close, assert_same_bits, assert_same_bytes, bf16_values, kmajor, say

pytestmark = pytest.mark.gpu

K = 8192
WRAP_ROWS = (1 << 32) // K  # 524288: the first row at or beyond 2^32 bytes
P_ROWS = 4095               # activation pool rows; 524288 % 4095 = 128
P_BLOCKS = 3                # weight pool: 3 blocks of 128 rows; 524288 % 384 = 128


@pytest.fixture(scope="module")
def dg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import moe_grouped_gemm_e4m3_amd as m
    m.lib()
    return m


def dev():
    return torch.device("cuda:0")


def _pool_tokens(dg, seed):
    """P_ROWS x K activation rows cast by both sides: device (q, s [K/128, P]) and oracle (q, s [P, K/128])."""
    a = synth.normal((P_ROWS, K), seed, synth.TID_A)
    q_d, s_d = dg.cast_fp8_per_token(torch.from_numpy(a).to(dev()))
    q_o, s_o = oracle.cast_per_token(a)
    assert_same_bytes(q_d, q_o, "pool A cast")
    assert_same_bits(s_d, kmajor(s_o), "pool A scales")
    return (q_d, s_d), (q_o, s_o)


def _weights(dg, G, N, seed):
    """G x N x K weights cast by both sides; device views [G,N,K] / [G,N/128,K/128]."""
    b = synth.normal((G, N, K), seed, synth.TID_B, std=0.02)
    q_d, s_d = dg.cast_fp8_per_block(torch.from_numpy(b.reshape(-1, K)).to(dev()))
    q_o, s_o = oracle.cast_per_block(b)
    assert_same_bytes(q_d.view(G, N, K), q_o.reshape(G, N, K), "B cast")
    assert_same_bits(s_d.view(G, N // 128, K // 128), s_o.reshape(G, N // 128, K // 128), "B scales")
    return (q_d.view(G, N, K), s_d.view(G, N // 128, K // 128)), (q_o.reshape(G, N, K), s_o.reshape(G, N // 128, K // 128))


def _tiled_rows(q_pool, s_pool, rows):
    """Device operand of `rows` rows, row r = pool row r mod P: codes [rows, K], scales [K/128, rows]."""
    idx = torch.arange(rows, device=dev(), dtype=torch.int64) % P_ROWS
    return q_pool.index_select(0, idx), s_pool.index_select(1, idx)


def _sample_rows(total, seed, extra=()):
    """The first rows, the rows around the 2^32-byte row, the last rows and random ones."""
    r = synth.rng(seed, 97)
    pick = np.concatenate([np.arange(0, 48), np.arange(WRAP_ROWS - 40, min(total, WRAP_ROWS + 88)),
                           np.arange(total - 48, total), r.integers(0, total, 384), np.asarray(extra, np.int64)])
    return np.unique(pick[(pick >= 0) & (pick < total)])


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _chosen(capfd):
    """Kernel names the library logged (DG_LOG) since the last read of the captured stderr."""
    torch.cuda.synchronize()
    return [ln.rsplit("-> ", 1)[-1].strip() for ln in capfd.readouterr().err.splitlines() if ln.startswith("[dg] ")]


def test_dense_activation_beyond_32_bit_offsets(dg, switches, capfd):
    M, N = WRAP_ROWS + 200, 256  # M*K >= 2^32, ragged last tile
    say("large dense M*K >= 2^32: M=%d N=%d K=%d" % (M, N, K))
    (qp, sp), (oqp, osp) = _pool_tokens(dg, seed=11)
    (qb, sb), (oqb, osb) = _weights(dg, 1, N, seed=11)
    qa, sa = _tiled_rows(qp, sp, M)
    switches.setenv("DG_LOG", "1")
    capfd.readouterr()
    d = dg.gemm_fp8_nt(qa, sa, qb[0], sb[0])
    assert _chosen(capfd) == ["tile2_256x128"]  # the register-staged fallback
    rows = _sample_rows(M, 11)
    y = bf16_values(d.index_select(0, torch.from_numpy(rows).to(dev())))
    del qa, sa, d
    _free()
    R = oracle.gemm(oqp[rows % P_ROWS], osp[rows % P_ROWS], oqb[0], osb[0])
    assert_close(y, R, "dense M=%d K=%d" % (M, K))


def test_contiguous_activation_beyond_32_bit_offsets(dg, switches, capfd):
    G, N = 4, 256
    blocks = WRAP_ROWS // 128 + 4  # M_total*K >= 2^32
    M = blocks * 128
    # four experts in order; a padding block in the first expert's span and the last block
    # padding; the last 50 rows of a block before the 2^32 row are routing padding
    eb = np.minimum(np.arange(blocks) * G // blocks, G - 1).astype(np.int32)
    eb[1000] = -1
    eb[-1] = -1
    mi = np.repeat(eb, 128)
    tail = (WRAP_ROWS // 128 - 3) * 128
    mi[tail + 78:tail + 128] = -1
    say("large contiguous M_total*K >= 2^32: G=%d M_total=%d N=%d K=%d" % (G, M, N, K))
    (qp, sp), (oqp, osp) = _pool_tokens(dg, seed=12)
    (qb, sb), (oqb, osb) = _weights(dg, G, N, seed=12)
    qa, sa = _tiled_rows(qp, sp, M)
    d = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    mi_d = torch.from_numpy(mi).to(dev())
    switches.setenv("DG_LOG", "1")
    capfd.readouterr()
    dg.grouped_gemm_contiguous(qa, sa, qb, sb, mi_d, d=d)
    assert _chosen(capfd) == ["tile2_128x256"]
    rows = _sample_rows(M, 12, extra=np.arange(1000 * 128 - 8, 1000 * 128 + 8))
    rows = rows[mi[rows] >= 0]
    y = bf16_values(d.index_select(0, torch.from_numpy(rows).to(dev())))
    del qa, sa, d
    _free()
    cols = np.arange(N)
    rr, cc = np.repeat(np.arange(rows.size), N), np.tile(cols, rows.size)
    R = oracle.gemm_pairs(oqp[rows % P_ROWS], osp[rows % P_ROWS], oqb, osb, rr, cc, group_of_row=mi[rows])
    assert_close(y.reshape(-1), R, "contiguous M_total=%d K=%d" % (M, K))


def test_masked_activation_beyond_32_bit_offsets(dg, switches, capfd):
    G, N = 1, 256
    M_max = WRAP_ROWS + 64  # M_max*K >= 2^32
    valid = M_max - 37      # rows from here on are left unwritten
    say("large masked M_max*K >= 2^32: G=%d M_max=%d valid=%d N=%d K=%d" % (G, M_max, valid, N, K))
    (qp, sp), (oqp, osp) = _pool_tokens(dg, seed=13)
    (qb, sb), (oqb, osb) = _weights(dg, G, N, seed=13)
    qa, sa = _tiled_rows(qp, sp, M_max)
    sentinel = torch.tensor(0x7FBF, dtype=torch.int16)  # a NaN pattern no result takes
    d = torch.empty((G, M_max, N), dtype=torch.bfloat16, device=dev())
    d.view(torch.int16).fill_(sentinel.item())
    mm = torch.tensor([valid], dtype=torch.int32, device=dev())
    switches.setenv("DG_LOG", "1")
    capfd.readouterr()
    dg.grouped_gemm_masked(qa.view(G, M_max, K), sa.view(G, K // 128, M_max), qb, sb, mm, d=d)
    assert _chosen(capfd) == ["tile2_256x128"]
    rows = _sample_rows(M_max, 13)
    got = d[0].index_select(0, torch.from_numpy(rows).to(dev()))
    untouched = got[torch.from_numpy(rows >= valid).to(dev())].view(torch.int16)
    assert bool((untouched == sentinel.item()).all()), "masked rows at or beyond the count were written"
    keep = rows < valid
    y = bf16_values(got)[keep]
    del qa, sa, d, got
    _free()
    r = rows[keep]
    R = oracle.gemm(oqp[r % P_ROWS], osp[r % P_ROWS], oqb[0], osb[0])
    assert_close(y, R, "masked M_max=%d K=%d" % (M_max, K))


def test_dense_weights_beyond_32_bit_offsets(dg, switches, capfd):
    M = 64                            # decode-sized
    N = WRAP_ROWS + 128               # N*K >= 2^32
    say("large dense N*K >= 2^32: M=%d N=%d K=%d" % (M, N, K))
    a = synth.normal((M, K), 14, synth.TID_A)
    qa, sa = dg.cast_fp8_per_token(torch.from_numpy(a).to(dev()))
    oqa, osa = oracle.cast_per_token(a)
    assert_same_bytes(qa, oqa, "A cast")
    assert_same_bits(sa, kmajor(osa), "A scales")
    # weight pool of three 128-row blocks; column n takes pool row n mod 384 and block
    # (n / 128) mod 3, so the block scales stay those of the rows they cover
    (qbp, sbp), (oqbp, osbp) = _weights(dg, 1, 128 * P_BLOCKS, seed=14)
    idx = torch.arange(N, device=dev(), dtype=torch.int64) % (128 * P_BLOCKS)
    qb = qbp[0].index_select(0, idx)
    sb = sbp[0].index_select(0, torch.arange(N // 128, device=dev(), dtype=torch.int64) % P_BLOCKS)
    switches.setenv("DG_LOG", "1")
    capfd.readouterr()
    d = dg.gemm_fp8_nt(qa, sa, qb, sb)
    assert _chosen(capfd) == ["decode_bn32_w8_k2"]  # the register-fed decode schedule
    r = synth.rng(14, 97)
    cols = np.unique(np.concatenate([np.arange(0, 256), np.arange(WRAP_ROWS - 256, N), r.integers(0, N, 1024)]))
    y = bf16_values(d.index_select(1, torch.from_numpy(cols).to(dev())))
    del qb, sb, d
    _free()
    rr, cc = np.repeat(np.arange(M), cols.size), np.tile(cols % (128 * P_BLOCKS), M)
    R = oracle.gemm_pairs(oqa, osa, oqbp[0], osbp[0], rr, cc)
    assert_close(y.reshape(-1), R, "dense N=%d K=%d" % (N, K))


@pytest.mark.parametrize("layout", ["contiguous", "masked"])
def test_grouped_weights_beyond_32_bit_offsets(dg, switches, capfd, layout):
    # one expert whose weights reach 2^32 bytes (N*K per group), 256 rows of which 200 are
    # routed / valid
    G, M, N, rows_valid = 1, 256, WRAP_ROWS + 128, 200
    say("large %s N*K >= 2^32: G=%d M=%d N=%d K=%d" % (layout, G, M, N, K))
    a = synth.normal((M, K), 15, synth.TID_A)
    qa, sa = dg.cast_fp8_per_token(torch.from_numpy(a).to(dev()))
    oqa, osa = oracle.cast_per_token(a)
    assert_same_bytes(qa, oqa, "A cast")
    assert_same_bits(sa, kmajor(osa), "A scales")
    (qbp, sbp), (oqbp, osbp) = _weights(dg, 1, 128 * P_BLOCKS, seed=15)
    idx = torch.arange(N, device=dev(), dtype=torch.int64) % (128 * P_BLOCKS)
    qb = qbp[0].index_select(0, idx).view(G, N, K)
    sb = sbp[0].index_select(0, torch.arange(N // 128, device=dev(), dtype=torch.int64) % P_BLOCKS).view(G, N // 128, K // 128)
    sentinel = 0x7FBF
    if layout == "contiguous":
        mi = np.full(M, -1, np.int32)
        mi[:rows_valid] = 0
        d = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
        d.view(torch.int16).fill_(sentinel)
        meta = torch.from_numpy(mi).to(dev())
        switches.setenv("DG_LOG", "1")
        capfd.readouterr()
        dg.grouped_gemm_contiguous(qa, sa, qb, sb, meta, d=d)
        assert _chosen(capfd) == ["tile2_128x128"]  # N is an odd multiple of 128
        out = d
    else:
        d = torch.empty((G, M, N), dtype=torch.bfloat16, device=dev())
        d.view(torch.int16).fill_(sentinel)
        meta = torch.tensor([rows_valid], dtype=torch.int32, device=dev())
        switches.setenv("DG_LOG", "1")
        capfd.readouterr()
        dg.grouped_gemm_masked(qa.view(G, M, K), sa.view(G, K // 128, M), qb, sb, meta, d=d)
        assert _chosen(capfd) == ["tile2_256x128"]
        out = d[0]
        # rows at or beyond the count keep their bytes
        assert bool((out[rows_valid:, ::4099].view(torch.int16) == sentinel).all())
    r = synth.rng(15, 97)
    cols = np.unique(np.concatenate([np.arange(0, 256), np.arange(WRAP_ROWS - 256, N), r.integers(0, N, 768)]))
    y = bf16_values(out[:rows_valid].index_select(1, torch.from_numpy(cols).to(dev())))
    del qb, sb, d, out
    _free()
    rr, cc = np.repeat(np.arange(rows_valid), cols.size), np.tile(cols % (128 * P_BLOCKS), rows_valid)
    R = oracle.gemm_pairs(oqa, osa, oqbp, osbp, rr, cc, group_of_row=np.zeros(M, np.int32))
    assert_close(y.reshape(-1), R, "%s N=%d K=%d" % (layout, N, K))
