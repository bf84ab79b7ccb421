"""The expert FFN entry point that allocates nothing (dg_moe_ffn_fp8_noalloc): its FP8
activation between the two GEMMs lives in the library's static device scratch instead of a
caller workspace. Its output must equal that of dg_moe_ffn_fp8 (same kernels, so bit for bit)
on consecutive calls, the second one smaller, so that nothing the first call left in the
scratch reaches the second one's results."""
import numpy as np
import pytest
import torch

import synth
from helpers import say, to_dev

pytestmark = pytest.mark.gpu

CONTIG, MASKED = 1, 2
SENTINEL = 0x7FBF  # a bf16 NaN pattern no computed row produces


@pytest.fixture(scope="module")
def dg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import moe_grouped_gemm_e4m3_amd as m
    m.lib()
    return m


def _weights(dg, G, H, I, seed, ue8m0):
    w1, w2 = synth.ffn_weights(G, H, I, seed)
    q1, s1 = dg.cast_fp8_per_block(to_dev(w1.reshape(G * 2 * I, H)), ue8m0=ue8m0)
    q2, s2 = dg.cast_fp8_per_block(to_dev(w2.reshape(G * H, I)), ue8m0=ue8m0)
    return (q1.view(G, 2 * I, H), s1.view(G, 2 * I // 128, H // 128), q2.view(G, H, I),
            s2.view(G, H // 128, I // 128))


def _both(dg, layout, x, sx, w, meta, expected_m, y_shape, ue8m0):
    """(y from the workspace entry point, y from the static-scratch one), both prefilled."""
    y_ws = torch.full(y_shape, SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    y_st = torch.full(y_shape, SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    dg.moe_ffn_fp8(layout, x, sx, *w, meta, expected_m=expected_m, y=y_ws, ue8m0=ue8m0)
    dg.moe_ffn_fp8_noalloc(layout, x, sx, *w, meta, expected_m=expected_m, y=y_st, ue8m0=ue8m0)
    torch.cuda.synchronize()
    return y_ws.view(torch.int16).cpu().numpy(), y_st.view(torch.int16).cpu().numpy()


@pytest.mark.parametrize("ue8m0", [False, True])
def test_noalloc_masked_matches_workspace(dg, ue8m0):
    for G, M_max, H, I, seed in [(8, 128, 1024, 512, 61), (4, 64, 512, 256, 62)]:
        say("ffn noalloc masked G=%d M_max=%d H=%d I=%d ue8m0=%s" % (G, M_max, H, I, ue8m0))
        mm = synth.masked_layout(G, M_max, seed)
        x = synth.normal((G, M_max, H), seed, synth.TID_A)
        xq, sx = dg.cast_fp8_per_token(to_dev(x), ue8m0=ue8m0)
        w = _weights(dg, G, H, I, seed, ue8m0)
        y_ws, y_st = _both(dg, MASKED, xq, sx, w, to_dev(mm), int(max(1, mm.mean())), (G, M_max, H), ue8m0)
        assert np.array_equal(y_ws, y_st)
        for g in range(G):  # rows beyond the valid count stay unwritten in both
            assert (y_st[g, int(mm[g]):] == np.int16(SENTINEL)).all()
            assert (y_st[g, :int(mm[g])] != np.int16(SENTINEL)).all()


@pytest.mark.parametrize("ue8m0", [False, True])
def test_noalloc_contiguous_matches_workspace(dg, ue8m0):
    for G, tokens, H, I, seed in [(4, 600, 1024, 512, 63), (2, 200, 512, 256, 64)]:
        say("ffn noalloc contiguous G=%d tokens=%d H=%d I=%d ue8m0=%s" % (G, tokens, H, I, ue8m0))
        mi, _ = synth.contiguous_layout(G, tokens, seed)
        x = synth.normal((mi.size, H), seed, synth.TID_A)
        x[mi < 0] = 0.0
        xq, sx = dg.cast_fp8_per_token(to_dev(x), ue8m0=ue8m0)
        w = _weights(dg, G, H, I, seed, ue8m0)
        y_ws, y_st = _both(dg, CONTIG, xq, sx, w, to_dev(mi), 0, (mi.size, H), ue8m0)
        routed = mi >= 0
        assert np.array_equal(y_ws[routed], y_st[routed])
        assert (y_st[routed] != np.int16(SENTINEL)).all()


def test_noalloc_rejects_calls_beyond_the_scratch(dg):
    # 15888 rows x I=2048 need 2112 * 15888 bytes > 32 MiB: refused before any launch
    G, M_max, H, I = 1, 15888, 128, 2048
    x = torch.zeros((G, M_max, H), dtype=torch.uint8, device="cuda:0")
    sx = torch.zeros((G, H // 128, M_max), dtype=torch.float32, device="cuda:0")
    w1 = torch.zeros((G, 2 * I, H), dtype=torch.uint8, device="cuda:0")
    s1 = torch.zeros((G, 2 * I // 128, H // 128), dtype=torch.float32, device="cuda:0")
    w2 = torch.zeros((G, H, I), dtype=torch.uint8, device="cuda:0")
    s2 = torch.zeros((G, H // 128, I // 128), dtype=torch.float32, device="cuda:0")
    mm = torch.full((G,), M_max, dtype=torch.int32, device="cuda:0")
    y = torch.full((G, M_max, H), SENTINEL, dtype=torch.int16, device="cuda:0").view(torch.bfloat16)
    with pytest.raises(dg.DGError) as e:
        dg.moe_ffn_fp8_noalloc(MASKED, x, sx, w1, s1, w2, s2, mm, y=y)
    assert e.value.status == 2 and "static scratch" in str(e.value)
    torch.cuda.synchronize()
    assert (y.view(torch.int16) == SENTINEL).all()
    # one row fewer fits
    y2 = dg.moe_ffn_fp8_noalloc(MASKED, x[:, :15887].contiguous(), sx[:, :, :15887].contiguous(), w1, s1, w2, s2,
                                mm - 1)
    torch.cuda.synchronize()
    assert (y2.float() == 0).all()
