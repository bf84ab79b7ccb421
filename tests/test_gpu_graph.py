"""The path captured in a HIP graph (how the benchmark launches it): every replay must equal
the eager result bit for bit, with eager work and synchronisations between replays."""
import numpy as np
import pytest
import torch

import synth
from helpers import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dg():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import moe_grouped_gemm_e4m3_amd as m
    m.lib()
    return m


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


# the shapes take the LDS decode kernel, the activation-resident decode kernel, and the tiles
@pytest.mark.parametrize("M,N,K", [(64, 7168, 2048), (64, 1024, 1536), (64, 24576, 1536), (300, 512, 1024)])
def test_cast_and_gemm_graph_replays_match_eager(dg, M, N, K):
    dev = torch.device("cuda:0")
    a32, b32 = synth.dense_inputs(M, N, K, seed=3)
    a = torch.from_numpy(a32).to(dev)
    qb, sb = dg.cast_fp8_per_block(torch.from_numpy(b32).to(dev))
    qa = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
    d = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step():
        dg.cast_fp8_per_token(a, qa, sa)
        dg.gemm_fp8_nt(qa, sa, qb, sb, d=d)

    say("graph replay M=%d N=%d K=%d" % (M, N, K))
    step()
    torch.cuda.synchronize()
    q_ref, s_ref, d_ref = qa.clone(), sa.clone(), d.clone()
    g = _capture(step)
    for r in range(3):
        qa.fill_(0); sa.fill_(-1.0); d.fill_(7.0)   # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(qa, q_ref), "replay %d: codes" % r
        assert torch.equal(sa.view(torch.int32), s_ref.view(torch.int32)), "replay %d: scales" % r
        assert torch.equal(d.view(torch.int16), d_ref.view(torch.int16)), "replay %d: output" % r


def test_grouped_graph_replays_match_eager(dg):
    dev = torch.device("cuda:0")
    G, Mm, N, K = 4, 128, 256, 512
    a, b, mm = synth.masked_inputs(G, Mm, N, K, seed=4)
    qa, sa = dg.cast_fp8_per_token(torch.from_numpy(a).to(dev))
    qb, sb = dg.cast_fp8_per_block(torch.from_numpy(b).to(dev))
    mmd = torch.from_numpy(mm).to(dev)
    d = torch.zeros((G, Mm, N), dtype=torch.bfloat16, device=dev)
    fn = lambda: dg.grouped_gemm_masked(qa, sa, qb, sb, mmd, d=d)
    say("graph replay masked")
    fn()
    torch.cuda.synchronize()
    ref = d.clone()
    g = _capture(fn)
    for r in range(3):
        d.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        rows = np.concatenate([gg * Mm + np.arange(int(mm[gg])) for gg in range(G)])
        dv, rv = d.view(G * Mm, N)[rows], ref.view(G * Mm, N)[rows]
        assert torch.equal(dv.view(torch.int16), rv.view(torch.int16)), "replay %d" % r


@pytest.mark.parametrize("layout", ["contiguous", "masked"])
def test_ffn_graph_replays_match_eager(dg, layout):
    # token cast + expert FFN (fused gate/up + SwiGLU + re-cast, then the down GEMM)
    dev = torch.device("cuda:0")
    G, H, I = 3, 384, 256
    if layout == "contiguous":
        mi, _ = synth.contiguous_layout(G, 300, 5)
        x32 = synth.normal((mi.size, H), 5, synth.TID_A)
        x32[mi < 0] = 0.0
        meta = torch.from_numpy(mi).to(dev)
        lay, sx_shape, rows = dg.LAYOUT_CONTIGUOUS, (H // 128, mi.size), (mi.size,)
    else:
        mm = np.array([70, 0, 128], np.int32)
        x32 = synth.normal((G, 128, H), 5, synth.TID_A)
        meta = torch.from_numpy(mm).to(dev)
        lay, sx_shape, rows = dg.LAYOUT_MASKED, (G, H // 128, 128), (G, 128)
    w1, w2 = synth.ffn_weights(G, H, I, 5)
    q1, s1 = dg.cast_fp8_per_block(torch.from_numpy(w1.reshape(-1, H)).to(dev))
    q2, s2 = dg.cast_fp8_per_block(torch.from_numpy(w2.reshape(-1, I)).to(dev))
    q1, s1 = q1.view(G, 2 * I, H), s1.view(G, 2 * I // 128, H // 128)
    q2, s2 = q2.view(G, H, I), s2.view(G, H // 128, I // 128)
    x = torch.from_numpy(x32).to(dev)
    qx = torch.empty(tuple(x.shape), dtype=torch.uint8, device=dev)
    sx = torch.empty(sx_shape, dtype=torch.float32, device=dev)
    hq = torch.zeros(rows + (I,), dtype=torch.uint8, device=dev)
    sh = torch.zeros((G, I // 128, 128) if layout == "masked" else (I // 128, mi.size), dtype=torch.float32,
                     device=dev)
    y = torch.zeros(rows + (H,), dtype=torch.bfloat16, device=dev)

    def step():
        dg.cast_fp8_per_token(x, qx, sx)
        dg.moe_ffn_fp8(lay, qx, sx, q1, s1, q2, s2, meta, expected_m=64, hq=hq, sfh=sh, y=y)

    say("graph replay ffn %s" % layout)
    step()
    torch.cuda.synchronize()
    hq_ref, sh_ref, y_ref = hq.clone(), sh.clone(), y.clone()
    g = _capture(step)
    for r in range(3):
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(hq, hq_ref), "replay %d: h codes" % r
        assert torch.equal(sh.view(torch.int32), sh_ref.view(torch.int32)), "replay %d: h scales" % r
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), "replay %d: y" % r
        qx.fill_(0); sx.fill_(-1.0)   # eager work between replays (recomputed by the next replay)
