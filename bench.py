"""Benchmark of the FP8 block-scaled GEMM path on one MI355X.

Default workload ("decode", dense + grouped at decode): two dense DeepSeek-V3-shaped layers
at M = 64 tokens, (N=7168, K=2048) and (N=24576, K=1536), and the two MoE expert layers in
the masked layout one GPU holds at decode (G=32 experts, 256-row buffers, valid rows
~U{0..256}), (N=4096, K=7168) and (N=7168, K=2048). One step = for each layer, the per-token
FP8 cast of its fp32 activations followed by its block-scaled FP8 GEMM (bf16 out). A masked
layer casts the valid rows of each expert only: the rows its GEMM reads.
Inputs are resident in HBM before timing starts. Every layer cycles through R_l copies of
its weights (R_l * |weights_l| >= 512 MiB) so the 256 MiB Infinity Cache cannot serve them.

Steps are captured in HIP graphs (one graph per weight copy, launched on torch's stream)
and replayed, so the measurement is GPU time rather than Python launch overhead.

Prints ONE JSON line. `value` is the GEMM FLOP rate over the whole step (cast included).
`roofline` is for the kernel that takes the most time in the step. Times come from HIP
events on the stream the kernels run on, between replays of graphs queued back to back, and
are medians over at least 10 replays and 100 launches. Each kernel gets two:
`in_step_us`, its marginal time in the step (a graph of the whole step over every weight
copy, minus the same graph without that one launch, the two alternating in three blocks of
replays), and `avg_us`, its launch duration (a graph of back-to-back launches of it alone
through the weight copies, >= 8 launches and about 200 us of work per graph). The roofline
uses `avg_us`, the figure a kernel trace reports. A cast timed alone reads an input that its
previous launch left in the caches, unlike in the step. `cpu_baseline` is the CPU oracle on the host cores over a bounded sample
of the same workload. `traffic` (HBM bytes per launch) is read from profiles/traffic.json
when that file was produced from the current kernel source.

Other workloads (--workload decode_dense|skinny128|skinny256|prefill|contiguous|masked|
ffn_contiguous|ffn_masked|ffn_masked_decode|tiny) print the same line shape.
--ue8m0 runs the same steps with power-of-two (UE8M0) scales: the _ue8m0 casts and GEMMs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8 block-scaled GEMM TFLOPS & % of MI355X FP8 MFMA peak (dense+grouped, M=64)"
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, published
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, published
RIDGE = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)  # flop per byte

# (kind, shape) per layer of each workload
WORKLOADS = {
    # the metric's configuration: dense decode at M=64 and the MoE masked (decode) layout
    "decode": {"desc": "dense M=64: (N=7168,K=2048) + (N=24576,K=1536); MoE masked G=32, M_max=256, "
                       "valid ~U{0..256}: (N=4096,K=7168) + (N=7168,K=2048)",
               "layers": [("dense", dict(M=64, N=7168, K=2048)), ("dense", dict(M=64, N=24576, K=1536)),
                          ("masked", dict(G=32, M_max=256, N=4096, K=7168)),
                          ("masked", dict(G=32, M_max=256, N=7168, K=2048))]},
    "decode_dense": {"desc": "dense decode M=64: (N=7168,K=2048) + (N=24576,K=1536)",
                     "layers": [("dense", dict(M=64, N=7168, K=2048)), ("dense", dict(M=64, N=24576, K=1536))]},
    # skinny M between decode and prefill, on the decode layers' shapes
    "skinny128": {"desc": "dense M=128: (N=7168,K=2048) + (N=24576,K=1536)",
                  "layers": [("dense", dict(M=128, N=7168, K=2048)), ("dense", dict(M=128, N=24576, K=1536))]},
    "skinny256": {"desc": "dense M=256: (N=7168,K=2048) + (N=24576,K=1536)",
                  "layers": [("dense", dict(M=256, N=7168, K=2048)), ("dense", dict(M=256, N=24576, K=1536))]},
    "prefill": {"desc": "dense prefill M=4096 with 1% x50 outliers: (N=7168,K=18432) + (N=36864,K=7168)",
                "layers": [("dense", dict(M=4096, N=7168, K=18432, outliers=True)),
                           ("dense", dict(M=4096, N=36864, K=7168, outliers=True))]},
    "contiguous": {"desc": "MoE contiguous G=8, 8192 routed rows padded to 128: (N=4096,K=7168) + (N=7168,K=2048)",
                   "layers": [("contiguous", dict(G=8, tokens=8192, N=4096, K=7168)),
                              ("contiguous", dict(G=8, tokens=8192, N=7168, K=2048))]},
    "masked": {"desc": "MoE masked G=32, M_max=256, valid ~U{0..256}: (N=4096,K=7168) + (N=7168,K=2048)",
               "layers": [("masked", dict(G=32, M_max=256, N=4096, K=7168)),
                          ("masked", dict(G=32, M_max=256, N=7168, K=2048))]},
    "tiny": {"desc": "dense M=128 N=256 K=512", "layers": [("dense", dict(M=128, N=256, K=512))]},
    # expert FFN: gate/up GEMM (N = 2I) with the SwiGLU + FP8 re-cast epilogue, then the
    # down GEMM (N = H, K = I); the same shapes as the contiguous / masked pairs above
    "ffn_contiguous": {"desc": "MoE expert FFN, contiguous G=8, 8192 routed rows padded to 128: H=7168, I=2048",
                       "layers": [("ffn_contiguous", dict(G=8, tokens=8192, H=7168, I=2048))]},
    "ffn_masked": {"desc": "MoE expert FFN, masked G=32, M_max=256, valid ~U{0..256}: H=7168, I=2048",
                   "layers": [("ffn_masked", dict(G=32, M_max=256, H=7168, I=2048))]},
    # decode-sized expert batches: 128 tokens x top-8 over 256 experts is 4 rows per expert on
    # average; one GPU's 32 experts with valid rows ~U{0..8} in 64-row buffers
    "ffn_masked_decode": {"desc": "MoE expert FFN at decode, masked G=32, M_max=64, valid ~U{0..8}: H=7168, I=2048",
                          "layers": [("ffn_masked", dict(G=32, M_max=64, H=7168, I=2048, max_count=8))]},
}
FFN_KINDS = ("ffn_contiguous", "ffn_masked")
FFN_WORKLOADS = ("ffn_contiguous", "ffn_masked", "ffn_masked_decode")


def weight_elems(kind, s):
    if kind in FFN_KINDS:
        return s["G"] * 3 * s["I"] * s["H"]
    return s.get("G", 1) * s["N"] * s["K"]


def swiglu_work(s, valid_rows, active):
    """Flops and HBM bytes of the fused gate/up launch: A, the W1 of the `active` experts (those
    with at least one valid row) and their scales in; the FP8 activation h and its per-token
    scales out."""
    H, I = s["H"], s["I"]
    flops = 2.0 * valid_rows * 2 * I * H
    byts = (valid_rows * H + active * 2 * I * H + 4 * valid_rows * H // 128
            + 4 * active * (2 * I // 128) * (H // 128) + valid_rows * I + 4 * valid_rows * I // 128)
    return flops, float(byts)


def layer_work(kind, s, valid_rows, active):
    """Algorithmic flops and HBM bytes of one GEMM launch: valid rows only, and the weights of
    the `active` groups only (an expert with no rows needs none of its weights)."""
    if kind in FFN_KINDS:  # the whole FFN: fused gate/up + down
        f1, b1 = swiglu_work(s, valid_rows, active)
        f2, b2 = layer_work(kind[4:], dict(G=s["G"], N=s["H"], K=s["I"]), valid_rows, active)
        return f1 + f2, b1 + b2
    N, K = s["N"], s["K"]
    G = active
    flops = 2.0 * valid_rows * N * K
    byts = (valid_rows * K            # A e4m3
            + G * N * K               # B e4m3
            + 4 * valid_rows * K // 128   # activation scales
            + 4 * G * (N // 128) * (K // 128)  # weight scales
            + 2 * valid_rows * N)     # bf16 out
    return flops, float(byts)


def cast_bytes(rows, K):
    return float(rows * K * 4 + rows * K + 4 * rows * K // 128)


def build_layer(dg, torch, kind, s, seed, copies, ue8m0=False):
    """Device inputs for one layer: fp32 activations, `copies` quantised weight copies."""
    import numpy as np
    import synth
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(1000 * seed + 17)
    ffn = kind in FFN_KINDS
    base = kind[4:] if ffn else kind
    if ffn:
        N, K = 2 * s["I"], s["H"]
    else:
        N, K = s["N"], s["K"]
    meta = None
    if base == "dense":
        rows = s["M"]
        valid = rows
        active = 1
        a = torch.randn((rows, K), generator=gen, device=dev, dtype=torch.float32)
        if s.get("outliers"):
            hit = torch.rand((rows, K), generator=gen, device=dev) < 0.01
            a = torch.where(hit, a * 50.0, a)
        G = 1
    elif base == "contiguous":
        mi, counts = synth.contiguous_layout(s["G"], s["tokens"], seed)
        rows = mi.size
        valid = int(counts.sum())
        active = int((counts > 0).sum())
        a = torch.randn((rows, K), generator=gen, device=dev, dtype=torch.float32)
        mi_d = torch.from_numpy(mi).to(dev)
        a[mi_d < 0] = 0.0
        meta = mi_d
        G = s["G"]
    else:
        mm = synth.masked_layout(s["G"], s["M_max"], seed, s.get("max_count"))
        rows = s["G"] * s["M_max"]
        valid = int(mm.sum())
        active = int((mm > 0).sum())
        a = torch.randn((s["G"], s["M_max"], K), generator=gen, device=dev, dtype=torch.float32)
        meta = torch.from_numpy(mm).to(dev)
        G = s["G"]
    ws = []
    for c in range(copies):
        w = torch.randn((G * N, K), generator=gen, device=dev, dtype=torch.float32) * 0.02
        qb, sb = dg.cast_fp8_per_block(w, ue8m0=ue8m0)
        del w
        if kind == "dense":
            ws.append((qb, sb))
        elif ffn:  # (gate/up, down) of every expert
            H, I = s["H"], s["I"]
            w = torch.randn((G * H, I), generator=gen, device=dev, dtype=torch.float32) * 0.02
            q2, s2 = dg.cast_fp8_per_block(w, ue8m0=ue8m0)
            del w
            ws.append((qb.view(G, N, K), sb.view(G, N // 128, K // 128), q2.view(G, H, I),
                       s2.view(G, H // 128, I // 128)))
        else:
            ws.append((qb.view(G, N, K), sb.view(G, N // 128, K // 128)))
    # activation scales are K-block-major: [K/128, rows], per group for the masked layout
    qa = torch.empty(tuple(a.shape), dtype=torch.uint8, device=dev)
    sa = torch.empty(tuple(a.shape[:-2]) + (K // 128, a.shape[-2]), dtype=torch.float32, device=dev)
    if base == "masked":
        d = torch.empty((s["G"], s["M_max"], N), dtype=torch.bfloat16, device=dev)
    else:
        d = torch.empty((rows, N), dtype=torch.bfloat16, device=dev)
    L = dict(kind=kind, s=s, a=a, qa=qa, sa=sa, ws=ws, d=d, meta=meta, rows=rows, valid=valid, active=active, G=G, ue8m0=ue8m0)
    if ffn:  # the FP8 activation between the GEMMs and the FFN output
        H, I = s["H"], s["I"]
        lead = (s["G"], s["M_max"]) if base == "masked" else (rows,)
        L["hq"] = torch.empty(lead + (I,), dtype=torch.uint8, device=dev)
        L["sh"] = torch.empty(((s["G"], I // 128, s["M_max"]) if base == "masked" else (I // 128, rows)),
                              dtype=torch.float32, device=dev)
        L["y"] = torch.empty(lead + (H,), dtype=torch.bfloat16, device=dev)
        L["layout"] = dg.LAYOUT_MASKED if base == "masked" else dg.LAYOUT_CONTIGUOUS
    return L


def expected_m(L):
    return max(1, L["valid"] // L["G"])


def cast_layer(dg, L):
    """The layer's per-token activation cast: in the masked layout, of the valid rows only
    (the rows its GEMM reads)."""
    if L["kind"].endswith("masked"):
        dg.cast_fp8_per_token_masked(L["a"], L["meta"], L["qa"], L["sa"], ue8m0=L["ue8m0"])
    else:
        dg.cast_fp8_per_token(L["a"], L["qa"], L["sa"], ue8m0=L["ue8m0"])


def run_layer(dg, L, copy_idx):
    """Cast the layer's activations, then its GEMM with weight copy `copy_idx`."""
    kind = L["kind"]
    u = L["ue8m0"]
    cast_layer(dg, L)
    if kind in FFN_KINDS:
        w1, s1, w2, s2 = L["ws"][copy_idx % len(L["ws"])]
        dg.moe_ffn_fp8(L["layout"], L["qa"], L["sa"], w1, s1, w2, s2, L["meta"], expected_m=expected_m(L),
                       hq=L["hq"], sfh=L["sh"], y=L["y"], ue8m0=u)
        return
    qb, sb = L["ws"][copy_idx % len(L["ws"])][:2]
    if kind == "dense":
        dg.gemm_fp8_nt(L["qa"], L["sa"], qb, sb, d=L["d"], ue8m0=u)
    elif kind == "contiguous":
        dg.grouped_gemm_contiguous(L["qa"], L["sa"], qb, sb, L["meta"], d=L["d"], ue8m0=u)
    else:
        dg.grouped_gemm_masked(L["qa"], L["sa"], qb, sb, L["meta"], expected_m=max(1, L["valid"] // L["G"]),
                               d=L["d"], ue8m0=u)


def load_traffic(workload, label):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from moe_grouped_gemm_e4m3_amd.profiling import source_hash
    rec = t.get(workload, {}).get(label)
    if not rec or rec.get("source_hash") != source_hash():
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(workload, budget_s, ue8m0=False):
    """The CPU oracle (unchanged) on a bounded sample of the workload: every layer's cast
    and GEMM over a row sample, repeated until ~budget_s seconds of work."""
    import numpy as np
    import oracle
    import synth
    sample_desc = []
    jobs = []
    if workload in FFN_WORKLOADS:
        # one expert's FFN over 64 tokens: cast, gate/up GEMM, SwiGLU, re-cast, down GEMM
        _, s = WORKLOADS[workload]["layers"][0]
        H, I, rows = s["H"], s["I"], 64
        x = synth.normal((rows, H), 0, synth.TID_A)
        w1, w2 = synth.ffn_weights(1, H, I, 0)
        w1q, s1 = oracle.cast_per_block(w1, pow2=ue8m0)
        w2q, s2 = oracle.cast_per_block(w2, pow2=ue8m0)
        del w1, w2
        mi = np.zeros(rows, np.int32)
        flops = 0.0
        t0 = time.perf_counter()
        reps = 0
        while True:
            xq, sx = oracle.cast_per_token(x, pow2=ue8m0)
            oracle.moe_ffn_contiguous(xq, sx, w1q, s1, w2q, s2, mi, ue8m0)
            flops += 2.0 * rows * 3 * I * H
            reps += 1
            if time.perf_counter() - t0 >= budget_s:
                break
        dt = time.perf_counter() - t0
        return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
                "sample": "one expert's FFN (cast, gate/up GEMM, SwiGLU, re-cast, down GEMM) over %d tokens, "
                          "H=%d I=%d, %d repetitions in %.1f s" % (rows, H, I, reps, dt)}
    for li, (kind, s) in enumerate(WORKLOADS[workload]["layers"]):
        N, K = s["N"], s["K"]
        rows = {"dense": s.get("M", 64), "contiguous": 64, "masked": 64}[kind]
        rows = min(rows, 64)
        a, _ = synth.dense_inputs(rows, 128, K, seed=li)
        G = s.get("G", 1)
        bcols = N if kind == "dense" and N * K * rows <= 2 ** 31 else min(N, 2048)
        b = synth.normal((bcols, K), li, synth.TID_B, 0.02)
        qb, sb = oracle.cast_per_block(b, pow2=ue8m0)
        jobs.append((a, qb, sb, rows, bcols, K))
        sample_desc.append("%dx%dx%d" % (rows, bcols, K))
    flops = 0.0
    t0 = time.perf_counter()
    reps = 0
    while True:
        for a, qb, sb, rows, bcols, K in jobs:
            qa, sa = oracle.cast_per_token(a, pow2=ue8m0)
            oracle.gemm(qa, sa, qb, sb)
            flops += 2.0 * rows * bcols * K
        reps += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "per-token cast + fp64 GEMM of %s (rows x N x K per layer), %d repetitions in %.1f s"
                      % (", ".join(sample_desc), reps, dt)}


def capture(torch, fn):
    """HIP graph of fn() on the current device (the binding launches on torch's current
    stream, which is the capture stream inside torch.cuda.graph)."""
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


def time_graphs(torch, graphs, n):
    """Replay graphs[i % len] for i < n between two events; returns ms."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(n):
        graphs[i % len(graphs)].replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1)


def replay_intervals(torch, graph, n):
    """Per-replay GPU times (ms) of n replays queued back to back, with an event between every
    two: the host queues them all before the first ends, so no interval holds host launch
    latency, except possibly the first, which is dropped. (Events around one replay at a time
    would include that latency: about 36 us per replay, measured on a one-launch graph.)"""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 2)]
    torch.cuda.synchronize()
    for i in range(n + 1):
        ev[i].record()
        graph.replay()
    ev[n + 1].record()
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(1, n + 1)]


def median(v):
    v = sorted(v)
    h = len(v) // 2
    return v[h] if len(v) % 2 else 0.5 * (v[h - 1] + v[h])


def warm_clocks(torch, graphs, seconds):
    """Untimed replays for about `seconds` of wall time: the GPU raises its clocks only after a
    stretch of sustained work, and a short first measurement would catch the ramp."""
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for g in graphs:
            g.replay()
        torch.cuda.synchronize()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode", choices=sorted(WORKLOADS))
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--ue8m0", action="store_true", help="power-of-two (UE8M0) scales")
    ap.add_argument("--kernel-reps", type=int, default=100,
                    help="launches per kernel in the per-kernel timing (at least 100)")
    ap.add_argument("--cache-bytes", type=float, default=512 * 2 ** 20,
                    help="minimum bytes of distinct weight copies cycled through")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 256 MiB device copy (reference kernel for HBM counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library runs each GEMM on one device and has no "
              "multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import moe_grouped_gemm_e4m3_amd as dg
    if not os.path.exists(dg.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    wl = WORKLOADS[args.workload]
    # weight copies per layer, so that every launch streams its weights from HBM, not from the
    # 256 MiB cache, in the step and in the per-kernel timing alike
    layer_copies = [int(min(64, max(1, math.ceil(args.cache_bytes / weight_elems(kind, s)))))
                    for kind, s in wl["layers"]]
    layers = [build_layer(dg, torch, kind, s, args.seed + i, layer_copies[i], args.ue8m0)
              for i, (kind, s) in enumerate(wl["layers"])]
    copies = max(layer_copies)  # one step graph per index; layer l uses copy index % R_l
    torch.cuda.synchronize()

    if args.copy_calibration:
        src = torch.empty(64 * 2 ** 20, dtype=torch.float32, device="cuda:0").fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def step(c):
        for L in layers:
            run_layer(dg, L, c)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # one graph per weight copy, each holding one whole step (casts + GEMMs)
    step_graphs = [capture(torch, lambda c=c: step(c)) for c in range(copies)]

    warm_clocks(torch, step_graphs, 0.5)

    # per-kernel timing: graphs of back-to-back launches of one kernel over the layer's
    # weight copies, replayed until at least `reps` launches and 10 replays
    reps = max(100, args.kernel_reps)
    kernels = []
    step_flops = 0.0
    for L in layers:
        f, _ = layer_work(L["kind"], L["s"], L["valid"], L["active"])
        step_flops += f
    def grouped(L, base, a, sa, qb, sb, d):
        u = L["ue8m0"]
        if base == "dense":
            dg.gemm_fp8_nt(a, sa, qb, sb, d=d, ue8m0=u)
        elif base == "contiguous":
            dg.grouped_gemm_contiguous(a, sa, qb, sb, L["meta"], d=d, ue8m0=u)
        else:
            dg.grouped_gemm_masked(a, sa, qb, sb, L["meta"], expected_m=expected_m(L), d=d, ue8m0=u)

    def seq_graph(launches, nc):
        """A graph that runs `launches` (each launch(c)) for weight copy c = 0 .. nc-1 in turn."""
        return capture(torch, lambda: [f(c) for c in range(nc) for f in launches])

    def paired_us(ga, gb, nc, n, blocks=3):
        """Median per-copy durations (us) of graphs ga and gb, replayed in alternating blocks of
        n back-to-back replays (so a drift of the clocks affects both alike)."""
        time_graphs(torch, [ga, gb], 2)
        ta, tb = [], []
        for _ in range(blocks):
            ta += [ms / nc * 1e3 for ms in replay_intervals(torch, ga, n)]
            tb += [ms / nc * 1e3 for ms in replay_intervals(torch, gb, n)]
        return median(ta), median(tb)

    # (layer index, label, launch(c), flops and bytes of one launch, part of the step, the
    # launches that precede it in its layer)
    entries = []
    for li, L in enumerate(layers):
        s_ = L["s"]
        kind = L["kind"]
        ffn = kind in FFN_KINDS
        base = kind[4:] if ffn else kind
        K = s_["H"] if ffn else s_["K"]
        cast_fn = lambda c, L=L: cast_layer(dg, L)
        cast_rows = L["valid"] if base == "masked" else L["rows"]
        entries.append((li, "cast", cast_fn, (0.0, cast_bytes(cast_rows, K)), True, []))
        if ffn:
            H, I = s_["H"], s_["I"]
            swiglu_fn = lambda c, L=L: dg.gemm_fp8_swiglu(L["layout"], L["qa"], L["sa"], *L["ws"][c % len(L["ws"])][:2],
                                                          L["meta"], expected_m=expected_m(L), hq=L["hq"], sfh=L["sh"],
                                                          ue8m0=L["ue8m0"])
            entries += [
                (li, "swiglu gate/up N=%d K=%d" % (2 * I, H), swiglu_fn, swiglu_work(s_, L["valid"], L["active"]),
                 True, [cast_fn]),
                (li, "down N=%d K=%d" % (H, I),
                 lambda c, L=L, base=base: grouped(L, base, L["hq"], L["sh"], *L["ws"][c % len(L["ws"])][2:], L["y"]),
                 layer_work(base, dict(G=s_["G"], N=H, K=I), L["valid"], L["active"]), True, [cast_fn, swiglu_fn]),
                # the same gate/up product as a plain GEMM with bf16 output: the cost of the epilogue
                (li, "plain gate/up (bf16 out, not in the step) N=%d K=%d" % (2 * I, H),
                 lambda c, L=L, base=base: grouped(L, base, L["qa"], L["sa"], *L["ws"][c % len(L["ws"])][:2], L["d"]),
                 layer_work(base, dict(G=s_["G"], N=2 * I, K=H), L["valid"], L["active"]), False, [cast_fn]),
            ]
        else:
            entries.append((li, "gemm", lambda c, L=L, base=base: grouped(L, base, L["qa"], L["sa"],
                                                                          *L["ws"][c % len(L["ws"])][:2], L["d"]),
                            layer_work(kind, s_, L["valid"], L["active"]), True, [cast_fn]))

    # Two times per kernel:
    #  - in_step_us: its marginal time in the step, the step graph over every weight copy minus
    #    the same graph without that one launch (with the step's cache state, inputs and
    #    neighbours; the cost of a graph replay cancels). Kernels outside the step: none.
    #  - avg_us: its launch duration, from a graph of back-to-back launches of it alone cycling
    #    through the weight copies, at least 8 launches and about 200 us of work per graph (so a
    #    replay's own cost is spread thin). The roofline uses this one, as a kernel trace would.
    step_seq = [(li, lab, fn) for li, lab, fn, _, in_step, _ in entries if in_step]
    n_step = max(10, math.ceil(reps / copies))
    full_graph = seq_graph([fn for _, _, fn in step_seq], copies)
    for li, lab, fn, (f, b), in_step, before in entries:
        L = layers[li]
        lc = len(L["ws"])
        marginal = None
        if in_step:
            g_without = seq_graph([g for lj, lb, g in step_seq if (lj, lb) != (li, lab)], copies)
            t_full, t_without = paired_us(full_graph, g_without, copies, n_step)
            del g_without
            marginal = t_full - t_without
            est = max(marginal, 1.0)
        else:
            est = 100.0
        per_graph = lc * max(1, math.ceil(max(8.0, 200.0 / est) / lc))  # launches per graph
        g_alone = seq_graph([fn], per_graph)
        n = max(10, math.ceil(reps / per_graph))
        time_graphs(torch, [g_alone], 2)
        avg_us = median([ms / per_graph * 1e3 for ms in replay_intervals(torch, g_alone, n)])
        del g_alone
        kind = L["kind"]
        ffn = kind in FFN_KINDS
        bound = "hbm" if (f == 0.0 or f / b < RIDGE) else "mfma"
        layer = kind if ffn else "%s N=%d K=%d" % (kind, L["s"]["N"], L["s"]["K"])
        kernels.append({"kernel": lab, "layer": layer, "avg_us": avg_us, "in_step_us": marginal,
                        "tflops": f / (avg_us * 1e-6) / 1e12, "gbs": b / (avg_us * 1e-6) / 1e9,
                        "bound": bound, "flops": f, "bytes": b, "launches": n * per_graph, "replays": n,
                        "in_step": in_step})
    del full_graph
    dom = max((k for k in kernels if k["in_step"]), key=lambda k: k["in_step_us"])

    # the whole step: W untimed warmup steps, then exactly K timed steps
    warm_clocks(torch, step_graphs, 0.2)
    time_graphs(torch, step_graphs, args.warmup)
    total_ms = time_graphs(torch, step_graphs, args.steps)
    ms_per_step = total_ms / args.steps
    if dom["bound"] == "hbm":
        achieved, peak, unit = dom["gbs"], PEAK_HBM_GBS, "GB/s"
    else:
        achieved, peak, unit = dom["tflops"], PEAK_FP8_TFLOPS, "TFLOP/s"
    traffic = load_traffic(args.workload + ("_ue8m0" if args.ue8m0 else ""), dom["layer"] + " " + dom["kernel"])

    value = step_flops / (ms_per_step * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3", "data": "synthetic",
        "config": {"workload": wl["desc"], "weight_copies": layer_copies,
                   "scales": "UE8M0 (powers of two)" if args.ue8m0 else "fp32 (amax / 448)",
                   "step": ("per-token FP8 cast of fp32 activations + expert FFN: gate/up GEMM with fused "
                            "SwiGLU and FP8 re-cast, then the down GEMM (bf16 out); replayed from HIP graphs"
                            if args.workload in FFN_WORKLOADS else
                            "per-token FP8 cast of fp32 activations + FP8 block-scaled GEMM (bf16 out), "
                            "per layer; replayed from HIP graphs")
                           + ("; masked layers cast their valid rows only" if any(
                               k.endswith("masked") for k, _ in wl["layers"]) else "")},
        "frac_of_fp8_peak": round(value / PEAK_FP8_TFLOPS, 5),
        "roofline": {"bound": dom["bound"], "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": dom["kernel"] + " " + dom["layer"], "algorithmic_bytes": dom["bytes"],
                     "algorithmic_flops": dom["flops"], "avg_us": round(dom["avg_us"], 3)},
        "kernels": [{k: (round(v, 3) if isinstance(v, float) else v) for k, v in kk.items()} for kk in kernels],
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(args.workload, args.cpu_budget, args.ue8m0)
        out["cpu_baseline"]["value"] = round(out["cpu_baseline"]["value"], 6)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
