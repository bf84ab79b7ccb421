"""Seeded synthetic inputs for the FP8 block-scaled GEMM path.

This module draws random numbers and builds routing layouts; it holds none of the
method's arithmetic (no quantisation, no scaling, no GEMM). Both the CPU oracle and the
HIP path take their inputs from here, each then quantising and multiplying on its own.

Workload shapes are DeepSeek-V3-like (hidden size 7168 from the DeepSeek-V3 repo review,
"Risks" 6; 256 routed experts with top-8 from its "Innovations" 3; 128x128 blocks). The
pages' own per-shape tables are missing, so these shapes stand in for them.

Recipes (one generator stream per (seed, tensor id), numpy PCG64):
  * activations A ~ N(0, 1) fp32; prefill activations additionally scale each element by
    50 with probability 0.01 (outliers);
  * weights B ~ N(0, 0.02) fp32 (0.02 is a standard deviation);
  * contiguous MoE layout: per-expert routed row counts ~ Multinomial(tokens, 1/G each),
    each expert's rows padded up to a multiple of 128; m_indices holds the expert id of
    each row, -1 on padding rows; padding rows of A are zero;
  * masked MoE layout: valid rows per expert ~ uniform on {0, ..., M_max} (inclusive), or on
    {0, ..., max_count} for decode-sized batches;
  * expert FFN weights: gate/up W1 [G, 2I, H] and down W2 [G, H, I], both ~ N(0, 0.02).
"""
from __future__ import annotations

import numpy as np

QBLK = 128

# tensor ids: one independent stream per role
TID_A, TID_B, TID_OUTLIER, TID_ROUTE, TID_MASK = 1, 2, 3, 4, 5
TID_W1, TID_W2 = 6, 7  # expert FFN: gate/up and down projections


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tensor_id])))


def normal(shape, seed: int, tensor_id: int, std: float = 1.0) -> np.ndarray:
    x = rng(seed, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def with_outliers(x: np.ndarray, seed: int, p: float = 0.01, factor: float = 50.0) -> np.ndarray:
    """Each element independently multiplied by `factor` with probability p."""
    hit = rng(seed, TID_OUTLIER).random(size=x.shape) < p
    y = x.copy()
    y[hit] *= np.float32(factor)
    return y


def contiguous_layout(G: int, tokens: int, seed: int, align: int = QBLK):
    """Returns (m_indices [M_total] int32, counts [G]) for the contiguous grouped layout."""
    counts = rng(seed, TID_ROUTE).multinomial(tokens, [1.0 / G] * G)
    padded = [((int(c) + align - 1) // align) * align for c in counts]
    m_indices = np.full(sum(padded), -1, np.int32)
    off = 0
    for g, (c, pc) in enumerate(zip(counts, padded)):
        m_indices[off:off + int(c)] = g
        off += pc
    return m_indices, counts.astype(np.int64)


def masked_layout(G: int, M_max: int, seed: int, max_count: int | None = None) -> np.ndarray:
    """masked_m [G] int32, each uniform on {0..max_count} (default max_count = M_max)."""
    hi = M_max if max_count is None else min(int(max_count), M_max)
    return rng(seed, TID_MASK).integers(0, hi + 1, size=G).astype(np.int32)


# Workload catalogue: shapes and recipes of the five configurations.
WORKLOADS = {
    "tiny": dict(kind="dense", M=128, N=256, K=512, outliers=False),
    "decode_n7168_k2048": dict(kind="dense", M=64, N=7168, K=2048, outliers=False),
    "decode_n24576_k1536": dict(kind="dense", M=64, N=24576, K=1536, outliers=False),
    "prefill_n7168_k18432": dict(kind="dense", M=4096, N=7168, K=18432, outliers=True),
    "prefill_n36864_k7168": dict(kind="dense", M=4096, N=36864, K=7168, outliers=True),
    "contig_g8_n4096_k7168": dict(kind="contiguous", G=8, tokens=8192, N=4096, K=7168),
    "contig_g8_n7168_k2048": dict(kind="contiguous", G=8, tokens=8192, N=7168, K=2048),
    "masked_g32_n4096_k7168": dict(kind="masked", G=32, M_max=256, N=4096, K=7168),
    "masked_g32_n7168_k2048": dict(kind="masked", G=32, M_max=256, N=7168, K=2048),
}


def dense_inputs(M: int, N: int, K: int, seed: int = 0, outliers: bool = False,
                 b_std: float = 0.02):
    """fp32 A [M,K] and B [N,K]."""
    a = normal((M, K), seed, TID_A)
    if outliers:
        a = with_outliers(a, seed)
    b = normal((N, K), seed, TID_B, std=b_std)
    return a, b


def contiguous_inputs(G: int, tokens: int, N: int, K: int, seed: int = 0, b_std: float = 0.02):
    """fp32 A [M_total,K] (zero on padding rows), B [G,N,K], m_indices [M_total]."""
    m_indices, _ = contiguous_layout(G, tokens, seed)
    a = normal((m_indices.size, K), seed, TID_A)
    a[m_indices < 0] = 0.0
    b = normal((G, N, K), seed, TID_B, std=b_std)
    return a, b, m_indices


def masked_inputs(G: int, M_max: int, N: int, K: int, seed: int = 0, b_std: float = 0.02):
    """fp32 A [G,M_max,K], B [G,N,K], masked_m [G]."""
    masked_m = masked_layout(G, M_max, seed)
    a = normal((G, M_max, K), seed, TID_A)
    b = normal((G, N, K), seed, TID_B, std=b_std)
    return a, b, masked_m


def ffn_weights(G: int, H: int, I: int, seed: int = 0, std: float = 0.02):
    """fp32 expert FFN weights: W1 [G,2I,H] (gate rows, then up rows), W2 [G,H,I]."""
    w1 = normal((G, 2 * I, H), seed, TID_W1, std=std)
    w2 = normal((G, H, I), seed, TID_W2, std=std)
    return w1, w2
