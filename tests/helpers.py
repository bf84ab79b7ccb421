"""Shared helpers for the GPU parity tests: run the same seeded inputs through the HIP path
(via the C-ABI binding) and through the CPU oracle, each side quantising on its own."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import synth


def say(msg: str) -> None:
    """Name the case before a GPU step (flushed, so a fault still leaves the name)."""
    print("[case] " + msg, flush=True)
    sys.stdout.flush()


def dev() -> torch.device:
    return torch.device("cuda:0")


def to_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to(dev())


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_values(t: torch.Tensor) -> np.ndarray:
    # rows a kernel leaves unwritten may hold signalling-NaN patterns; their cast is not an error
    with np.errstate(invalid="ignore"):
        return t.float().cpu().numpy().astype(np.float64)


def gpu_cast_tokens(dg, a_f32: np.ndarray, ue8m0: bool = False):
    """Per-token cast on the GPU of [M,K] or [G,M,K]; returns device (q, sf) with sf in the
    library's K-block-major layout ([K/128,M] or [G,K/128,M])."""
    return dg.cast_fp8_per_token(to_dev(a_f32), ue8m0=ue8m0)


def kmajor(s: np.ndarray) -> np.ndarray:
    """Oracle per-token scales [..., M, K/128] in the library's layout [..., K/128, M]."""
    return np.ascontiguousarray(np.swapaxes(s, -1, -2))


def gpu_cast_blocks(dg, w_f32: np.ndarray, ue8m0: bool = False):
    return dg.cast_fp8_per_block(to_dev(w_f32), ue8m0=ue8m0)


def oracle_cast_tokens(a_f32: np.ndarray):
    shp = a_f32.shape
    q, s = oracle.cast_per_token(a_f32.reshape(-1, shp[-1]))
    return q.reshape(shp), s.reshape(*shp[:-1], shp[-1] // 128)


def assert_same_bytes(gpu_q: torch.Tensor, cpu_q: np.ndarray, what: str) -> None:
    g = gpu_q.cpu().numpy()
    if not np.array_equal(g, cpu_q):
        bad = np.argwhere(g != cpu_q)
        raise AssertionError("%s: %d byte mismatches, first at %s (gpu %#x, oracle %#x)" % (
            what, len(bad), tuple(bad[0]), g[tuple(bad[0])], cpu_q[tuple(bad[0])]))


def assert_same_bits(gpu_s: torch.Tensor, cpu_s: np.ndarray, what: str) -> None:
    g = gpu_s.cpu().numpy().astype(np.float32)
    if not np.array_equal(g.view(np.uint32), cpu_s.astype(np.float32).view(np.uint32)):
        bad = np.argwhere(g.view(np.uint32) != cpu_s.astype(np.float32).view(np.uint32))
        raise AssertionError("%s: %d scale mismatches, first at %s (gpu %r, oracle %r)" % (
            what, len(bad), tuple(bad[0]), g[tuple(bad[0])], cpu_s[tuple(bad[0])]))


def assert_close(y: np.ndarray, R: np.ndarray, what: str, mask=None) -> dict:
    res = oracle.compare(y, R, mask)
    assert res["ok"], "%s: %s" % (what, res)
    return res


def quantised_dense(dg, M, N, K, seed=0, outliers=False, ue8m0=False):
    """Seeded fp32 inputs, quantised by both sides; byte/bit equality of the casts asserted.
    Returns (device q/s tensors, oracle q/s arrays)."""
    a, b = synth.dense_inputs(M, N, K, seed, outliers)
    qa_d, sa_d = gpu_cast_tokens(dg, a, ue8m0)
    qb_d, sb_d = gpu_cast_blocks(dg, b, ue8m0)
    qa, sa = oracle.cast_per_token(a, pow2=ue8m0)
    qb, sb = oracle.cast_per_block(b, pow2=ue8m0)
    assert_same_bytes(qa_d, qa, "A cast %dx%d" % (M, K))
    assert_same_bits(sa_d, kmajor(sa), "A scales %dx%d" % (M, K))
    assert_same_bytes(qb_d, qb, "B cast %dx%d" % (N, K))
    assert_same_bits(sb_d, sb, "B scales %dx%d" % (N, K))
    return (qa_d, sa_d, qb_d, sb_d), (qa, sa, qb, sb)
