"""Seeded synthetic inputs for the quantized-decode workloads.

Only random draws and storage-format casts live here; none of the method's
arithmetic (no quantizer, no packing rule, no product).  Both the HIP path and
the CPU oracle are fed from these arrays.

Generator: NumPy PCG64 (``numpy.random.default_rng(seed)``).  Multi-M
workloads draw activations once at the largest M and slice the first rows, so
the weights are shared across M.

INT4 AWQ weight words are drawn as uniform 32-bit integers: each of the eight
4-bit fields of a uniform word is itself uniform on 0..15 and independent of
the others, which is exactly "codes uniform on 0..15, packed eight to a word",
whatever the nibble order.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEEDS = {"int4_gemv_512": 1, "kv_cache": 2, "w8a8_qkv": 3, "w8a8_down": 4, "int4_qkv": 5}


def rng(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 storage bits (uint16) through torch's CPU cast (RNE)."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


# --------------------------------------------------------------------------
# KV cache: fp32 [num_tokens, head_dim], N(0,1) with ~1% outliers scaled x10.

def kv_cache(num_tokens: int = 32768, head_dim: int = 128, seed: int = 2,
             outlier_frac: float = 0.01, outlier_gain: float = 10.0) -> np.ndarray:
    g = rng(seed)
    x = g.normal(0.0, 1.0, (num_tokens, head_dim)).astype(np.float32)
    mask = g.random((num_tokens, head_dim)) < outlier_frac
    x[mask] *= np.float32(outlier_gain)
    return x


def attn_decode(num_tokens: int = 4096, num_kv_heads: int = 8, num_q_heads: int = 32, head_dim: int = 128,
                seed: int = 11):
    """One decode token's queries and the cache it reads: (q fp32 [Hq, D],
    k fp32 [T, Hkv, D], v fp32 [T, Hkv, D]); K and V rows have the KV cache's
    value distribution (4096 tokens x 8 heads = the 32768 x 128 cache), q is
    N(0, 1)."""
    g = rng(seed)
    q = g.normal(0.0, 1.0, (num_q_heads, head_dim)).astype(np.float32)
    rows = num_tokens * num_kv_heads
    k = kv_cache(rows, head_dim, seed=seed + 1).reshape(num_tokens, num_kv_heads, head_dim)
    v = kv_cache(rows, head_dim, seed=seed + 2).reshape(num_tokens, num_kv_heads, head_dim)
    return q, k, v


# --------------------------------------------------------------------------
# W8A8: bf16 activations N(0,1); fp32 weights N(0, 0.02) to be quantized.

@dataclass
class W8A8Inputs:
    x_bf16: np.ndarray              # uint16 [M_max, K]
    up_bf16: np.ndarray | None      # uint16 [M_max, K] (SwiGLU variant) or None
    weights: list                   # fp32 [n_i, K] per segment


def w8a8(m_max: int, k: int, seg_n, seed: int, with_up: bool = False,
         w_std: float = 0.02) -> W8A8Inputs:
    g = rng(seed)
    x = to_bf16_bits(g.normal(0.0, 1.0, (m_max, k)).astype(np.float32))
    w = g.normal(0.0, w_std, (int(sum(seg_n)), k)).astype(np.float32)
    up = to_bf16_bits(g.normal(0.0, 1.0, (m_max, k)).astype(np.float32)) if with_up else None
    segs, off = [], 0
    for n in seg_n:
        segs.append(w[off:off + n])
        off += n
    return W8A8Inputs(x, up, segs)


def w8a8_qkv(seed: int = 3) -> W8A8Inputs:
    """Per-row fused QKV: M up to 32, K=4096, segments 4096 + 1024 + 1024."""
    return w8a8(32, 4096, (4096, 1024, 1024), seed)


def w8a8_down(seed: int = 4, with_up: bool = False) -> W8A8Inputs:
    """128x128 block-scaled down projection: M up to 256, K=14336, N=4096."""
    return w8a8(256, 14336, (4096,), seed, with_up=with_up)


# --------------------------------------------------------------------------
# INT4 AWQ: fp32 activations N(0,1); per projection uniform words, scales
# U(0.001, 0.02) and zeros U(0, 15) per (group, column).

@dataclass
class AwqProj:
    qweight: np.ndarray   # uint32 [K, n/8]
    scales: np.ndarray    # fp32 [K/gs, n]
    zeros: np.ndarray     # fp32 [K/gs, n]


def awq_proj(g: np.random.Generator, k: int, n: int, group_size: int) -> AwqProj:
    qw = g.integers(0, 2 ** 32, (k, n // 8), dtype=np.uint64).astype(np.uint32)
    s = g.uniform(0.001, 0.02, (k // group_size, n)).astype(np.float32)
    z = g.uniform(0.0, 15.0, (k // group_size, n)).astype(np.float32)
    return AwqProj(qw, s, z)


def int4_awq(m_max: int, k: int, ns, group_size: int, seed: int):
    """Returns (x fp32 [m_max, K], [AwqProj per projection])."""
    g = rng(seed)
    x = g.normal(0.0, 1.0, (m_max, k)).astype(np.float32)
    projs = [awq_proj(g, k, n, group_size) for n in ns]
    return x, projs


def int4_gemv_512(seed: int = 1):
    """Single projection: M=1, K=512, N=512, group 128."""
    return int4_awq(1, 512, (512,), 128, seed)


def int4_qkv(seed: int = 5):
    """Fused Q/K/V at an 8B-class shape: M up to 128, K=4096, 4096/1024/1024."""
    return int4_awq(128, 4096, (4096, 1024, 1024), 128, seed)
