"""Algorithmic work of the path, the numerators of every throughput figure.

[HJ] counts a GEMM of shapes ``(m, k) x (k, n)`` as ``2 m k n`` FLOPs and
neglects activations, dropout and the all-reduce's additions (MLP,
single-card forward and backward; TP forward); backward is twice forward.
The attention core is credited only with the (query, key) pairs the causal
mask leaves visible: ``QK^T`` and ``PV`` are ``2 d`` FLOPs per pair each.
"""
from __future__ import annotations


def causal_pairs(s: int, causal: bool = True) -> int:
    """Visible (query, key) pairs of one sequence and head: keys at or before
    the query under the causal mask (``s (s + 1) / 2``), all ``s^2`` without it."""
    return s * (s + 1) // 2 if causal else s * s


def gemm(m: int, k: int, n: int) -> int:
    return 2 * m * k * n


def mlp_shard(tokens: int, h: int, f: int, act: str) -> int:
    """Per-rank MLP forward + backward: ``12 T h f`` (GeLU) or ``18 T h f`` (SwiGLU)."""
    n_first = 1 if act == "gelu" else 2
    fwd = n_first * gemm(tokens, h, f) + gemm(tokens, f, h)
    return 3 * fwd


def attn_core(b: int, s: int, q: int, d: int, causal: bool = True) -> int:
    """Forward attention core of ``q`` local query heads: ``4 d`` per visible pair."""
    return 4 * d * b * q * causal_pairs(s, causal)


def attn_shard_fwd(b: int, s: int, h: int, q: int, kv: int, d: int, causal: bool = True) -> int:
    """Per-rank attention forward: QKV GEMM, core and output projection."""
    T = b * s
    return gemm(T, h, (q + 2 * kv) * d) + attn_core(b, s, q, d, causal) + gemm(T, q * d, h)
