"""Seeded synthetic inputs for the tensor-parallel layer shard workloads.

This module holds only data generation: shapes, seeds, normal draws and the
rounding of draws to bfloat16 so that the GPU path and the CPU oracle see the
very same numbers.  It holds none of the layer's arithmetic.

Workloads (one per named configuration, sizes as in the page notation:
``T = b*s`` tokens, hidden size ``h``, intermediate size ``h_ffn``, TP degree
``t``, per-rank intermediate width ``f = h_ffn / t``):

====  ======================  ====  =====  ======  ==  =====================
id    family                  T     h      h_ffn   t   dtype
====  ======================  ====  =====  ======  ==  =====================
1     GeLU MLP                64    128    512     2   fp32
2     GPT-style GeLU MLP      2048  1024   4096    4   bf16, dropout p=0.1
3     Llama SwiGLU MLP        4096  4096   11008   8   bf16
4     GQA attention shard     4096  4096   -       8   bf16 (32 q / 8 kv, d=128)
5     full layer (attn+MLP)   8192  8192   28672   8   bf16 (64 q / 8 kv, d=128)
====  ======================  ====  =====  ======  ==  =====================

Every tensor is drawn from numpy's PCG64 seeded with
``SeedSequence([1000*cfg + tensor_id, rank])``; a sharded weight is drawn one
rank slice at a time and the unsharded weight is the concatenation of the
slices in rank order, so any subset of ranks can be produced without the rest.
Tensor ids: X=1, W1/Wg=2, Wu=3, W2/Wdown=4, Wqkv=5 (Wq, Wk, Wv: 51, 52, 53),
Wo=9, b1=6, b2=7, dOut=8; the dropout seed is ``1000*cfg + 99``.

Initialisation follows the configurations: ``N(0, 1/fan_in)`` is read as a
variance (std ``fan_in**-0.5``); ``N(0, 0.02)`` and ``N(0, 0.01)`` as standard
deviations.  Configurations that state no distribution inherit from their
family (2 from 1, 4 and 5 from 3).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

from . import flops as F

TENSOR_IDS = dict(X=1, W1=2, Wu=3, W2=4, Wq=51, Wk=52, Wv=53, Wo=9, b1=6, b2=7, dOut=8)


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) >> 16
    out = (bits.astype(np.uint32) << 16).view(np.float32)
    return out.reshape(a.shape)


def _draw(cfg: int, name: str, rank: int, shape, std: float, bf16: bool) -> np.ndarray:
    ss = np.random.SeedSequence([1000 * cfg + TENSOR_IDS[name], rank])
    g = np.random.Generator(np.random.PCG64(ss))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return round_to_bf16(x) if bf16 else x


@dataclasses.dataclass(frozen=True)
class MLPConfig:
    cfg: int
    b: int
    s: int
    h: int
    h_ffn: int
    t: int
    act: str              # "gelu" or "swiglu"
    dtype: str            # "fp32" or "bf16"
    p_drop: float
    bias: bool
    std_w1: Optional[float]   # None: 1/sqrt(fan_in)
    std_w2: Optional[float]
    std_b: float = 0.01

    @property
    def tokens(self) -> int:
        return self.b * self.s

    @property
    def f(self) -> int:
        return self.h_ffn // self.t

    @property
    def seed(self) -> int:
        return 1000 * self.cfg + 99

    @property
    def bf16(self) -> bool:
        return self.dtype == "bf16"

    def flops_per_rank(self) -> int:
        """fwd+bwd algorithmic FLOPs of one rank's shard: 12*T*h*f (GeLU) or 18*T*h*f (SwiGLU)."""
        return F.mlp_shard(self.tokens, self.h, self.f, self.act)


@dataclasses.dataclass(frozen=True)
class AttnConfig:
    cfg: int
    b: int
    s: int
    h: int
    n_q: int
    n_kv: int
    d: int
    t: int
    std_w: float = 0.02

    @property
    def tokens(self) -> int:
        return self.b * self.s

    @property
    def q(self) -> int:
        return self.n_q // self.t

    @property
    def kv(self) -> int:
        return self.n_kv // self.t

    def flops_per_rank(self) -> int:
        """Forward FLOPs of one rank: QKV and output GEMMs plus the causal core (unmasked pairs only)."""
        return F.attn_shard_fwd(self.b, self.s, self.h, self.q, self.kv, self.d, causal=True)

    def flops_bwd_per_rank(self) -> int:
        """Backward FLOPs of one rank: twice each forward term (input- and weight-gradient products)."""
        return 2 * self.flops_per_rank()


MLP_CONFIGS = {
    1: MLPConfig(1, 1, 64, 128, 512, 2, "gelu", "fp32", 0.0, True, None, None),
    2: MLPConfig(2, 4, 512, 1024, 4096, 4, "gelu", "bf16", 0.1, True, None, None),
    3: MLPConfig(3, 2, 2048, 4096, 11008, 8, "swiglu", "bf16", 0.0, False, 0.02, 0.02),
    5: MLPConfig(5, 4, 2048, 8192, 28672, 8, "swiglu", "bf16", 0.0, False, 0.02, 0.02),
}

ATTN_CONFIGS = {
    4: AttnConfig(4, 2, 2048, 4096, 32, 8, 128, 8),
    5: AttnConfig(5, 4, 2048, 8192, 64, 8, 128, 8),
}


def custom_mlp(cfg: int, b: int, s: int, h: int, h_ffn: int, t: int, act: str,
               dtype: str = "bf16", p_drop: float = 0.0, bias: bool = False) -> MLPConfig:
    """A small workload of the same family, for tests that must run in seconds."""
    std = None if act == "gelu" else 0.02
    return MLPConfig(cfg, b, s, h, h_ffn, t, act, dtype, p_drop, bias, std, std)


def custom_attn(cfg: int, b: int, s: int, h: int, n_q: int, n_kv: int, d: int, t: int) -> AttnConfig:
    return AttnConfig(cfg, b, s, h, n_q, n_kv, d, t)


def mlp_activation(c: MLPConfig, rows: Optional[np.ndarray] = None):
    """X [T,h] and the upstream gradient dOut [T,h] (both replicated across ranks)."""
    X = _draw(c.cfg, "X", 0, (c.tokens, c.h), 1.0, c.bf16)
    dOut = _draw(c.cfg, "dOut", 0, (c.tokens, c.h), 1.0, c.bf16)
    if rows is not None:
        X, dOut = X[rows], dOut[rows]
    return X, dOut


def mlp_rank_weights(c: MLPConfig, rank: int) -> dict:
    """Rank ``rank``'s shard: W1_i [h,f] (gate for SwiGLU), Wu_i [h,f] or None,
    W2_i [f,h], b1_i [f] or None; plus the replicated b2 [h] or None."""
    std1 = c.std_w1 if c.std_w1 is not None else 1.0 / math.sqrt(c.h)
    std2 = c.std_w2 if c.std_w2 is not None else 1.0 / math.sqrt(c.h_ffn)
    f = c.f
    out = dict(
        W1=_draw(c.cfg, "W1", rank, (c.h, f), std1, c.bf16),
        Wu=_draw(c.cfg, "Wu", rank, (c.h, f), std1, c.bf16) if c.act == "swiglu" else None,
        W2=_draw(c.cfg, "W2", rank, (f, c.h), std2, c.bf16),
        b1=_draw(c.cfg, "b1", rank, (f,), c.std_b, c.bf16) if c.bias else None,
        b2=_draw(c.cfg, "b2", 0, (c.h,), c.std_b, c.bf16) if c.bias else None,
    )
    return out


def mlp_full_weights(c: MLPConfig) -> dict:
    """Unsharded weights: rank slices concatenated in rank order."""
    shards = [mlp_rank_weights(c, r) for r in range(c.t)]
    cat = lambda k, ax: None if shards[0][k] is None else np.concatenate([s[k] for s in shards], axis=ax)
    return dict(W1=cat("W1", 1), Wu=cat("Wu", 1), W2=cat("W2", 0), b1=cat("b1", 0), b2=shards[0]["b2"])


def attn_activation(c: AttnConfig) -> np.ndarray:
    return _draw(c.cfg, "X", 0, (c.tokens, c.h), 1.0, True)


def attn_upstream_grad(c: AttnConfig) -> np.ndarray:
    """dZ [T,h]: gradient of the attention sublayer's output, the same on every rank."""
    return _draw(c.cfg, "dOut", 0, (c.tokens, c.h), 1.0, True)


def attn_rank_weights(c: AttnConfig, rank: int) -> dict:
    """Wqkv_i [h, (q+2kv)d] with columns [Q heads | K heads | V heads] (head-major,
    d each) and Wo_i [q*d, h]."""
    d = c.d
    Wq = _draw(c.cfg, "Wq", rank, (c.h, c.q * d), c.std_w, True)
    Wk = _draw(c.cfg, "Wk", rank, (c.h, c.kv * d), c.std_w, True)
    Wv = _draw(c.cfg, "Wv", rank, (c.h, c.kv * d), c.std_w, True)
    Wo = _draw(c.cfg, "Wo", rank, (c.q * d, c.h), c.std_w, True)
    return dict(Wqkv=np.ascontiguousarray(np.concatenate([Wq, Wk, Wv], axis=1)), Wo=Wo)
