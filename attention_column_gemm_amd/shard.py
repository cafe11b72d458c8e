"""Per-rank shard objects over the C ABI, with torch-allocated buffers.

Torch provides device memory and the stream; every arithmetic step is a call
into libtpshard.  Buffers are allocated once per object so that repeated
steps (the benchmark) allocate nothing.
"""
from __future__ import annotations

import numpy as np

from . import binding as B
from . import validate as V


def _torch():
    import torch
    if not torch.cuda.is_available():
        raise RuntimeError("a HIP GPU is required: libtpshard runs only on gfx950")
    return torch


def to_device(a, dtype: str, device="cuda"):
    """numpy array (fp32 holding bf16-exact values for bf16) -> device tensor of the storage type."""
    torch = _torch()
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    t = t.to(device)
    return t.to(torch.bfloat16) if dtype == "bf16" else t


def to_numpy(t):
    return None if t is None else t.detach().float().cpu().numpy()


class MLPShard:
    """One rank's MLP shard: weights and activation buffers on the device."""

    def __init__(self, tokens, h, h_ffn, t, rank, act="gelu", dtype="bf16", device="cuda"):
        torch = _torch()
        self.torch = torch
        self.tokens, self.h, self.h_ffn, self.t, self.rank = tokens, h, h_ffn, t, rank
        self.f, self.col0 = B.tp_mlp_shard_cols(h_ffn, t, rank, B.TP_BF16 if dtype == "bf16" else B.TP_F32)
        self.act, self.dtype = act, dtype
        self.tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.desc = B.mlp_desc(tokens, h, h_ffn, t, rank, B.TP_BF16 if dtype == "bf16" else B.TP_F32,
                               B.TP_GELU if act == "gelu" else B.TP_SWIGLU)
        nsav = 1 if act == "gelu" else 2
        T, f = tokens, self.f
        e = lambda *shape, dt=None: torch.empty(*shape, dtype=dt or self.tdt, device=device)
        self.saved = e(nsav, T, f)
        self.H = e(T, f)
        self.Z = e(T, h)
        self.dY = e(T, h)
        self.dA = e(nsav, T, f)
        self.dW1 = e(nsav, h, f, dt=torch.float32)
        self.dW2 = e(f, h, dt=torch.float32)
        self.db1 = e(f, dt=torch.float32) if act == "gelu" else None
        self.db2 = e(h, dt=torch.float32)
        self.dX = e(T, h)
        self.device = device

    def load(self, X, W1, Wu, b1, W2, dOut=None):
        """Upload numpy inputs (the seeded generator's output)."""
        d = lambda a: to_device(a, self.dtype, self.device)
        self.X, self.W1, self.Wu, self.b1, self.W2 = d(X), d(W1), d(Wu), d(b1), d(W2)
        self.dOut = d(dOut)
        return self

    def forward(self, stream=None):
        B.tp_mlp_shard_fwd(self.desc, self.X, self.W1, self.Wu, self.b1, self.W2, self.saved, self.H, self.Z, stream)
        return self.Z

    def backward(self, p_drop=0.0, seed=0, want_db2=True, want_db1=True, write_dY=None, stream=None):
        """``write_dY``: None -> dY is written only when p_drop > 0 (else dOut is used directly)."""
        if write_dY is None:
            write_dY = p_drop > 0
        B.tp_mlp_shard_bwd(self.desc, self.dOut, p_drop, seed, self.X, self.W1, self.Wu, self.W2, self.saved, self.H,
                           self.dY if write_dY else None, self.db2 if want_db2 else None, self.dA, self.dW1,
                           self.db1 if (want_db1 and self.act == "gelu") else None, self.dW2, self.dX, stream)
        return self.dX


class AttnShard:
    """One rank's attention shard (forward and backward)."""

    def __init__(self, b, s, h, n_q, n_kv, d, t, rank, causal=True, device="cuda"):
        torch = _torch()
        self.b, self.s, self.h, self.n_q, self.n_kv, self.d, self.t, self.rank = b, s, h, n_q, n_kv, d, t, rank
        self.q, self.kv, self.q0, self.kv0 = B.tp_attn_shard_heads(n_q, n_kv, t, rank)
        self.desc = B.attn_desc(b, s, h, n_q, n_kv, d, t, rank, B.TP_BF16, 1 if causal else 0)
        T = b * s
        e = lambda *shape, dt=torch.bfloat16: torch.empty(*shape, dtype=dt, device=device)
        self.QKV = e(T, (self.q + 2 * self.kv) * d)
        self.O = e(T, self.q * d)
        self.lse = e(b, self.q, s, dt=torch.float32)
        self.Z = e(T, h)
        self.device = device

    def load(self, X, Wqkv, Wo):
        self.X, self.Wqkv, self.Wo = (to_device(a, "bf16", self.device) for a in (X, Wqkv, Wo))
        return self

    def forward(self, want_lse=True, stream=None):
        B.tp_attn_shard_fwd(self.desc, self.X, self.Wqkv, self.Wo, self.QKV, self.O,
                            self.lse if want_lse else None, self.Z, stream)
        return self.Z

    def alloc_backward(self):
        """Buffers of the backward pass (allocated once, reused by every call)."""
        torch = _torch()
        if getattr(self, "dQKV", None) is None:
            T, h, d = self.b * self.s, self.h, self.d
            e = lambda *shape, dt=torch.bfloat16: torch.empty(*shape, dtype=dt, device=self.device)
            self.dO = e(T, self.q * d)
            self.stats = e(self.b, self.q, self.s, 2, dt=torch.float32)
            self.dQKV = e(T, (self.q + 2 * self.kv) * d)
            self.dWqkv = e(h, (self.q + 2 * self.kv) * d, dt=torch.float32)
            self.dWo = e(self.q * d, h, dt=torch.float32)
            self.dX = e(T, h)
        return self

    def backward(self, dZ, stream=None):
        """Gradients for the upstream gradient ``dZ`` [T, h] (needs a forward with lse)."""
        self.alloc_backward()
        V.like("dZ", dZ, (self.b * self.s, self.h), self.X.dtype, self.X.device, optional=False)
        B.tp_attn_shard_bwd(self.desc, dZ, self.X, self.Wqkv, self.Wo, self.QKV, self.O, self.lse, self.dO,
                            self.stats, self.dQKV, self.dWqkv, self.dWo, self.dX, stream)
        return self.dX


def _rows_cols(shape):
    if len(shape) < 1:
        raise ValueError("partials and slices need at least one dimension (rows)")
    return shape[0], int(np.prod(shape[1:], dtype=np.int64)) if len(shape) > 1 else 1


def sum_partials(partials, bias=None, p_drop=0.0, seed=0, out=None, stream=None, residual=None):
    """Emulated all-reduce of same-shaped device tensors (rank order), with the
    residual add fused when ``residual`` is given."""
    torch = _torch()
    shape, code, dev = V.group("partials", partials)
    rows, cols = _rows_cols(shape)
    dt = partials[0].dtype
    V.vector("bias", bias, cols, dt, dev)
    V.like("residual", residual, shape, dt, dev)
    if out is None:
        out = torch.empty_like(partials[0])
    V.like("out", out, shape, dt, dev)
    if residual is None:
        B.tp_sum_partials(rows, cols, len(partials), code, list(partials), bias, p_drop, seed, out, stream)
    else:
        B.tp_sum_partials_residual(rows, cols, len(partials), code, list(partials), bias, p_drop, seed, residual,
                                   out, stream)
    return out


def reduce_scatter(partials, rank, bias=None, p_drop=0.0, seed=0, residual_r=None, out=None, stream=None):
    """Rank ``rank``'s token slice of the emulated all-reduce (Megatron-SP first half)."""
    torch = _torch()
    shape, code, dev = V.group("partials", partials)
    rows, cols = _rows_cols(shape)
    t = len(partials)
    if rows % t:
        raise ValueError(f"rows {rows} do not divide over t = {t} ranks")
    dt = partials[0].dtype
    sl = (rows // t,) + tuple(shape[1:])
    V.vector("bias", bias, cols, dt, dev)
    V.like("residual_r", residual_r, sl, dt, dev)
    if out is None:
        out = torch.empty(sl, dtype=dt, device=dev)
    V.like("out", out, sl, dt, dev)
    B.tp_reduce_scatter(rows, cols, t, rank, code, list(partials), bias, p_drop, seed, residual_r, out, stream)
    return out


def all_gather(slices, out=None, stream=None):
    """The full tensor from the ranks' token slices (Megatron-SP second half)."""
    torch = _torch()
    shape, code, dev = V.group("slices", slices)
    rows, cols = _rows_cols(shape)
    full = (rows * len(slices),) + tuple(shape[1:])
    if out is None:
        out = torch.empty(full, dtype=slices[0].dtype, device=dev)
    V.like("out", out, full, slices[0].dtype, dev)
    B.tp_all_gather(rows, cols, len(slices), code, list(slices), out, stream)
    return out


_NORMS = {"rms": B.TP_NORM_RMS, "layer": B.TP_NORM_LAYER}


def sum_partials_norm(partials, norm="rms", gamma=None, beta=None, eps=1e-6, bias=None, p_drop=0.0, seed=0,
                      residual=None, out=None, normed=None, stream=None):
    """Emulated all-reduce with the residual add and the next sublayer's
    token-wise norm fused: returns (out, normed)."""
    torch = _torch()
    shape, code, dev = V.group("partials", partials)
    rows, cols = _rows_cols(shape)
    dt = partials[0].dtype
    for name, vec in (("bias", bias), ("gamma", gamma), ("beta", beta)):
        V.vector(name, vec, cols, dt, dev)
    V.like("residual", residual, shape, dt, dev)
    out = torch.empty_like(partials[0]) if out is None else out
    normed = torch.empty_like(partials[0]) if normed is None else normed
    V.like("out", out, shape, dt, dev)
    V.like("normed", normed, shape, dt, dev)
    B.tp_sum_partials_norm(rows, cols, len(partials), code, list(partials), bias, p_drop, seed, residual,
                           _NORMS[norm], gamma, beta, eps, out, normed, stream)
    return out, normed


def reduce_scatter_norm(partials, rank, norm="rms", gamma=None, beta=None, eps=1e-6, bias=None, p_drop=0.0, seed=0,
                        residual_r=None, out=None, normed=None, stream=None):
    """Rank ``rank``'s token slice of the block output and its norm
    (Megatron-SP: reduce-scatter, then the token-wise norm on the slice)."""
    torch = _torch()
    shape, code, dev = V.group("partials", partials)
    rows, cols = _rows_cols(shape)
    t = len(partials)
    if rows % t:
        raise ValueError(f"rows {rows} do not divide over t = {t} ranks")
    dt = partials[0].dtype
    sl = (rows // t,) + tuple(shape[1:])
    for name, vec in (("bias", bias), ("gamma", gamma), ("beta", beta)):
        V.vector(name, vec, cols, dt, dev)
    V.like("residual_r", residual_r, sl, dt, dev)
    out = torch.empty(sl, dtype=dt, device=dev) if out is None else out
    normed = torch.empty(sl, dtype=dt, device=dev) if normed is None else normed
    V.like("out", out, sl, dt, dev)
    V.like("normed", normed, sl, dt, dev)
    B.tp_reduce_scatter_norm(rows, cols, t, rank, code, list(partials), bias, p_drop, seed, residual_r,
                             _NORMS[norm], gamma, beta, eps, out, normed, stream)
    return out, normed
