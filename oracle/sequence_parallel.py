"""The closing all-reduce of a TP block with a fused residual add, and its
Megatron-SP split into reduce-scatter and all-gather.

Test infrastructure (see ``oracle``).  All arithmetic in float64.

[LP] "ラブパラ" II.III Computational Details lists, among the token-wise fused
operators, a fused bias + dropout + residual add and a fused all-reduce +
residual add.  Read together with the MLP's output path (the partials summed
by operator g, the bias added once, dropout after the sum; [TP1], [L11]
section 3, [HJ]), the closing step of a block is::

    Out = R + Dropout_{p,seed}(sum_i Z_i + b)

with ``R`` the block's residual input, added once, after dropout (the
residual path itself is never dropped).

[LP] III.III Block Layout Contract: the all-reduce at the end of a TP block
can be split into a reduce-scatter of ``(b, s, H)`` to a ``1/t`` token slice
per rank, the token-wise operations (bias, dropout, residual) run on that
slice only, and an all-gather at the next block's entry restores ``(b, s,
H)``.  Rank ``r`` owns token rows ``[r T/t, (r+1) T/t)``; the dropout mask of
an element is that of its position in the full ``[T, H]`` tensor, so the
split changes nothing in the result (reading: the rows are split in rank
order and ``T`` must divide by ``t``).

The same passage puts the token-wise norm between the two halves: after the
reduce-scatter each rank normalises its own token slice (its name there is
layernorm; [LP] II.III lists fused layernorm / RMSnorm among the token-wise
operators, and [L11] section 3 hands the MLP input gradient back to an
RMSNorm in the Llama layout).  Readings taken: the norm is the next
sublayer's pre-norm, applied to the block output ``Out`` (the new residual
stream) of each of the rank's rows; both outputs are kept, ``Out`` for the
residual path and ``norm(Out)`` for the all-gather into the next sublayer.

* RMSNorm: ``y = x / sqrt(mean(x^2) + eps) * gamma``
* LayerNorm: ``y = (x - mean(x)) / sqrt(var(x) + eps) * gamma + beta``, with
  the biased variance ``mean((x - mean(x))^2)``

over the ``H`` features of one token; ``gamma`` (and ``beta``) are
replicated ``[H]`` vectors, ``None`` meaning ones (zeros).
"""
from __future__ import annotations

import numpy as np

from . import dropout


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def sum_partials_residual(partials, bias=None, p=0.0, seed=0, residual=None, rows=None):
    """``residual + Dropout(sum_i P_i + bias)``, partials summed in rank order.

    ``rows``: the global row indices of the given (full-width) rows, for the
    dropout mask; ``None`` means all rows from 0.
    """
    acc = np.zeros_like(_f64(partials[0]))
    for P in partials:
        acc = acc + _f64(P)
    if bias is not None:
        acc = acc + _f64(bias)
    out = dropout.apply(acc, seed, p, rows)
    if residual is not None:
        out = out + _f64(residual)
    return out


def slice_rows(T: int, t: int, rank: int) -> np.ndarray:
    """Token rows of rank ``rank`` after the reduce-scatter."""
    if T % t:
        raise ValueError("T must divide by t")
    n = T // t
    return np.arange(rank * n, (rank + 1) * n)


def reduce_scatter(partials, t, rank, bias=None, p=0.0, seed=0, residual_r=None):
    """Rank ``rank``'s slice of the block output: only its rows of each partial
    are summed, then bias, dropout (global indices) and its residual slice."""
    rows = slice_rows(_f64(partials[0]).shape[0], t, rank)
    return sum_partials_residual([_f64(P)[rows] for P in partials], bias, p, seed, residual_r, rows=rows)


def all_gather(slices):
    """The full tensor from the ranks' slices, in rank order."""
    return np.concatenate([_f64(s) for s in slices], axis=0)


def rms_norm(x, gamma=None, eps=1e-6):
    """Token-wise RMSNorm over the last axis."""
    x = _f64(x)
    y = x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)
    return y if gamma is None else y * _f64(gamma)


def layer_norm(x, gamma=None, beta=None, eps=1e-5):
    """Token-wise LayerNorm over the last axis (biased variance)."""
    x = _f64(x)
    mu = np.mean(x, axis=-1, keepdims=True)
    var = np.mean((x - mu) ** 2, axis=-1, keepdims=True)
    y = (x - mu) / np.sqrt(var + eps)
    if gamma is not None:
        y = y * _f64(gamma)
    if beta is not None:
        y = y + _f64(beta)
    return y


def norm(x, kind, gamma=None, beta=None, eps=1e-6):
    if kind == "rms":
        if beta is not None:
            raise ValueError("RMSNorm has no shift")
        return rms_norm(x, gamma, eps)
    if kind == "layer":
        return layer_norm(x, gamma, beta, eps)
    raise ValueError(f"unknown norm {kind!r}")


def sum_partials_norm(partials, bias=None, p=0.0, seed=0, residual=None, kind="rms", gamma=None, beta=None,
                      eps=1e-6, rows=None):
    """``Out = residual + Dropout(sum_i P_i + bias)`` and ``norm(Out)``."""
    out = sum_partials_residual(partials, bias, p, seed, residual, rows)
    return out, norm(out, kind, gamma, beta, eps)


def reduce_scatter_norm(partials, t, rank, bias=None, p=0.0, seed=0, residual_r=None, kind="rms", gamma=None,
                        beta=None, eps=1e-6):
    """Rank ``rank``'s slice of the block output and the norm of that slice."""
    out = reduce_scatter(partials, t, rank, bias, p, seed, residual_r)
    return out, norm(out, kind, gamma, beta, eps)
