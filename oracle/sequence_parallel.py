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
