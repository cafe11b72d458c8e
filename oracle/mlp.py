"""MLP of a Megatron-style layer: unsharded definition and per-rank shards.

Test infrastructure (see ``oracle``).  All arithmetic in float64.

Layout: row-major, tokens ``T = b*s`` on rows ([L11] section 1 notation;
[LP] O.I), weights stored ``[in, out]`` so that the layer is ``X W`` (the
semantic orientation [L11] section 1 asks for, independent of how a framework
stores ``Linear.weight``).

Sharding ([L11] sections 2-3; [TP1] column split, MLP and attention;
[HJ] TP forward): with TP degree ``t`` and ``f = h_ffn / t``, rank ``i`` owns
columns ``[i f, (i+1) f)`` of ``W1`` (gate and up for SwiGLU) and of ``b1``, and
rows ``[i f, (i+1) f)`` of ``W2``.  The column-parallel first GEMM needs the
replicated input only; the activation acts elementwise on the rank's own
columns; the row-parallel second GEMM yields a full-shape partial ``Z_i``; the
forward all-reduce (operator g of [TP1]) sums the partials, after which the
output bias is added once ([L11] section 3, last paragraph) and dropout
applied ([HJ]; [LP] I.III).

Open points and the readings taken:

* GeLU is the erf form; SwiGLU is ``SiLU(X Wg) * (X Wu)`` (see
  :mod:`oracle.activations`).
* The first layer's bias ``b1`` is column-sharded with ``W1`` and added before
  the activation (the pages only speak of the row-parallel bias).
* [HJ]'s single-card backward writes the activation gradient as ``LZ * W2``
  without a transpose; the shapes only work with ``dH = dY W2^T``, which is
  what is computed here.
"""
from __future__ import annotations

import numpy as np

from . import activations as act_fn
from . import dropout


def _f64(a):
    return None if a is None else np.asarray(a, dtype=np.float64)


def shard_cols(h_ffn: int, t: int, rank: int, unit: int = 1) -> slice:
    """Intermediate columns owned by ``rank``.

    An even split when ``t`` divides ``h_ffn`` ([L11] section 2).  Otherwise
    ([TP1], GQA paragraph: a non-dividing size needs an uneven split or
    padding) the columns are cut into contiguous ranges, in rank order, as
    even as whole ``unit``-column blocks allow: with ``u = h_ffn / unit``
    blocks, every rank gets ``u // t`` blocks and the first ``u % t`` ranks one
    more (a rank may get none).  ``unit`` must divide ``h_ffn``.
    """
    if h_ffn % unit:
        raise ValueError("unit must divide h_ffn")
    u = h_ffn // unit
    base, extra = divmod(u, t)
    start = unit * (rank * base + min(rank, extra))
    return slice(start, start + unit * (base + (1 if rank < extra else 0)))


# ----------------------------------------------------------------------------
# Unsharded definition ([HJ] MLP single-card forward/backward; [TP1] MLP)
# ----------------------------------------------------------------------------

def forward(X, W1, W2, *, act="gelu", Wu=None, b1=None, b2=None, p=0.0, seed=0, rows=None):
    """Out = Dropout(act(X W1 [+b1]) W2 [+ b2]).

    ``rows`` gives the global token indices of the rows of ``X`` (for the
    dropout counter); default ``0..T-1``.  Returns a dict of every
    intermediate.
    """
    X, W1, W2, Wu, b1, b2 = map(_f64, (X, W1, W2, Wu, b1, b2))
    out = {}
    if act == "gelu":
        A = X @ W1
        if b1 is not None:
            A = A + b1
        H = act_fn.gelu(A)
        out["A"] = A
    elif act == "swiglu":
        G = X @ W1
        U = X @ Wu
        H = act_fn.silu(G) * U
        out["G"], out["U"] = G, U
    else:
        raise ValueError(act)
    Y = H @ W2
    if b2 is not None:
        Y = Y + b2
    out["H"], out["Y"] = H, Y
    out["Out"] = dropout.apply(Y, seed, p, rows)
    return out


def backward(dOut, X, W1, W2, *, act="gelu", Wu=None, b1=None, b2=None, p=0.0, seed=0, rows=None):
    """Gradients of ``L = <dOut, Out>`` for the unsharded MLP.

    Dropout backward multiplies by the same mask and ``1/(1-p)`` ([HJ] MLP,
    single-card backward); the output weight's gradient is ``H^T dY`` and the
    activation's input gradient ``dY W2^T`` ([HJ]; [L11] section 2,
    row-parallel layer); the first layer mirrors it ([L11] section 2,
    column-parallel layer).
    """
    fw = forward(X, W1, W2, act=act, Wu=Wu, b1=b1, b2=b2, p=p, seed=seed, rows=rows)
    X, W1, W2, Wu = map(_f64, (X, W1, W2, Wu))
    dY = dropout.apply(dOut, seed, p, rows)
    g = {"dY": dY, "db2": dY.sum(axis=0), "dW2": fw["H"].T @ dY}
    dH = dY @ W2.T
    if act == "gelu":
        dA = dH * act_fn.gelu_grad(fw["A"])
        g["dA"] = dA
        g["db1"] = dA.sum(axis=0)
        g["dW1"] = X.T @ dA
        g["dX"] = dA @ W1.T
    else:
        G, U = fw["G"], fw["U"]
        dU = dH * act_fn.silu(G)
        dG = dH * U * act_fn.silu_grad(G)
        g["dG"], g["dU"] = dG, dU
        g["dW1"] = X.T @ dG
        g["dWu"] = X.T @ dU
        g["dX"] = dG @ W1.T + dU @ Wu.T
    g["fwd"] = fw
    return g


# ----------------------------------------------------------------------------
# One rank's shard ([L11] sections 2-3; [HJ] TP forward/backward)
# ----------------------------------------------------------------------------

def shard_forward(X, W1_i, W2_i, *, act="gelu", Wu_i=None, b1_i=None):
    """Column-parallel GEMM + local activation, then row-parallel GEMM.

    Returns ``saved`` (``A_i`` for GeLU, ``G_i``/``U_i`` for SwiGLU), ``H_i`` and the
    partial ``Z_i = H_i W2_i`` (no output bias: it is added after the sum).
    """
    X, W1_i, W2_i, Wu_i, b1_i = map(_f64, (X, W1_i, W2_i, Wu_i, b1_i))
    res = {}
    if act == "gelu":
        A = X @ W1_i
        if b1_i is not None:
            A = A + b1_i
        H = act_fn.gelu(A)
        res["A"] = A
    else:
        G = X @ W1_i
        U = X @ Wu_i
        H = act_fn.silu(G) * U
        res["G"], res["U"] = G, U
    res["H"] = H
    res["Z"] = H @ W2_i
    return res


def sum_partials(partials, bias=None, p=0.0, seed=0, rows=None):
    """Emulated all-reduce: ``Dropout(sum_i P_i + bias)``, summed in rank order.

    The bias is added exactly once, after the sum ([L11] section 3); dropout
    follows the all-reduce ([LP] I.III; [HJ]).
    """
    acc = np.zeros_like(np.asarray(partials[0], dtype=np.float64))
    for P in partials:
        acc = acc + np.asarray(P, dtype=np.float64)
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float64)
    return dropout.apply(acc, seed, p, rows)


def shard_backward(dOut, X, W1_i, W2_i, saved, H_i, *, act="gelu", Wu_i=None, p=0.0, seed=0, rows=None):
    """One rank's backward.

    dOut is replicated (after the forward all-reduce every rank holds the same
    output, so its gradient is the same everywhere: [HJ] TP backward).
    ``dY`` undoes dropout; ``dW2_i = H_i^T dY`` and ``dH_i = dY W2_i^T`` are local
    (row-parallel layer, [L11] section 2); the activation backward is local
    on the rank's columns; ``dW1_i = X^T dA_i`` is local and ``dX_i = dA_i W1_i^T``
    is a partial that the backward all-reduce (operator f of [TP1]) sums.
    For SwiGLU the gate and up contributions are added before that sum
    ([L11] section 3).
    """
    X, W1_i, W2_i, Wu_i, H_i = map(_f64, (X, W1_i, W2_i, Wu_i, H_i))
    dY = dropout.apply(dOut, seed, p, rows)
    g = {"dY": dY, "db2": dY.sum(axis=0), "dW2": H_i.T @ dY}
    dH = dY @ W2_i.T
    if act == "gelu":
        dA = dH * act_fn.gelu_grad(_f64(saved["A"]))
        g["dA"] = dA
        g["db1"] = dA.sum(axis=0)
        g["dW1"] = X.T @ dA
        g["dX"] = dA @ W1_i.T
    else:
        G, U = _f64(saved["G"]), _f64(saved["U"])
        dU = dH * act_fn.silu(G)
        dG = dH * U * act_fn.silu_grad(G)
        g["dG"], g["dU"] = dG, dU
        g["dW1"] = X.T @ dG
        g["dWu"] = X.T @ dU
        g["dX"] = dG @ W1_i.T + dU @ Wu_i.T
    return g


def shard_step(dOut, X, W1_i, W2_i, *, act="gelu", Wu_i=None, b1_i=None, p=0.0, seed=0, rows=None):
    """Forward then backward of one shard, with the saved tensors taken from the forward."""
    fw = shard_forward(X, W1_i, W2_i, act=act, Wu_i=Wu_i, b1_i=b1_i)
    bw = shard_backward(dOut, X, W1_i, W2_i, fw, fw["H"], act=act, Wu_i=Wu_i, p=p, seed=seed, rows=rows)
    return fw, bw


def column_sample(dOut, X, W1_i, W2_i, cols, *, act="gelu", Wu_i=None, b1_i=None, p=0.0, seed=0):
    """Weight gradients of a subset of a shard's intermediate columns.

    Restricting a shard to some of its intermediate columns is itself a valid
    column split ([L11] section 2: every output column of the first GEMM is
    complete on the rank that owns it), so ``dW1_i[:, cols]``, ``dW2_i[cols, :]``
    and ``db1_i[cols]`` are exactly the gradients of the sub-shard made of
    those columns.  Costs O(T h |cols|).
    """
    cols = np.asarray(cols)
    sub = lambda W, ax: None if W is None else np.take(W, cols, axis=ax)
    return shard_step(dOut, X, sub(W1_i, 1), sub(W2_i, 0), act=act, Wu_i=sub(Wu_i, 1),
                      b1_i=sub(b1_i, 0), p=p, seed=seed)
