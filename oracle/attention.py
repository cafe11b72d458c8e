"""Causal grouped-query self-attention, unsharded and per TP rank (forward).

Test infrastructure (see ``oracle``).  All arithmetic in float64.

What is computed ([HJ] Attention, single-card forward; [L11] section 4;
[LP] I.III): ``Q = X Wq``, ``K = X Wk``, ``V = X Wv``; per sequence and head
``S = Q K^T / sqrt(d)``; row softmax; ``O = P V``; heads concatenated
head-major; ``Z = O Wo``.

Readings taken where the pages are silent:

* Scale ``1/sqrt(d)`` ([LP] II.III lists the fused "divide by the dim scale"
  with mask and softmax; [HJ] omits it).
* Causal mask inside each sequence: key position ``<=`` query position.
  The diagonal is always visible, so no row is empty.
* Rows are tokens ``r = beta*s + sigma``; attention never crosses sequences.
* Grouped-query attention: global query head ``j`` reads KV head
  ``j // (n_q / n_kv)``; a rank owns whole groups ([L11] section 4; [LP]
  I.III), i.e. query heads ``[i q, (i+1) q)`` and KV heads ``[i kv, (i+1) kv)``.
* A rank's QKV weight has columns ``[Q heads | K heads | V heads]``, d each.
* No RoPE, attention dropout or projection biases.
* ``lse`` is the natural-log sum of ``exp`` of the scaled, masked scores of a
  row (the per-row statistic a flash-style kernel keeps).
"""
from __future__ import annotations

import numpy as np


def _f64(a):
    return np.asarray(a, dtype=np.float64)


def core(Q, K, V, *, b, s, n_q, n_kv, d, causal=True):
    """Attention core on head-major packed ``Q [T, n_q d]``, ``K, V [T, n_kv d]``.

    Returns ``O [T, n_q d]`` and ``lse [b, n_q, s]``.
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    if n_q % n_kv:
        raise ValueError("n_q must divide by n_kv")
    group = n_q // n_kv
    T = b * s
    O = np.zeros((T, n_q * d))
    lse = np.zeros((b, n_q, s))
    scale = 1.0 / np.sqrt(d)
    allowed = np.tril(np.ones((s, s), dtype=bool)) if causal else np.ones((s, s), dtype=bool)
    for beta in range(b):
        rows = slice(beta * s, (beta + 1) * s)
        for j in range(n_q):
            g = j // group
            q = Q[rows, j * d:(j + 1) * d]
            k = K[rows, g * d:(g + 1) * d]
            v = V[rows, g * d:(g + 1) * d]
            S = (q @ k.T) * scale
            S = np.where(allowed, S, -np.inf)
            m = S.max(axis=1, keepdims=True)
            E = np.exp(S - m)
            den = E.sum(axis=1, keepdims=True)
            P = E / den
            O[rows, j * d:(j + 1) * d] = P @ v
            lse[beta, j, :] = (m + np.log(den))[:, 0]
    return O, lse


def forward(X, Wq, Wk, Wv, Wo, *, b, s, n_q, n_kv, d, causal=True):
    """Unsharded attention sublayer; returns Q, K, V, O, lse, Z."""
    X = _f64(X)
    Q, K, V = X @ _f64(Wq), X @ _f64(Wk), X @ _f64(Wv)
    O, lse = core(Q, K, V, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d, causal=causal)
    return dict(Q=Q, K=K, V=V, O=O, lse=lse, Z=O @ _f64(Wo))


def shard_forward(X, Wqkv_i, Wo_i, *, b, s, q, kv, d, causal=True):
    """One rank: its QKV column shard, local heads' attention, row-parallel out-projection.

    ``Z_i`` is a partial of the full output; the forward all-reduce sums them
    ([L11] section 4).
    """
    X = _f64(X)
    QKV = X @ _f64(Wqkv_i)
    Q = QKV[:, :q * d]
    K = QKV[:, q * d:(q + kv) * d]
    V = QKV[:, (q + kv) * d:(q + 2 * kv) * d]
    O, lse = core(Q, K, V, b=b, s=s, n_q=q, n_kv=kv, d=d, causal=causal)
    return dict(QKV=QKV, O=O, lse=lse, Z=O @ _f64(Wo_i))


def shard_forward_rows(X, Wqkv_i, Wo_i, rows, *, b, s, q, kv, d):
    """Sampled rows of one rank's causal attention output.

    A query row needs the keys and values of its own sequence up to its own
    position only, so each sampled row is computed from that prefix.
    Returns ``O[rows]``, ``lse[:, rows]`` (as ``[q, len(rows)]``) and ``Z[rows]``.
    """
    X = _f64(X)
    Wqkv_i = _f64(Wqkv_i)
    rows = np.asarray(rows)
    group = q // kv
    scale = 1.0 / np.sqrt(d)
    O = np.zeros((len(rows), q * d))
    lse = np.zeros((q, len(rows)))
    Wq = Wqkv_i[:, :q * d]
    Wk = Wqkv_i[:, q * d:(q + kv) * d]
    Wv = Wqkv_i[:, (q + kv) * d:]
    cache = {}
    for n, r in enumerate(rows):
        beta, sigma = divmod(int(r), s)
        if beta not in cache:
            xs = X[beta * s:(beta + 1) * s]
            cache = {beta: (xs @ Wk, xs @ Wv)}
        K, V = cache[beta]
        qrow = X[r] @ Wq
        for j in range(q):
            g = j // group
            k = K[:sigma + 1, g * d:(g + 1) * d]
            v = V[:sigma + 1, g * d:(g + 1) * d]
            sc = (k @ qrow[j * d:(j + 1) * d]) * scale
            m = sc.max()
            e = np.exp(sc - m)
            O[n, j * d:(j + 1) * d] = (e @ v) / e.sum()
            lse[j, n] = m + np.log(e.sum())
    return dict(O=O, lse=lse, Z=O @ _f64(Wo_i))
