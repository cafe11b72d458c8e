"""Causal grouped-query self-attention, unsharded and per TP rank, forward and backward.

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


def shard_heads(n_q: int, n_kv: int, t: int, rank: int):
    """The heads rank ``rank`` owns: ``(q, kv, q0, kv0)`` -- its number of query
    and KV heads and the first of each.

    A rank holds whole GQA groups, the query heads with their KV head ([L11]
    section 4; [LP] I.III).  ``n_kv >= t``: the ``n_kv`` groups are dealt out in
    rank order, the first ``n_kv % t`` ranks taking one more ([TP1], GQA
    paragraph: a non-dividing count needs an uneven split).  ``n_kv < t``: each
    KV head is replicated on ``t / n_kv`` consecutive ranks, which split its
    query heads evenly ([LP] III.III: when the split is not complete several
    cards share one KV projection, a parameter replica); this needs ``t`` to be
    a multiple of ``n_kv`` and the group size a multiple of ``t / n_kv``.
    """
    if n_q % n_kv:
        raise ValueError("n_q must divide by n_kv")
    group = n_q // n_kv
    if n_kv >= t:
        base, extra = divmod(n_kv, t)
        kv = base + (1 if rank < extra else 0)
        kv0 = rank * base + min(rank, extra)
        return kv * group, kv, kv0 * group, kv0
    if t % n_kv or group % (t // n_kv):
        raise ValueError("replicated KV heads need t % n_kv == 0 and (n_q/n_kv) % (t/n_kv) == 0")
    r = t // n_kv
    g, sub = divmod(rank, r)
    q = group // r
    return q, 1, g * group + sub * q, g


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


def core_backward(Q, K, V, dO, *, b, s, n_q, n_kv, d, causal=True):
    """Gradients of the attention core with respect to ``Q, K, V``.

    [HJ] Attention, single-card backward: with ``P`` the row softmax of the
    scaled, masked scores, ``dV = P^T dO`` and ``dP = dO V^T``; the softmax
    backward of a row ``y = softmax(x)`` is ``dx = y * (dy - <dy, y>)``, so
    ``dS = P * (dP - rowsum(P * dP))``; then ``dQ = dS K / sqrt(d)`` and
    ``dK = dS^T Q / sqrt(d)``.  [LP] I.O: the scores are recomputed here, not
    stored.  With grouped-query attention the gradients of a KV head add up
    over the query heads that read it (the chain rule through the shared use).
    Returns ``dQ [T, n_q d]``, ``dK, dV [T, n_kv d]``.
    """
    Q, K, V, dO = _f64(Q), _f64(K), _f64(V), _f64(dO)
    if n_q % n_kv:
        raise ValueError("n_q must divide by n_kv")
    group = n_q // n_kv
    T = b * s
    dQ = np.zeros((T, n_q * d))
    dK = np.zeros((T, n_kv * d))
    dV = np.zeros((T, n_kv * d))
    scale = 1.0 / np.sqrt(d)
    allowed = np.tril(np.ones((s, s), dtype=bool)) if causal else np.ones((s, s), dtype=bool)
    for beta in range(b):
        rows = slice(beta * s, (beta + 1) * s)
        for j in range(n_q):
            g = j // group
            q = Q[rows, j * d:(j + 1) * d]
            k = K[rows, g * d:(g + 1) * d]
            v = V[rows, g * d:(g + 1) * d]
            do = dO[rows, j * d:(j + 1) * d]
            S = np.where(allowed, (q @ k.T) * scale, -np.inf)
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            dP = do @ v.T
            dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            dQ[rows, j * d:(j + 1) * d] = (dS @ k) * scale
            dK[rows, g * d:(g + 1) * d] += (dS.T @ q) * scale
            dV[rows, g * d:(g + 1) * d] += P.T @ do
    return dQ, dK, dV


def backward(dZ, X, Wq, Wk, Wv, Wo, *, b, s, n_q, n_kv, d, causal=True):
    """Unsharded attention sublayer backward for the upstream gradient ``dZ``.

    [HJ] Attention, single-card backward, in its order: ``dWo = O^T dZ``,
    ``dO = dZ Wo^T``; the core's ``dQ, dK, dV``; then the projection weights
    ``dWq = X^T dQ`` (likewise K, V) and the input gradient
    ``dX = dQ Wq^T + dK Wk^T + dV Wv^T``.
    """
    X, dZ = _f64(X), _f64(dZ)
    Wq, Wk, Wv, Wo = _f64(Wq), _f64(Wk), _f64(Wv), _f64(Wo)
    f = forward(X, Wq, Wk, Wv, Wo, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d, causal=causal)
    dWo = f["O"].T @ dZ
    dO = dZ @ Wo.T
    dQ, dK, dV = core_backward(f["Q"], f["K"], f["V"], dO, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d, causal=causal)
    return dict(dO=dO, dQ=dQ, dK=dK, dV=dV, dWq=X.T @ dQ, dWk=X.T @ dK, dWv=X.T @ dV, dWo=dWo,
                dX=dQ @ Wq.T + dK @ Wk.T + dV @ Wv.T)


def shard_backward(dZ, X, Wqkv_i, Wo_i, *, b, s, q, kv, d, causal=True):
    """One rank's attention backward.

    The upstream gradient ``dZ`` of the sublayer output is the same on every
    rank (the backward of the forward all-reduce is the identity; [TP1]
    operators f and g).  The rank forms ``dWo_i = O_i^T dZ`` and
    ``dO_i = dZ Wo_i^T`` for its heads, its heads' ``dQ, dK, dV`` packed like
    ``QKV_i`` (``[Q heads | K heads | V heads]``), ``dWqkv_i = X^T dQKV_i`` and
    the partial input gradient ``dX_i = dQKV_i Wqkv_i^T``, which the backward
    all-reduce at the QKV input sums over ranks ([TP1], attention's
    communication; [L11] section 4).
    """
    X, dZ, Wqkv_i, Wo_i = _f64(X), _f64(dZ), _f64(Wqkv_i), _f64(Wo_i)
    f = shard_forward(X, Wqkv_i, Wo_i, b=b, s=s, q=q, kv=kv, d=d, causal=causal)
    QKV = f["QKV"]
    dO = dZ @ Wo_i.T
    dQ, dK, dV = core_backward(QKV[:, :q * d], QKV[:, q * d:(q + kv) * d], QKV[:, (q + kv) * d:], dO,
                               b=b, s=s, n_q=q, n_kv=kv, d=d, causal=causal)
    dQKV = np.concatenate([dQ, dK, dV], axis=1)
    return dict(QKV=QKV, O=f["O"], lse=f["lse"], dO=dO, dQKV=dQKV, dWo=f["O"].T @ dZ,
                dWqkv=X.T @ dQKV, dX=dQKV @ Wqkv_i.T)
