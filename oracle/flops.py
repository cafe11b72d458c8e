"""Algorithmic FLOP counts (test infrastructure; see ``oracle``).

[HJ] counts a GEMM of shapes ``(m, k) x (k, n)`` as ``2 m k n`` FLOPs and
neglects the activation, dropout and the all-reduce's additions (MLP,
single-card forward and backward; TP forward).  Its totals for a GeLU MLP
with ``d_ff = 4 d``: forward ``16 B S d^2``, backward twice that, and ``1/n``
of each per rank under ``n``-way TP.  For attention (MHA, no causal saving):
forward ``8 B S d^2 + 4 B S^2 d``, backward ``16 B S d^2 + 8 B S^2 d``
(Attention, single-card backward): every projection GEMM and both core
products get an input-gradient and a weight-gradient (or second-operand)
product; recomputing the scores is not counted.
"""


def gemm(m: int, k: int, n: int) -> int:
    return 2 * m * k * n


def mlp_shard(tokens: int, h: int, f: int, act: str) -> dict:
    """Per-rank FLOPs of the MLP shard with intermediate width ``f``.

    Forward: one (GeLU) or two (SwiGLU: gate and up) ``[T,h]x[h,f]`` GEMMs and
    the ``[T,f]x[f,h]`` GEMM.  Backward: two GEMMs per forward GEMM (the input
    and the weight gradient), so twice the forward.
    """
    n_first = 1 if act == "gelu" else 2
    fwd = n_first * gemm(tokens, h, f) + gemm(tokens, f, h)
    bwd = 2 * fwd
    return dict(fwd=fwd, bwd=bwd, total=fwd + bwd)


def attention_pairs(s: int, causal: bool = True) -> int:
    """(query, key) pairs of one sequence and head that the mask leaves
    visible: every key at or before the query (``1 + 2 + ... + s``) under the
    causal mask, all ``s^2`` without it."""
    return s * (s + 1) // 2 if causal else s * s


def attention_shard_fwd(b: int, s: int, h: int, q: int, kv: int, d: int, causal: bool = True) -> dict:
    """Per-rank forward FLOPs: QKV GEMM, core (QK^T and PV over the key/query
    pairs actually computed) and the output projection."""
    T = b * s
    pairs = attention_pairs(s, causal)
    qkv = gemm(T, h, (q + 2 * kv) * d)
    core = 2 * (2 * d) * b * q * pairs
    out = gemm(T, q * d, h)
    return dict(qkv=qkv, core=core, out=out, total=qkv + core + out)


def attention_shard_bwd(b: int, s: int, h: int, q: int, kv: int, d: int, causal: bool = True) -> dict:
    """Per-rank backward FLOPs: twice each forward term ([HJ] Attention,
    single-card backward) -- ``dWo`` and ``dO`` for the output projection,
    ``dP``/``dV`` and ``dQ``/``dK`` for the core over the computed pairs,
    ``dWqkv`` and ``dX`` for the QKV projection."""
    f = attention_shard_fwd(b, s, h, q, kv, d, causal)
    return dict(qkv=2 * f["qkv"], core=2 * f["core"], out=2 * f["out"], total=2 * f["total"])
