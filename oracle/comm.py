"""Tensor-parallel all-reduce count and bytes per layer (test infrastructure).

[L11] section 5 (formulas lost in the page's extraction; the prose survives)
and [TP1] "communication cost": a classic Transformer layer does four
activation all-reduces per microbatch -- one after the attention output
projection and one after the MLP down projection in forward (operator g),
one at the attention QKV input and one at the MLP input in backward
(operator f).  One all-reduce carries a ``[b*s, h]`` activation of ``delta``
bytes per element ([LP] O.I: fp32 4, bf16 2), so its logical payload is
``b*s*h*delta``.  A ring all-reduce is a reduce-scatter followed by an
all-gather ([L11] section 5; [LP] O.II), each moving ``(t-1)/t`` of the
payload per rank, so a rank sends ``2 (t-1)/t`` payloads; [L11] warns not to
report the logical size as the bytes on the wire, so both are returned.
[LP] II.II drops the ``(t-1)/t`` factor and quotes ``2 delta b S H`` per
all-reduce and ``8 delta b S H`` per layer, the large-``t`` limit of the same
count.
"""
from __future__ import annotations

from fractions import Fraction


def comm_bytes(tokens: int, h: int, t: int, delta: int) -> dict:
    if tokens < 0 or h < 0 or t < 1 or delta < 1:
        raise ValueError("bad arguments")
    payload = tokens * h * delta
    ring = Fraction(2 * (t - 1), t) * payload
    n_fwd, n_bwd = 2, 2
    n = n_fwd + n_bwd
    return dict(n_allreduce_fwd=n_fwd, n_allreduce_bwd=n_bwd,
                payload_bytes=payload, ring_bytes_per_rank=float(ring),
                layer_payload_bytes=n * payload, layer_ring_bytes_per_rank=float(n * ring),
                ring_exact=ring)
