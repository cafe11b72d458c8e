"""One tensor-parallel rank's share of a Megatron-style Transformer layer on
AMD MI355X (gfx950).

The computation lives in ``libtpshard.so`` (HIP kernels behind the C ABI of
``include/tp_shard.h``); :mod:`attention_column_gemm_amd.binding` exposes its
functions under the same names, and :mod:`attention_column_gemm_amd.shard`
wraps them into per-rank forward/backward calls that allocate their outputs
with torch (device memory and streams only).
:mod:`attention_column_gemm_amd.inputs` generates the seeded synthetic
workloads.  The library is loaded on first use; build it with
``python -m attention_column_gemm_amd.build``.
"""
from .binding import (TP_BF16, TP_F32, TP_GELU, TP_SWIGLU, TPError, attn_desc, mlp_desc,  # noqa: F401
                      tp_attn_shard_fwd, tp_comm_bytes, tp_mlp_shard_bwd, tp_mlp_shard_fwd, tp_sum_partials)
