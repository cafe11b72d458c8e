"""CPU oracle for one tensor-parallel rank's share of a Megatron-style layer.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
float64 reference that the GPU library is checked against.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it; the
GPU library never calls it and shares no code with it.

Everything is computed in float64 with numpy (a matmul is the only library
primitive used for the dense contractions; scipy's ``erf`` and ``expit`` give
the activation functions).  Inputs are whatever numbers the GPU sees (fp32 or
bf16-valued), promoted to float64; intermediates are never rounded.

Pages cited (by title and section):

* [L11]  grasp.study Lesson 11, "张量并行线性层分片与前反向通信量计算"
         (tensor-parallel linear sharding and fwd/bwd communication volume),
         sections 1-6.
* [LP]   cnblogs "ラブパラ" (a survey of parallelisms): O.I Notation,
         O.II Collective Communication, I.O Activations, I.III Tensor
         Parallelism, II.II Communication Approaches, II.III Computational
         Details, II.V Agnostic to Implementation, III.III Block Layout
         Contract.
* [HJ]   hjcheng0602.cn "tensorparallel/tp": MLP (single-card forward and
         backward, TP forward and backward) and Attention sections.
* [TP1]  "Tensor Parallelism张量并行（一）": row split, column split, MLP and
         attention, the f and g operators, communication cost.

Modules:

* :mod:`oracle.activations` - GeLU (erf form), SiLU and their derivatives.
* :mod:`oracle.dropout`     - the counter-based dropout mask.
* :mod:`oracle.mlp`         - unsharded and per-shard MLP forward/backward,
                              and the emulated all-reduce (sum of partials).
* :mod:`oracle.attention`   - causal GQA attention, unsharded and per shard,
                              forward and backward.
* :mod:`oracle.sequence_parallel` - the closing all-reduce with a fused residual
                              add, and its Megatron-SP reduce-scatter / all-gather split.
* :mod:`oracle.comm`        - all-reduce count and bytes per layer.
* :mod:`oracle.flops`       - algorithmic FLOP counts.

Parity status: every function here is pinned by a test in
``tests/test_oracle_*.py`` except where its docstring says "parity unpinned".
"""
from . import activations, dropout, mlp, attention, sequence_parallel, comm, flops  # noqa: F401
