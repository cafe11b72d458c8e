"""The shard calls replayed from a captured HIP graph.

The library allocates nothing and issues no memset: every call is a fixed
sequence of kernel launches on the caller's stream, so a caller can capture a
whole step once and replay it.  Each replay must reproduce the eager results
bit for bit (the kernels are deterministic), with eager work of the program's
own between the replays.
"""
import pytest

from attention_column_gemm_amd import inputs as I
from parity import banner, need_gpu

pytestmark = pytest.mark.gpu


def _replay_and_compare(torch, run, outputs, scribble):
    """Eager reference, capture, then three replays each preceded by eager
    work that overwrites the outputs."""
    run()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outputs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for replay in range(3):
        scribble()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(ref, outputs)):
            assert torch.equal(a, b), f"replay {replay}: output {i} differs from the eager run"


MLP_CASES = {
    # GeLU with both biases and dropout, two ranks, both all-reduces
    "gelu_bias_dropout_t2": I.custom_mlp(301, 2, 200, 512, 2048, 2, "gelu", "bf16", p_drop=0.1, bias=True),
    # SwiGLU whose column GEMM splits its last round of tiles in two K halves
    # (fp32 partial tiles kept in Z_i's memory until the row GEMM overwrites it)
    "swiglu_split_tail_t1": I.custom_mlp(303, 2, 2000, 1056, 2104, 1, "swiglu", "bf16"),
}


@pytest.mark.parametrize("name", list(MLP_CASES))
def test_mlp_step_replays_from_a_graph(name):
    torch = need_gpu()
    from attention_column_gemm_amd.shard import MLPShard, sum_partials, to_device
    c = MLP_CASES[name]
    banner(f"graph mlp {name} T={c.tokens} h={c.h} h_ffn={c.h_ffn} t={c.t} p={c.p_drop}")
    X, dOut = I.mlp_activation(c)
    shards = []
    for rank in range(c.t):
        w = I.mlp_rank_weights(c, rank)
        shards.append(MLPShard(c.tokens, c.h, c.h_ffn, c.t, rank, act=c.act, dtype=c.dtype).load(
            X, w["W1"], w["Wu"], w["b1"], w["W2"], dOut))
    b2 = I.mlp_rank_weights(c, 0)["b2"]
    b2 = None if b2 is None else to_device(b2, c.dtype)
    out = torch.empty(c.tokens, c.h, dtype=torch.bfloat16, device="cuda")
    dx = torch.empty(c.tokens, c.h, dtype=torch.bfloat16, device="cuda")

    def run():
        for sh in shards:
            sh.forward()
            sh.backward(c.p_drop, c.seed)
        sum_partials([sh.Z for sh in shards], b2, c.p_drop, c.seed, out=out)
        sum_partials([sh.dX for sh in shards], out=dx)

    outputs = [out, dx] + [t for sh in shards
                           for t in (sh.saved, sh.H, sh.Z, sh.dY if c.p_drop > 0 else None,  # dY: written with dropout only
                                     sh.db2, sh.dA, sh.dW1, sh.db1, sh.dW2, sh.dX)]
    outputs = [t for t in outputs if t is not None]

    def scribble():
        for t in outputs:
            t.fill_(3.0)
        shards[0].forward()  # an eager call of the library between replays

    _replay_and_compare(torch, run, outputs, scribble)


def test_attention_step_replays_from_a_graph():
    """Causal attention with h = 2048, where the forward's, dK/dV's and dQ's
    splits of their heavier blocks all apply."""
    torch = need_gpu()
    from attention_column_gemm_amd.shard import AttnShard, to_device
    c = I.custom_attn(302, 1, 256, 2048, 4, 1, 128, 1)
    banner(f"graph attention b={c.b} s={c.s} h={c.h} n_q={c.n_q} n_kv={c.n_kv} d={c.d}")
    X = I.attn_activation(c)
    w = I.attn_rank_weights(c, 0)
    sh = AttnShard(c.b, c.s, c.h, c.n_q, c.n_kv, c.d, c.t, 0).load(X, w["Wqkv"], w["Wo"]).alloc_backward()
    dZ = to_device(I.attn_upstream_grad(c), "bf16")

    def run():
        sh.forward()
        sh.backward(dZ)

    outputs = [sh.QKV, sh.O, sh.lse, sh.Z, sh.dO, sh.dQKV, sh.dWqkv, sh.dWo, sh.dX]

    def scribble():
        for t in outputs:
            t.fill_(-2.0)

    _replay_and_compare(torch, run, outputs, scribble)
