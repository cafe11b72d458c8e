"""GPU parity of uneven shards: FFN widths that t does not divide (including
ranks with no columns), GQA groups dealt out unevenly, and KV heads
replicated over several ranks.  Full weights are drawn once and cut by the
library's split; the oracle cuts them by its own rule (the two rules are
checked equal on the CPU), and the per-rank results must also add up to the
unsharded layer."""
import numpy as np
import pytest

from attention_column_gemm_amd import inputs as I
from oracle import attention as OA
from oracle import mlp as O
from parity import TOL, banner, check, need_gpu

pytestmark = pytest.mark.gpu
BF = TOL["bf16"]


def _np(t):
    return t.detach().float().cpu().numpy()


MLP_CASES = {
    # name: (b, s, h, h_ffn, t, act, p, bias)
    "gelu_1000_t3": (2, 40, 256, 1000, 3, "gelu", 0.1, True),
    "swiglu_1000_t3": (1, 96, 264, 1000, 3, "swiglu", 0.0, False),
    "swiglu_64_t16_empty_ranks": (1, 48, 128, 64, 16, "swiglu", 0.0, False),
}


@pytest.mark.parametrize("name", list(MLP_CASES))
def test_uneven_mlp_shards(name):
    torch = need_gpu()
    b, s, h, hf, t, act, p, bias = MLP_CASES[name]
    banner(f"uneven mlp {name}")
    from attention_column_gemm_amd.shard import MLPShard, sum_partials, to_device
    c1 = I.custom_mlp(300 + len(name), b, s, h, hf, 1, act, "bf16", p_drop=p, bias=bias)
    X, dOut = I.mlp_activation(c1)
    w = I.mlp_full_weights(c1)
    gZ, gdX, Zs, dXs = [], [], [], []
    for r in range(t):
        sh = MLPShard(c1.tokens, h, hf, t, r, act=act, dtype="bf16")
        c = O.shard_cols(hf, t, r, 8)
        assert (sh.col0, sh.col0 + sh.f) == (c.start, c.stop)
        cut = lambda a, ax: None if a is None else np.ascontiguousarray(a[:, c] if ax == 1 else a[c])
        W1, Wu, W2, b1 = cut(w["W1"], 1), cut(w["Wu"], 1), cut(w["W2"], 0), cut(w["b1"], 0)
        sh.load(X, W1, Wu, b1, W2, dOut).forward()
        sh.backward(p, c1.seed, want_db2=False, want_db1=bias)
        torch.cuda.synchronize()
        fw, bw = O.shard_step(dOut, X, W1, W2, act=act, Wu_i=Wu, b1_i=b1, p=p, seed=c1.seed)
        check(f"r{r}.Z_i (f={sh.f})", _np(sh.Z), fw["Z"], BF)
        check(f"r{r}.dX_i", _np(sh.dX), bw["dX"], BF)
        if sh.f:
            check(f"r{r}.H_i", _np(sh.H), fw["H"], BF)
            check(f"r{r}.dW2_i", _np(sh.dW2), bw["dW2"], BF)
            check(f"r{r}.dW1_i", _np(sh.dW1[0]), bw["dW1"], BF)
        else:
            assert not np.any(_np(sh.Z)) and not np.any(_np(sh.dX))
        gZ.append(sh.Z)
        gdX.append(sh.dX)
        Zs.append(fw["Z"])
        dXs.append(bw["dX"])
    Z = sum_partials(gZ)
    dX = sum_partials(gdX)
    torch.cuda.synchronize()
    full = O.forward(X, w["W1"], w["W2"], act=act, Wu=w["Wu"], b1=w["b1"])
    fb = O.backward(dOut, X, w["W1"], w["W2"], act=act, Wu=w["Wu"], b1=w["b1"], p=p, seed=c1.seed)
    check("sum Z_i = unsharded H W2", _np(Z), full["H"] @ np.asarray(w["W2"], np.float64), BF)
    check("sum dX_i = unsharded dX", _np(dX), fb["dX"], BF)


ATTN_CASES = {
    # name: (b, s, h, n_q, n_kv, d, t)
    "uneven_groups_d128": (2, 72, 192, 12, 3, 128, 2),
    "uneven_groups_d64_t3": (1, 100, 128, 10, 5, 64, 3),
    "replicated_kv_d128": (2, 64, 128, 8, 2, 128, 4),
    "replicated_kv_d64_t8": (1, 80, 128, 16, 2, 64, 8),
}


@pytest.mark.parametrize("name", list(ATTN_CASES))
def test_uneven_and_replicated_attention_shards(name):
    torch = need_gpu()
    b, s, h, n_q, n_kv, d, t = ATTN_CASES[name]
    banner(f"uneven attention {name}")
    from attention_column_gemm_amd.shard import AttnShard, sum_partials, to_device
    c1 = I.custom_attn(400 + len(name), b, s, h, n_q, n_kv, d, 1)
    X = I.attn_activation(c1)
    w = I.attn_rank_weights(c1, 0)
    dZ = I.attn_upstream_grad(c1)
    Wq, Wk, Wv = w["Wqkv"][:, :n_q * d], w["Wqkv"][:, n_q * d:(n_q + n_kv) * d], w["Wqkv"][:, (n_q + n_kv) * d:]
    gZ, gdX = [], []
    dWk, dWv = np.zeros(Wk.shape), np.zeros(Wv.shape)
    fb = OA.backward(dZ, X, Wq, Wk, Wv, w["Wo"], b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)
    for r in range(t):
        q, kv, q0, kv0 = OA.shard_heads(n_q, n_kv, t, r)
        sh = AttnShard(b, s, h, n_q, n_kv, d, t, r)
        assert (sh.q, sh.kv, sh.q0, sh.kv0) == (q, kv, q0, kv0)
        cq, ck = slice(q0 * d, (q0 + q) * d), slice(kv0 * d, (kv0 + kv) * d)
        Wqkv = np.ascontiguousarray(np.concatenate([Wq[:, cq], Wk[:, ck], Wv[:, ck]], 1))
        Wo = np.ascontiguousarray(w["Wo"][cq])
        sh.load(X, Wqkv, Wo).forward()
        sh.backward(to_device(dZ, "bf16"))
        torch.cuda.synchronize()
        ref = OA.shard_backward(dZ, X, Wqkv, Wo, b=b, s=s, q=q, kv=kv, d=d)
        check(f"r{r}.O_i (q={q} kv={kv})", _np(sh.O), ref["O"], BF)
        check(f"r{r}.dQKV_i", _np(sh.dQKV), ref["dQKV"], BF)
        check(f"r{r}.dWqkv_i", _np(sh.dWqkv), ref["dWqkv"], BF)
        check(f"r{r}.dWo_i", _np(sh.dWo), ref["dWo"], BF)
        check(f"r{r}.dX_i", _np(sh.dX), ref["dX"], BF)
        dWk[:, ck] += _np(sh.dWqkv)[:, q * d:(q + kv) * d]
        dWv[:, ck] += _np(sh.dWqkv)[:, (q + kv) * d:]
        gZ.append(sh.Z)
        gdX.append(sh.dX)
    Z = sum_partials(gZ)
    dX = sum_partials(gdX)
    torch.cuda.synchronize()
    full = OA.forward(X, Wq, Wk, Wv, w["Wo"], b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)
    check("sum Z_i = unsharded Z", _np(Z), full["Z"], BF)
    check("sum dX_i = unsharded dX", _np(dX), fb["dX"], BF)
    check("replicas' dWk add up", dWk, fb["dWk"], BF)
    check("replicas' dWv add up", dWv, fb["dWv"], BF)
