"""GPU parity of the attention shard forward (QKV GEMM, causal GQA flash
attention, row-parallel output projection) against the float64 oracle."""
import numpy as np
import pytest

from attention_column_gemm_amd import inputs as I
from oracle import attention as OA
from oracle import mlp as O
from parity import TOL, banner, check, edge_indices, need_gpu

pytestmark = pytest.mark.gpu
BF = TOL["bf16"]


def _np(t):
    return t.detach().float().cpu().numpy()


def _run(c, rank, causal=True):
    from attention_column_gemm_amd.shard import AttnShard
    X = I.attn_activation(c)
    w = I.attn_rank_weights(c, rank)
    sh = AttnShard(c.b, c.s, c.h, c.n_q, c.n_kv, c.d, c.t, rank, causal=causal).load(X, w["Wqkv"], w["Wo"])
    sh.forward()
    return sh, X, w


SMALL = {
    # (config, causal)
    "gqa4_d128_ragged": (I.custom_attn(201, 2, 200, 256, 16, 4, 128, 2), True),
    "gqa2_d128_t4": (I.custom_attn(202, 1, 136, 264, 16, 8, 128, 4), True),
    "mha_d64_noncausal": (I.custom_attn(203, 3, 72, 128, 4, 4, 64, 2), False),
    "gqa8_d64_causal": (I.custom_attn(204, 2, 264, 192, 16, 2, 64, 2), True),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_attention_all_ranks_full_parity(name):
    torch = need_gpu()
    c, causal = SMALL[name]
    banner(f"attn {name} b={c.b} s={c.s} h={c.h} n_q={c.n_q} n_kv={c.n_kv} d={c.d} t={c.t} causal={causal}")
    from attention_column_gemm_amd.shard import sum_partials
    gZ, Zs = [], []
    for rank in range(c.t):
        sh, X, w = _run(c, rank, causal)
        torch.cuda.synchronize()
        ref = OA.shard_forward(X, w["Wqkv"], w["Wo"], b=c.b, s=c.s, q=c.q, kv=c.kv, d=c.d, causal=causal)
        check(f"r{rank}.QKV_i", _np(sh.QKV), ref["QKV"], BF)
        check(f"r{rank}.O_i", _np(sh.O), ref["O"], BF)
        check(f"r{rank}.lse_i", _np(sh.lse), ref["lse"], BF)
        check(f"r{rank}.Z_i", _np(sh.Z), ref["Z"], BF)
        # attention core alone, from the GPU's own bf16 QKV (isolates the flash kernel)
        q, kv, d = c.q, c.kv, c.d
        QKV = _np(sh.QKV)
        Oc, lc = OA.core(QKV[:, :q * d], QKV[:, q * d:(q + kv) * d], QKV[:, (q + kv) * d:], b=c.b, s=c.s,
                         n_q=q, n_kv=kv, d=d, causal=causal)
        check(f"r{rank}.core(O_i)", _np(sh.O), Oc, 1e-2)
        gZ.append(sh.Z)
        Zs.append(ref["Z"])
    Z = sum_partials(gZ)
    torch.cuda.synchronize()
    check("Z = sum Z_i", _np(Z), O.sum_partials(Zs), BF)


@pytest.mark.slow
def test_attention_cfg4_all_ranks():
    """GQA attention shard, bf16: b=2 s=2048 h=4096 32q/8kv d=128 t=8."""
    torch = need_gpu()
    c = I.ATTN_CONFIGS[4]
    banner("attn cfg4 full size, 8 ranks")
    from attention_column_gemm_amd.shard import sum_partials
    rows = edge_indices(c.tokens, extra=8, seed=7)
    gZ, Zr = [], []
    for rank in range(c.t):
        sh, X, w = _run(c, rank)
        torch.cuda.synchronize()
        if rank in (0, c.t - 1):
            ref = OA.shard_forward(X, w["Wqkv"], w["Wo"], b=c.b, s=c.s, q=c.q, kv=c.kv, d=c.d)
            check(f"r{rank}.QKV_i", _np(sh.QKV), ref["QKV"], BF)
            check(f"r{rank}.O_i", _np(sh.O), ref["O"], BF)
            check(f"r{rank}.lse_i", _np(sh.lse), ref["lse"], BF)
            check(f"r{rank}.Z_i", _np(sh.Z), ref["Z"], BF)
            Zr.append(ref["Z"][rows])
        else:
            ref = OA.shard_forward_rows(X, w["Wqkv"], w["Wo"], rows, b=c.b, s=c.s, q=c.q, kv=c.kv, d=c.d)
            check(f"r{rank}.O_i rows", _np(sh.O)[rows], ref["O"], BF)
            check(f"r{rank}.Z_i rows", _np(sh.Z)[rows], ref["Z"], BF)
            Zr.append(ref["Z"])
        gZ.append(sh.Z.clone())
        del sh
    Z = sum_partials(gZ)
    torch.cuda.synchronize()
    check("Z rows = sum Z_i", _np(Z)[rows], O.sum_partials(Zr), BF)


@pytest.mark.slow
def test_attention_cfg5_rank0_sampled():
    """Full-layer attention shard, bf16: b=4 s=2048 h=8192 64q/8kv d=128 t=8, rank 0."""
    need_gpu()
    c = I.ATTN_CONFIGS[5]
    banner("attn cfg5 full size, rank 0, sampled rows")
    sh, X, w = _run(c, 0)
    rows = edge_indices(c.tokens, extra=8, seed=8)
    ref = OA.shard_forward_rows(X, w["Wqkv"], w["Wo"], rows, b=c.b, s=c.s, q=c.q, kv=c.kv, d=c.d)
    check("O_i rows", _np(sh.O)[rows], ref["O"], BF)
    lse = _np(sh.lse).transpose(1, 0, 2).reshape(c.q, -1)[:, rows]
    check("lse_i rows", lse, ref["lse"], BF)
    check("Z_i rows", _np(sh.Z)[rows], ref["Z"], BF)
