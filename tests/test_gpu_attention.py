"""GPU parity of the attention shard forward (QKV GEMM, causal GQA flash
attention, row-parallel output projection) and backward (dO and dWo GEMMs,
flash backward, dWqkv and partial dX GEMMs) against the float64 oracle."""
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


# ------------------------------------------------------------------ backward

BWD_SMALL = dict(SMALL)
BWD_SMALL["s1_single_token"] = (I.custom_attn(205, 3, 1, 128, 4, 2, 64, 2), True)
BWD_SMALL["s33_d128_gqa4"] = (I.custom_attn(206, 2, 33, 136, 8, 2, 128, 2), True)


def _run_bwd(c, rank, causal=True):
    from attention_column_gemm_amd.shard import to_device
    sh, X, w = _run(c, rank, causal)
    dZ = I.attn_upstream_grad(c)
    sh.backward(to_device(dZ, "bf16"))
    return sh, X, w, dZ


def _check_bwd(tag, c, sh, X, w, dZ, causal):
    ref = OA.shard_backward(dZ, X, w["Wqkv"], w["Wo"], b=c.b, s=c.s, q=c.q, kv=c.kv, d=c.d, causal=causal)
    check(f"{tag}.dO_i", _np(sh.dO), ref["dO"], BF)
    check(f"{tag}.dQKV_i", _np(sh.dQKV), ref["dQKV"], BF)
    check(f"{tag}.dWqkv_i", _np(sh.dWqkv), ref["dWqkv"], BF)
    check(f"{tag}.dWo_i", _np(sh.dWo), ref["dWo"], BF)
    check(f"{tag}.dX_i", _np(sh.dX), ref["dX"], BF)
    # the core alone, from the GPU's own bf16 QKV and dO (isolates the flash backward)
    q, kv, d = c.q, c.kv, c.d
    QKV = _np(sh.QKV)
    dQ, dK, dV = OA.core_backward(QKV[:, :q * d], QKV[:, q * d:(q + kv) * d], QKV[:, (q + kv) * d:], _np(sh.dO),
                                  b=c.b, s=c.s, n_q=q, n_kv=kv, d=d, causal=causal)
    got = _np(sh.dQKV)
    check(f"{tag}.core dQ", got[:, :q * d], dQ, 1e-2)
    check(f"{tag}.core dK", got[:, q * d:(q + kv) * d], dK, 1e-2)
    check(f"{tag}.core dV", got[:, (q + kv) * d:], dV, 1e-2)
    return ref


@pytest.mark.parametrize("name", list(BWD_SMALL))
def test_attention_backward_all_ranks_full_parity(name):
    torch = need_gpu()
    c, causal = BWD_SMALL[name]
    banner(f"attn bwd {name} b={c.b} s={c.s} h={c.h} n_q={c.n_q} n_kv={c.n_kv} d={c.d} t={c.t} causal={causal}")
    from attention_column_gemm_amd.shard import sum_partials
    gdX, rdX = [], []
    for rank in range(c.t):
        sh, X, w, dZ = _run_bwd(c, rank, causal)
        torch.cuda.synchronize()
        ref = _check_bwd(f"r{rank}", c, sh, X, w, dZ, causal)
        gdX.append(sh.dX)
        rdX.append(ref["dX"])
    dX = sum_partials(gdX)
    torch.cuda.synchronize()
    check("dX = sum dX_i", _np(dX), O.sum_partials(rdX), BF)


def test_attention_backward_is_deterministic():
    torch = need_gpu()
    c, causal = SMALL["gqa4_d128_ragged"]
    banner("attn bwd determinism")
    from attention_column_gemm_amd.shard import to_device
    sh, X, w, dZ = _run_bwd(c, 1, causal)
    first = [t.clone() for t in (sh.dQKV, sh.dWqkv, sh.dWo, sh.dX)]
    sh.backward(to_device(dZ, "bf16"))
    torch.cuda.synchronize()
    for a, b in zip(first, (sh.dQKV, sh.dWqkv, sh.dWo, sh.dX)):
        assert torch.equal(a, b)


@pytest.mark.slow
def test_attention_backward_cfg4_first_and_last_rank():
    """GQA attention shard backward, bf16: b=2 s=2048 h=4096 32q/8kv d=128 t=8."""
    torch = need_gpu()
    c = I.ATTN_CONFIGS[4]
    for rank in (0, c.t - 1):
        banner(f"attn bwd cfg4 full size, rank {rank}")
        sh, X, w, dZ = _run_bwd(c, rank)
        torch.cuda.synchronize()
        _check_bwd(f"r{rank}", c, sh, X, w, dZ, True)
        del sh


@pytest.mark.slow
def test_attention_backward_cfg5_rank0():
    """Full-layer attention shard backward, bf16: b=4 s=2048 h=8192 64q/8kv d=128 t=8, rank 0."""
    torch = need_gpu()
    c = I.ATTN_CONFIGS[5]
    banner("attn bwd cfg5 full size, rank 0")
    sh, X, w, dZ = _run_bwd(c, 0)
    torch.cuda.synchronize()
    _check_bwd("r0", c, sh, X, w, dZ, True)


SPLIT_BWD = {
    # (config, causal, dQ split expected): dX_i's memory holds dQ's partials only in the last case
    "gqa4_d128_ragged": (SMALL["gqa4_d128_ragged"][0], True, False),
    "gqa8_d64_causal": (SMALL["gqa8_d64_causal"][0], True, False),
    "mqa4_d128_h2048": (I.custom_attn(207, 1, 256, 2048, 4, 1, 128, 1), True, True),
}


@pytest.mark.parametrize("name", list(SPLIT_BWD))
def test_attention_backward_key_block_split(name, lib_options):
    """The causal dK/dV kernel runs its heavier half of key blocks as two
    work-groups each (fp32 halves in dWqkv_i's memory), and dQ its heavier
    half of query blocks as two work-groups over the halves of their keys
    (fp32 halves in dX_i's memory, when it holds them); second kernels add
    the halves.  Against the oracle with the splits on and off; the runs
    differ in rounding where a split ran (proof that it ran), and dWqkv_i
    and dX_i, written over the halves afterwards, are right in both."""
    torch = need_gpu()
    c, causal, dq_split = SPLIT_BWD[name]
    got = {}
    for split in ("1", "0"):
        lib_options(split_tail=int(split))
        banner(f"attn bwd key split={split} {name}")
        sh, X, w, dZ = _run_bwd(c, 0, causal)
        torch.cuda.synchronize()
        _check_bwd(f"split{split}", c, sh, X, w, dZ, causal)
        got[split] = sh.dQKV.clone()
        del sh
    q, kv, d = c.q, c.kv, c.d
    kvcols = slice(q * d, (q + 2 * kv) * d)
    assert not torch.equal(got["1"][:, kvcols], got["0"][:, kvcols]), "the key-block split did not run"
    same_q = torch.equal(got["1"][:, :q * d], got["0"][:, :q * d])
    assert same_q != dq_split, "the dQ split ran where it should not, or did not run where it should"


FWD_SPLIT = {
    # (config, causal, split expected)
    # 8 query blocks, the heavier 4 as two halves each
    "mqa4_d128_h2048": (SPLIT_BWD["mqa4_d128_h2048"][0], True, True),
    # Z_i's memory too small for the halves: runs unsplit both ways
    "gqa4_d128_ragged_no_room": (SMALL["gqa4_d128_ragged"][0], True, False),
    # h = 4096, one sequence of 256
    "mqa4_d128_h4096": (I.custom_attn(208, 1, 256, 4096, 4, 1, 128, 1), True, True),
    # two sequences of 200 (ragged last block): the heavier 3 of 7 query blocks per sequence split
    "mqa4_d128_s200_ragged": (I.custom_attn(209, 2, 200, 4096, 4, 1, 128, 1), True, True),
}


@pytest.mark.parametrize("name", list(FWD_SPLIT))
def test_attention_forward_query_block_split(name, lib_options):
    """A causal forward whose launch leaves work-group slots empty runs its
    heavier half of query blocks as two work-groups over the halves of the
    keys (softmax state in Z_i's memory, merged by a second kernel).  O_i,
    lse_i and Z_i against the oracle with the split on and off; O_i differs
    in rounding where the split ran (proof that it ran)."""
    torch = need_gpu()
    c, causal, expect = FWD_SPLIT[name]
    ref = None
    got = {}
    for split in ("1", "0"):
        lib_options(split_tail=int(split))
        banner(f"attn fwd query split={split} {name}")
        sh, X, w = _run(c, 0, causal)
        torch.cuda.synchronize()
        if ref is None:
            ref = OA.shard_forward(X, w["Wqkv"], w["Wo"], b=c.b, s=c.s, q=c.q, kv=c.kv, d=c.d, causal=causal)
        check(f"split{split}.O_i", _np(sh.O), ref["O"], BF)
        check(f"split{split}.lse_i", _np(sh.lse), ref["lse"], BF)
        check(f"split{split}.Z_i", _np(sh.Z), ref["Z"], BF)
        q, kv, d = c.q, c.kv, c.d
        QKV = _np(sh.QKV)
        Oc, lc = OA.core(QKV[:, :q * d], QKV[:, q * d:(q + kv) * d], QKV[:, (q + kv) * d:], b=c.b, s=c.s,
                         n_q=q, n_kv=kv, d=d, causal=causal)
        check(f"split{split}.core(O_i)", _np(sh.O), Oc, 1e-2)
        check(f"split{split}.core(lse_i)", _np(sh.lse), lc, 1e-3)
        got[split] = sh.O.clone()
        del sh
    assert torch.equal(got["1"], got["0"]) != expect, "the query-block split ran where it should not, or did not run"


def test_attention_backward_pair_half_width_tail():
    """The paired dWqkv + dX launch at h = 4088, T = 4000 with eight local
    query heads and one KV head: 16 x 5 + 16 x 16 = 336 large tiles, 80 in
    the last round, so dX's last five tile rows run as 256 x 128 tiles
    (ragged in both directions).  Every backward output against the oracle."""
    torch = need_gpu()
    c = I.custom_attn(210, 4, 1000, 4088, 8, 1, 128, 1)
    banner(f"attn bwd pair half-width tail b={c.b} s={c.s} h={c.h} n_q={c.n_q} n_kv={c.n_kv} d={c.d}")
    sh, X, w, dZ = _run_bwd(c, 0, True)
    torch.cuda.synchronize()
    _check_bwd("tail", c, sh, X, w, dZ, True)


FWD_PAIRED = {
    # one round of paired query blocks (>= 256 work-groups of eight waves): 16 query blocks of 32 rows,
    # 4 heads per work-group half, 32 head groups
    "gqa8_d128_b16_s512": I.custom_attn(211, 16, 512, 256, 8, 1, 128, 1),
    # ragged last query block (rows 480..499) and sequence
    "gqa8_d128_b16_s500_ragged": I.custom_attn(212, 16, 500, 256, 8, 1, 128, 1),
    "gqa8_d64_b16_s512": I.custom_attn(213, 16, 512, 256, 8, 1, 64, 1),
    # 15 query blocks: the middle job holds one block only
    "gqa8_d128_b16_s480_odd": I.custom_attn(214, 16, 480, 256, 8, 1, 128, 1),
    # groups of 4 and 2 (64-row blocks: two row tiles per head in a half)
    "gqa4_d128_b32_s512": I.custom_attn(215, 32, 512, 256, 8, 2, 128, 1),
    "gqa2_d64_b32_s512": I.custom_attn(216, 32, 512, 256, 4, 2, 64, 1),
}


@pytest.mark.parametrize("name", list(FWD_PAIRED))
def test_attention_forward_paired_blocks(name, lib_options):
    """A causal forward with at least one full round of paired query blocks
    runs each work-group over blocks pr and npb-1-pr, its two wave sets
    taking alternate 64-key blocks and merging through LDS.  O_i, lse_i and
    Z_i against the oracle with the pairing on and off (the plain kernel);
    O_i differs in rounding between them (proof that it ran)."""
    torch = need_gpu()
    c = FWD_PAIRED[name]
    ref = None
    got = {}
    for split in (1, 0):
        lib_options(split_tail=split)
        banner(f"attn fwd paired={split} {name} b={c.b} s={c.s} n_q={c.n_q} n_kv={c.n_kv} d={c.d}")
        sh, X, w = _run(c, 0, True)
        torch.cuda.synchronize()
        if ref is None:
            ref = OA.shard_forward(X, w["Wqkv"], w["Wo"], b=c.b, s=c.s, q=c.q, kv=c.kv, d=c.d, causal=True)
        check(f"paired{split}.O_i", _np(sh.O), ref["O"], BF)
        check(f"paired{split}.lse_i", _np(sh.lse), ref["lse"], BF)
        check(f"paired{split}.Z_i", _np(sh.Z), ref["Z"], BF)
        q, kv, d = c.q, c.kv, c.d
        QKV = _np(sh.QKV)
        Oc, lc = OA.core(QKV[:, :q * d], QKV[:, q * d:(q + kv) * d], QKV[:, (q + kv) * d:], b=c.b, s=c.s,
                         n_q=q, n_kv=kv, d=d, causal=True)
        check(f"paired{split}.core(O_i)", _np(sh.O), Oc, 1e-2)
        check(f"paired{split}.core(lse_i)", _np(sh.lse), lc, 1e-3)
        got[split] = sh.O.clone()
        del sh
    assert not torch.equal(got[1], got[0]), "the paired kernel did not run"


DS_HANDOVER = {
    # causal dS tiles that fit in dX_i's memory: dK/dV hands them to dQ
    "gqa4_d128_s256_h1024": I.custom_attn(221, 2, 256, 1024, 8, 2, 128, 2),
    # ragged sequence, d = 64
    "gqa4_d64_s200_h1024_ragged": I.custom_attn(222, 2, 200, 1024, 8, 2, 64, 2),
    # more tiles than dX_i holds: the last ones go to dWqkv_i's memory after the dK/dV halves
    "mqa4_d128_s512_h1024_overflow": I.custom_attn(223, 1, 512, 1024, 4, 1, 128, 1),
}


@pytest.mark.parametrize("name", list(DS_HANDOVER))
def test_attention_backward_ds_handover(name, lib_options):
    """Where the causal dS tiles fit in dX_i's memory (and dWqkv_i's after
    the dK/dV halves), the dK/dV kernel stores them and dQ is computed from
    them without recomputing the scores.  One forward, then the backward with
    the hand-over on and off: both against the oracle, and dQ bit-identical
    (the handed-over tiles hold the values the recompute forms, and dQ's
    products run in the same order)."""
    torch = need_gpu()
    from attention_column_gemm_amd.shard import to_device
    c = DS_HANDOVER[name]
    lib_options(split_tail=1)
    banner(f"attn bwd dS hand-over {name} b={c.b} s={c.s} h={c.h} n_q={c.n_q} n_kv={c.n_kv} d={c.d}")
    sh, X, w = _run(c, 0, True)
    dZ = I.attn_upstream_grad(c)
    got = {}
    for split in (1, 0):
        lib_options(split_tail=split)
        sh.backward(to_device(dZ, "bf16"))
        torch.cuda.synchronize()
        _check_bwd(f"handover{split}", c, sh, X, w, dZ, True)
        got[split] = sh.dQKV[:, :c.q * c.d].clone()
    assert torch.equal(got[1], got[0]), "dQ from the handed-over dS tiles differs from the recompute"


def test_attention_backward_ds_not_fitting(lib_options):
    """Causal dS tiles that do not fit in dX_i's and dWqkv_i's memory: dQ
    recomputes the scores, and with split_tail on its heaviest query blocks
    are split in two (their fp32 halves in dX_i's memory).  One forward, then
    the backward with the split on and off, both against the oracle; dQ
    differs between the two in rounding only, which shows the split ran."""
    torch = need_gpu()
    from attention_column_gemm_amd.shard import to_device
    c = I.custom_attn(224, 1, 1024, 512, 4, 1, 64, 1)
    nqt = (c.s + 31) // 32
    tiles = c.b * c.q * nqt * (nqt + 1) // 2
    room = c.b * c.s * c.h * 2 + c.h * (c.q + 2 * c.kv) * c.d * 4
    assert tiles * 2048 > room, "the shape no longer exceeds the hand-over's room"
    lib_options(split_tail=1)
    banner(f"attn bwd dS not fitting b={c.b} s={c.s} h={c.h} n_q={c.n_q} n_kv={c.n_kv} d={c.d}")
    sh, X, w = _run(c, 0, True)
    dZ = I.attn_upstream_grad(c)
    got = {}
    for split in (1, 0):
        lib_options(split_tail=split)
        sh.backward(to_device(dZ, "bf16"))
        torch.cuda.synchronize()
        _check_bwd(f"nofit{split}", c, sh, X, w, dZ, True)
        got[split] = sh.dQKV[:, :c.q * c.d].clone()
    assert not torch.equal(got[1], got[0]), "dQ's split query blocks did not run"
