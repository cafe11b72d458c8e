"""GPU parity of the MLP shard (forward, backward, emulated all-reduces)
against the float64 oracle, through the C ABI.

Small workloads are compared element by element on every output of every
rank and on the summed outputs; the full-size workloads are compared on
sampled token rows (forward outputs and input gradients) and sampled
intermediate columns (weight and bias gradients), in the tile configuration
the benchmark uses.
"""
import os

import numpy as np
import pytest

from attention_column_gemm_amd import binding as B
from attention_column_gemm_amd import inputs as I
from oracle import mlp as O
from parity import TOL, banner, check, edge_indices, need_gpu

pytestmark = pytest.mark.gpu


def _gpu_rank(c, rank, X, dOut, w, write_dY=True):
    from attention_column_gemm_amd.shard import MLPShard
    sh = MLPShard(c.tokens, c.h, c.h_ffn, c.t, rank, act=c.act, dtype=c.dtype)
    sh.load(X, w["W1"], w["Wu"], w["b1"], w["W2"], dOut)
    sh.forward()
    sh.backward(c.p_drop, c.seed, want_db2=True, want_db1=True, write_dY=write_dY)
    sh.wrote_dY = write_dY
    return sh


def _np(t):
    return t.detach().float().cpu().numpy()


def _compare_rank(c, sh, fw, bw, rows=None, tol=None, tag=""):
    tol = tol or TOL[c.dtype]
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    if c.act == "gelu":
        check(f"{tag}A_i", sel(_np(sh.saved[0])), fw["A"], tol)
        check(f"{tag}dA_i", sel(_np(sh.dA[0])), bw["dA"], tol)
    else:
        check(f"{tag}G_i", sel(_np(sh.saved[0])), fw["G"], tol)
        check(f"{tag}U_i", sel(_np(sh.saved[1])), fw["U"], tol)
        check(f"{tag}dG_i", sel(_np(sh.dA[0])), bw["dG"], tol)
        check(f"{tag}dU_i", sel(_np(sh.dA[1])), bw["dU"], tol)
    check(f"{tag}H_i", sel(_np(sh.H)), fw["H"], tol)
    check(f"{tag}Z_i", sel(_np(sh.Z)), fw["Z"], tol)
    if sh.wrote_dY:
        check(f"{tag}dY", sel(_np(sh.dY)), bw["dY"], tol)
    check(f"{tag}dX_i", sel(_np(sh.dX)), bw["dX"], tol)


def _compare_rank_grads(c, sh, bw, cols=None, tol=None, tag=""):
    tol = tol or TOL[c.dtype]
    cs = (lambda a, ax: a) if cols is None else (lambda a, ax: np.take(a, cols, axis=ax))
    check(f"{tag}dW1_i", cs(_np(sh.dW1[0]), 1), bw["dW1"], tol)
    if c.act == "swiglu":
        check(f"{tag}dWu_i", cs(_np(sh.dW1[1]), 1), bw["dWu"], tol)
    else:
        check(f"{tag}db1_i", cs(_np(sh.db1), 0), bw["db1"], tol)
    check(f"{tag}dW2_i", cs(_np(sh.dW2), 0), bw["dW2"], tol)


SMALL = {
    "cfg1_gelu_fp32_t2": I.MLP_CONFIGS[1],
    "ragged_gelu_bias_dropout_t4": I.custom_mlp(101, 2, 164, 264, 544, 4, "gelu", "bf16", p_drop=0.15, bias=True),
    "ragged_swiglu_t2": I.custom_mlp(102, 1, 328, 264, 688, 2, "swiglu", "bf16"),
    "ragged_gelu_fp32_t3": I.custom_mlp(103, 3, 45, 132, 3 * 76, 3, "gelu", "fp32", p_drop=0.3, bias=True),
    # K loops of one and two 64-deep tiles: the loop body never runs, or runs once with the
    # refill past the last tile (h = 40: dH has one K tile; f = 48 per rank: dX has one per segment)
    "tinyK_swiglu_t4": I.custom_mlp(104, 2, 50, 40, 192, 4, "swiglu", "bf16"),
    "tinyK_gelu_bias_dropout_t2": I.custom_mlp(105, 1, 70, 128, 144, 2, "gelu", "bf16", p_drop=0.1, bias=True),
}


@pytest.mark.parametrize("tile", ["auto", "large", "small", "tiny"])
@pytest.mark.parametrize("name", list(SMALL))
def test_mlp_all_ranks_full_parity(name, tile, lib_options):
    torch = need_gpu()
    c = SMALL[name]
    if tile != "auto":
        if c.dtype == "fp32":
            pytest.skip("tile override applies to the bf16 matrix-core GEMM only")
        lib_options(tile={"large": B.TP_TILE_LARGE, "small": B.TP_TILE_SMALL, "tiny": B.TP_TILE_TINY}[tile])
    banner(f"mlp {name} tile={tile} T={c.tokens} h={c.h} h_ffn={c.h_ffn} t={c.t} {c.act} {c.dtype} p={c.p_drop}")
    from attention_column_gemm_amd.shard import sum_partials, to_device
    X, dOut = I.mlp_activation(c)
    shards, Zs, dXs = [], [], []
    for rank in range(c.t):
        w = I.mlp_rank_weights(c, rank)
        sh = _gpu_rank(c, rank, X, dOut, w)
        fw, bw = O.shard_step(dOut, X, w["W1"], w["W2"], act=c.act, Wu_i=w["Wu"], b1_i=w["b1"], p=c.p_drop,
                              seed=c.seed)
        torch.cuda.synchronize()
        _compare_rank(c, sh, fw, bw, tag=f"r{rank}.")
        _compare_rank_grads(c, sh, bw, tag=f"r{rank}.")
        if rank == 0:
            check("db2", _np(sh.db2), bw["db2"], TOL[c.dtype])
        shards.append(sh)
        Zs.append(fw["Z"])
        dXs.append(bw["dX"])
    b2 = I.mlp_rank_weights(c, 0)["b2"]
    out = sum_partials([s.Z for s in shards], to_device(b2, c.dtype), c.p_drop, c.seed)
    dx = sum_partials([s.dX for s in shards])
    torch.cuda.synchronize()
    check("Out = g(sum Z_i)", _np(out), O.sum_partials(Zs, b2, c.p_drop, c.seed), TOL[c.dtype])
    check("dX = f(sum dX_i)", _np(dx), O.sum_partials(dXs), TOL[c.dtype])
    # the emulated all-reduce against the unsharded layer
    full = I.mlp_full_weights(c)
    ref = O.backward(dOut, X, full["W1"], full["W2"], act=c.act, Wu=full["Wu"], b1=full["b1"], b2=full["b2"],
                     p=c.p_drop, seed=c.seed)
    check("Out vs unsharded", _np(out), ref["fwd"]["Out"], TOL[c.dtype])
    check("dX vs unsharded", _np(dx), ref["dX"], TOL[c.dtype])


def test_mlp_cfg2_full_parity_and_determinism():
    """GPT-style GeLU MLP, bf16, T=2048 h=1024 h_ffn=4096 t=4, dropout 0.1."""
    torch = need_gpu()
    c = I.MLP_CONFIGS[2]
    banner("mlp cfg2 full parity, all 4 ranks")
    from attention_column_gemm_amd.shard import sum_partials, to_device
    X, dOut = I.mlp_activation(c)
    Zs, dXs, gZ, gdX = [], [], [], []
    for rank in range(c.t):
        w = I.mlp_rank_weights(c, rank)
        sh = _gpu_rank(c, rank, X, dOut, w)
        fw, bw = O.shard_step(dOut, X, w["W1"], w["W2"], act=c.act, b1_i=w["b1"], p=c.p_drop, seed=c.seed)
        torch.cuda.synchronize()
        _compare_rank(c, sh, fw, bw, tag=f"r{rank}.")
        _compare_rank_grads(c, sh, bw, tag=f"r{rank}.")
        if rank == 0:
            check("db2", _np(sh.db2), bw["db2"], TOL[c.dtype])
            # run-twice determinism: bit-identical outputs
            first = [x.clone() for x in (sh.Z, sh.dX, sh.dW1, sh.dW2, sh.db1, sh.db2, sh.dA)]
            sh.forward()
            sh.backward(c.p_drop, c.seed, write_dY=True)
            torch.cuda.synchronize()
            for a, b in zip(first, (sh.Z, sh.dX, sh.dW1, sh.dW2, sh.db1, sh.db2, sh.dA)):
                assert torch.equal(a, b)
        Zs.append(fw["Z"]); dXs.append(bw["dX"]); gZ.append(sh.Z); gdX.append(sh.dX)
    b2 = I.mlp_rank_weights(c, 0)["b2"]
    out = sum_partials(gZ, to_device(b2, c.dtype), c.p_drop, c.seed)
    dx = sum_partials(gdX)
    torch.cuda.synchronize()
    check("Out = g(sum Z_i)", _np(out), O.sum_partials(Zs, b2, c.p_drop, c.seed), TOL[c.dtype])
    check("dX = f(sum dX_i)", _np(dx), O.sum_partials(dXs), TOL[c.dtype])


def _sampled_rank(c, rank, X, dOut, w, rows, cols):
    """The launch sequence the benchmark times (dY is written only when p > 0)."""
    torch = need_gpu()
    sh = _gpu_rank(c, rank, X, dOut, w, write_dY=c.p_drop > 0)
    torch.cuda.synchronize()
    fw, bw = O.shard_step(dOut[rows], X[rows], w["W1"], w["W2"], act=c.act, Wu_i=w["Wu"], b1_i=w["b1"],
                          p=c.p_drop, seed=c.seed, rows=rows)
    _compare_rank(c, sh, fw, bw, rows=rows, tag=f"r{rank}.rows.")
    _, cbw = O.column_sample(dOut, X, w["W1"], w["W2"], cols, act=c.act, Wu_i=w["Wu"], b1_i=w["b1"],
                             p=c.p_drop, seed=c.seed)
    _compare_rank_grads(c, sh, cbw, cols=cols, tag=f"r{rank}.cols.")
    return sh, fw, bw


@pytest.mark.slow
def test_mlp_cfg3_all_ranks_sampled():
    """Llama SwiGLU MLP, bf16, T=4096 h=4096 h_ffn=11008 t=8 (f=1376): every rank,
    sampled rows/columns, plus the summed output on the sampled rows."""
    torch = need_gpu()
    c = I.MLP_CONFIGS[3]
    banner("mlp cfg3 full size, 8 ranks, sampled")
    from attention_column_gemm_amd.shard import sum_partials
    X, dOut = I.mlp_activation(c)
    rows = edge_indices(c.tokens, extra=8, seed=3)
    cols = edge_indices(c.f, tiles=(64, 128, 256), extra=4, seed=4)
    gZ, gdX, Zr, dXr = [], [], [], []
    for rank in range(c.t):
        w = I.mlp_rank_weights(c, rank)
        sh, fw, bw = _sampled_rank(c, rank, X, dOut, w, rows, cols)
        gZ.append(sh.Z.clone()); gdX.append(sh.dX.clone()); Zr.append(fw["Z"]); dXr.append(bw["dX"])
        del sh
    out = sum_partials(gZ)
    dx = sum_partials(gdX)
    torch.cuda.synchronize()
    check("Out rows = sum Z_i", _np(out)[rows], O.sum_partials(Zr), TOL["bf16"])
    check("dX rows = sum dX_i", _np(dx)[rows], O.sum_partials(dXr), TOL["bf16"])


@pytest.mark.slow
def test_mlp_cfg5_rank0_sampled():
    """Full-layer MLP shard, bf16, T=8192 h=8192 h_ffn=28672 t=8 (f=3584),
    rank 0 as timed by the benchmark: sampled rows and columns."""
    need_gpu()
    c = I.MLP_CONFIGS[5]
    banner("mlp cfg5 full size, rank 0, sampled")
    X, dOut = I.mlp_activation(c)
    w = I.mlp_rank_weights(c, 0)
    rows = edge_indices(c.tokens, extra=8, seed=5)
    cols = edge_indices(c.f, tiles=(64, 128, 256), extra=4, seed=6)
    _sampled_rank(c, 0, X, dOut, w, rows, cols)


SPLIT_CASES = {
    # column GEMM: 16 x 17 = 272 tiles of 256 x 128, ragged in rows and columns; the last 16 are
    # split, their partial tiles (8.4 MB) fitting in Z_i's memory (T h bf16 = 8.4 MB)
    "col_T4000_h1056_f2104": (106, 2, 2000, 1056, 2104),
    # one ragged row of 272 column tiles: K = h = 200 in four 64-deep tiles (two per half); Z_i's
    # memory (0.1 MB) is too small for the partials, so this runs unsplit both ways
    "col_T250_h200_f34800_no_room": (107, 1, 250, 200, 34800),
}


@pytest.mark.parametrize("name", list(SPLIT_CASES))
def test_mlp_split_tail_parity(name, lib_options):
    """A column GEMM whose last round of large tiles is at most half full runs
    it as two K halves per tile (fp32 partial tiles in Z_i's memory), finished
    by a kernel that adds the halves and runs the SwiGLU epilogue.  Forward
    outputs against the oracle with the split on and off; where the split
    applies, the two runs differ in rounding (proof that it ran)."""
    torch = need_gpu()
    from attention_column_gemm_amd.shard import MLPShard
    cfg, b, s, h, h_ffn = SPLIT_CASES[name]
    c = I.custom_mlp(cfg, b, s, h, h_ffn, 1, "swiglu", "bf16")
    X, dOut = I.mlp_activation(c)
    w = I.mlp_rank_weights(c, 0)
    fw = O.shard_forward(X, w["W1"], w["W2"], act=c.act, Wu_i=w["Wu"])
    outs = {}
    for split in ("1", "0"):
        lib_options(split_tail=int(split))
        banner(f"mlp split tail={split} T={c.tokens} h={c.h} f={c.f}")
        sh = MLPShard(c.tokens, c.h, c.h_ffn, c.t, 0, act=c.act, dtype=c.dtype)
        sh.load(X, w["W1"], w["Wu"], w["b1"], w["W2"], dOut)
        sh.forward()
        torch.cuda.synchronize()
        tol = TOL[c.dtype]
        check(f"split{split}.G_i", _np(sh.saved[0]), fw["G"], tol)
        check(f"split{split}.U_i", _np(sh.saved[1]), fw["U"], tol)
        check(f"split{split}.H_i", _np(sh.H), fw["H"], tol)
        check(f"split{split}.Z_i", _np(sh.Z), fw["Z"], tol)
        outs[split] = sh.saved[0].clone()
        del sh
    ran = not torch.equal(outs["1"], outs["0"])
    assert ran == ("no_room" not in name), "the split ran where it should not, or did not run where it should"


PAIR_TAIL_CASES = {
    # dWg, dWu (15 x 4 tiles of 256 x 128) + dX (18 x 15 tiles of 256 x 256): 330 tiles, the last
    # round holding 74, so dX's last five tile rows run as 145 tiles of 256 x 128; ragged in T, h, f
    "swiglu_dW1_dX_T4400_h3704_f504": I.custom_mlp(108, 2, 2200, 3704, 504, 1, "swiglu", "bf16"),
    # dH (5 x 16) + dW2 (16 x 16): 336 tiles, the last round holding 80, so dW2's last five tile
    # rows run at half width; GeLU with both biases and dropout, ragged in T, h and f
    "gelu_dH_dW2_T1200_h3960_f3960": I.custom_mlp(109, 2, 600, 3960, 3960, 1, "gelu", "bf16", p_drop=0.1,
                                                  bias=True),
}


@pytest.mark.parametrize("name", list(PAIR_TAIL_CASES))
def test_mlp_pair_half_width_tail_parity(name, lib_options):
    """A paired backward launch whose last round of large tiles is at most
    half full runs problem 2's last tile rows as 256 x 128 tiles.  Every
    output against the oracle with the tail on and off; each output element
    sums the same K tiles in the same order either way, so the two runs are
    bit-identical."""
    torch = need_gpu()
    c = PAIR_TAIL_CASES[name]
    X, dOut = I.mlp_activation(c)
    w = I.mlp_rank_weights(c, 0)
    fw, bw = O.shard_step(dOut, X, w["W1"], w["W2"], act=c.act, Wu_i=w["Wu"], b1_i=w["b1"], p=c.p_drop, seed=c.seed)
    runs = {}
    for split in ("1", "0"):
        lib_options(split_tail=int(split))
        banner(f"mlp pair tail={split} {name}")
        sh = _gpu_rank(c, 0, X, dOut, w)
        torch.cuda.synchronize()
        _compare_rank(c, sh, fw, bw, tag=f"split{split}.")
        _compare_rank_grads(c, sh, bw, tag=f"split{split}.")
        check(f"split{split}.db2", _np(sh.db2), bw["db2"], TOL[c.dtype])
        runs[split] = [t.clone() for t in (sh.dA, sh.dW1, sh.dW2, sh.dX)]
        del sh
    for a, b in zip(runs["1"], runs["0"]):
        assert torch.equal(a, b), "the half-width tail changed a result"
