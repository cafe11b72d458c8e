"""Pins of the CPU oracle to facts outside itself (CPU only).

Each test checks the oracle against something the pages or mathematics fix:
tabulated values, closed forms, invariants the pages state, brute force on
tiny inputs written with Python loops and ``math``, finite differences of the
forward pass, and a simulated ring all-reduce.  The tests are chosen so that
a plausible slip in the oracle (a dropped term, a sign, a wrong index, a
transposed operand, the bias counted per rank) fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import activations as A
from oracle import attention as att
from oracle import comm, dropout, flops, mlp
from oracle import sequence_parallel as sp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- activations

def test_gelu_matches_tabulated_normal_cdf():
    pts = json.load(open(os.path.join(GOLDEN, "normal_cdf.json")))["points"]
    for p in pts:
        x = p["x"]
        assert abs(A.normal_cdf(x) - p["Phi"]) < 1e-14
        assert abs(A.gelu(x) - x * p["Phi"]) < 1e-14


def test_activation_closed_forms():
    x = np.linspace(-6, 6, 101)
    assert A.gelu(0.0) == 0.0 and A.silu(0.0) == 0.0
    # GeLU(-x) = GeLU(x) - x and SiLU(-x) = SiLU(x) - x (Phi(-x) = 1 - Phi(x), sigma(-x) = 1 - sigma(x))
    np.testing.assert_allclose(A.gelu(-x), A.gelu(x) - x, atol=1e-14)
    np.testing.assert_allclose(A.silu(-x), A.silu(x) - x, atol=1e-14)
    assert abs(A.gelu_grad(0.0) - 0.5) < 1e-15 and abs(A.silu_grad(0.0) - 0.5) < 1e-15
    # sigma(1) = e / (1 + e)
    assert abs(A.silu(1.0) - 0.7310585786300049) < 1e-15
    # saturation: identity for large positive, zero for large negative inputs
    assert A.gelu(40.0) == 40.0 and A.gelu(-1000.0) == 0.0
    assert A.silu(40.0) == 40.0 and A.silu(-1000.0) == 0.0


@pytest.mark.parametrize("fn,grad", [(A.gelu, A.gelu_grad), (A.silu, A.silu_grad)])
def test_activation_derivative_finite_difference(fn, grad):
    x = np.linspace(-5, 5, 57)
    e = 1e-6
    fd = (fn(x + e) - fn(x - e)) / (2 * e)
    np.testing.assert_allclose(grad(x), fd, atol=1e-8)


# -------------------------------------------------------------------- dropout

def test_splitmix64_published_vectors():
    g = json.load(open(os.path.join(GOLDEN, "splitmix64.json")))
    for v in g["vectors"]:
        want = [int(o, 0) for o in v["outputs"]]
        got = [int(x) for x in dropout.splitmix64_nth(v["seed"], np.arange(1, len(want) + 1))]
        assert got == want


def test_dropout_threshold_and_identity():
    assert dropout.drop_threshold(0.0) == 0
    assert dropout.drop_threshold(0.5) == 2 ** 31
    assert dropout.drop_threshold(0.25) == 2 ** 30
    Y = _rng(0).standard_normal((5, 7))
    np.testing.assert_array_equal(dropout.apply(Y, 123, 0.0), Y)
    with pytest.raises(ValueError):
        dropout.drop_threshold(1.0)


def test_dropout_keep_fraction_and_values():
    rows, cols, p = 2048, 1024, 0.1
    m = dropout.keep_mask(2099, rows, cols, p)
    n = rows * cols
    frac = m.mean()
    sigma = math.sqrt(p * (1 - p) / n)
    assert abs(frac - (1 - p)) < 6 * sigma
    Y = np.ones((4, 9))
    out = dropout.apply(Y, 7, 0.25)
    vals = set(np.unique(out).tolist())
    assert vals <= {0.0, 1.0 / 0.75}


def test_dropout_mask_depends_only_on_global_index():
    """The mask of a row subset equals those rows of the full mask, so it is
    the same whatever the TP degree or the tiling ([LP] II.V)."""
    full = dropout.keep_mask(5, 64, 48, 0.3)
    rows = np.array([0, 3, 17, 63])
    np.testing.assert_array_equal(dropout.keep_mask(5, rows, 48, 0.3), full[rows])
    # flat index r*cols + c: element (r, c) of a [64, 48] tensor and element r*48+c of a [1, 3072] one agree
    flat = dropout.keep_mask(5, 1, 64 * 48, 0.3).reshape(64, 48)
    np.testing.assert_array_equal(flat, full)


# ------------------------------------------------------------------- MLP fwd

def _brute_mlp(X, W1, W2, act, Wu=None, b1=None, b2=None):
    """Pure-Python loops over the definition; math.erf / math.exp only."""
    T, h = len(X), len(X[0])
    f = len(W1[0])
    out = [[0.0] * h for _ in range(T)]
    for r in range(T):
        Hrow = []
        for j in range(f):
            a = sum(X[r][k] * W1[k][j] for k in range(h))
            if act == "gelu":
                if b1 is not None:
                    a += b1[j]
                Hrow.append(a * 0.5 * (1.0 + math.erf(a / math.sqrt(2.0))))
            else:
                u = sum(X[r][k] * Wu[k][j] for k in range(h))
                Hrow.append(a / (1.0 + math.exp(-a)) * u)
        for c in range(h):
            y = sum(Hrow[j] * W2[j][c] for j in range(f))
            if b2 is not None:
                y += b2[c]
            out[r][c] = y
    return np.array(out)


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_mlp_forward_brute_force(act):
    g = _rng(1)
    T, h, hf = 3, 4, 6
    X = g.standard_normal((T, h))
    W1 = g.standard_normal((h, hf))
    Wu = g.standard_normal((h, hf)) if act == "swiglu" else None
    W2 = g.standard_normal((hf, h))
    b1 = g.standard_normal(hf) if act == "gelu" else None
    b2 = g.standard_normal(h)
    want = _brute_mlp(X.tolist(), W1.tolist(), W2.tolist(), act,
                      None if Wu is None else Wu.tolist(),
                      None if b1 is None else b1.tolist(), b2.tolist())
    got = mlp.forward(X, W1, W2, act=act, Wu=Wu, b1=b1, b2=b2)["Out"]
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-13)


def test_mlp_forward_saturated_integer_case():
    """Pre-activations of +/-1000 make GeLU and SiLU exact identities or zeros,
    so the layer is exactly linear in integers and checkable by hand.

    X rows are one-hot, so row r of A is row r's one-hot pick of W1 plus b1;
    the orientation of W1 and W2, the bias placement, the gate/up roles and the
    single addition of b2 are all visible in the integers.
    """
    L = 1000.0
    # h=3 inputs, h_ffn=4 intermediate, T=3 tokens
    X = np.eye(3)
    W1 = np.array([[L, -L, L, -L], [-L, L, L, -L], [L, L, -L, -L]])
    b1 = np.array([1.0, 2.0, 3.0, -2.0])       # GeLU case: shifts but keeps signs
    W2 = np.array([[1.0, 0.0, 2.0], [0.0, 3.0, 0.0], [1.0, 1.0, 1.0], [5.0, 5.0, 5.0]])
    b2 = np.array([10.0, 20.0, 30.0])
    out = mlp.forward(X, W1, W2, act="gelu", b1=b1, b2=b2)["Out"]
    # token 0: A = [L+1, -L+2, L+3, -L-2] -> H = [L+1, 0, L+3, 0]
    want0 = np.array([(L + 1) * 1 + (L + 3) * 1, (L + 3) * 1, (L + 1) * 2 + (L + 3) * 1]) + b2
    np.testing.assert_array_equal(out[0], want0)
    # token 2: A = [L+1, L+2, -L+3, -L-2] -> H = [L+1, L+2, 0, 0]
    want2 = np.array([(L + 1), 3 * (L + 2), 2 * (L + 1)]) + b2
    np.testing.assert_array_equal(out[2], want2)

    # SwiGLU: SiLU on the gate (W1), identity factor from up (Wu)
    Wu = np.array([[2.0, 3.0, 4.0, 5.0], [6.0, 7.0, 8.0, 9.0], [1.0, 1.0, 1.0, 1.0]])
    out = mlp.forward(X, W1, W2, act="swiglu", Wu=Wu, b2=b2)["Out"]
    # token 1: gate = [-L, L, L, -L] -> SiLU = [0, L, L, 0]; up = [6,7,8,9] -> H = [0, 7L, 8L, 0]
    want1 = np.array([8 * L, 21 * L + 8 * L, 8 * L]) + b2
    np.testing.assert_array_equal(out[1], want1)


def _mlp_case(seed, T=5, h=6, hf=8, act="gelu", bias=True):
    g = _rng(seed)
    return dict(
        X=g.standard_normal((T, h)), W1=g.standard_normal((h, hf)) / 2,
        Wu=g.standard_normal((h, hf)) / 2 if act == "swiglu" else None,
        W2=g.standard_normal((hf, h)) / 2,
        b1=g.standard_normal(hf) if (bias and act == "gelu") else None,
        b2=g.standard_normal(h) if bias else None,
        dOut=g.standard_normal((T, h)))


def _shards(c, t, act):
    hf = c["W1"].shape[1]
    res = []
    for i in range(t):
        sl = mlp.shard_cols(hf, t, i)
        res.append(dict(W1=c["W1"][:, sl], W2=c["W2"][sl, :],
                        Wu=None if c["Wu"] is None else c["Wu"][:, sl],
                        b1=None if c["b1"] is None else c["b1"][sl]))
    return res


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("t", [1, 2, 4])
def test_sum_of_partials_equals_unsharded(act, t):
    """Sigma_i Z_i = H W2 ([L11] section 3; [TP1] MLP), column pieces of H and
    dW1/db1 and row pieces of dW2 are the unsharded ones ([L11] section 2), and
    Sigma_i dX_i = dX ([TP1] operator f)."""
    c = _mlp_case(10 + t, act=act)
    p, seed = 0.2, 77
    full = mlp.backward(c["dOut"], c["X"], c["W1"], c["W2"], act=act, Wu=c["Wu"], b1=c["b1"],
                        b2=c["b2"], p=p, seed=seed)
    parts, dxs, Hs, dW1s, dW2s, db1s, dWus = [], [], [], [], [], [], []
    for s in _shards(c, t, act):
        fw, bw = mlp.shard_step(c["dOut"], c["X"], s["W1"], s["W2"], act=act, Wu_i=s["Wu"],
                                b1_i=s["b1"], p=p, seed=seed)
        parts.append(fw["Z"]); Hs.append(fw["H"]); dxs.append(bw["dX"])
        dW1s.append(bw["dW1"]); dW2s.append(bw["dW2"])
        if act == "gelu":
            db1s.append(bw["db1"])
        else:
            dWus.append(bw["dWu"])
    out = mlp.sum_partials(parts, c["b2"], p, seed)
    rel = lambda a, b: np.abs(a - b).max() / np.abs(b).max()
    assert rel(out, full["fwd"]["Out"]) < 1e-12
    assert rel(np.concatenate(Hs, 1), full["fwd"]["H"]) < 1e-13
    assert rel(mlp.sum_partials(dxs), full["dX"]) < 1e-12
    assert rel(np.concatenate(dW1s, 1), full["dW1"]) < 1e-12
    assert rel(np.concatenate(dW2s, 0), full["dW2"]) < 1e-12
    if act == "gelu":
        assert rel(np.concatenate(db1s), full["db1"]) < 1e-12
    else:
        assert rel(np.concatenate(dWus, 1), full["dWu"]) < 1e-12


def test_bias_added_per_rank_is_counted_t_times():
    """Adding the row-parallel output bias on every rank before the sum
    counts it t times ([L11] section 3, last paragraph)."""
    c = _mlp_case(3)
    t = 4
    parts = [mlp.shard_forward(c["X"], s["W1"], s["W2"], b1_i=s["b1"])["Z"] for s in _shards(c, t, "gelu")]
    right = mlp.sum_partials(parts, c["b2"])
    wrong = mlp.sum_partials([P + c["b2"] for P in parts])
    np.testing.assert_allclose(wrong - right, np.broadcast_to((t - 1) * c["b2"], right.shape), atol=1e-12)


def test_row_first_split_does_not_commute_with_gelu():
    """GeLU(X1 A1 + X2 A2) != GeLU(X1 A1) + GeLU(X2 A2) ([TP1] row split)."""
    g = _rng(4)
    X, Aw = g.standard_normal((4, 6)), g.standard_normal((6, 5))
    lhs = A.gelu(X[:, :3] @ Aw[:3] + X[:, 3:] @ Aw[3:])
    rhs = A.gelu(X[:, :3] @ Aw[:3]) + A.gelu(X[:, 3:] @ Aw[3:])
    assert np.abs(lhs - rhs).max() > 1e-2
    # while the column split commutes ([TP1] column split)
    np.testing.assert_allclose(A.gelu(X @ Aw), np.concatenate([A.gelu(X @ Aw[:, :2]), A.gelu(X @ Aw[:, 2:])], 1),
                               atol=1e-14)


# ------------------------------------------------------------------- MLP bwd

def _loss(c, act, p, seed, **over):
    cc = dict(c, **over)
    o = mlp.forward(cc["X"], cc["W1"], cc["W2"], act=act, Wu=cc["Wu"], b1=cc["b1"], b2=cc["b2"],
                    p=p, seed=seed)["Out"]
    return float((o * c["dOut"]).sum())


@pytest.mark.parametrize("act,p", [("gelu", 0.0), ("gelu", 0.3), ("swiglu", 0.0), ("swiglu", 0.25)])
def test_backward_central_differences(act, p):
    """Every gradient of L = <dOut, Out> against central differences of the
    forward pass (T=4, h=5, h_ffn=6)."""
    c = _mlp_case(20, T=4, h=5, hf=6, act=act)
    seed = 31
    g = mlp.backward(c["dOut"], c["X"], c["W1"], c["W2"], act=act, Wu=c["Wu"], b1=c["b1"], b2=c["b2"],
                     p=p, seed=seed)
    names = {"X": "dX", "W1": "dW1", "W2": "dW2", "b2": "db2"}
    if act == "gelu":
        names["b1"] = "db1"
    else:
        names["Wu"] = "dWu"
    e = 1e-6
    for name, gname in names.items():
        base = c[name]
        fd = np.zeros_like(base)
        for idx in np.ndindex(base.shape):
            plus, minus = base.copy(), base.copy()
            plus[idx] += e
            minus[idx] -= e
            fd[idx] = (_loss(c, act, p, seed, **{name: plus}) - _loss(c, act, p, seed, **{name: minus})) / (2 * e)
        np.testing.assert_allclose(g[gname], fd, rtol=1e-6, atol=1e-7 * max(1.0, np.abs(fd).max()),
                                   err_msg=f"{act} p={p} {gname}")


def test_t1_shard_equals_unsharded():
    """t = 1 is the single-card layer ([L11] section 6: correctness against a
    single-card baseline)."""
    c = _mlp_case(6, act="swiglu", bias=False)
    full = mlp.backward(c["dOut"], c["X"], c["W1"], c["W2"], act="swiglu", Wu=c["Wu"])
    fw, bw = mlp.shard_step(c["dOut"], c["X"], c["W1"], c["W2"], act="swiglu", Wu_i=c["Wu"])
    np.testing.assert_allclose(fw["Z"], full["fwd"]["Y"], rtol=1e-14, atol=1e-14)
    for k in ("dX", "dW1", "dWu", "dW2"):
        np.testing.assert_allclose(bw[k], full[k], rtol=1e-13, atol=1e-13)


def test_column_sample_and_row_sample_match_full_shard():
    c = _mlp_case(8, T=9, h=6, hf=10, act="gelu")
    p, seed = 0.1, 5
    fw, bw = mlp.shard_step(c["dOut"], c["X"], c["W1"], c["W2"], b1_i=c["b1"], p=p, seed=seed)
    cols = np.array([0, 4, 9])
    sub_fw, sub_bw = mlp.column_sample(c["dOut"], c["X"], c["W1"], c["W2"], cols, b1_i=c["b1"], p=p, seed=seed)
    np.testing.assert_allclose(sub_bw["dW1"], bw["dW1"][:, cols], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sub_bw["dW2"], bw["dW2"][cols], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sub_bw["db1"], bw["db1"][cols], rtol=1e-13, atol=1e-14)
    rows = np.array([1, 5, 8])
    rfw, rbw = mlp.shard_step(c["dOut"][rows], c["X"][rows], c["W1"], c["W2"], b1_i=c["b1"], p=p, seed=seed,
                              rows=rows)
    np.testing.assert_allclose(rfw["Z"], fw["Z"][rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(rbw["dX"], bw["dX"][rows], rtol=1e-13, atol=1e-14)


# ----------------------------------------------------------------- attention

def _brute_attn(Q, K, V, b, s, n_q, n_kv, d):
    group = n_q // n_kv
    T = b * s
    O = [[0.0] * (n_q * d) for _ in range(T)]
    for beta in range(b):
        for j in range(n_q):
            g = j // group
            for i in range(s):
                r = beta * s + i
                sc = []
                for k in range(i + 1):
                    rk = beta * s + k
                    sc.append(sum(Q[r][j * d + e] * K[rk][g * d + e] for e in range(d)) / math.sqrt(d))
                m = max(sc)
                w = [math.exp(x - m) for x in sc]
                z = sum(w)
                for e in range(d):
                    O[r][j * d + e] = sum(w[k] * V[beta * s + k][g * d + e] for k in range(i + 1)) / z
    return np.array(O)


def test_attention_brute_force_gqa():
    g = _rng(12)
    b, s, n_q, n_kv, d = 2, 5, 4, 2, 3
    Q = g.standard_normal((b * s, n_q * d))
    K = g.standard_normal((b * s, n_kv * d))
    V = g.standard_normal((b * s, n_kv * d))
    O, lse = att.core(Q, K, V, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)
    want = _brute_attn(Q.tolist(), K.tolist(), V.tolist(), b, s, n_q, n_kv, d)
    np.testing.assert_allclose(O, want, rtol=1e-13, atol=1e-13)


def test_attention_closed_forms():
    g = _rng(13)
    b, s, n_q, n_kv, d = 2, 6, 4, 2, 8
    K = g.standard_normal((b * s, n_kv * d))
    V = g.standard_normal((b * s, n_kv * d))
    # Q = 0: uniform weights over the causal prefix -> prefix mean, lse = log(count)
    O, lse = att.core(np.zeros((b * s, n_q * d)), K, V, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)
    for beta in range(b):
        for j in range(n_q):
            gh = j // (n_q // n_kv)
            v = V[beta * s:(beta + 1) * s, gh * d:(gh + 1) * d]
            want = np.cumsum(v, 0) / np.arange(1, s + 1)[:, None]
            np.testing.assert_allclose(O[beta * s:(beta + 1) * s, j * d:(j + 1) * d], want, atol=1e-14)
            np.testing.assert_allclose(lse[beta, j], np.log(np.arange(1, s + 1)), atol=1e-14)
    # s = 1: the only visible key is the token itself -> O = V of the group's KV head
    O1, _ = att.core(g.standard_normal((3, n_q * d)), K[:3], V[:3], b=3, s=1, n_q=n_q, n_kv=n_kv, d=d)
    for j in range(n_q):
        gh = j // 2
        np.testing.assert_allclose(O1[:, j * d:(j + 1) * d], V[:3, gh * d:(gh + 1) * d], atol=1e-15)
    # two keys with scaled scores 0 and ln 3: weights 1/4 and 3/4
    dd = 4
    q = np.zeros((2, dd)); q[1, 0] = 1.0
    k = np.zeros((2, dd)); k[1, 0] = math.log(3.0) * math.sqrt(dd)
    v = np.array([[1.0, 0, 0, 0], [0, 1.0, 0, 0]])
    O2, lse2 = att.core(q, k, v, b=1, s=2, n_q=1, n_kv=1, d=dd)
    np.testing.assert_allclose(O2[1], [0.25, 0.75, 0, 0], atol=1e-15)
    assert abs(lse2[0, 0, 1] - math.log(4.0)) < 1e-14


def test_attention_sum_over_ranks_equals_unsharded():
    """Head-sharded QKV + row-parallel out-projection: Sigma_i Z_i = Z ([L11] section 4)."""
    g = _rng(14)
    b, s, h, n_q, n_kv, d, t = 2, 7, 16, 8, 4, 4, 2
    X = g.standard_normal((b * s, h))
    Wq, Wk, Wv = (g.standard_normal((h, n * d)) / 4 for n in (n_q, n_kv, n_kv))
    Wo = g.standard_normal((n_q * d, h)) / 4
    full = att.forward(X, Wq, Wk, Wv, Wo, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)
    q, kv = n_q // t, n_kv // t
    Z = np.zeros_like(full["Z"])
    for i in range(t):
        Wqkv = np.concatenate([Wq[:, i * q * d:(i + 1) * q * d], Wk[:, i * kv * d:(i + 1) * kv * d],
                               Wv[:, i * kv * d:(i + 1) * kv * d]], 1)
        sh = att.shard_forward(X, Wqkv, Wo[i * q * d:(i + 1) * q * d], b=b, s=s, q=q, kv=kv, d=d)
        np.testing.assert_allclose(sh["O"], full["O"][:, i * q * d:(i + 1) * q * d], rtol=1e-13, atol=1e-14)
        Z += sh["Z"]
        rows = np.array([0, 3, 7, 13])
        sr = att.shard_forward_rows(X, Wqkv, Wo[i * q * d:(i + 1) * q * d], rows, b=b, s=s, q=q, kv=kv, d=d)
        np.testing.assert_allclose(sr["Z"], sh["Z"][rows], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(sr["lse"], sh["lse"].transpose(1, 0, 2).reshape(q, -1)[:, rows], atol=1e-12)
    np.testing.assert_allclose(Z, full["Z"], rtol=1e-12, atol=1e-13)


def _attn_case(seed, b=2, s=4, h=6, n_q=4, n_kv=2, d=3):
    g = _rng(seed)
    X = g.standard_normal((b * s, h))
    Wq, Wk, Wv = (g.standard_normal((h, n * d)) / 2 for n in (n_q, n_kv, n_kv))
    Wo = g.standard_normal((n_q * d, h)) / 2
    dZ = g.standard_normal((b * s, h))
    return dict(X=X, Wq=Wq, Wk=Wk, Wv=Wv, Wo=Wo, dZ=dZ, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)


def test_attention_backward_central_differences():
    """Every gradient of L = <dZ, Z> against central differences (GQA, causal, two sequences)."""
    c = _attn_case(21)
    kw = dict(b=c["b"], s=c["s"], n_q=c["n_q"], n_kv=c["n_kv"], d=c["d"])
    got = att.backward(c["dZ"], c["X"], c["Wq"], c["Wk"], c["Wv"], c["Wo"], **kw)
    names = ["X", "Wq", "Wk", "Wv", "Wo"]

    def loss():
        return float((att.forward(*(c[n] for n in names), **kw)["Z"] * c["dZ"]).sum())

    eps = 1e-6
    for n in names:
        arr = c[n]
        num = np.zeros_like(arr)
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            lp = loss()
            arr[idx] = keep - eps
            lm = loss()
            arr[idx] = keep
            num[idx] = (lp - lm) / (2 * eps)
        g = got["d" + n]
        assert np.abs(num - g).max() <= 1e-6 * np.abs(g).max(), n


def test_attention_backward_closed_forms():
    g = _rng(22)
    b, s, n_q, n_kv, d = 2, 6, 4, 2, 5
    group = n_q // n_kv
    K = g.standard_normal((b * s, n_kv * d))
    V = g.standard_normal((b * s, n_kv * d))
    dO = g.standard_normal((b * s, n_q * d))
    # Q = 0: every visible key has weight 1/(i+1), so dV[k] = sum over the group's heads and over
    # queries i >= k of dO[i] / (i+1), and dK = dS^T Q / sqrt(d) = 0.
    dQ, dK, dV = att.core_backward(np.zeros((b * s, n_q * d)), K, V, dO, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)
    np.testing.assert_allclose(dK, 0.0, atol=1e-15)
    for beta in range(b):
        for gh in range(n_kv):
            want = np.zeros((s, d))
            for j in range(gh * group, (gh + 1) * group):
                do = dO[beta * s:(beta + 1) * s, j * d:(j + 1) * d]
                w = do / np.arange(1, s + 1)[:, None]
                want += np.cumsum(w[::-1], 0)[::-1]
            np.testing.assert_allclose(dV[beta * s:(beta + 1) * s, gh * d:(gh + 1) * d], want, atol=1e-13)
    # s = 1: one visible key with weight 1 -> dS = 0, so dQ = dK = 0 and dV = the group's summed dO
    Q1 = g.standard_normal((3, n_q * d))
    dQ1, dK1, dV1 = att.core_backward(Q1, K[:3], V[:3], dO[:3], b=3, s=1, n_q=n_q, n_kv=n_kv, d=d)
    np.testing.assert_allclose(dQ1, 0.0, atol=1e-15)
    np.testing.assert_allclose(dK1, 0.0, atol=1e-15)
    for gh in range(n_kv):
        want = sum(dO[:3, j * d:(j + 1) * d] for j in range(gh * group, (gh + 1) * group))
        np.testing.assert_allclose(dV1[:, gh * d:(gh + 1) * d], want, atol=1e-15)


def test_attention_backward_shards_match_unsharded():
    """Rank i's dWqkv_i holds the unsharded dWq/dWk/dWv columns of its heads, dWo_i the
    unsharded dWo rows of its heads, and the backward all-reduce of dX_i gives dX
    ([TP1] operators f and g; [L11] section 4)."""
    g = _rng(23)
    b, s, h, n_q, n_kv, d, t = 2, 5, 12, 8, 4, 3, 2
    X = g.standard_normal((b * s, h))
    Wq, Wk, Wv = (g.standard_normal((h, n * d)) / 3 for n in (n_q, n_kv, n_kv))
    Wo = g.standard_normal((n_q * d, h)) / 3
    dZ = g.standard_normal((b * s, h))
    full = att.backward(dZ, X, Wq, Wk, Wv, Wo, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)
    q, kv = n_q // t, n_kv // t
    dX = np.zeros_like(full["dX"])
    for i in range(t):
        cq, ckv = slice(i * q * d, (i + 1) * q * d), slice(i * kv * d, (i + 1) * kv * d)
        Wqkv = np.concatenate([Wq[:, cq], Wk[:, ckv], Wv[:, ckv]], 1)
        sh = att.shard_backward(dZ, X, Wqkv, Wo[cq], b=b, s=s, q=q, kv=kv, d=d)
        want = np.concatenate([full["dWq"][:, cq], full["dWk"][:, ckv], full["dWv"][:, ckv]], 1)
        np.testing.assert_allclose(sh["dWqkv"], want, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sh["dWo"], full["dWo"][cq], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sh["dO"], full["dO"][:, cq], rtol=1e-12, atol=1e-12)
        dX += sh["dX"]
    np.testing.assert_allclose(dX, full["dX"], rtol=1e-11, atol=1e-12)


# ------------------------------------------------------------ uneven shards

def test_uneven_column_split_is_a_partition():
    for h_ffn, t, unit in [(512, 2, 1), (1000, 3, 8), (24, 2, 8), (40, 8, 8), (13, 4, 1), (12, 5, 4)]:
        got = [mlp.shard_cols(h_ffn, t, r, unit) for r in range(t)]
        assert got[0].start == 0 and got[-1].stop == h_ffn
        for a, b in zip(got, got[1:]):
            assert a.stop == b.start
        sizes = [c.stop - c.start for c in got]
        assert all(sz % unit == 0 for sz in sizes) and max(sizes) - min(sizes) <= unit
        assert sizes == sorted(sizes, reverse=True)
        if h_ffn % (t * unit) == 0:
            assert sizes == [h_ffn // t] * t


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_uneven_mlp_shards_match_unsharded(act):
    """Uneven (and empty) column shards: Sigma_i Z_i and Sigma_i dX_i equal the
    unsharded layer, the column pieces of H and dW1 concatenate to it, the row
    pieces of dW2 stack to it ([L11] sections 2-3 hold for any column split)."""
    g = _rng(41)
    T, h, hf = 5, 6, 13
    X = g.standard_normal((T, h))
    W1, Wu = g.standard_normal((h, hf)), g.standard_normal((h, hf))
    W2, b1 = g.standard_normal((hf, h)), g.standard_normal(hf)
    dOut = g.standard_normal((T, h))
    wu = Wu if act == "swiglu" else None
    bb = b1 if act == "gelu" else None
    full = mlp.forward(X, W1, W2, act=act, Wu=wu, b1=bb)
    fb = mlp.backward(dOut, X, W1, W2, act=act, Wu=wu, b1=bb)
    for t in (2, 3, 5, 16):
        Z = np.zeros((T, h))
        dX = np.zeros((T, h))
        Hs, dW1s, dW2s = [], [], []
        for r in range(t):
            c = mlp.shard_cols(hf, t, r)
            fw, bw = mlp.shard_step(dOut, X, W1[:, c], W2[c], act=act, Wu_i=None if wu is None else wu[:, c],
                                    b1_i=None if bb is None else bb[c])
            Z += fw["Z"]
            dX += bw["dX"]
            Hs.append(fw["H"])
            dW1s.append(bw["dW1"])
            dW2s.append(bw["dW2"])
        np.testing.assert_allclose(Z, full["Y"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dX, fb["dX"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(np.concatenate(Hs, 1), full["H"], rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(np.concatenate(dW1s, 1), fb["dW1"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(np.concatenate(dW2s, 0), fb["dW2"], rtol=1e-12, atol=1e-12)


def test_head_split_rules():
    """Every query head on exactly one rank, with its KV head local; KV heads
    either dealt out whole or replicated on t/n_kv ranks."""
    for n_q, n_kv, t in [(8, 2, 2), (12, 3, 2), (10, 5, 4), (8, 2, 4), (16, 4, 8), (32, 8, 8), (6, 6, 4), (8, 1, 8)]:
        group = n_q // n_kv
        owner = {}
        kv_owners = {}
        for r in range(t):
            q, kv, q0, kv0 = att.shard_heads(n_q, n_kv, t, r)
            for j in range(q0, q0 + q):
                assert j not in owner
                owner[j] = r
                assert kv0 <= j // group < kv0 + kv           # the head's KV head is local
            for gh in range(kv0, kv0 + kv):
                kv_owners.setdefault(gh, []).append(r)
        assert sorted(owner) == list(range(n_q))
        assert sorted(kv_owners) == list(range(n_kv))
        reps = {len(v) for v in kv_owners.values()}
        assert reps == ({1} if n_kv >= t else {t // n_kv})
    for bad in [(8, 3, 2), (12, 4, 8), (8, 2, 6), (8, 4, 6)]:
        with pytest.raises(ValueError):
            att.shard_heads(*bad, 0)


@pytest.mark.parametrize("n_q,n_kv,t", [(12, 3, 2), (8, 2, 4), (16, 2, 8), (10, 5, 3)])
def test_uneven_and_replicated_attention_shards_match_unsharded(n_q, n_kv, t):
    """Sigma_i Z_i = Z and Sigma_i dX_i = dX; the Q column blocks of dWqkv_i
    are the unsharded dWq columns of the rank's heads; the K/V blocks of the
    ranks that hold the same (replicated) KV head add up to its unsharded dWk,
    dWv (the gradient of a parameter replica is reduced over its replicas)."""
    if n_kv < t and (t % n_kv or (n_q // n_kv) % (t // n_kv)):
        pytest.skip("not a supported split")
    g = _rng(42)
    b, s, h, d = 2, 5, 12, 3
    X = g.standard_normal((b * s, h))
    Wq, Wk, Wv = (g.standard_normal((h, n * d)) / 3 for n in (n_q, n_kv, n_kv))
    Wo = g.standard_normal((n_q * d, h)) / 3
    dZ = g.standard_normal((b * s, h))
    full = att.forward(X, Wq, Wk, Wv, Wo, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)
    fb = att.backward(dZ, X, Wq, Wk, Wv, Wo, b=b, s=s, n_q=n_q, n_kv=n_kv, d=d)
    Z, dX = np.zeros_like(full["Z"]), np.zeros_like(fb["dX"])
    dWk, dWv = np.zeros_like(fb["dWk"]), np.zeros_like(fb["dWv"])
    for r in range(t):
        q, kv, q0, kv0 = att.shard_heads(n_q, n_kv, t, r)
        cq, ck = slice(q0 * d, (q0 + q) * d), slice(kv0 * d, (kv0 + kv) * d)
        Wqkv = np.concatenate([Wq[:, cq], Wk[:, ck], Wv[:, ck]], 1)
        Z += att.shard_forward(X, Wqkv, Wo[cq], b=b, s=s, q=q, kv=kv, d=d)["Z"]
        sh = att.shard_backward(dZ, X, Wqkv, Wo[cq], b=b, s=s, q=q, kv=kv, d=d)
        dX += sh["dX"]
        np.testing.assert_allclose(sh["dWqkv"][:, :q * d], fb["dWq"][:, cq], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(sh["dWo"], fb["dWo"][cq], rtol=1e-12, atol=1e-12)
        dWk[:, ck] += sh["dWqkv"][:, q * d:(q + kv) * d]
        dWv[:, ck] += sh["dWqkv"][:, (q + kv) * d:]
    np.testing.assert_allclose(Z, full["Z"], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(dX, fb["dX"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dWk, fb["dWk"], rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(dWv, fb["dWv"], rtol=1e-11, atol=1e-12)


# ------------------------------------------- fused residual and Megatron-SP

def _partials(seed, t=4, T=12, h=16):
    g = _rng(seed)
    return [g.standard_normal((T, h)) for _ in range(t)], g.standard_normal(h), g.standard_normal((T, h))


def test_residual_is_added_once_and_never_dropped():
    """With all partials and the bias zero, the block output is exactly the
    residual at any dropout rate and any t: the residual path is added once,
    after dropout ([LP] II.III fused bias + dropout + residual add)."""
    for t in (1, 3):
        P, b, R = _partials(31, t=t)
        Z = [np.zeros_like(p) for p in P]
        for p in (0.0, 0.1, 0.5):
            out = sp.sum_partials_residual(Z, np.zeros_like(b), p, 7, R)
            assert np.array_equal(out, R)


def test_residual_fusion_adds_the_residual_to_the_plain_all_reduce():
    P, b, R = _partials(32)
    for p in (0.0, 0.25):
        plain = mlp.sum_partials(P, b, p, 11)
        fused = sp.sum_partials_residual(P, b, p, 11, R)
        np.testing.assert_array_equal(fused, plain + R)
        np.testing.assert_array_equal(sp.sum_partials_residual(P, b, p, 11, None), plain)


def test_reduce_scatter_then_all_gather_equals_the_all_reduce():
    """[LP] III.III: the all-reduce split into reduce-scatter (token slices,
    token-wise bias/dropout/residual on the slice) and all-gather gives the
    same tensor, element for element, in rank order."""
    for t in (1, 2, 4):
        P, b, R = _partials(33 + t, t=t, T=4 * t + 8 * t, h=24)
        T = P[0].shape[0]
        for p in (0.0, 0.3):
            full = sp.sum_partials_residual(P, b, p, 5, R)
            slices = []
            for r in range(t):
                rows = sp.slice_rows(T, t, r)
                assert rows[0] == r * (T // t) and len(rows) == T // t
                slices.append(sp.reduce_scatter(P, t, r, b, p, 5, R[rows]))
            np.testing.assert_array_equal(sp.all_gather(slices), full)
    with pytest.raises(ValueError):
        sp.slice_rows(10, 4, 0)


def test_reduce_scatter_slices_partition_the_sum():
    """p = 0, no bias, no residual: the slices are the rows of sum_i P_i, and a
    slice does not depend on the other ranks' rows of the partials."""
    P, _, _ = _partials(36, t=4, T=16, h=8)
    for r in range(4):
        rows = sp.slice_rows(16, 4, r)
        got = sp.reduce_scatter(P, 4, r)
        np.testing.assert_array_equal(got, sum(p[rows] for p in P))
        Q = [p.copy() for p in P]
        for q in Q:
            q[np.setdiff1d(np.arange(16), rows)] = np.nan
        np.testing.assert_array_equal(sp.reduce_scatter(Q, 4, r), got)


# ---------------------------------------------------------------------- comm

def _ring_allreduce_bytes(t, n_per_chunk, delta, seed=0):
    """Simulate a ring all-reduce (reduce-scatter then all-gather) of t vectors
    and count the bytes each rank sends."""
    g = _rng(seed)
    data = [g.integers(-5, 5, size=t * n_per_chunk) for _ in range(t)]
    want = sum(data)
    buf = [d.copy().reshape(t, n_per_chunk) for d in data]
    sent = [0] * t
    for step in range(t - 1):        # reduce-scatter
        msgs = []
        for r in range(t):
            c = (r - step) % t
            msgs.append(((r + 1) % t, c, buf[r][c].copy()))
            sent[r] += n_per_chunk * delta
        for dst, c, v in msgs:
            buf[dst][c] += v
    for step in range(t - 1):        # all-gather
        msgs = []
        for r in range(t):
            c = (r + 1 - step) % t
            msgs.append(((r + 1) % t, c, buf[r][c].copy()))
            sent[r] += n_per_chunk * delta
        for dst, c, v in msgs:
            buf[dst][c] = v
    for r in range(t):
        np.testing.assert_array_equal(buf[r].reshape(-1), want)
    return sent


@pytest.mark.parametrize("t", [1, 2, 3, 4, 8])
def test_comm_bytes_against_simulated_ring(t):
    tokens, h, delta = 6, 4 * t, 2          # payload splits into t equal chunks
    r = comm.comm_bytes(tokens, h, t, delta)
    sent = _ring_allreduce_bytes(t, tokens * h // t, delta)
    assert all(x == sent[0] for x in sent)
    assert r["ring_bytes_per_rank"] == sent[0]
    assert r["payload_bytes"] == tokens * h * delta
    assert r["n_allreduce_fwd"] + r["n_allreduce_bwd"] == 4     # [L11] section 5; [TP1] communication cost
    assert r["layer_ring_bytes_per_rank"] == 4 * sent[0]


def test_comm_bytes_large_t_limit_and_dtypes():
    """[LP] II.II quotes 8 delta b S H per layer with (t-1)/t dropped."""
    r = comm.comm_bytes(4096, 4096, 10 ** 6, 2)
    assert abs(r["layer_ring_bytes_per_rank"] / (8 * 2 * 4096 * 4096) - 1) < 1e-5
    assert comm.comm_bytes(64, 128, 2, 4)["payload_bytes"] == 32768     # fp32, delta = 4
    assert comm.comm_bytes(64, 128, 1, 4)["ring_bytes_per_rank"] == 0


# --------------------------------------------------------------------- flops

def test_flops_match_page_totals():
    """[HJ]: GeLU MLP with d_ff = 4d: forward 16 B S d^2, backward 32 B S d^2,
    per rank /n; attention forward 8 B S d^2 + 4 B S^2 d without causal saving."""
    B, S, d = 3, 5, 8
    one = flops.mlp_shard(B * S, d, 4 * d, "gelu")
    assert one["fwd"] == 16 * B * S * d * d and one["bwd"] == 32 * B * S * d * d
    n = 4
    per = flops.mlp_shard(B * S, d, 4 * d // n, "gelu")
    assert per["fwd"] * n == one["fwd"] and per["bwd"] * n == one["bwd"]
    heads, dh = 2, d // 2
    a = flops.attention_shard_fwd(B, S, d, heads, heads, dh, causal=False)
    assert a["total"] == 8 * B * S * d * d + 4 * B * S * S * d
    ab = flops.attention_shard_bwd(B, S, d, heads, heads, dh, causal=False)
    assert ab["total"] == 16 * B * S * d * d + 8 * B * S * S * d


@pytest.mark.parametrize("s", [1, 2, 3, 5, 8, 17, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_pair_count_brute_force(s, causal):
    """The pairs the attention core is credited with ([HJ] Attention: QK^T and
    PV are 2 d FLOPs per computed pair) are the pairs the oracle's mask leaves
    visible.  Counted two ways that do not use the closed form: a loop over
    (query, key) positions, and the oracle's own attention with Q = 0, whose
    uniform weights make exp(lse) the number of visible keys of each row."""
    loop = sum(1 for sq in range(s) for sk in range(s) if (sk <= sq or not causal))
    g = _rng(900 + s)
    b, d = 2, 4
    K, V = g.standard_normal((b * s, d)), g.standard_normal((b * s, d))
    _, lse = att.core(np.zeros((b * s, d)), K, V, b=b, s=s, n_q=1, n_kv=1, d=d, causal=causal)
    counted = np.exp(lse)
    assert np.allclose(counted, np.rint(counted), atol=1e-9)
    per_seq = int(np.rint(counted).sum()) // b
    assert per_seq == loop
    assert flops.attention_pairs(s, causal) == loop
    q, dh = 3, 8
    core = flops.attention_shard_fwd(b, s, 16, q, 1, dh, causal)["core"]
    assert core == 4 * dh * b * q * loop
    # the product side's accounting (bench and the workload tables) counts the same pairs
    from attention_column_gemm_amd import flops as PF
    assert PF.causal_pairs(s, causal) == loop
    assert PF.attn_core(b, s, q, dh, causal) == core
    assert PF.attn_shard_fwd(b, s, 16, q, 1, dh, causal) == flops.attention_shard_fwd(b, s, 16, q, 1, dh,
                                                                                         causal)["total"]


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
def test_product_side_mlp_flops_match_oracle(act):
    from attention_column_gemm_amd import flops as PF
    for T, h, f in [(5, 6, 8), (8192, 8192, 3584), (4096, 4096, 1376)]:
        assert PF.mlp_shard(T, h, f, act) == flops.mlp_shard(T, h, f, act)["total"]


@pytest.mark.parametrize("act", ["gelu", "swiglu"])
@pytest.mark.parametrize("t", [2, 4])
def test_missing_rank_fails_the_sum_invariant(act, t):
    """Negative test of the Sigma-invariant ([L11] sections 2-3; [TP1]
    operators f and g): leaving any one rank's partial Z_i out of the forward
    sum, or its dX_i out of the backward sum, no longer gives the unsharded
    result, while the complete sums do."""
    c = _mlp_case(40 + t, act=act, bias=False)
    full = mlp.backward(c["dOut"], c["X"], c["W1"], c["W2"], act=act, Wu=c["Wu"])
    Zs, dXs = [], []
    for s in _shards(c, t, act):
        fw, bw = mlp.shard_step(c["dOut"], c["X"], s["W1"], s["W2"], act=act, Wu_i=s["Wu"])
        Zs.append(fw["Z"])
        dXs.append(bw["dX"])
    rel = lambda a, b: np.abs(a - b).max() / np.abs(b).max()
    assert rel(mlp.sum_partials(Zs), full["fwd"]["Out"]) < 1e-12
    assert rel(mlp.sum_partials(dXs), full["dX"]) < 1e-12
    for miss in range(t):
        keep = [i for i in range(t) if i != miss]
        assert rel(mlp.sum_partials([Zs[i] for i in keep]), full["fwd"]["Out"]) > 1e-3, miss
        assert rel(mlp.sum_partials([dXs[i] for i in keep]), full["dX"]) > 1e-3, miss


# ------------------------------------------------- norm on the token slice

def _norm_loops(x, kind, gamma, beta, eps):
    """Pure-Python loops, one token at a time, from the definitions."""
    out = []
    for row in x.tolist():
        n = len(row)
        if kind == "rms":
            ms = sum(v * v for v in row) / n
            r = 1.0 / math.sqrt(ms + eps)
            out.append([row[j] * r * gamma[j] for j in range(n)])
        else:
            mu = sum(row) / n
            var = sum((v - mu) ** 2 for v in row) / n
            r = 1.0 / math.sqrt(var + eps)
            out.append([(row[j] - mu) * r * gamma[j] + beta[j] for j in range(n)])
    return np.array(out)


@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_norm_brute_force(kind):
    g = _rng(50)
    x = g.standard_normal((5, 7)) * 3 + 1
    gamma, beta = g.standard_normal(7), g.standard_normal(7)
    eps = 1e-3
    got = sp.norm(x, kind, gamma, beta if kind == "layer" else None, eps)
    ref = _norm_loops(x, kind, gamma, beta if kind == "layer" else np.zeros(7), eps)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


def test_norm_closed_forms():
    """[3, 4, 0, 0]: RMS 2.5, so RMSNorm gives [1.2, 1.6, 0, 0]; mean 1.75 and
    variance 3.1875 for LayerNorm.  A constant row c maps to sign(c) gamma
    under RMSNorm (eps = 0) and to beta under LayerNorm.  RMSNorm of a
    zero-mean row is LayerNorm's with beta = 0."""
    x = np.array([[3.0, 4.0, 0.0, 0.0]])
    np.testing.assert_allclose(sp.rms_norm(x, eps=0.0), [[1.2, 1.6, 0.0, 0.0]], rtol=1e-15)
    ln = sp.layer_norm(x, eps=0.0)
    np.testing.assert_allclose(ln, (x - 1.75) / math.sqrt(3.1875), rtol=1e-14)
    gamma, beta = np.array([1.0, -2.0, 0.5, 3.0]), np.array([0.1, 0.2, -0.3, 0.4])
    for c in (2.5, -0.75):
        row = np.full((1, 4), c)
        np.testing.assert_allclose(sp.rms_norm(row, gamma, eps=0.0), [np.sign(c) * gamma], rtol=1e-15)
        np.testing.assert_array_equal(sp.layer_norm(row, gamma, beta, eps=1e-5), [beta])
    g = _rng(51)
    z = g.standard_normal((3, 6))
    z -= z.mean(axis=1, keepdims=True)
    np.testing.assert_allclose(sp.rms_norm(z, gamma=np.arange(6.0), eps=1e-4),
                               sp.layer_norm(z, gamma=np.arange(6.0), eps=1e-4), rtol=1e-13, atol=1e-14)


@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_norm_invariants(kind):
    """Scale invariance norm(c x) = norm(x) for c > 0 (eps = 0); unit RMS
    (RMSNorm) or zero mean and unit variance (LayerNorm) with gamma = 1."""
    g = _rng(52)
    x = g.standard_normal((4, 32)) + 0.5
    for c in (0.01, 3.0, 1e4):
        np.testing.assert_allclose(sp.norm(c * x, kind, eps=0.0), sp.norm(x, kind, eps=0.0), rtol=1e-12)
    y = sp.norm(x, kind, eps=0.0)
    if kind == "rms":
        np.testing.assert_allclose(np.sqrt((y * y).mean(axis=1)), 1.0, rtol=1e-13)
    else:
        np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-14)
        np.testing.assert_allclose(y.var(axis=1), 1.0, rtol=1e-13)


def test_norm_matches_torch_reference_routines():
    """Special cases that reduce to library routines: torch's layer_norm and
    rms_norm in float64 on the CPU."""
    import torch
    g = _rng(53)
    x = g.standard_normal((6, 40)) * 2
    gamma, beta = g.standard_normal(40), g.standard_normal(40)
    tx = torch.from_numpy(x)
    ln = torch.nn.functional.layer_norm(tx, (40,), torch.from_numpy(gamma), torch.from_numpy(beta), eps=1e-5)
    np.testing.assert_allclose(sp.layer_norm(x, gamma, beta, 1e-5), ln.numpy(), rtol=1e-12, atol=1e-12)
    rn = torch.nn.functional.rms_norm(tx, (40,), torch.from_numpy(gamma), eps=1e-6)
    np.testing.assert_allclose(sp.rms_norm(x, gamma, 1e-6), rn.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("kind", ["rms", "layer"])
def test_norm_on_slices_equals_norm_of_the_all_reduce(kind):
    """[LP] III.III: the token-wise norm on each rank's slice, then the
    all-gather, gives the norm of the full all-reduce, element for element;
    the residual slices gather to the full block output."""
    g = _rng(54)
    for t in (1, 2, 4):
        P, b, R = _partials(55 + t, t=t, T=6 * t, h=20)
        gamma, beta = g.standard_normal(20), (g.standard_normal(20) if kind == "layer" else None)
        T = P[0].shape[0]
        for p in (0.0, 0.2):
            full_out, full_n = sp.sum_partials_norm(P, b, p, 9, R, kind, gamma, beta, 1e-5)
            outs, normeds = [], []
            for r in range(t):
                rows = sp.slice_rows(T, t, r)
                o, n = sp.reduce_scatter_norm(P, t, r, b, p, 9, R[rows], kind, gamma, beta, 1e-5)
                outs.append(o)
                normeds.append(n)
            np.testing.assert_array_equal(sp.all_gather(outs), full_out)
            np.testing.assert_array_equal(sp.all_gather(normeds), full_n)
            np.testing.assert_allclose(full_n, sp.norm(sp.sum_partials_residual(P, b, p, 9, R), kind, gamma, beta,
                                                       1e-5), rtol=0, atol=0)
    with pytest.raises(ValueError):
        sp.norm(np.ones((1, 3)), "rms", None, np.ones(3))
    with pytest.raises(ValueError):
        sp.norm(np.ones((1, 3)), "batch")
