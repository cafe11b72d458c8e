"""tp_attn_shard_bwd_noalloc (the attention backward with its per-row
statistics in the library's fixed device array) against tp_attn_shard_bwd on
the same inputs, and both against the float64 oracle: two calls in a row,
the second on a smaller problem, so the array holds the first call's
statistics when the second starts."""
import pytest

from attention_column_gemm_amd import inputs as I
from oracle import attention as OA
from parity import TOL, banner, check, need_gpu

pytestmark = pytest.mark.gpu

CASES = [
    # larger first: b=2, s=300, h=512, 8 q / 2 kv heads over t=2 (q=4, kv=1), d=128
    ("b2_s300_h512_gqa4_d128", I.custom_attn(501, 2, 300, 512, 8, 2, 128, 2)),
    # then smaller: b=1, s=130, h=256, 4 q / 2 kv heads, t=1, d=64 (ragged last blocks)
    ("b1_s130_h256_gqa2_d64", I.custom_attn(502, 1, 130, 256, 4, 2, 64, 1)),
]


def _outputs(torch, sh):
    T, h, d = sh.b * sh.s, sh.h, sh.d
    e = lambda *shape, dt=torch.bfloat16: torch.full(shape, float("nan"), dtype=dt, device="cuda")
    return dict(dO=e(T, sh.q * d), dQKV=e(T, (sh.q + 2 * sh.kv) * d),
                dWqkv=e(h, (sh.q + 2 * sh.kv) * d, dt=torch.float32), dWo=e(sh.q * d, h, dt=torch.float32),
                dX=e(T, h))


def test_noalloc_backward_matches_the_allocating_entry_point():
    torch = need_gpu()
    from attention_column_gemm_amd import binding as B
    from attention_column_gemm_amd.shard import AttnShard, to_device
    for name, c in CASES:
        banner(f"attention backward no-alloc {name}")
        X = I.attn_activation(c)
        w = I.attn_rank_weights(c, 0)
        dZ = to_device(I.attn_upstream_grad(c), "bf16")
        sh = AttnShard(c.b, c.s, c.h, c.n_q, c.n_kv, c.d, c.t, 0).load(X, w["Wqkv"], w["Wo"])
        sh.forward(want_lse=True)
        sh.backward(dZ)
        torch.cuda.synchronize()
        o = _outputs(torch, sh)
        B.tp_attn_shard_bwd_noalloc(sh.desc, dZ, sh.X, sh.Wqkv, sh.Wo, sh.QKV, sh.O, sh.lse, o["dO"], o["dQKV"],
                                    o["dWqkv"], o["dWo"], o["dX"])
        torch.cuda.synchronize()
        for k, ref in (("dO", sh.dO), ("dQKV", sh.dQKV), ("dWqkv", sh.dWqkv), ("dWo", sh.dWo), ("dX", sh.dX)):
            assert torch.equal(o[k], ref), f"{name}: {k} differs from tp_attn_shard_bwd"
        r = OA.shard_backward(I.attn_upstream_grad(c), X, w["Wqkv"], w["Wo"], b=c.b, s=c.s, q=c.q, kv=c.kv, d=c.d)
        for k in ("dO", "dQKV", "dWqkv", "dWo", "dX"):
            check(f"{name}.{k}", o[k].float().cpu().numpy(), r[k], TOL["bf16"])
        del sh, o

