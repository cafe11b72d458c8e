"""GPU parity of the emulated all-reduce (rank-ordered sum, bias once,
dropout) and bit-exactness of the dropout mask."""
import numpy as np
import pytest

from oracle import dropout as OD
from oracle import mlp as O
from parity import TOL, banner, check, need_gpu

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    from attention_column_gemm_amd.shard import to_device
    return to_device(a, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("t,rows,cols,p,bias", [
    (1, 7, 8, 0.0, False), (2, 64, 128, 0.0, True), (4, 37, 264, 0.1, True), (8, 300, 1024, 0.25, False),
    (3, 0, 16, 0.1, True),
])
def test_sum_partials_parity(dtype, t, rows, cols, p, bias):
    torch = need_gpu()
    banner(f"sum_partials {dtype} t={t} rows={rows} cols={cols} p={p} bias={bias}")
    from attention_column_gemm_amd.inputs import round_to_bf16
    from attention_column_gemm_amd.shard import sum_partials
    rng = np.random.default_rng(t * 1000 + cols)
    parts = [rng.standard_normal((rows, cols)).astype(np.float32) for _ in range(t)]
    b = rng.standard_normal(cols).astype(np.float32) if bias else None
    if dtype == "bf16":
        parts = [round_to_bf16(x) for x in parts]
        b = None if b is None else round_to_bf16(b)
    seed = 12345 + t
    out = sum_partials([_dev(x, dtype) for x in parts], _dev(b, dtype), p, seed)
    torch.cuda.synchronize()
    ref = O.sum_partials(parts, b, p, seed)
    check("out", out.float().cpu().numpy(), ref, TOL[dtype] if dtype == "bf16" else 1e-6)
    if p > 0 and rows > 0:
        # the kept set is an integer decision: bit-identical to the oracle's mask
        kept_gpu = out.float().cpu().numpy() != 0.0
        kept_ref = OD.keep_mask(seed, rows, cols, p) & (np.abs(sum(parts) + (0 if b is None else b)) > 0)
        np.testing.assert_array_equal(kept_gpu, kept_ref)


def test_dropout_mask_bitwise_large():
    """Mask of a [2048, 1024] output at p = 0.1 (the GPT-style workload)."""
    torch = need_gpu()
    banner("dropout mask [2048,1024] p=0.1")
    from attention_column_gemm_amd.shard import sum_partials
    ones = torch.ones(2048, 1024, dtype=torch.bfloat16, device="cuda")
    seed = 2099
    out = sum_partials([ones], None, 0.1, seed)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy()
    keep = OD.keep_mask(seed, 2048, 1024, 0.1)
    np.testing.assert_array_equal(got != 0.0, keep)
    # kept values carry the scale 1/(1 - p) rounded to bf16
    assert np.all(np.abs(got[keep] - 1.0 / 0.9) < 1.0 / 0.9 * 2 ** -8)


def test_dropout_mask_independent_of_t():
    """Summing the same total split over t = 1, 2, 4, 8 partials gives the same mask."""
    torch = need_gpu()
    banner("dropout mask vs t")
    from attention_column_gemm_amd.shard import sum_partials
    masks = []
    for t in (1, 2, 4, 8):
        parts = [torch.full((64, 256), 1.0 / t, dtype=torch.float32, device="cuda") for _ in range(t)]
        out = sum_partials(parts, None, 0.3, 77)
        torch.cuda.synchronize()
        masks.append(out.cpu().numpy() != 0)
    for m in masks[1:]:
        np.testing.assert_array_equal(m, masks[0])
    np.testing.assert_array_equal(masks[0], OD.keep_mask(77, 64, 256, 0.3))
