"""Shared helpers of the GPU parity tests (not a test module).

Error metric (one number per output tensor): ``max|gpu - ref| / max|ref|``,
the largest deviation relative to the tensor's largest reference magnitude.
Element-wise relative error is ill-posed where the reference is ~0 (GeLU and
dropout zeros), so the norm-wise form is the gate.  Bars: 1e-4 for tensors
stored in fp32 end to end, 2e-2 for bf16 storage with fp32 accumulation,
against the float64 oracle.
"""
import sys

import numpy as np
import pytest

TOL = {"fp32": 1e-4, "bf16": 2e-2}


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    from attention_column_gemm_amd import binding
    binding.lib()  # raises when the HIP library is missing: never silently skipped
    return torch


def rel_err(gpu, ref) -> float:
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if ref.size == 0:
        return 0.0
    den = np.abs(ref).max()
    num = np.abs(gpu - ref).max()
    if den == 0.0:
        return float(num)
    return float(num / den)


def check(name, gpu, ref, tol, log=None):
    e = rel_err(gpu, ref)
    msg = f"  {name:<24s} max-rel-err {e:.3e} (bar {tol:.0e})"
    print(msg, flush=True)
    if log is not None:
        log.append((name, e))
    assert np.all(np.isfinite(np.asarray(gpu, dtype=np.float64))), f"{name}: non-finite values"
    assert e <= tol, msg


def banner(text):
    print(f"\n[gpu-case] {text}", flush=True)
    sys.stdout.flush()


def edge_indices(n, tiles=(32, 64, 128, 256), extra=0, seed=0):
    """Sample indices: both ends, both sides of each tile edge, plus random ones."""
    s = {0, n - 1}
    for t in tiles:
        for k in list(range(t, n, t))[:6] + [(n - 1) // t * t]:
            if 0 < k < n:
                s.update({k - 1, k})
    rng = np.random.default_rng(seed)
    if extra:
        s.update(rng.integers(0, n, size=extra).tolist())
    return np.array(sorted(i for i in s if 0 <= i < n))
