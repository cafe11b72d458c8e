"""Host-side checks of tensor arguments, made before anything is handed to
the library.

The C ABI sees raw device pointers, so it cannot tell a tensor's dtype,
shape or layout; a wrong one would make a kernel read past an allocation.
These checks run on any torch tensor (CPU tensors included, so they are
testable without a GPU) and raise ``TypeError`` for a storage type the
library does not take and ``ValueError`` for everything else.
"""
from __future__ import annotations

TP_F32, TP_BF16 = 0, 1


def storage_code(dtype) -> int:
    """The library's storage code of a torch dtype: bf16 or fp32, nothing else."""
    import torch
    if dtype == torch.bfloat16:
        return TP_BF16
    if dtype == torch.float32:
        return TP_F32
    raise TypeError(f"storage type {dtype} is not provided (bf16 or fp32 only)")


def elem_bytes(code: int) -> int:
    return 2 if code == TP_BF16 else 4


def _dense(name, x):
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (the library reads dense row-major memory)")


def group(name, tensors):
    """Tensors that must agree: the same shape, storage type and device, all
    contiguous.  Returns (shape, storage code, device)."""
    tensors = list(tensors)
    if not tensors:
        raise ValueError(f"{name}: at least one tensor is required")
    x0 = tensors[0]
    code = storage_code(x0.dtype)
    for i, x in enumerate(tensors):
        if x is None:
            raise ValueError(f"{name}[{i}]: missing")
        _dense(f"{name}[{i}]", x)
        if x.dtype != x0.dtype:
            raise TypeError(f"{name}[{i}]: dtype {x.dtype} differs from {name}[0]'s {x0.dtype}")
        if x.device != x0.device:
            raise ValueError(f"{name}[{i}]: on {x.device}, {name}[0] on {x0.device}")
        if tuple(x.shape) != tuple(x0.shape):
            raise ValueError(f"{name}[{i}]: shape {tuple(x.shape)} differs from {name}[0]'s {tuple(x0.shape)}")
    return tuple(x0.shape), code, x0.device


def like(name, x, shape, dtype, device, optional=True):
    """``x`` must have exactly ``shape``, ``dtype`` and ``device`` and be
    contiguous (or be None when optional)."""
    if x is None:
        if optional:
            return
        raise ValueError(f"{name}: missing")
    _dense(name, x)
    if x.dtype != dtype:
        raise TypeError(f"{name}: dtype {x.dtype}, expected {dtype}")
    if x.device != device:
        raise ValueError(f"{name}: on {x.device}, expected {device}")
    if tuple(x.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(x.shape)}, expected {tuple(shape)}")


def vector(name, x, n, dtype, device):
    """An optional vector of exactly ``n`` elements (a bias)."""
    if x is None:
        return
    _dense(name, x)
    if x.dtype != dtype:
        raise TypeError(f"{name}: dtype {x.dtype}, expected {dtype}")
    if x.device != device:
        raise ValueError(f"{name}: on {x.device}, expected {device}")
    if x.numel() != n:
        raise ValueError(f"{name}: {x.numel()} elements, expected {n}")


def at_least(name, x, n_elems, code):
    """A tensor handed to the ABI as a raw pointer: storage type ``code`` and
    at least the ``n_elems`` elements the call will touch.  Integers (raw
    addresses) and None pass unchecked: the caller vouches for them."""
    if x is None or isinstance(x, int) or not hasattr(x, "numel"):
        return
    _dense(name, x)
    try:
        got = storage_code(x.dtype)
    except TypeError as e:
        raise TypeError(f"{name}: {e}") from None
    if got != code:
        raise TypeError(f"{name}: dtype {x.dtype} does not match the call's storage type")
    if x.numel() < n_elems:
        raise ValueError(f"{name}: {x.numel()} elements, the call touches {n_elems}")


def at_least_f32(name, x, n_elems):
    """As :func:`at_least` for the fp32-only outputs (weight and bias gradients, statistics)."""
    at_least(name, x, n_elems, TP_F32)
