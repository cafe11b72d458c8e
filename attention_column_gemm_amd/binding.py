"""Thin ctypes binding of libtpshard (include/tp_shard.h).

Argument marshalling only: tensors become device pointers, the stream becomes
a ``hipStream_t``, and a negative status becomes a :class:`TPError`.  Every
step of the computation runs in the library's HIP kernels; there is no
fallback.  Functions carry the C names and argument order.

Tensor arguments may be ``torch.Tensor`` objects on the GPU (their
``data_ptr()`` is passed), plain integers (raw device addresses) or ``None``
for optional NULL arguments.  ``stream=None`` means torch's current stream.
"""
from __future__ import annotations

import ctypes
import os
import re

from . import validate as V

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB_PATH = os.path.join(PKG, "libtpshard.so")
HEADER = os.path.join(ROOT, "include", "tp_shard.h")

TP_F32, TP_BF16 = 0, 1
TP_GELU, TP_SWIGLU = 0, 1
TP_OK, TP_EINVAL, TP_ENOTDIV, TP_EDTYPE, TP_EALIGN, TP_EHIP, TP_EUNSUPPORTED = 0, -1, -2, -3, -4, -5, -6
TP_ENOSCRATCH = -7
TP_TILE_AUTO, TP_TILE_LARGE, TP_TILE_SMALL, TP_TILE_TINY = 0, 1, 2, 3
TP_NORM_RMS, TP_NORM_LAYER = 0, 1


class TPError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


class tp_mlp_desc(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int64), ("h", ctypes.c_int64), ("h_ffn", ctypes.c_int64),
                ("t", ctypes.c_int32), ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("act", ctypes.c_int32)]


class tp_attn_desc(ctypes.Structure):
    _fields_ = [("b", ctypes.c_int64), ("s", ctypes.c_int64), ("h", ctypes.c_int64),
                ("n_q", ctypes.c_int32), ("n_kv", ctypes.c_int32), ("d", ctypes.c_int32), ("t", ctypes.c_int32),
                ("rank", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32)]


class tp_comm(ctypes.Structure):
    _fields_ = [("n_allreduce_fwd", ctypes.c_int32), ("n_allreduce_bwd", ctypes.c_int32),
                ("payload_bytes", ctypes.c_uint64), ("ring_bytes_per_rank", ctypes.c_double),
                ("layer_payload_bytes", ctypes.c_uint64), ("layer_ring_bytes_per_rank", ctypes.c_double)]


_lib = None
_VP = ctypes.c_void_p


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m attention_column_gemm_amd.build`")
        # torch first: its HIP libraries ask for libamdhip64 by file name, not by soname, so
        # loading this library (which asks for the soname) first would leave two HIP runtimes
        # in the process, and torch's tensors and streams would be foreign to the one that
        # launches the kernels here (every launch then fails).  Loaded after torch, the soname
        # resolves to torch's runtime.
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        L.tp_mlp_shard_fwd.argtypes = [ctypes.POINTER(tp_mlp_desc)] + [_VP] * 8 + [_VP]
        L.tp_mlp_shard_bwd.argtypes = ([ctypes.POINTER(tp_mlp_desc), _VP, ctypes.c_float, ctypes.c_uint64]
                                       + [_VP] * 6 + [_VP, _VP, _VP, _VP, _VP, _VP, _VP] + [_VP])
        L.tp_attn_shard_fwd.argtypes = [ctypes.POINTER(tp_attn_desc)] + [_VP] * 7 + [_VP]
        L.tp_attn_shard_bwd.argtypes = [ctypes.POINTER(tp_attn_desc)] + [_VP] * 13 + [_VP]
        L.tp_attn_shard_bwd_noalloc.argtypes = [ctypes.POINTER(tp_attn_desc)] + [_VP] * 12 + [_VP]
        L.tp_sum_partials.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(_VP), _VP, ctypes.c_float, ctypes.c_uint64, _VP, _VP]
        L.tp_sum_partials_residual.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                               ctypes.POINTER(_VP), _VP, ctypes.c_float, ctypes.c_uint64, _VP,
                                               _VP, _VP]
        L.tp_reduce_scatter.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.c_int32, ctypes.POINTER(_VP), _VP, ctypes.c_float, ctypes.c_uint64,
                                        _VP, _VP, _VP]
        L.tp_sum_partials_norm.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(_VP), _VP, ctypes.c_float, ctypes.c_uint64, _VP,
                                           ctypes.c_int32, _VP, _VP, ctypes.c_float, _VP, _VP, _VP]
        L.tp_reduce_scatter_norm.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.POINTER(_VP), _VP, ctypes.c_float,
                                             ctypes.c_uint64, _VP, ctypes.c_int32, _VP, _VP, ctypes.c_float, _VP,
                                             _VP, _VP]
        L.tp_all_gather.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.POINTER(_VP), _VP, _VP]
        L.tp_mlp_shard_cols.argtypes = [ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                        ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
        L.tp_attn_shard_heads.argtypes = [ctypes.c_int32] * 4 + [ctypes.POINTER(ctypes.c_int32)] * 4
        L.tp_comm_bytes.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.POINTER(tp_comm)]
        L.tp_set_options.argtypes = [ctypes.c_int32, ctypes.c_int32]
        L.tp_get_options.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
        L.tp_profile_arm.argtypes = [ctypes.POINTER(_VP), ctypes.c_int32]
        L.tp_status_string.argtypes = [ctypes.c_int]
        L.tp_status_string.restype = ctypes.c_char_p
        for name in ("tp_mlp_shard_fwd", "tp_mlp_shard_bwd", "tp_attn_shard_fwd", "tp_attn_shard_bwd",
                     "tp_attn_shard_bwd_noalloc",
                     "tp_sum_partials", "tp_sum_partials_residual", "tp_reduce_scatter", "tp_all_gather",
                     "tp_sum_partials_norm", "tp_reduce_scatter_norm", "tp_mlp_shard_cols", "tp_attn_shard_heads", "tp_comm_bytes", "tp_set_options",
                     "tp_get_options", "tp_profile_arm"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def declared_functions() -> list:
    """Names of the functions include/tp_shard.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(tp_\w+)\s*\(", text, flags=re.M)))


def status_string(status: int) -> str:
    return lib().tp_status_string(int(status)).decode()


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        if hasattr(x, "is_cuda") and not x.is_cuda:
            raise ValueError("tensor arguments must live in GPU memory")
        if hasattr(x, "is_contiguous") and not x.is_contiguous():
            raise ValueError("tensor arguments must be contiguous (the library reads dense row-major memory)")
        return x.data_ptr()
    raise TypeError(f"cannot pass {type(x)} as a device pointer")


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc: int, where: str):
    if rc != TP_OK:
        raise TPError(rc, where)


def _mlp_sizes(desc):
    """(T, h, f, n_saved) of a descriptor, or None when the library would reject it anyway."""
    try:
        f, _ = tp_mlp_shard_cols(desc.h_ffn, desc.t, desc.rank, desc.dtype)
    except (TPError, ctypes.ArgumentError):
        return None
    return desc.tokens, desc.h, f, (1 if desc.act == TP_GELU else 2)


def _attn_sizes(desc):
    """(T, h, q*d, (q+2kv)*d, b*q*s) of a descriptor, or None when the library would reject it anyway."""
    try:
        q, kv, _, _ = tp_attn_shard_heads(desc.n_q, desc.n_kv, desc.t, desc.rank)
    except (TPError, ctypes.ArgumentError):
        return None
    return desc.b * desc.s, desc.h, q * desc.d, (q + 2 * kv) * desc.d, desc.b * q * desc.s


def _need(code, **sized):
    for name, (x, n) in sized.items():
        V.at_least(name, x, n, code)


def _need_f32(**sized):
    for name, (x, n) in sized.items():
        V.at_least_f32(name, x, n)


def tp_mlp_shard_fwd(desc: tp_mlp_desc, X, W1_i, Wu_i, b1_i, W2_i, saved_i, H_i, Z_i, stream=None):
    z = _mlp_sizes(desc)
    if z:
        T, h, f, ns = z
        _need(desc.dtype, X=(X, T * h), W1_i=(W1_i, h * f), Wu_i=(Wu_i, h * f), b1_i=(b1_i, f), W2_i=(W2_i, f * h),
              saved_i=(saved_i, ns * T * f), H_i=(H_i, T * f), Z_i=(Z_i, T * h))
    _check(lib().tp_mlp_shard_fwd(ctypes.byref(desc), _ptr(X), _ptr(W1_i), _ptr(Wu_i), _ptr(b1_i), _ptr(W2_i),
                                  _ptr(saved_i), _ptr(H_i), _ptr(Z_i), _stream(stream)), "tp_mlp_shard_fwd")


def tp_mlp_shard_bwd(desc: tp_mlp_desc, dOut, p_drop: float, seed: int, X, W1_i, Wu_i, W2_i, saved_i, H_i,
                     dY, db2, dA_i, dW1_i, db1_i, dW2_i, dX_i, stream=None):
    z = _mlp_sizes(desc)
    if z:
        T, h, f, ns = z
        _need(desc.dtype, dOut=(dOut, T * h), X=(X, T * h), W1_i=(W1_i, h * f), Wu_i=(Wu_i, h * f),
              W2_i=(W2_i, f * h), saved_i=(saved_i, ns * T * f), H_i=(H_i, T * f), dY=(dY, T * h),
              dA_i=(dA_i, ns * T * f), dX_i=(dX_i, T * h))
        _need_f32(db2=(db2, h), dW1_i=(dW1_i, ns * h * f), db1_i=(db1_i, f), dW2_i=(dW2_i, f * h))
    _check(lib().tp_mlp_shard_bwd(ctypes.byref(desc), _ptr(dOut), float(p_drop), int(seed) & (2 ** 64 - 1),
                                  _ptr(X), _ptr(W1_i), _ptr(Wu_i), _ptr(W2_i), _ptr(saved_i), _ptr(H_i), _ptr(dY),
                                  _ptr(db2), _ptr(dA_i), _ptr(dW1_i), _ptr(db1_i), _ptr(dW2_i), _ptr(dX_i),
                                  _stream(stream)), "tp_mlp_shard_bwd")


def tp_attn_shard_fwd(desc: tp_attn_desc, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, Z_i, stream=None):
    z = _attn_sizes(desc)
    if z:
        T, h, nq, nqkv, rows = z
        _need(TP_BF16, X=(X, T * h), Wqkv_i=(Wqkv_i, h * nqkv), Wo_i=(Wo_i, nq * h), QKV_i=(QKV_i, T * nqkv),
              O_i=(O_i, T * nq), Z_i=(Z_i, T * h))
        _need_f32(lse_i=(lse_i, rows))
    _check(lib().tp_attn_shard_fwd(ctypes.byref(desc), _ptr(X), _ptr(Wqkv_i), _ptr(Wo_i), _ptr(QKV_i), _ptr(O_i),
                                   _ptr(lse_i), _ptr(Z_i), _stream(stream)), "tp_attn_shard_fwd")


def tp_attn_shard_bwd(desc: tp_attn_desc, dZ, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dO_i, stats_i, dQKV_i, dWqkv_i,
                      dWo_i, dX_i, stream=None):
    z = _attn_sizes(desc)
    if z:
        T, h, nq, nqkv, rows = z
        _need(TP_BF16, dZ=(dZ, T * h), X=(X, T * h), Wqkv_i=(Wqkv_i, h * nqkv), Wo_i=(Wo_i, nq * h),
              QKV_i=(QKV_i, T * nqkv), O_i=(O_i, T * nq), dO_i=(dO_i, T * nq), dQKV_i=(dQKV_i, T * nqkv),
              dX_i=(dX_i, T * h))
        _need_f32(lse_i=(lse_i, rows), stats_i=(stats_i, 2 * rows), dWqkv_i=(dWqkv_i, h * nqkv),
                  dWo_i=(dWo_i, nq * h))
    _check(lib().tp_attn_shard_bwd(ctypes.byref(desc), _ptr(dZ), _ptr(X), _ptr(Wqkv_i), _ptr(Wo_i), _ptr(QKV_i),
                                   _ptr(O_i), _ptr(lse_i), _ptr(dO_i), _ptr(stats_i), _ptr(dQKV_i), _ptr(dWqkv_i),
                                   _ptr(dWo_i), _ptr(dX_i), _stream(stream)), "tp_attn_shard_bwd")


def tp_attn_shard_bwd_noalloc(desc: tp_attn_desc, dZ, X, Wqkv_i, Wo_i, QKV_i, O_i, lse_i, dO_i, dQKV_i, dWqkv_i,
                              dWo_i, dX_i, stream=None):
    z = _attn_sizes(desc)
    if z:
        T, h, nq, nqkv, rows = z
        _need(TP_BF16, dZ=(dZ, T * h), X=(X, T * h), Wqkv_i=(Wqkv_i, h * nqkv), Wo_i=(Wo_i, nq * h),
              QKV_i=(QKV_i, T * nqkv), O_i=(O_i, T * nq), dO_i=(dO_i, T * nq), dQKV_i=(dQKV_i, T * nqkv),
              dX_i=(dX_i, T * h))
        _need_f32(lse_i=(lse_i, rows), dWqkv_i=(dWqkv_i, h * nqkv), dWo_i=(dWo_i, nq * h))
    _check(lib().tp_attn_shard_bwd_noalloc(ctypes.byref(desc), _ptr(dZ), _ptr(X), _ptr(Wqkv_i), _ptr(Wo_i),
                                           _ptr(QKV_i), _ptr(O_i), _ptr(lse_i), _ptr(dO_i), _ptr(dQKV_i),
                                           _ptr(dWqkv_i), _ptr(dWo_i), _ptr(dX_i), _stream(stream)),
           "tp_attn_shard_bwd_noalloc")


def _need_list(code, name, xs, n):
    for i, x in enumerate(xs):
        V.at_least(f"{name}[{i}]", x, n, code)


def tp_sum_partials(rows: int, cols: int, t: int, dtype: int, partials, bias, p_drop: float, seed: int, out,
                    stream=None):
    _need_list(dtype, "partials", partials, rows * cols)
    _need(dtype, bias=(bias, cols), out=(out, rows * cols))
    arr = (_VP * max(1, len(partials)))(*[_ptr(p) for p in partials])
    _check(lib().tp_sum_partials(int(rows), int(cols), int(t), int(dtype), arr, _ptr(bias), float(p_drop),
                                 int(seed) & (2 ** 64 - 1), _ptr(out), _stream(stream)), "tp_sum_partials")


def tp_sum_partials_residual(rows: int, cols: int, t: int, dtype: int, partials, bias, p_drop: float, seed: int,
                             residual, out, stream=None):
    _need_list(dtype, "partials", partials, rows * cols)
    _need(dtype, bias=(bias, cols), residual=(residual, rows * cols), out=(out, rows * cols))
    arr = (_VP * max(1, len(partials)))(*[_ptr(p) for p in partials])
    _check(lib().tp_sum_partials_residual(int(rows), int(cols), int(t), int(dtype), arr, _ptr(bias), float(p_drop),
                                          int(seed) & (2 ** 64 - 1), _ptr(residual), _ptr(out), _stream(stream)),
           "tp_sum_partials_residual")


def tp_reduce_scatter(rows: int, cols: int, t: int, rank: int, dtype: int, partials, bias, p_drop: float, seed: int,
                      residual_r, out_r, stream=None):
    _need_list(dtype, "partials", partials, rows * cols)
    n = rows // t if t > 0 else 0
    _need(dtype, bias=(bias, cols), residual_r=(residual_r, n * cols), out_r=(out_r, n * cols))
    arr = (_VP * max(1, len(partials)))(*[_ptr(p) for p in partials])
    _check(lib().tp_reduce_scatter(int(rows), int(cols), int(t), int(rank), int(dtype), arr, _ptr(bias),
                                   float(p_drop), int(seed) & (2 ** 64 - 1), _ptr(residual_r), _ptr(out_r),
                                   _stream(stream)), "tp_reduce_scatter")


def tp_sum_partials_norm(rows: int, cols: int, t: int, dtype: int, partials, bias, p_drop: float, seed: int,
                         residual, norm: int, gamma, beta, eps: float, out, normed, stream=None):
    _need_list(dtype, "partials", partials, rows * cols)
    _need(dtype, bias=(bias, cols), residual=(residual, rows * cols), gamma=(gamma, cols), beta=(beta, cols),
          out=(out, rows * cols), normed=(normed, rows * cols))
    arr = (_VP * max(1, len(partials)))(*[_ptr(p) for p in partials])
    _check(lib().tp_sum_partials_norm(int(rows), int(cols), int(t), int(dtype), arr, _ptr(bias), float(p_drop),
                                      int(seed) & (2 ** 64 - 1), _ptr(residual), int(norm), _ptr(gamma), _ptr(beta),
                                      float(eps), _ptr(out), _ptr(normed), _stream(stream)), "tp_sum_partials_norm")


def tp_reduce_scatter_norm(rows: int, cols: int, t: int, rank: int, dtype: int, partials, bias, p_drop: float,
                           seed: int, residual_r, norm: int, gamma, beta, eps: float, out_r, normed_r, stream=None):
    _need_list(dtype, "partials", partials, rows * cols)
    n = rows // t if t > 0 else 0
    _need(dtype, bias=(bias, cols), residual_r=(residual_r, n * cols), gamma=(gamma, cols), beta=(beta, cols),
          out_r=(out_r, n * cols), normed_r=(normed_r, n * cols))
    arr = (_VP * max(1, len(partials)))(*[_ptr(p) for p in partials])
    _check(lib().tp_reduce_scatter_norm(int(rows), int(cols), int(t), int(rank), int(dtype), arr, _ptr(bias),
                                        float(p_drop), int(seed) & (2 ** 64 - 1), _ptr(residual_r), int(norm),
                                        _ptr(gamma), _ptr(beta), float(eps), _ptr(out_r), _ptr(normed_r),
                                        _stream(stream)), "tp_reduce_scatter_norm")


def tp_all_gather(rows_per_rank: int, cols: int, t: int, dtype: int, slices, out, stream=None):
    _need_list(dtype, "slices", slices, rows_per_rank * cols)
    _need(dtype, out=(out, t * rows_per_rank * cols))
    arr = (_VP * max(1, len(slices)))(*[_ptr(p) for p in slices])
    _check(lib().tp_all_gather(int(rows_per_rank), int(cols), int(t), int(dtype), arr, _ptr(out), _stream(stream)),
           "tp_all_gather")


def tp_set_options(tile: int = TP_TILE_AUTO, split_tail: int = 1):
    _check(lib().tp_set_options(int(tile), int(split_tail)), "tp_set_options")


def tp_get_options():
    """(tile, split_tail) currently in force."""
    a, b = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().tp_get_options(ctypes.byref(a), ctypes.byref(b)), "tp_get_options")
    return a.value, b.value


class options:
    """Context manager: ``with options(tile=TP_TILE_SMALL, split_tail=0): ...``
    sets the library's launch options and restores the previous ones on exit."""

    def __init__(self, tile=None, split_tail=None):
        self.tile, self.split_tail = tile, split_tail

    def __enter__(self):
        self.saved = tp_get_options()
        tp_set_options(self.saved[0] if self.tile is None else self.tile,
                       self.saved[1] if self.split_tail is None else self.split_tail)
        return self

    def __exit__(self, *exc):
        tp_set_options(*self.saved)
        return False


def tp_mlp_shard_cols(h_ffn: int, t: int, rank: int, dtype: int):
    """(f_i, col0): the intermediate columns rank ``rank`` owns."""
    f, c0 = ctypes.c_int64(), ctypes.c_int64()
    _check(lib().tp_mlp_shard_cols(int(h_ffn), int(t), int(rank), int(dtype), ctypes.byref(f), ctypes.byref(c0)),
           "tp_mlp_shard_cols")
    return f.value, c0.value


def tp_attn_shard_heads(n_q: int, n_kv: int, t: int, rank: int):
    """(q_i, kv_i, q0, kv0): the heads rank ``rank`` owns."""
    v = [ctypes.c_int32() for _ in range(4)]
    _check(lib().tp_attn_shard_heads(int(n_q), int(n_kv), int(t), int(rank), *[ctypes.byref(x) for x in v]),
           "tp_attn_shard_heads")
    return tuple(x.value for x in v)


def tp_comm_bytes(tokens: int, h: int, t: int, delta: int) -> tp_comm:
    out = tp_comm()
    _check(lib().tp_comm_bytes(int(tokens), int(h), int(t), int(delta), ctypes.byref(out)), "tp_comm_bytes")
    return out


def mlp_desc(tokens, h, h_ffn, t, rank=0, dtype=TP_BF16, act=TP_GELU) -> tp_mlp_desc:
    return tp_mlp_desc(tokens, h, h_ffn, t, rank, dtype, act)


def attn_desc(b, s, h, n_q, n_kv, d, t, rank=0, dtype=TP_BF16, causal=1) -> tp_attn_desc:
    return tp_attn_desc(b, s, h, n_q, n_kv, d, t, rank, dtype, causal)
