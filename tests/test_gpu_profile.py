"""The per-kernel profiling hook (tp_profile_arm) on a real launch sequence:
each armed event pair spans its kernels in order and the hook changes no
result."""
import ctypes

import pytest

from attention_column_gemm_amd import binding as B
from attention_column_gemm_amd import inputs as I
from parity import banner, need_gpu

pytestmark = pytest.mark.gpu


def test_profile_hook_brackets_each_forward_kernel():
    torch = need_gpu()
    from attention_column_gemm_amd.shard import MLPShard
    c = I.custom_mlp(106, 2, 256, 512, 2048, 2, "swiglu", "bf16")
    banner(f"profile hook: SwiGLU MLP forward T={c.tokens} h={c.h} h_ffn={c.h_ffn} t={c.t}")
    X, dOut = I.mlp_activation(c)
    w = I.mlp_rank_weights(c, 0)
    sh = MLPShard(c.tokens, c.h, c.h_ffn, c.t, 0, act=c.act, dtype=c.dtype)
    sh.load(X, w["W1"], w["Wu"], w["b1"], w["W2"], dOut)
    sh.forward()
    torch.cuda.synchronize()
    ref_H, ref_Z = sh.H.clone(), sh.Z.clone()

    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
    ev = []
    for _ in range(4):  # two scopes: the column GEMM (with its epilogue) and the row GEMM
        e = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(e)) == 0
        ev.append(e)

    def ms(a, b):
        f = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(f), a, b) == 0
        return f.value

    try:
        arr = (ctypes.c_void_p * 4)(*[e.value for e in ev])
        assert B.lib().tp_profile_arm(arr, 4) == B.TP_OK
        sh.forward()
        sh.forward()   # the hook disarmed itself after two scopes: this call launches plainly
        torch.cuda.synchronize()
        col, row, gap = ms(ev[0], ev[1]), ms(ev[2], ev[3]), ms(ev[1], ev[2])
        print(f"  column GEMM {col * 1e3:.1f} us, row GEMM {row * 1e3:.1f} us, between {gap * 1e3:.1f} us", flush=True)
        assert 0.0 < col < 1000.0 and 0.0 < row < 1000.0
        assert gap >= 0.0, "the second scope started before the first one ended"
        assert torch.equal(sh.H, ref_H) and torch.equal(sh.Z, ref_Z), "the hook changed a result"
    finally:
        B.lib().tp_profile_arm(None, 0)
        for e in ev:
            hip.hipEventDestroy(e)
