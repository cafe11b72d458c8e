"""Benchmark: one TP rank's layer shard on one MI355X, through the C ABI.

A step is one pass of the whole hot path for rank 0 of the chosen workload:
attention shard forward (QKV GEMM, causal GQA attention, output projection),
its emulated all-reduce, the MLP shard forward, its emulated all-reduce, the
MLP shard backward and its emulated all-reduce, the attention shard backward
(taking the reduced MLP input gradient as its upstream gradient) and its
emulated all-reduce, plus the host-side all-reduce accounting.  Inputs are
seeded synthetic tensors already resident in HBM when timing starts.

The reported metric is the per-rank MLP forward+backward throughput
(algorithmic FLOPs 18*T*h*f for SwiGLU, 12*T*h*f for GeLU, over the measured
time of the MLP shard's forward and backward calls) and its fraction of the
MI355X bf16 dense matrix-core peak; every kernel's time, the emulated
all-reduces' HBM bandwidth and the attention shard are reported beside it.

Beside it, outside the step, the block-closing all-reduce with the residual
add fused and its Megatron-SP split (one rank's reduce-scatter, the
all-gather) are timed at the same [T, h] shape, and rank 0 of two uneven
splits (an FFN width t does not divide, KV heads replicated over ranks).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload cfg5|cfg3|cfg2] [--no-cpu] [--no-extras]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from attention_column_gemm_amd import flops as F  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 matrix-core peak (published)
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E bandwidth (published)
METRIC = "per-rank TP MLP fwd+bwd TFLOP/s and % of bf16 MFMA peak on 1 MI355X"

WORKLOADS = {
    # name: (mlp config id, attention config id or None)
    "cfg5": (5, 5),
    "cfg3": (3, 4),
    "cfg2": (2, None),
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "attention_column_gemm_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


class HipEvents:
    """Raw hipEvent_t handles for the library's per-kernel profiling hook."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e)
        return evs

    def elapsed_ms(self, a, b) -> float:
        f = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(f), a, b)
        assert rc == 0, f"hipEventElapsedTime failed ({rc})"
        return f.value


def kernel_plan(mc, ac):
    """Kernels one step enqueues, in order: (label, row, flops, bytes)."""
    T, h, f = mc.tokens, mc.h, mc.f
    d = 2 if mc.bf16 else 4
    plan = []
    if ac is not None:
        Ta, ha, q, kv, dh = ac.tokens, ac.h, ac.q, ac.kv, ac.d
        plan += [("attn_qkv_gemm", "a8", 2 * Ta * ha * (q + 2 * kv) * dh, None),
                 ("attn_core", "a8", F.attn_core(ac.b, ac.s, q, dh), None),
                 ("attn_out_gemm", "a8", 2 * Ta * q * dh * ha, None),
                 ("allreduce_attn_sum", "a3", None, (ac.t + 1) * Ta * ha * 2)]
    n1 = 1 if mc.act == "gelu" else 2
    plan += [("mlp_fwd_col_gemm_act", "a1", 2 * T * h * f * n1, None),
             ("mlp_fwd_row_gemm", "a2", 2 * T * f * h, None),
             ("allreduce_fwd_sum", "a3", None, (mc.t + 1) * T * h * d + (h * d if mc.bias else 0))]
    if mc.p_drop > 0:
        plan.append(("mlp_bwd_dropout", "a4", None, 2 * T * h * d))
    if mc.bias:
        plan.append(("mlp_bwd_db2_colsum", "a4", None, T * h * d + 4 * h))
    if mc.bf16:
        # dH (with the activation backward) and dW2 are independent: one paired launch
        plan.append(("mlp_bwd_dH_dW2_gemm_act", "a5", 2 * 2 * T * h * f, None))
    else:
        plan += [("mlp_bwd_dH_gemm_act", "a5", 2 * T * h * f, None),
                 ("mlp_bwd_dW2_gemm", "a5", 2 * T * f * h, None)]
    if mc.bias and mc.act == "gelu":
        plan.append(("mlp_bwd_db1_colsum", "a5", None, T * f * d + 4 * f))
    if mc.bf16:
        # dW1 (dWg, dWu) and dX are independent and share one paired launch
        plan.append(("mlp_bwd_dW1_dX_gemm", "a6", 2 * T * h * f * n1 * 2, None))
    else:
        plan += [("mlp_bwd_dW1_gemm", "a6", 2 * T * h * f * n1, None),
                 ("mlp_bwd_dX_gemm", "a6", 2 * T * f * h * n1, None)]
    plan.append(("allreduce_bwd_sum", "a7", None, (mc.t + 1) * T * h * d))
    if ac is not None:
        # attention backward: algorithmic FLOPs per kernel (the score and dP
        # recomputations are not counted): dK/dV do dP, dV and dK, dQ does dQ
        pairs = ac.b * q * F.causal_pairs(ac.s)
        # dO with dWo, and dWqkv with dX, run as paired launches
        plan += [("attn_bwd_dO_dWo_gemm", "f1", 2 * 2 * Ta * ha * q * dh, None),
                 ("attn_bwd_stats", "f1", None, 2 * Ta * q * dh * 2 + ac.b * q * ac.s * 12),
                 ("attn_bwd_dkv", "f1", 6 * dh * pairs, None),
                 ("attn_bwd_dq", "f1", 2 * dh * pairs, None),
                 ("attn_bwd_dWqkv_dX_gemm", "f1", 2 * 2 * Ta * ha * (q + 2 * kv) * dh, None),
                 ("allreduce_attn_bwd_sum", "a7", None, (ac.t + 1) * Ta * ha * 2)]
    return plan


def time_split_and_residual(torch, mc, partials, residual, bias, reps=10):
    """The block-closing all-reduce with the residual fused, and its
    Megatron-SP split (one rank's reduce-scatter, the all-gather), at the
    workload's [T, h] shape; HBM bytes each call must move."""
    from attention_column_gemm_amd.shard import (all_gather, reduce_scatter, reduce_scatter_norm, sum_partials,
                                                 sum_partials_norm)
    t, T, h = mc.t, mc.tokens, mc.h
    d = 2 if mc.bf16 else 4
    n = T // t
    out = torch.empty_like(partials[0])
    sl = torch.empty((n, h), dtype=partials[0].dtype, device="cuda")
    slices = [sl] + [sl.clone() for _ in range(t - 1)]
    full = torch.empty_like(partials[0])
    normed = torch.empty_like(partials[0])
    sl_n = torch.empty_like(sl)
    gamma = torch.ones(h, dtype=partials[0].dtype, device="cuda")
    bb = h * d if bias is not None else 0
    calls = {
        "allreduce_residual_fused": (lambda: sum_partials(partials, bias, mc.p_drop, mc.seed, out=out,
                                                          residual=residual),
                                     (t + 2) * T * h * d + bb, "f3"),
        "sp_reduce_scatter_rank0": (lambda: reduce_scatter(partials, 0, bias, mc.p_drop, mc.seed,
                                                           residual_r=residual[:n], out=sl),
                                    T * h * d + 2 * n * h * d + bb, "f2"),
        "sp_all_gather": (lambda: all_gather(slices, out=full), 2 * T * h * d, "f2"),
        "allreduce_residual_rmsnorm_fused": (lambda: sum_partials_norm(partials, "rms", gamma, None, 1e-5, bias,
                                                                       mc.p_drop, mc.seed, residual=residual,
                                                                       out=out, normed=normed),
                                             (t + 3) * T * h * d + bb + h * d, "f2"),
        "sp_reduce_scatter_rmsnorm_rank0": (lambda: reduce_scatter_norm(partials, 0, "rms", gamma, None, 1e-5, bias,
                                                                        mc.p_drop, mc.seed, residual_r=residual[:n],
                                                                        out=sl, normed=sl_n),
                                            T * h * d + 3 * n * h * d + bb + h * d, "f2"),
    }
    res = []
    for name, (fn, nbytes, row) in calls.items():
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        res.append({"kernel": name, "row": row, "avg_ms": round(ms, 5), "bytes": nbytes,
                    "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
                    "frac_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)})
    return res


def time_uneven_shards(torch, reps=5):
    """Uneven splits run the same kernels on the rank's own share: the Llama
    SwiGLU MLP (T=4096, h=4096, h_ffn=11008) over t=3 ranks (widths 3672,
    3672, 3664) and the full-layer attention (64 q / 8 kv heads, d=128) over
    t=16 ranks (each KV head replicated on two ranks), rank 0, fwd+bwd."""
    import numpy as np
    from attention_column_gemm_amd import inputs as I
    from attention_column_gemm_amd.shard import AttnShard, MLPShard, to_device
    out = []
    rng = np.random.default_rng(0)

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    T, h, hf, t = 4096, 4096, 11008, 3
    sh = MLPShard(T, h, hf, t, 0, act="swiglu", dtype="bf16")
    g = lambda *shape, std=0.02: I.round_to_bf16(rng.standard_normal(shape).astype(np.float32) * std)
    sh.load(g(T, h, std=1.0), g(h, sh.f), g(h, sh.f), None, g(sh.f, h), g(T, h, std=1.0))
    ms = timed(lambda: (sh.forward(), sh.backward(0.0, 0, want_db2=False, want_db1=False)))
    fl = 18 * T * h * sh.f
    out.append({"case": f"SwiGLU MLP h_ffn={hf} over t={t}, rank 0 (f={sh.f})", "row": "f4", "avg_ms": round(ms, 4),
                "tflops": round(fl / (ms * 1e-3) / 1e12, 2)})
    del sh
    b, s, h, n_q, n_kv, d, t = 4, 2048, 8192, 64, 8, 128, 16
    ash = AttnShard(b, s, h, n_q, n_kv, d, t, 0)
    ash.load(g(b * s, h, std=1.0), g(h, (ash.q + 2 * ash.kv) * d), g(ash.q * d, h))
    dZ = to_device(g(b * s, h, std=1.0), "bf16")
    ms = timed(lambda: (ash.forward(), ash.backward(dZ)))
    fl = 3 * F.attn_shard_fwd(b, s, h, ash.q, ash.kv, d)
    out.append({"case": f"attention {n_q}q/{n_kv}kv d={d} over t={t} (KV replicated on 2 ranks), rank 0 "
                        f"(q={ash.q}, kv={ash.kv})", "row": "f4", "avg_ms": round(ms, 4),
                "tflops": round(fl / (ms * 1e-3) / 1e12, 2)})
    return out


def host_identity():
    """The host the CPU baseline ran on: logical CPUs, the CPUs this process
    may use, the CPU model, and the BLAS threads numpy's BLAS runs."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    blas = None
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": affinity, "cpu_model": model, "blas_threads": blas}


def cpu_baseline(mc, X, dOut, w, budget_s=12.0):
    """The float64 oracle on a bounded token slice of the same rank-0 shard."""
    import numpy as np
    from oracle import mlp as O
    host = host_identity()
    W = {k: (None if v is None else np.asarray(v, dtype=np.float64)) for k, v in w.items()}
    n, elapsed = 16, 0.0
    while True:
        t0 = time.perf_counter()
        O.shard_step(dOut[:n], X[:n], W["W1"], W["W2"], act=mc.act, Wu_i=W["Wu"], b1_i=W["b1"], p=mc.p_drop,
                     seed=mc.seed, rows=np.arange(n))
        elapsed = time.perf_counter() - t0
        if elapsed * 2 > budget_s or n * 2 > mc.tokens:
            break
        n *= 2
    flops = F.mlp_shard(n, mc.h, mc.f, mc.act)
    cores = host["blas_threads"] or host["affinity_cpus"] or host["nproc"] or 1
    return {"value": round(flops / elapsed / 1e12, 6), "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"rank-0 MLP shard fwd+bwd of workload {mc.cfg} on its first {n} of {mc.tokens} tokens "
                      f"(all weights; {flops / 1e9:.1f} GFLOP in float64 numpy/BLAS, {elapsed:.1f} s)",
            "threads_used": host["blas_threads"], **{k: v for k, v in host.items() if k != "blas_threads"}}


def time_mlp_workload(torch, mcid, steps, warmup=10):
    """MLP shard fwd+bwd of another workload, rank 0, timed like the headline
    (the span of the forward and backward calls per step, mean over steps)."""
    from attention_column_gemm_amd import inputs as I
    from attention_column_gemm_amd.shard import MLPShard
    mc = I.MLP_CONFIGS[mcid]
    X, dOut = I.mlp_activation(mc)
    w = I.mlp_rank_weights(mc, 0)
    sh = MLPShard(mc.tokens, mc.h, mc.h_ffn, mc.t, 0, act=mc.act, dtype=mc.dtype)
    sh.load(X, w["W1"], w["Wu"], w["b1"], w["W2"], dOut)
    run = lambda: (sh.forward(), sh.backward(mc.p_drop, mc.seed, want_db2=mc.bias, want_db1=mc.bias))
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in evs:
        a.record()
        run()
        b.record()
    torch.cuda.synchronize()
    ms = sum(a.elapsed_time(b) for a, b in evs) / steps
    fl = mc.flops_per_rank()
    tf = fl / (ms * 1e-3) / 1e12
    # The same calls captured once in a HIP graph and replayed: the kernels'
    # own rate, without the host's per-call issue time between launches
    # (the library allocates nothing and issues no memset, so a step
    # captures as a fixed sequence of kernel launches).
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        run()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    gevs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in gevs:
        a.record()
        g.replay()
        b.record()
    torch.cuda.synchronize()
    gms = sum(a.elapsed_time(b) for a, b in gevs) / steps
    gtf = fl / (gms * 1e-3) / 1e12
    del g, sh
    return {"workload": f"{mc.act} MLP shard fwd+bwd, T={mc.tokens} h={mc.h} h_ffn={mc.h_ffn} t={mc.t} "
                        f"(f={mc.f}), {mc.dtype}, p_drop={mc.p_drop}, bias={mc.bias}, rank 0",
            "cfg": mcid, "steps": steps, "mlp_ms": round(ms, 4), "flops": fl, "tflops": round(tf, 2),
            "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "graph_replay": {"mlp_ms": round(gms, 4), "tflops": round(gtf, 2),
                             "pct_of_bf16_peak": round(100 * gtf / PEAK_BF16_TFLOPS, 2)}}


def tp_record(mc, ac, per_step):
    """The per-layer record of a TP experiment ([L11] section 6): TP degree
    and rank, shapes, the layout of every linear, the all-reduces (count,
    logical payload and dtype) and their time over the timed steps (mean,
    P95; on one GPU every emulated all-reduce runs alone on the stream, so
    its whole time is exposed)."""
    import numpy as np
    dt = "bf16" if mc.bf16 else "fp32"
    delta = 2 if mc.bf16 else 4
    layouts = {"mlp": {"W1 (gate)" if mc.act == "swiglu" else "W1": "column (output dim split, input replicated)",
                       **({"Wu (up)": "column (output dim split, input replicated)"} if mc.act == "swiglu" else {}),
                       "W2 (down)" if mc.act == "swiglu" else "W2": "row (input dim split, output partial)"}}
    if ac is not None:
        layouts["attention"] = {"Wqkv": f"column by head ({ac.q} q / {ac.kv} kv heads of {ac.n_q} / {ac.n_kv})",
                                "Wo": "row (input dim split by head, output partial)"}
    ars = []
    names = [("allreduce_attn_fwd", "allreduce_attn_fwd", "g after the attention output projection"),
             ("allreduce_fwd", "allreduce_fwd", "g after the MLP down/W2 projection"),
             ("allreduce_bwd", "allreduce_bwd", "f at the MLP input (sum of dX_i)"),
             ("allreduce_attn_bwd", "allreduce_attn_bwd", "f at the attention input (sum of dX_i)")]
    for label, key, where in names:
        if key not in per_step:
            continue
        v = np.asarray(per_step[key])
        ars.append({"where": where, "payload_bytes": mc.tokens * mc.h * delta, "dtype": dt,
                    "mean_ms": round(float(v.mean()), 5), "p95_ms": round(float(np.percentile(v, 95)), 5),
                    "exposed_ms": round(float(v.mean()), 5)})
    return {"t": mc.t, "rank": 0, "tokens": mc.tokens, "h": mc.h, "h_ffn": mc.h_ffn,
            "layouts": layouts, "allreduce_dtype": dt,
            "allreduces_per_layer": 4 if ac is not None else 2, "allreduces": ars}


def load_traffic(kernel_label, workload):
    """HBM bytes per launch from the rocprofv3 PMC summary, if taken on the current sources
    and on this workload."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
    except Exception:
        return None
    if rec.get("source_hash") != source_hash() or rec.get("workload") != workload:
        return None
    ent = rec.get("kernels", {}).get(kernel_label)
    return None if ent is None else ent.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="cfg5", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the separate timing of the fused-residual all-reduce and its reduce-scatter / "
                         "all-gather split (profiling runs: keeps the step's kernels last)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after timing, run a plain device copy of this many MiB (a known-size reference for "
                         "HBM traffic counters); not part of the timed region")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one rank's shard on ONE GPU; --gpus {args.gpus} is not supported "
              "(the all-reduce is emulated on one device; multi-GPU runs are out of scope).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from attention_column_gemm_amd import binding as B
    from attention_column_gemm_amd import inputs as I
    from attention_column_gemm_amd.shard import AttnShard, MLPShard, sum_partials, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    mcid, acid = WORKLOADS[args.workload]
    mc = I.MLP_CONFIGS[mcid]
    ac = I.ATTN_CONFIGS[acid] if acid is not None else None

    log(f"[bench] workload {args.workload}: generating inputs")
    X, dOut = I.mlp_activation(mc)
    w = I.mlp_rank_weights(mc, 0)
    mlp = MLPShard(mc.tokens, mc.h, mc.h_ffn, mc.t, 0, act=mc.act, dtype=mc.dtype)
    mlp.load(X, w["W1"], w["Wu"], w["b1"], w["W2"], dOut)
    b2 = to_device(w["b2"], mc.dtype)
    attn = None
    if ac is not None:
        Xa = I.attn_activation(ac)
        wa = I.attn_rank_weights(ac, 0)
        attn = AttnShard(ac.b, ac.s, ac.h, ac.n_q, ac.n_kv, ac.d, ac.t, 0).load(Xa, wa["Wqkv"], wa["Wo"])
        del Xa

    # Rank 0's own partials come from its kernels each step; the other t-1
    # ranks' partials are stand-ins holding rank 0's values (the reduction's
    # cost does not depend on the values it reads).
    def others(ref, t):
        return [ref.clone() for _ in range(t - 1)]

    mlp.forward()
    mlp.backward(mc.p_drop, mc.seed, want_db2=mc.bias, want_db1=mc.bias)
    z_others, dx_others = others(mlp.Z, mc.t), others(mlp.dX, mc.t)
    out = torch.empty_like(mlp.Z)
    dxsum = torch.empty_like(mlp.dX)
    if attn is not None:
        assert ac.tokens == mc.tokens and ac.h == mc.h, "the attention backward takes the MLP's input gradient"
        attn.forward(want_lse=True)
        attn.backward(dxsum)
        za_others = others(attn.Z, ac.t)
        zasum = torch.empty_like(attn.Z)
        dxa_others = others(attn.dX, ac.t)
        dxasum = torch.empty_like(attn.dX)
    torch.cuda.synchronize()

    plan = kernel_plan(mc, ac)
    nk = len(plan)
    hip = HipEvents()
    stream = torch.cuda.current_stream()
    comm = B.tp_comm_bytes(mc.tokens, mc.h, mc.t, 2 if mc.bf16 else 4)

    def step(kev=None):
        if kev is not None:
            arr = (ctypes.c_void_p * (2 * nk))(*[e.value for e in kev])
            rc = B.lib().tp_profile_arm(arr, 2 * nk)
            assert rc == 0
        marks = []
        ev = lambda: torch.cuda.Event(enable_timing=True)
        if attn is not None:
            e0 = ev(); e0.record()
            attn.forward(want_lse=True)
            e1 = ev(); e1.record()
            sum_partials([attn.Z] + za_others, None, 0.0, 0, out=zasum)
            e2 = ev(); e2.record()
            marks += [("attention_fwd", e0, e1), ("allreduce_attn_fwd", e1, e2)]
        e0 = ev(); e0.record()
        mlp.forward()
        e1 = ev(); e1.record()
        sum_partials([mlp.Z] + z_others, b2, mc.p_drop, mc.seed, out=out)
        e2 = ev(); e2.record()
        mlp.backward(mc.p_drop, mc.seed, want_db2=mc.bias, want_db1=mc.bias)
        e3 = ev(); e3.record()
        sum_partials([mlp.dX] + dx_others, None, 0.0, 0, out=dxsum)
        e4 = ev(); e4.record()
        marks += [("mlp_fwd", e0, e1), ("mlp_bwd", e2, e3), ("allreduce_fwd", e1, e2), ("allreduce_bwd", e3, e4)]
        if attn is not None:
            attn.backward(dxsum)
            e5 = ev(); e5.record()
            sum_partials([attn.dX] + dxa_others, None, 0.0, 0, out=dxasum)
            e6 = ev(); e6.record()
            marks += [("attention_bwd", e4, e5), ("allreduce_attn_bwd", e5, e6)]
        B.tp_comm_bytes(mc.tokens, mc.h, mc.t, 2 if mc.bf16 else 4)   # a9: host-only accounting
        return marks

    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    kevs = [hip.create(2 * nk) for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    all_marks = [step() for _ in range(args.steps)]
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    # per-kernel durations: the same number of steps again, right after, with
    # the library's events armed around every kernel (kept out of the steps
    # above, whose spans give the headline value)
    log(f"[bench] per-kernel timing over {args.steps} more steps")
    for i in range(args.steps):
        step(kevs[i])
    torch.cuda.synchronize()

    kern_ms = np.zeros(nk)
    for kev in kevs:
        for i in range(nk):
            kern_ms[i] += hip.elapsed_ms(kev[2 * i], kev[2 * i + 1])
    kern_ms /= args.steps
    per_step = {}
    for marks in all_marks:
        for name, a, b in marks:
            per_step.setdefault(name, []).append(a.elapsed_time(b))
    span = {k: sum(v) / len(v) for k, v in per_step.items()}

    mlp_flops = mc.flops_per_rank()
    mlp_ms = span["mlp_fwd"] + span["mlp_bwd"]
    value = mlp_flops / (mlp_ms * 1e-3) / 1e12

    kernels = []
    for (label, row, flops, nbytes), ms in zip(plan, kern_ms):
        k = {"kernel": label, "row": row, "avg_ms": round(ms, 5)}
        if flops:
            k["tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
            k["frac_bf16_peak"] = round(flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)
        if nbytes:
            k["gbs"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
            k["frac_hbm_peak"] = round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)
        kernels.append(k)
    # dominant kernel: the longest one
    di = int(np.argmax(kern_ms))
    dl, _, dflops, dbytes = plan[di]
    if dflops:
        ach = dflops / (kern_ms[di] * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dl, "achieved": round(ach, 2), "peak": PEAK_BF16_TFLOPS,
                "unit": "TFLOP/s", "frac": round(ach / PEAK_BF16_TFLOPS, 4), "flops_per_launch": dflops,
                "avg_ms": round(float(kern_ms[di]), 5), "traffic": load_traffic(dl, args.workload)}
    else:
        ach = dbytes / (kern_ms[di] * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dl, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4), "bytes_per_launch": dbytes,
                "avg_ms": round(float(kern_ms[di]), 5), "traffic": load_traffic(dl, args.workload)}

    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if mc.bf16 else "f32",
        "data": "synthetic",
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "config": {
            "workload": {"cfg5": "full per-rank layer shard (attention + SwiGLU MLP, fwd+bwd), rank 0 of t=8",
                         "cfg3": "Llama SwiGLU MLP shard + GQA attention shard, fwd+bwd, rank 0 of t=8",
                         "cfg2": "GPT GeLU MLP shard fwd+bwd with dropout 0.1, rank 0 of t=4"}[args.workload],
            "tokens": mc.tokens, "b": mc.b, "s": mc.s, "h": mc.h, "h_ffn": mc.h_ffn, "t": mc.t, "f": mc.f,
            "act": mc.act, "p_drop": mc.p_drop, "bias": mc.bias,
            **({"attn": {"b": ac.b, "s": ac.s, "h": ac.h, "n_q": ac.n_q, "n_kv": ac.n_kv, "d": ac.d, "t": ac.t}}
               if ac is not None else {}),
        },
        "mlp_ms_per_step": round(mlp_ms, 4),
        "mlp_flops_per_step": mlp_flops,
        "spans_ms": {k: round(v, 4) for k, v in span.items()},
        "kernels": kernels,
        "roofline": roof,
        "comm": {"n_allreduce_per_layer": comm.n_allreduce_fwd + comm.n_allreduce_bwd,
                 "payload_bytes": comm.payload_bytes, "ring_bytes_per_rank": comm.ring_bytes_per_rank},
        "tp_record": tp_record(mc, ac, per_step),
        "wall_s_timed": round(wall, 3),
        "source_hash": source_hash(),
    }
    if attn is not None:
        af = I.ATTN_CONFIGS[acid].flops_per_rank()
        res["attention_fwd_tflops"] = round(af / (span["attention_fwd"] * 1e-3) / 1e12, 2)
        ab = I.ATTN_CONFIGS[acid].flops_bwd_per_rank()
        res["attention_bwd_tflops"] = round(ab / (span["attention_bwd"] * 1e-3) / 1e12, 2)
    if mc.tokens % mc.t == 0 and not args.no_extras:
        res["split_and_residual"] = time_split_and_residual(torch, mc, [mlp.Z] + z_others, mlp.X, b2)
    if args.workload == "cfg5" and not args.no_extras:
        del attn, mlp, z_others, dx_others, za_others, dxa_others
        torch.cuda.empty_cache()
        res["uneven_shards"] = time_uneven_shards(torch)
    if args.workload == "cfg5" and not args.no_extras:
        log("[bench] other workloads' MLP fwd+bwd")
        res["other_workloads"] = [time_mlp_workload(torch, 3, args.steps), time_mlp_workload(torch, 2, args.steps)]
        torch.cuda.empty_cache()
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 2
        src = torch.empty(n, dtype=torch.bfloat16, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        res["copy_calibration_mib"] = args.copy_calibration_mib
        del src, dst
    if not args.no_cpu:
        log("[bench] CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(mc, X, dOut, w)
    else:
        res["cpu_baseline"] = None
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
