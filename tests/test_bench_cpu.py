"""Host-side checks of the benchmark script's contract (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, cwd=ROOT)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "ONE GPU" in (r.stdout + r.stderr)


def test_unknown_workload_is_rejected():
    r = _run("--workload", "cfg9")
    assert r.returncode != 0


def _bench_module():
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_traffic_figures_apply_only_to_their_workload_and_sources():
    import json
    bench = _bench_module()
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic.json")))
    label, ent = next(iter(rec["kernels"].items()))
    current = rec["source_hash"] == bench.source_hash()
    got = bench.load_traffic(label, rec["workload"])
    assert got == (ent["bytes_per_launch"] if current else None)
    other = "cfg2" if rec["workload"] != "cfg2" else "cfg3"
    assert bench.load_traffic(label, other) is None


def test_kernel_plan_matches_the_paired_launches():
    """bf16 backward GEMM pairs are one launch each; fp32 shards keep them apart."""
    from attention_column_gemm_amd import inputs as I
    bench = _bench_module()
    plan = [p[0] for p in bench.kernel_plan(I.MLP_CONFIGS[5], I.ATTN_CONFIGS[5])]
    assert "mlp_bwd_dH_dW2_gemm_act" in plan and "mlp_bwd_dW1_dX_gemm" in plan
    assert "attn_bwd_dO_dWo_gemm" in plan and "attn_bwd_dWqkv_dX_gemm" in plan
    fp32 = [p[0] for p in bench.kernel_plan(I.MLP_CONFIGS[1], None)]
    assert "mlp_bwd_dH_gemm_act" in fp32 and "mlp_bwd_dX_gemm" in fp32
    # the paired entries carry both problems' FLOPs
    c = I.MLP_CONFIGS[5]
    total = sum(p[2] or 0 for p in bench.kernel_plan(c, None) if p[0].startswith("mlp_"))
    assert total == c.flops_per_rank()


def test_tp_record_fields():
    """[L11] section 6's record: layouts per linear, all-reduce count, payload,
    dtype, mean and P95 time."""
    from attention_column_gemm_amd import inputs as I
    bench = _bench_module()
    steps = {"allreduce_attn_fwd": [0.2, 0.21, 0.25], "allreduce_fwd": [0.2, 0.2, 0.2],
             "allreduce_bwd": [0.1, 0.3, 0.2], "allreduce_attn_bwd": [0.2] * 3}
    r = bench.tp_record(I.MLP_CONFIGS[5], I.ATTN_CONFIGS[5], steps)
    assert r["allreduces_per_layer"] == 4 and len(r["allreduces"]) == 4
    assert r["allreduce_dtype"] == "bf16"
    assert set(r["layouts"]) == {"mlp", "attention"}
    assert "column" in r["layouts"]["mlp"]["W1 (gate)"] and "row" in r["layouts"]["mlp"]["W2 (down)"]
    for a in r["allreduces"]:
        assert a["payload_bytes"] == 8192 * 8192 * 2 and a["p95_ms"] >= a["mean_ms"] - 1e-12
    r1 = bench.tp_record(I.MLP_CONFIGS[1], None, {"allreduce_fwd": [1.0], "allreduce_bwd": [2.0]})
    assert r1["allreduce_dtype"] == "fp32" and r1["allreduces"][0]["payload_bytes"] == 64 * 128 * 4


def test_host_identity_fields():
    bench = _bench_module()
    h = bench.host_identity()
    assert h["nproc"] >= 1 and h["affinity_cpus"] >= 1
    assert set(h) == {"nproc", "affinity_cpus", "cpu_model", "blas_threads"}
