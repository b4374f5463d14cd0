"""The benchmark's command-line contract on the CPU: more than one GPU is
refused with a message (the step runs on one GPU; nothing is launched), and
the flags parse, and the parity block of the line is computed and gated as
stated."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=120)


def test_more_than_one_gpu_is_refused():
    for n in ("2", "8"):
        r = run("--gpus", n)
        assert r.returncode == 2, r
        assert "one GPU" in r.stderr and r.stdout == ""


def test_help_lists_the_legs():
    r = run("--help")
    assert r.returncode == 0
    for flag in ("--steps", "--warmup", "--workload", "--zero2", "--offload", "--amp", "--composed", "--cpu-sample",
                 "--no-skipped-leg", "--fused-final"):
        assert flag in r.stdout, flag


def test_parity_statistics_of_the_bench_line():
    # the bench line's parity block, computed here from the oracle's own step
    # on the tiny workload (standing in for the device's first step), then with
    # planted differences
    import numpy as np

    import bench
    import oracle
    import synth
    from synth.workloads import workload

    w = workload(0)
    spec = w.tensors[0]
    S = 1 << 14
    st = lambda k, r=0: synth.stream_id(k, spec.tensor_id, r)
    grads = [synth.host_bf16(S, w.seed, st(synth.KIND_GRAD, r), w.grad_std, start=spec.start) for r in range(w.M)]
    master = synth.host_f32(S, w.seed, st(synth.KIND_MASTER), w.master_std, start=spec.start)
    z32 = np.zeros(S, np.float32)
    new, _ = oracle.zero_step([oracle.TensorState(grads, master, z32, z32, None)], oracle.HParams(**w.hparams()))
    first = {"master": new[0].master.copy(), "exp_avg": new[0].exp_avg.copy(), "exp_avg_sq": new[0].exp_avg_sq.copy(),
             "param_out": new[0].param_out.copy()}
    cpu, par = bench.cpu_baseline(w, S, first)
    assert cpu["kind"] == "oracle" and cpu["cpu_model"]
    assert par["gates"] == "pass" and par["elements"] == S
    assert par["max_ulp"] == {"master": 0, "exp_avg": 0, "exp_avg_sq": 0, "param_out": 0}
    assert par["bit_identical"]["master"] == 1.0
    first["exp_avg_sq"].view(np.uint32)[7] += 5  # 5 ulps: inside the stated tolerance at v ~ 1e-12, outside 4 ulps
    par = bench.parity_stats(first, new[0])
    assert par["gates"] == "FAIL" and par["max_ulp"]["exp_avg_sq"] == 5
    first["exp_avg_sq"].view(np.uint32)[7] -= 5
    first["param_out"][3] += 2
    assert bench.parity_stats(first, new[0])["gates"] == "FAIL"
