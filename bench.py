"""Benchmark of the fused per-rank ZeRO-1 shard step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload I]

A step is one zero_step call over the workload's shard: fold the M bf16
gradient replicas in fp32, unscale, check, norm (+ clip/skip when the
workload asks), AdamW on the fp32 master/m/v, bf16 emit. Inputs are seeded
synthetic data generated on the device before the timed region. The default
workload is the 7.5B-parameter model at 64-way ZeRO-1: one rank's
117,187,500-parameter shard reducing 64 replicas.

Prints one JSON line: params updated per second, the live HBM roofline of
the step kernels (algorithmic bytes / average step duration from HIP events
on the launch stream), the counter-measured HBM traffic when a profile of the
current kernel source is on file, and the CPU oracle timed on a bounded
sample of the same workload.

--zero2 times the ZeRO-2 streaming form instead (default workload: the
ragged Llama-7B-shaped bucket list): each step reduces every gradient bucket
(reduce_bucket_size 5e7 elements, backward order) into the fp32 shard
accumulators with zero_bucket_reduce, for --micro-batches micro-batches,
then applies zero_step_accumulated.

--offload times the CPU-offloaded form (default workload: the 7.5B shard):
the fold and norm on the GPU, the fp32 gradient to pinned host memory, AdamW
on host threads over host-resident state, the bf16 shard back to the device.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, AMD public specification
METRIC = "params updated/s + HBM GB/s (% of peak), fused ZeRO-1 reduce+AdamW shard step"
CSRC = os.path.join(ROOT, "sharded_optimizer_step_amd", "csrc")
# Every source that decides what runs on the device: the kernels, and the host
# planner that picks each pass's tile geometry and launches them.
LIBRARY_SOURCES = [os.path.join(CSRC, f) for f in ("zero_kernels.hip", "zero_api.cpp", "zero_internal.h")]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# How the seeded inputs are drawn (synth/): "N(0, s)" is read as zero mean,
# standard deviation s, drawn as a scaled Irwin-Hall sum of eight 16-bit
# uniforms from Philox4x32-10 counters; bf16 replicas are the top 16 bits
# of the fp32 draw.
INPUTS = ("seeded synthetic: Philox4x32-10 counters, N(0, s) read as s times an Irwin-Hall sum of 8 uniforms "
          "(mean 0, variance 1, support +-4.9), bf16 replicas by truncation of the fp32 draw")


def kernel_source_hash() -> str:
    """Hash of the library's device kernels and host planner, comments and
    blank space removed: a profile stays valid across comment edits and goes
    stale on any change of the code that decides which kernels run and how."""
    import re
    h = hashlib.sha256()
    for path in LIBRARY_SOURCES:
        src = open(path, encoding="utf-8").read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)   # block comments
        src = re.sub(r"//[^\n]*", " ", src)                  # line comments (no '//' in these sources' strings)
        h.update(os.path.basename(path).encode() + b"\0" + " ".join(src.split()).encode() + b"\0")
    return h.hexdigest()[:16]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", type=int, default=None,
                   help="0..4, see synth/workloads.py (default 2; 3 with --zero2)")
    p.add_argument("--cpu-sample", type=int, default=1 << 26,
                   help="elements of the shard the CPU oracle runs on (0: skip the CPU baseline)")
    p.add_argument("--calib-copy", action="store_true",
                   help="only run a plain 4 GiB device copy (HBM counter calibration)")
    p.add_argument("--stagger", type=int, default=0, help="bytes added between consecutive replica bases")
    p.add_argument("--zero2", action="store_true",
                   help="the ZeRO-2 streaming step: per-bucket zero_bucket_reduce, then zero_step_accumulated")
    p.add_argument("--micro-batches", type=int, default=1, help="--zero2: micro-batches accumulated per step")
    p.add_argument("--fused-final", action="store_true",
                   help="--zero2: each bucket's last micro-batch folded and applied in one pass (zero_bucket_step; "
                        "no clipping or skipping), then zero_step_accumulated with no tensors for the record")
    p.add_argument("--streams", type=int, default=None,
                   help="--zero2: side streams the buckets alternate over (1: the launch stream; default 2, "
                        "3 with --fused-final)")
    p.add_argument("--offload", action="store_true",
                   help="the CPU-offloaded step: zero_offload_step with the optimizer state in host memory")
    p.add_argument("--threads", type=int, default=0, help="--offload: host threads (0: the CPU affinity mask)")
    p.add_argument("--composed", action="store_true",
                   help="the same step through the three composed entry points (zero_shard_reduce, "
                        "zero_grad_check_norm, zero_adamw_step; single-tensor workloads)")
    p.add_argument("--no-skipped-leg", action="store_true",
                   help="leave out the skipped-steps leg of a workload with inf injection (a trace of clean steps only)")
    p.add_argument("--amp", action="store_true",
                   help="step with zero_step_amp: the loss scale held on the device, starting at the workload's "
                        "1/grad_scale (a power of two), window 1000, hysteresis 2")
    return p.parse_args()


def calib_copy(steps: int):
    import torch
    n = 1 << 30  # 4 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": 4 * n, "calib_copy_bytes_written": 4 * n, "launches": steps}))


def build_workload(w, stagger: int):
    import torch

    import sharded_optimizer_step_amd as z
    import synth

    dev = torch.device("cuda:0")
    tensors = []
    for spec in w.tensors:
        n = spec.n
        grads = []
        if stagger:
            # one allocation, rows padded to 256 B plus a per-row stagger
            row = (2 * n + 255) // 256 * 256 + stagger
            assert row % 16 == 0
            packed = torch.empty(w.M * row // 2, dtype=torch.bfloat16, device=dev)
            rows = [packed[r * row // 2:r * row // 2 + n] for r in range(w.M)]
        else:
            rows = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(w.M)]
        for r, g in enumerate(rows):
            st = synth.stream_id(synth.KIND_GRAD, spec.tensor_id, r)
            synth.device_bf16(g, w.seed, st, w.grad_std, start=spec.start)
            grads.append(g)
        st = lambda k: synth.stream_id(k, spec.tensor_id, 0)
        master = synth.device_f32(torch.empty(n, device=dev), w.seed, st(synth.KIND_MASTER), w.master_std,
                                  start=spec.start)
        m = torch.zeros(n, device=dev)
        v = torch.zeros(n, device=dev)
        if w.m_std:
            synth.device_f32(m, w.seed, st(synth.KIND_EXP_AVG), w.m_std, start=spec.start)
        if w.v_std:
            synth.device_f32(v, w.seed, st(synth.KIND_EXP_AVG_SQ), w.v_std, start=spec.start, absval=True)
        out = torch.empty(n, dtype=torch.bfloat16, device=dev)
        tensors.append(z.ZeroTensor(grads, master, m, v, out))
    torch.cuda.synchronize()
    return tensors


def snapshot_first_step(tensors, sample: int) -> dict:
    """The first `sample` elements of the first tensor's state and bf16
    output, copied to the host (after the first step from the seeded state)."""
    import numpy as np
    import torch
    t = tensors[0]
    k = min(sample, t.master.numel())
    torch.cuda.synchronize()
    return {"master": t.master[:k].cpu().numpy(), "exp_avg": t.exp_avg[:k].cpu().numpy(),
            "exp_avg_sq": t.exp_avg_sq[:k].cpu().numpy(),
            "param_out": t.param_out[:k].view(torch.int16).cpu().numpy().view(np.uint16)}


def _ordered(x, bits: int):
    import numpy as np
    if bits == 32:
        u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.int64)
        return np.where(u >= 2**31, 2**31 - u, u)
    u = np.ascontiguousarray(x, np.uint16).astype(np.int64)
    return np.where(u >= 0x8000, 0x8000 - u, u)


def parity_stats(got: dict, want) -> dict:
    """The device's first step against the oracle's on the same elements: per
    field the largest relative error with no floor, the largest distance in
    units in the last place (binary32; bf16 for the output), the share of
    elements that are bit-identical, and the verdict of the parity gates
    (|d| <= max(2e-6 |ref|, 1e-7) and <= 4 ulp on master, m, v; <= 1 bf16 ulp
    on the output)."""
    import numpy as np
    out = {"elements": int(want.master.size), "max_rel_no_floor": {}, "max_ulp": {}, "bit_identical": {}}
    ok = True
    for name, w in (("master", want.master), ("exp_avg", want.exp_avg), ("exp_avg_sq", want.exp_avg_sq)):
        g = got[name]
        gd, wd = g.astype(np.float64), w.astype(np.float64)
        same = (gd == wd) | (np.isnan(gd) & np.isnan(wd))
        with np.errstate(invalid="ignore", divide="ignore"):
            err = np.where(same, 0.0, np.abs(gd - wd))
            nz = np.abs(wd) > 0
            rel = float(np.max(err[nz] / np.abs(wd[nz]))) if nz.any() else 0.0
        ulp = np.where(same, 0, np.abs(_ordered(g, 32) - _ordered(w, 32)))
        ok &= bool(np.all(same | (err <= np.maximum(2e-6 * np.abs(wd), 1e-7)))) and int(ulp.max()) <= 4
        out["max_rel_no_floor"][name] = float(f"{rel:.3g}")
        out["max_ulp"][name] = int(ulp.max())
        out["bit_identical"][name] = float(f"{np.mean(same):.6f}")
    d = np.abs(_ordered(got["param_out"], 16) - _ordered(want.param_out, 16))
    ok &= int(d.max()) <= 1
    out["max_ulp"]["param_out"] = int(d.max())
    out["bit_identical"]["param_out"] = float(f"{np.mean(d == 0):.6f}")
    out["gates"] = "pass" if ok else "FAIL"
    return out


def cpu_baseline(w, sample: int, first=None):
    """The oracle, as it is, on the first `sample` elements of the workload's
    first tensor, with all M replicas, on one host core, then on every core.
    `first`: the device's state after its first step on the same elements
    (snapshot_first_step); the oracle's result is compared with it when the
    sample's step is the whole step's on those elements (no clipping, or the
    sample is the whole shard). Returns (cpu_baseline, parity or None)."""
    import oracle
    import synth

    spec = w.tensors[0]
    S = min(sample, spec.n)
    st = lambda k, r=0: synth.stream_id(k, spec.tensor_id, r)
    grads = [synth.host_bf16(S, w.seed, st(synth.KIND_GRAD, r), w.grad_std, start=spec.start) for r in range(w.M)]
    import numpy as np
    master = synth.host_f32(S, w.seed, st(synth.KIND_MASTER), w.master_std, start=spec.start)
    m = synth.host_f32(S, w.seed, st(synth.KIND_EXP_AVG), w.m_std, start=spec.start) if w.m_std else \
        np.zeros(S, np.float32)
    v = synth.host_f32(S, w.seed, st(synth.KIND_EXP_AVG_SQ), w.v_std, start=spec.start, absval=True) if w.v_std \
        else np.zeros(S, np.float32)
    hp = oracle.HParams(**{k: val for k, val in w.hparams().items()})
    t0 = time.perf_counter()
    new, _ = oracle.zero_step([oracle.TensorState(grads, master, m, v, None)], hp)
    dt = time.perf_counter() - t0
    # the same oracle on every core of the process's affinity mask: one call
    # per contiguous slice of the sample, from a thread each (ctypes releases
    # the interpreter lock during the call)
    from concurrent.futures import ThreadPoolExecutor
    k = max(1, len(os.sched_getaffinity(0)))
    bounds = [(S * j // k, S * (j + 1) // k) for j in range(k)]
    parts = [oracle.TensorState([g[a:b] for g in grads], master[a:b], m[a:b], v[a:b], None) for a, b in bounds]
    t1 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=k) as ex:
        list(ex.map(lambda st: oracle.zero_step([st], hp), parts))
    dt_all = time.perf_counter() - t1
    cpu = {"value": S / dt, "unit": "params/s", "cores": 1, "kind": "oracle", "cpu_model": cpu_model(),
           "sample": f"first {S:,} elements of the shard with all {w.M} replicas ({dt:.1f} s, single thread)",
           "all_cores": {"value": S / dt_all, "cores": k,
                         "sample": f"the same sample in {k} contiguous slices, one thread each ({dt_all:.2f} s)"}}
    parity = None
    if first is not None and first["master"].size == S and (not w.hparams()["max_grad_norm"] > 0 or S == w.n_total):
        parity = {"sample": f"first {S:,} elements of {spec.name} after the first (untimed) step from the seeded "
                            f"state, against the oracle's step on the same elements", **parity_stats(first, new[0])}
    return cpu, parity


def skipped_steps(a, w, tensors, step, res, stream) -> dict:
    """After the clean steps: the seeded +inf values of an odd run planted in
    the replicas, K more steps timed (each must come back skipped: the fold
    pass runs, the update pass exits), then the replicas restored."""
    import torch

    import sharded_optimizer_step_amd as z
    import synth

    spec = w.tensors[0]
    pos = synth.inject_positions(w.seed, 1, w.M, spec.n, w.inject_rate)
    g16 = [g.view(torch.int16) for g in tensors[0].grads]
    saved = [(r, i, int(g16[r][i].item())) for r, i in pos]
    for r, i in pos:
        g16[r][i] = 0x7F80  # +inf
    K = a.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(K):
        step(a.warmup + K + i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    r = z.read_result(res)
    for rr, i, v in saved:
        g16[rr][i] = v
    torch.cuda.synchronize()
    if r["status"] != 0 or r["found_inf"] != 1 or r["skipped"] != 1:
        raise RuntimeError(f"an injected step was not skipped: {r}")
    ms = ev[0].elapsed_time(ev[1]) / K
    n = w.n_total
    return {"infs_planted": len(pos), "ms_per_step": round(ms, 4),
            "hbm_gbs": round((2 * w.M + 4) * n / (ms * 1e-3) / 1e9, 1), "bytes_per_param": 2 * w.M + 4}


def zero2_line(a, w, tensors) -> dict:
    """Times the ZeRO-2 streaming step; returns the fields of the JSON line."""
    import torch

    import sharded_optimizer_step_amd as z
    from synth.workloads import zero2_buckets

    K = max(1, a.micro_batches)
    buckets = zero2_buckets(w)
    n = w.n_total
    # one contiguous fp32 accumulator for the whole shard, a view per tensor
    flat = torch.empty(n, dtype=torch.float32, device="cuda")
    accs, pos = [], 0
    for spec in w.tensors:
        accs.append(flat[pos:pos + spec.n])
        pos += spec.n
    parts = z.new_bucket_partials(len(buckets))
    reducers = [z.BucketReducer([z.GradShard(tensors[t].grads, accs[t]) for t in idx], parts[32 * b:32 * b + 32])
                for b, idx in enumerate(buckets)]
    ats = [z.AccTensor(acc, t.master, t.exp_avg, t.exp_avg_sq, t.param_out) for acc, t in zip(accs, tensors)]
    sws = z.workspace(z.zero_step_accumulated_workspace_bytes(ats))
    hp0 = w.hparams()
    hp = z.HParams(**hp0)
    fused = a.fused_final
    if fused:
        if hp.max_grad_norm > 0 or hp.skip_on_nonfinite:
            sys.exit("bench.py --fused-final: the workload clips or skips, so its update waits for the norm")
        steppers = [z.BucketStepper([z.BucketTensor(tensors[t].grads, accs[t] if K > 1 else None, tensors[t].master,
                                                    tensors[t].exp_avg, tensors[t].exp_avg_sq, tensors[t].param_out)
                                     for t in idx], parts[32 * b:32 * b + 32]) for b, idx in enumerate(buckets)]
    res = z.new_result()
    stream = torch.cuda.current_stream()
    # buckets are independent (own accumulators, workspace and partial), so a
    # loop that overlaps communication issues them on side streams; bucket b
    # always goes to the same one, which orders its micro-batches
    NS = max(1, a.streams if a.streams is not None else (3 if a.fused_final else 2))
    # the step's buckets together write more than the Infinity Cache holds:
    # their state stores stream out (zero_step decides this by itself)
    stream_flag = z.BUCKET_STREAM_STORES if n > z.STREAM_STORES_MIN_PARAMS else 0
    side = [torch.cuda.Stream() for _ in range(NS)] if NS > 1 else [stream]

    def step(i, ev=None):
        hp.step = hp0["step"] + i
        stamp = i + 1
        if NS > 1:
            for sd in side:
                sd.wait_stream(stream)
        for k in range(K):
            if fused and k == K - 1:
                for b, sp in enumerate(steppers):
                    sp.step((z.BUCKET_ACCUMULATE if k else 0) | stream_flag, hp, stamp, side[b % NS])
                continue
            flags = (z.BUCKET_ACCUMULATE if k else 0) | (z.BUCKET_FINAL if k == K - 1 else 0)
            for b, rd in enumerate(reducers):
                rd.reduce(flags, hp.grad_scale, stamp, side[b % NS])
        if NS > 1:
            for sd in side:
                stream.wait_stream(sd)
        if ev is not None:
            ev.record(stream)
        if fused:  # the record from the bucket partials alone
            z.zero_step_accumulated([], hp, parts, len(buckets), stamp, 0.0, None, res, stream)
        else:
            z.zero_step_accumulated(ats, hp, parts, len(buckets), stamp, 0.0, sws, res, stream)

    first = None
    for i in range(a.warmup):
        step(i)
        if i == 0 and K == 1 and a.cpu_sample > 0:
            # one micro-batch: the first step from the seeded state is the ZeRO-1 step's
            first = snapshot_first_step(tensors, a.cpu_sample)
    torch.cuda.synchronize()
    r = z.read_result(res)
    if r["status"] != 0:
        raise RuntimeError(f"step status {r}")
    S = a.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(S + 1)]
    mid = [torch.cuda.Event(enable_timing=True) for _ in range(S)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(S):
        step(a.warmup + i, mid[i])
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[S])
    per_ms = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(S))
    reduce_ms = sum(ev[i].elapsed_time(mid[i]) for i in range(S)) / S
    update_ms = sum(mid[i].elapsed_time(ev[i + 1]) for i in range(S)) / S
    avg_ms = total_ms / S
    # algorithmic bytes per shard parameter: the first micro-batch reads M
    # replicas and writes the fp32 sum, later ones also read it back; the
    # step reads g and the state, writes the state and the bf16 shard. With
    # the fused final pass the last micro-batch reads M replicas (and the sum
    # of the earlier ones) and the state, and writes the state and the shard.
    if fused:
        b_reduce = 2 * w.M * (K - 1) + 4 + 8 * (K - 2) if K > 1 else 0
        b_update = 2 * w.M + 26 + (4 if K > 1 else 0)
        names = ("fused final passes", "bucket reduces")
    else:
        b_reduce = 2 * w.M * K + 4 + 8 * (K - 1)
        b_update = 30
        names = ("update", "bucket reduces")
    bpp = b_reduce + b_update
    if fused:
        # the final passes run in the first phase, the record (a few us) in the second
        dom = (names[0], b_update, reduce_ms + update_ms) if K == 1 else (names[0] + " and reduces", bpp,
                                                                          reduce_ms + update_ms)
    else:
        dom = (names[0], b_update, update_ms) if update_ms >= reduce_ms else (names[1], b_reduce, reduce_ms)
    achieved = dom[1] * n / (dom[2] * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE) and K == 1 and not a.stagger:
        ent = json.load(open(TRAFFIC_FILE)).get(f"{w.index}_zero2_K1" + ("_fused" if fused else ""))
        if ent and ent.get("kernel_source_sha256_16") == kernel_source_hash() and ent.get("kernel") == dom[0]:
            traffic = ent["bytes_per_launch"]
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    cfg = {"workload": w.name + f", ZeRO-2 streaming: {len(buckets)} buckets of reduce_bucket_size 5e7 "
                                f"in backward order, {K} micro-batch(es)"
                                + (", the last one fused with the update" if fused else ""),
           "shard_params": n, "M": w.M, "tensors": len(w.tensors), "buckets": len(buckets), "micro_batches": K,
           "reduce_streams": NS,
           "state_stores_streamed": bool(fused and stream_flag),
           "bytes_per_param": bpp, "step_t": hp0["step"],
           "hbm_gbs": round(bpp * n / (avg_ms * 1e-3) / 1e9, 1),
           **({"bucket_phase_ms": round(reduce_ms, 4), "record_ms": round(update_ms, 4)} if fused else
              {"reduce_ms": round(reduce_ms, 4), "reduce_gbs": round(b_reduce * n / (reduce_ms * 1e-3) / 1e9, 1),
               "update_ms": round(update_ms, 4), "update_gbs": round(b_update * n / (update_ms * 1e-3) / 1e9, 1)}),
           "roofline_kernel": dom[0],
           "step_ms_min": round(per_ms[0], 4), "step_ms_median": round(per_ms[S // 2], 4)}
    return {"value": n / (avg_ms * 1e-3), "ms_per_step": avg_ms, "config": cfg, "roofline": roofline, "first": first}


PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction: the MI355X host link (public specification)


def offload_line(a, w, tensors) -> dict:
    """Times the CPU-offloaded step; returns the fields of the JSON line. The
    step is synchronous (it returns once the host state is updated), so it is
    timed on the host clock between device synchronizations."""
    import torch

    import sharded_optimizer_step_amd as z

    ots = [z.OffloadTensor(t.grads, t.master.cpu(), t.exp_avg.cpu(), t.exp_avg_sq.cpu(), t.param_out)
           for t in tensors]
    for t in tensors:  # the optimizer state now lives in host memory only
        t.master = t.exp_avg = t.exp_avg_sq = None
    torch.cuda.empty_cache()
    ws = z.workspace(z.zero_offload_workspace_bytes(ots, w.M))
    hws = z.host_workspace(z.zero_offload_host_workspace_bytes(ots))
    hp0 = w.hparams()
    hp = z.HParams(**hp0)
    stream = torch.cuda.current_stream()
    threads = a.threads
    for i in range(a.warmup):
        hp.step = hp0["step"] + i
        r = z.zero_offload_step(ots, hp, 0.0, ws, hws, threads, stream)
    torch.cuda.synchronize()
    if r["status"] != 0:
        raise RuntimeError(f"step status {r}")
    S = a.steps
    per = []
    torch.cuda.synchronize()
    t_all = time.perf_counter()
    for i in range(S):
        hp.step = hp0["step"] + a.warmup + i
        t0 = time.perf_counter()
        z.zero_offload_step(ots, hp, 0.0, ws, hws, threads, stream)
        per.append(time.perf_counter() - t0)
    torch.cuda.synchronize()
    total_s = time.perf_counter() - t_all
    n = w.n_total
    # the two limits of the offloaded step, each timed alone
    g_dev = torch.empty(n, dtype=torch.float32, device="cuda")
    g_host = torch.empty(n, dtype=torch.float32, pin_memory=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        g_host.copy_(g_dev, non_blocking=True)
    torch.cuda.synchronize()
    d2h_gbs = 3 * 4 * n / (time.perf_counter() - t0) / 1e9
    h = ots[0]
    k = h.master.numel()
    out_h = torch.zeros(k, dtype=torch.bfloat16, pin_memory=True)
    g_host[:k].zero_()
    host_s = []
    for _ in range(3):
        t0 = time.perf_counter()
        z.zero_offload_adamw_host(h.master, h.exp_avg, h.exp_avg_sq, g_host[:k], out_h, hp, 1.0, threads)
        host_s.append(time.perf_counter() - t0)
    host_pps = k / min(host_s)
    step_s = total_s / S
    link = 6 * n / step_s / 1e9  # 4 B of gradient down, 2 B of bf16 up per parameter
    roofline = {"bound": "pcie", "achieved": round(4 * n / step_s / 1e9, 2), "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                "frac": round(4 * n / step_s / 1e9 / PCIE_PEAK_GBS, 4), "traffic": None}
    cfg = {"workload": w.name + ", CPU-offloaded optimizer (state in host memory)", "shard_params": n, "M": w.M,
           "tensors": len(w.tensors), "host_threads": threads or len(os.sched_getaffinity(0)),
           "link_bytes_per_param": 6, "link_gbs": round(link, 2), "d2h_copy_gbs": round(d2h_gbs, 2),
           "host_update_params_per_s": round(host_pps), "hbm_state_bytes_saved": 12 * n, "step_t": hp0["step"],
           "step_ms_min": round(1e3 * min(per), 3), "step_ms_median": round(1e3 * sorted(per)[S // 2], 3)}
    return {"value": n / step_s, "ms_per_step": 1e3 * step_s, "config": cfg, "roofline": roofline}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: the step runs on one GPU (asked for --gpus {a.gpus}); "
              "the multi-GPU layout is a design, not a measured path", file=sys.stderr)
        sys.exit(2)
    import torch

    import sharded_optimizer_step_amd as z
    from synth.workloads import workload

    torch.cuda.set_device(0)
    if a.calib_copy:
        calib_copy(max(a.steps, 1))
        return
    if a.workload is None:
        a.workload = 3 if a.zero2 else 2
    if a.zero2 and a.offload:
        sys.exit("bench.py: --zero2 and --offload are separate legs")
    w = workload(a.workload)
    tensors = build_workload(w, a.stagger)
    if a.zero2 or a.offload:
        if a.amp:
            sys.exit("bench.py: --zero2 and --offload run with a fixed loss scale")
        out = zero2_line(a, w, tensors) if a.zero2 else offload_line(a, w, tensors)
        cpu, parity = cpu_baseline(w, a.cpu_sample, out.get("first")) if a.cpu_sample > 0 else (None, None)
        line = {"metric": METRIC, "value": out["value"], "unit": "params/s", "n_gpus": 1, "steps": a.steps,
                "warmup": a.warmup, "ms_per_step": out["ms_per_step"], "higher_is_better": True, "scaling": "weak",
                "vs_baseline": None, "dtype": "f32", "data": "synthetic", "config": {**out["config"], "inputs": INPUTS},
                "roofline": out["roofline"], "cpu_baseline": cpu, "parity": parity}
        print(json.dumps(line), flush=True)
        return
    hp0 = w.hparams()
    hp = z.HParams(**hp0)
    res = z.new_result()
    stream = torch.cuda.current_stream()
    if a.composed:
        if a.amp or len(tensors) != 1:
            sys.exit("bench.py --composed: single-tensor workloads, fixed loss scale")
        T = tensors[0]
        g = torch.empty(T.master.numel(), dtype=torch.float32, device="cuda")
        ws = z.workspace(z.zero_grad_check_norm_workspace_bytes(g.numel()))

        def step(i):
            hp.step = hp0["step"] + i
            z.zero_shard_reduce(T.grads, hp.grad_scale, g, stream)
            z.zero_grad_check_norm(g, hp, 0.0, ws, res, stream)
            z.zero_adamw_step(T.master, T.exp_avg, T.exp_avg_sq, g, T.param_out, hp, res, stream)
    elif a.amp:
        import math
        power = -math.log2(hp.grad_scale)
        if power != int(power):
            sys.exit(f"bench.py --amp: workload grad_scale {hp.grad_scale} is not a power of two")
        lscfg = z.LossScaleConfig(initial_scale_power=int(power), window=1000, hysteresis=2, min_scale=1.0)
        hp.grad_scale = 1.0  # the multiplier now comes from the device state
        ls = z.new_loss_scale()
        z.zero_loss_scale_init(lscfg, ls, stream)
        ws = z.workspace(z.zero_step_amp_workspace_bytes(tensors, w.M, hp))
        runner = z.StepRunner(tensors, ws, res)  # the tensor list marshalled once, as a training loop would

        def step(i):
            hp.step = hp0["step"] + i
            runner.step_amp(hp, lscfg, ls, 0.0, stream)
    else:
        ws = z.workspace(z.zero_step_workspace_bytes(tensors, w.M, hp))
        runner = z.StepRunner(tensors, ws, res)  # the tensor list marshalled once, as a training loop would

        def step(i):
            hp.step = hp0["step"] + i
            runner.step(hp, 0.0, stream)

    first = None
    for i in range(a.warmup):
        step(i)
        if i == 0 and a.cpu_sample > 0:  # the first step from the seeded state, for the parity sample
            first = snapshot_first_step(tensors, a.cpu_sample)
    torch.cuda.synchronize()
    r = z.read_result(res)
    if r["status"] != 0:
        raise RuntimeError(f"step status {r}")
    K = a.steps
    # the K timed steps, with events on the stream the kernels run on at the
    # two ends only (an event between steps costs about 0.2% of a 2.9 ms step)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(K):
        step(a.warmup + i)
    ev[1].record(stream)
    torch.cuda.synchronize()
    total_ms = ev[0].elapsed_time(ev[1])
    avg_ms = total_ms / K
    # the spread from steps with an event between each, after the timed region
    ks = min(K, 10)
    pev = [torch.cuda.Event(enable_timing=True) for _ in range(ks + 1)]
    pev[0].record(stream)
    for i in range(ks):
        step(a.warmup + K + i)
        pev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_ms = sorted(pev[i].elapsed_time(pev[i + 1]) for i in range(ks))
    n = w.n_total
    bpp = w.bytes_per_param() if not a.amp else 2 * w.M + 34  # the AMP step is always two-pass
    if a.composed:
        bpp = 2 * w.M + 38  # reduce 2M + 4, check 4, update 30
    achieved = bpp * n / (avg_ms * 1e-3) / 1e9
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tf = json.load(open(TRAFFIC_FILE))
        ent = tf.get(str(a.workload))
        if (ent and ent.get("kernel_source_sha256_16") == kernel_source_hash() and not a.amp and not a.composed
                and not a.stagger):
            # the one fused launch of a single-pass step; both launches of a two-pass step
            traffic = ent["bytes_per_launch"] if not w.two_pass else ent.get("bytes_per_step")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic}
    skipped = (skipped_steps(a, w, tensors, step, res, stream)
               if w.inject_rate > 0 and not a.composed and not a.no_skipped_leg else None)
    cpu, parity = None, None
    if a.cpu_sample > 0:
        cpu, parity = cpu_baseline(w, a.cpu_sample, first)
    line = {
        "metric": METRIC, "value": n / (total_ms * 1e-3 / K), "unit": "params/s", "n_gpus": 1, "steps": K,
        "warmup": a.warmup, "ms_per_step": total_ms / K, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "shard_params": n, "M": w.M, "tensors": len(w.tensors),
                   "bytes_per_param": bpp, "two_pass": w.two_pass or a.amp, "step_t": hp0["step"],
                   "loss_scale": "dynamic, on device" if a.amp else "fixed",
                   # above this size the library streams the state stores (zero_step decides)
                   "state_stores_streamed": (not a.composed) and n > z.STREAM_STORES_MIN_PARAMS,
                   **({"form": "composed: zero_shard_reduce, zero_grad_check_norm, zero_adamw_step"}
                      if a.composed else {}),
                   "hbm_gbs": round(bpp * n / (total_ms * 1e-3 / K) / 1e9, 1),
                   # the single-pass traffic model (2M + 26 B) over the same time, for a two-pass step
                   **({"hbm_gbs_at_2M_plus_26": round((2 * w.M + 26) * n / (total_ms * 1e-3 / K) / 1e9, 1)}
                      if bpp != 2 * w.M + 26 else {}),
                   "step_ms_min": round(per_ms[0], 4), "step_ms_median": round(per_ms[len(per_ms) // 2], 4),
                   "inputs": INPUTS,
                   **({"skipped_steps": skipped} if skipped else {})},
        "roofline": roofline, "cpu_baseline": cpu, "parity": parity,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
