"""GPU parity of every C-ABI entry point against the CPU oracle, on seeded
inputs that span several 2048-element tiles, ragged tails, unaligned heads,
scalar-only layouts and the degenerate cases of the step.

Gates: the fp32 reduced sum and found_inf bit-exact; master/m/v within
max(2e-6 |ref|, 1e-7); the bf16 output within 1 ulp; a finite norm within
1e-5 relative."""
import math

import numpy as np
import pytest
import torch

import oracle
import sharded_optimizer_step_amd as z
import synth
from cases import (Case, Stats, assert_state_matches, assert_tensor_matches, bits_equal, build, hp_oracle,
                   ordered32, run_step, to_np_f32, to_np_u16, ulp_gate, ULP_GATE)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    z.lib()  # the HIP library must be there: fail loudly otherwise
    torch.cuda.set_device(0)
    yield


def _bf16_dev(h: np.ndarray, off: int = 0) -> torch.Tensor:
    base = torch.empty(h.size + off + 8, dtype=torch.int16, device="cuda")
    v = base[off:off + h.size]
    v.copy_(torch.from_numpy(h.view(np.int16)))
    return v.view(torch.bfloat16)


# ---------------------------------------------------------------- generator

def test_device_generator_matches_host_bitwise():
    n, start = 1_000_003, 12_345
    st = synth.stream_id(synth.KIND_GRAD, 7, 3)
    g = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    synth.device_bf16(g, 1002, st, 1e-4, start=start)
    assert np.array_equal(to_np_u16(g), synth.host_bf16(n, 1002, st, 1e-4, start=start))
    f = torch.empty(n, dtype=torch.float32, device="cuda")
    for ab in (False, True):
        synth.device_f32(f, 1003, st, 1e-8, start=start, absval=ab)
        assert bits_equal(to_np_f32(f), synth.host_f32(n, 1003, st, 1e-8, start=start, absval=ab))


# ---------------------------------------------------------------- zero_shard_reduce

@pytest.mark.parametrize("M,n,scale", [(1, 4099, 1.0), (2, 2048, 1.0), (3, 2049, 0.25), (4, 100_003, 2.0**-16),
                                       (8, 262_144, 1.0), (16, 10_007, 1.0 / 3.0), (33, 5_000, 1.0),
                                       (64, 70_001, 1.0), (65, 3_001, 0.5), (130, 2_111, 1.0 / 130)])
def test_shard_reduce_bit_exact(M, n, scale):
    rng = np.random.default_rng(M * 1000 + n)
    hs = [synth.host_bf16(n, 11, synth.stream_id(0, 0, r), 1e-3) for r in range(M)]
    # a few wide-range values stress the rounding of the fold
    for r in range(M):
        k = rng.integers(0, n, 8)
        hs[r][k] = rng.integers(0, 0x7F00, 8).astype(np.uint16) | (rng.integers(0, 2, 8).astype(np.uint16) << 15)
    ds = [_bf16_dev(h) for h in hs]
    out = torch.full((n,), float("nan"), device="cuda")
    z.zero_shard_reduce(ds, scale, out)
    want = oracle.reduce(hs, scale)
    got = to_np_f32(out)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan)
    assert bits_equal(got[~nan], want[~nan])


@pytest.mark.parametrize("offs", [[1, 1, 1, 1, 2], [3, 3, 3, 3, 6], [1, 2, 3, 0, 0], [0, 0, 0, 0, 1]])
def test_shard_reduce_unaligned_layouts(offs):
    # shared misalignment -> vector path with a scalar head; mixed -> scalar path
    M, n = 4, 9_999
    hs = [synth.host_bf16(n, 12, synth.stream_id(0, 1, r), 1e-3) for r in range(M)]
    ds = [_bf16_dev(h, offs[r]) for r, h in enumerate(hs)]
    base = torch.empty(n + offs[M] + 8, dtype=torch.float32, device="cuda")
    out = base[offs[M]:offs[M] + n]
    z.zero_shard_reduce(ds, 1.0, out)
    assert bits_equal(to_np_f32(out), oracle.reduce(hs))


def test_shard_reduce_special_values():
    M, n = 4, 4096
    hs = [synth.host_bf16(n, 13, synth.stream_id(0, 2, r), 1e-3) for r in range(M)]
    hs[0][0:4] = [0x8000, 0x8000, 0x0000, 0x8000]   # signed zeros
    hs[1][0:4] = [0x8000, 0x0000, 0x8000, 0x8000]
    hs[2][0:4] = [0x8000, 0x8000, 0x8000, 0x8000]
    hs[3][0:4] = [0x8000, 0x8000, 0x8000, 0x0000]
    hs[0][10:14] = [0x0001, 0x807F, 0x0040, 0x7F7F]  # subnormals, bf16 max
    hs[1][10:14] = [0x0001, 0x0002, 0x8040, 0x7F7F]  # max + max overflows fp32
    hs[2][20] = 0x7F80
    hs[3][21] = 0xFF80
    hs[1][22], hs[2][22] = 0x7F80, 0xFF80          # +inf + -inf = NaN
    hs[0][23] = 0x7FC1
    order = [[0x3F80, 0x3380, 0x3380, 0xBF80]]      # 1, 2^-24, 2^-24, -1 -> 0 in ascending order
    for r in range(M):
        hs[r][30] = order[0][r]
    ds = [_bf16_dev(h) for h in hs]
    out = torch.empty(n, dtype=torch.float32, device="cuda")
    z.zero_shard_reduce(ds, 1.0, out)
    got, want = to_np_f32(out), oracle.reduce(hs)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan) and nan[22] and nan[23]
    assert bits_equal(got[~nan], want[~nan])
    assert got[30] == 0.0 and np.isinf(got[13])


# ---------------------------------------------------------------- zero_grad_check_norm

@pytest.mark.parametrize("n,max_norm,skip,ext,bad", [
    (2048, 0.0, 0, 0.0, None), (100_003, 1.0, 0, 0.0, None), (100_003, 0.01, 1, 0.0, None),
    (55_555, 0.5, 0, 3.0, None), (4099, 1.0, 1, 0.0, "inf"), (4099, 1.0, 0, 0.0, "nan"), (1, 1.0, 0, 0.0, None),
    (0, 1.0, 0, 2.25, None)])
def test_check_norm(n, max_norm, skip, ext, bad):
    g = synth.host_f32(n, 21, synth.stream_id(0, 3, 0), 3e-3)
    if bad == "inf" and n:
        g[n // 2] = np.inf
    if bad == "nan" and n:
        g[n - 1] = np.nan
    gd = torch.from_numpy(g.copy()).cuda()
    ws = z.workspace(z.zero_grad_check_norm_workspace_bytes(n))
    res = z.new_result()
    hp = z.HParams(max_grad_norm=max_norm, skip_on_nonfinite=skip)
    z.zero_grad_check_norm(gd, hp, ext, ws, res)
    r = z.read_result(res)
    s, f = oracle.check(g)
    o = oracle.finalize(s, ext, f, max_norm, skip)
    assert r["found_inf"] == o.found_inf and r["skipped"] == o.skipped and r["status"] == 0
    if o.found_inf == 0:
        assert math.isclose(r["sumsq"], o.sumsq, rel_tol=1e-12)
        assert abs(r["grad_norm"] - o.grad_norm) <= 1e-5 * o.grad_norm + 1e-30
        assert abs(r["clip_coef"] - o.clip_coef) <= 1e-6 * o.clip_coef
    else:
        assert not math.isfinite(r["grad_norm"])


# ---------------------------------------------------------------- zero_adamw_step

@pytest.mark.parametrize("n,t,coef", [(2048, 1, None), (100_003, 100, 0.37), (4097, 1000, None), (3, 5000, 0.5),
                                      (262_144, 10, None)])
def test_adamw_step(n, t, coef):
    hp = z.HParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=t)
    seed = 31 + t
    th = synth.host_f32(n, seed, synth.stream_id(1, 0, 0), 0.02)
    m = synth.host_f32(n, seed, synth.stream_id(2, 0, 0), 1e-5)
    v = synth.host_f32(n, seed, synth.stream_id(3, 0, 0), 1e-8, absval=True)
    g = synth.host_f32(n, seed, synth.stream_id(0, 0, 0), 1e-4)
    if t == 1:
        m[:] = 0
        v[:] = 0
    D = [torch.from_numpy(a.copy()).cuda() for a in (th, m, v, g)]
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    res = None
    if coef is not None:
        # a record that carries the clip coefficient, written by the library
        gd = torch.from_numpy(g.copy()).cuda()
        s, _ = oracle.check(g)
        max_norm = coef * (math.sqrt(s) + 1e-6)
        res = z.new_result()
        z.zero_grad_check_norm(gd, z.HParams(max_grad_norm=max_norm), 0.0,
                               z.workspace(z.zero_grad_check_norm_workspace_bytes(n)), res)
        coef = oracle.finalize(s, 0.0, 0, max_norm, 0).clip_coef  # the oracle's own coefficient
        assert abs(z.read_result(res)["clip_coef"] - coef) <= 1e-6 * coef
    z.zero_adamw_step(D[0], D[1], D[2], D[3], out, hp, res)
    wt, wm, wv, wo = oracle.adamw(th, m, v, g, hp_oracle(hp), coef if coef is not None else 1.0)
    same_coef = coef is None or z.read_result(res)["clip_coef"] == coef
    assert_state_matches(to_np_f32(D[0]), to_np_f32(D[1]), to_np_f32(D[2]), to_np_u16(out), wt, wm, wv, wo,
                         f"adamw n={n} t={t}", ulp_max=ULP_GATE if same_coef else None)


def test_adamw_step_respects_a_skipped_record():
    n = 5000
    g = synth.host_f32(n, 41, synth.stream_id(0, 0, 0), 1e-4)
    g[17] = np.inf
    gd = torch.from_numpy(g).cuda()
    res = z.new_result()
    z.zero_grad_check_norm(gd, z.HParams(skip_on_nonfinite=1), 0.0,
                           z.workspace(z.zero_grad_check_norm_workspace_bytes(n)), res)
    st = [torch.full((n,), 0.5, device="cuda") for _ in range(3)]
    out = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    z.zero_adamw_step(st[0], st[1], st[2], gd, out, z.HParams(step=3), res)
    assert all(bool((x == 0.5).all()) for x in st) and bool((out.view(torch.int16) == 0).all())
    assert z.read_result(res)["skipped"] == 1


# ---------------------------------------------------------------- zero_step (fused)

HP_SINGLE = z.HParams(lr=1e-3, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, step=10)


@pytest.mark.parametrize("M", [1, 2, 3, 4, 8, 16, 32, 64, 65])
def test_zero_step_single_pass(M):
    n = 70_001 if M <= 16 else 9_001
    case = Case([n], M, seed=50 + M)
    dts, hts = build(case)
    r, _ = run_step(dts, HP_SINGLE)
    new, ro = oracle.zero_step(hts, hp_oracle(HP_SINGLE))
    st = Stats()
    assert_tensor_matches(dts[0], new[0], f"M={M}", st)
    assert r["found_inf"] == 0 and r["skipped"] == 0 and r["status"] == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    assert r["clip_coef"] == 1.0
    print(f"M={M} max rel {st.max_rel} max ulp {st.max_ulp}")


@pytest.mark.parametrize("M", [4, 20])
def test_zero_step_single_pass_long_burst_tiles(M):
    # The single-pass geometries with 16 vectors per thread (256 x 16 up to
    # M = 16, 512 x 16 above) update their state two vectors at a time. The
    # large tensor gives the grid over two tiles per CU, and its last tile
    # ends inside a pair: 1141 vectors, so lanes 53-63 of the second wave hold
    # the pair's first vector but not its second. Beside it, a 5-element
    # tensor with no whole vector and a 4099-element one with a head and a
    # tail share the launch. Every element checked.
    tile = 32768 if M <= 16 else 65536
    sizes = [130 * tile + 1141 * 8 + 5, 5, 4099]
    offs = [[0] * (M + 4), [0] * (M + 4), [3] * (M + 4)]
    case = Case(sizes, M, seed=55 + M, offsets=offs)
    dts, hts = build(case)
    r, _ = run_step(dts, HP_SINGLE)
    new, ro = oracle.zero_step(hts, hp_oracle(HP_SINGLE))
    st = Stats()
    for i, (d, h) in enumerate(zip(dts, new)):
        assert_tensor_matches(d, h, f"M={M} tensor {i}", st)
    assert r["found_inf"] == 0 and r["skipped"] == 0 and r["status"] == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    print(f"M={M} max rel {st.max_rel} max ulp {st.max_ulp}")


@pytest.mark.parametrize("max_norm,skip,scale", [(1e-3, 0, 1.0), (1.0, 0, 1.0), (0.0, 1, 1.0),
                                                 (1e-3, 1, 2.0**-16)])
def test_zero_step_two_pass(max_norm, skip, scale):
    M = 8
    case = Case([100_003, 512, 2049], M, seed=60, grad_std=1e-3 / scale)
    dts, hts = build(case)
    hp = z.HParams(step=100, max_grad_norm=max_norm, skip_on_nonfinite=skip, grad_scale=scale)
    r, _ = run_step(dts, hp)
    new, ro = oracle.zero_step(hts, hp_oracle(hp))
    for i, (d, h) in enumerate(zip(dts, new)):
        assert_tensor_matches(d, h, f"tensor {i}", ulp_max=ulp_gate((r, ro)))
    assert r["found_inf"] == 0 and r["skipped"] == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    assert abs(r["clip_coef"] - ro.clip_coef) <= 1e-6 * ro.clip_coef
    if max_norm == 1e-3:
        assert ro.clip_coef < 1.0


def test_zero_step_two_pass_with_many_tiles_per_cu():
    # 67M elements: the first pass has over four 65536-element tiles per CU,
    # where it switches to its long-burst geometry; every element checked
    M = 3
    case = Case([1024 * 65536 + 12_345, 4099], M, seed=61, grad_std=1e-4)
    dts, hts = build(case)
    hp = z.HParams(step=100, max_grad_norm=0.5, skip_on_nonfinite=1)
    r, _ = run_step(dts, hp)
    new, ro = oracle.zero_step(hts, hp_oracle(hp))
    st = Stats()
    for i, (d, h) in enumerate(zip(dts, new)):
        assert_tensor_matches(d, h, f"tensor {i}", st, ulp_max=ulp_gate((r, ro)))
    assert r["found_inf"] == 0 and r["skipped"] == 0 and ro.clip_coef < 1.0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    assert abs(r["clip_coef"] - ro.clip_coef) <= 1e-6 * ro.clip_coef
    print(st)


@pytest.mark.parametrize("extra", [-1, 1])
def test_zero_step_at_the_stream_threshold(extra):
    # One parameter below and one above ZERO_STREAM_STORES_MIN_PARAMS: plain
    # and streamed whole-line state stores in the single pass (256 x 16,
    # paired update), with a second tensor that ends inside a 512-element
    # block and a third with a scalar head and tail; every element checked
    M = 3
    n = z.STREAM_STORES_MIN_PARAMS + extra
    sizes = [n - 70_003 - 4099, 70_003, 4099]
    offs = [[0] * (M + 4), [0] * (M + 4), [3] * (M + 4)]
    case = Case(sizes, M, seed=66 + extra, offsets=offs)
    dts, hts = build(case)
    r, _ = run_step(dts, HP_SINGLE)
    new, ro = oracle.zero_step(hts, hp_oracle(HP_SINGLE))
    st = Stats()
    for i, (d, h) in enumerate(zip(dts, new)):
        assert_tensor_matches(d, h, f"n {n} tensor {i}", st)
    assert r["found_inf"] == 0 and r["skipped"] == 0 and r["status"] == 0
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    print(f"n={n}", st)


def test_zero_step_ragged_unaligned_bucket():
    sizes = [512, 0, 1, 7, 8, 4099, 11_011, 4097, 2048, 2047, 2049, 300_001]
    M = 4
    rng = np.random.default_rng(70)
    offs = []
    for t, n in enumerate(sizes):
        if t % 3 == 0:
            offs.append([0] * (M + 4))                      # aligned
        elif t % 3 == 1:
            # shared misalignment: bf16 offset k and fp32 offset k mod 4 meet
            # 16-byte alignment at the same element -> vector path with a head
            k = int(rng.integers(1, 8))
            offs.append([k] * M + [k % 4] * 3 + [k])
        else:
            offs.append([int(x) for x in rng.integers(0, 8, M + 4)])  # mixed: scalar path
    case = Case(sizes, M, seed=71, offsets=offs)
    for hp in (z.HParams(step=7), z.HParams(step=7, max_grad_norm=2e-3)):
        dts, hts = build(case)
        r, _ = run_step(dts, hp)
        new, ro = oracle.zero_step(hts, hp_oracle(hp))
        for i, (d, h) in enumerate(zip(dts, new)):
            assert_tensor_matches(d, h, f"tensor {i} n={sizes[i]}", ulp_max=ulp_gate((r, ro)))
        assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm


@pytest.mark.parametrize("what", ["pinf", "ninf", "nan", "pinf_ninf", "overflow"])
def test_zero_step_skip_leaves_state_unchanged(what):
    M = 4
    case = Case([20_000, 513], M, seed=80)
    dts, hts = build(case)
    g = dts[0].grads
    i16 = [x.view(torch.int16) for x in g]
    if what == "pinf":
        i16[2][777] = 0x7F80
    elif what == "ninf":
        i16[0][19_999] = -128  # 0xFF80
    elif what == "nan":
        i16[3][5] = 0x7FC1
    elif what == "pinf_ninf":
        i16[1][8] = 0x7F80
        i16[2][8] = -128
    else:
        i16[0][9] = 0x7F7F
        i16[1][9] = 0x7F7F
        i16[2][9] = 0
        i16[3][9] = 0
    before = [(to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq), to_np_u16(d.param_out))
              for d in dts]
    hp = z.HParams(step=3, max_grad_norm=1.0, skip_on_nonfinite=1)
    r, _ = run_step(dts, hp)
    assert r["found_inf"] == 1 and r["skipped"] == 1 and r["status"] == 0
    for d, b in zip(dts, before):
        after = (to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq), to_np_u16(d.param_out))
        assert all(bits_equal(x, y) for x, y in zip(after, b))
    # without the skip switch the flag is still raised and the update runs
    dts, _ = build(case)
    dts[0].grads[1].view(torch.int16)[3] = 0x7F80
    r, _ = run_step(dts, z.HParams(step=3))
    assert r["found_inf"] == 1 and r["skipped"] == 0
    assert not np.isfinite(to_np_f32(dts[0].master)[3])


def test_zero_step_external_sumsq():
    case = Case([30_000], 2, seed=90)
    dts, hts = build(case)
    hp = z.HParams(step=5, max_grad_norm=0.1)
    r, _ = run_step(dts, hp, external=0.01)
    new, ro = oracle.zero_step(hts, hp_oracle(hp), 0.01)
    assert abs(r["grad_norm"] - ro.grad_norm) <= 1e-5 * ro.grad_norm
    assert_tensor_matches(dts[0], new[0], ulp_max=ulp_gate((r, ro)))


def test_zero_step_is_bitwise_repeatable():
    case = Case([300_001, 4096, 513], 8, seed=91)
    outs = []
    for _ in range(2):
        dts, _ = build(case)
        r, _ = run_step(dts, z.HParams(step=9, max_grad_norm=5e-3))
        outs.append((r, [(to_np_f32(d.master), to_np_f32(d.exp_avg), to_np_f32(d.exp_avg_sq),
                          to_np_u16(d.param_out)) for d in dts]))
    assert outs[0][0] == outs[1][0]
    for a, b in zip(outs[0][1], outs[1][1]):
        assert all(bits_equal(x, y) for x, y in zip(a, b))


def test_fused_equals_composed_entry_points():
    M, n = 8, 200_003
    case = Case([n], M, seed=92)
    hp = z.HParams(step=4)
    dts, _ = build(case)
    run_step(dts, hp)
    d2, _ = build(case)
    g = torch.empty(n, dtype=torch.float32, device="cuda")
    z.zero_shard_reduce(d2[0].grads, hp.grad_scale, g)
    res = z.new_result()
    z.zero_grad_check_norm(g, hp, 0.0, z.workspace(z.zero_grad_check_norm_workspace_bytes(n)), res)
    z.zero_adamw_step(d2[0].master, d2[0].exp_avg, d2[0].exp_avg_sq, g, d2[0].param_out, hp, res)
    for a, b in ((dts[0].master, d2[0].master), (dts[0].exp_avg, d2[0].exp_avg),
                 (dts[0].exp_avg_sq, d2[0].exp_avg_sq)):
        assert bits_equal(to_np_f32(a), to_np_f32(b))
    assert np.array_equal(to_np_u16(dts[0].param_out), to_np_u16(d2[0].param_out))


def test_resume_equals_uninterrupted():
    case = Case([50_001, 700], 4, seed=93)
    hp = lambda t: z.HParams(step=t, max_grad_norm=1e-2)
    a, _ = build(case)
    for t in range(1, 6):
        run_step(a, hp(t))
    b, _ = build(case)
    for t in range(1, 3):
        run_step(b, hp(t))
    saved = [[x.clone() for x in (d.master, d.exp_avg, d.exp_avg_sq)] for d in b]
    c, _ = build(case)  # fresh buffers, state restored from the saved copy
    for d, s in zip(c, saved):
        d.master.copy_(s[0])
        d.exp_avg.copy_(s[1])
        d.exp_avg_sq.copy_(s[2])
    for t in range(3, 6):
        run_step(c, hp(t))
    for x, y in zip(a, c):
        assert bits_equal(to_np_f32(x.master), to_np_f32(y.master))
        assert bits_equal(to_np_f32(x.exp_avg_sq), to_np_f32(y.exp_avg_sq))


def test_stale_workspace_is_detected_and_forget_recovers():
    case = Case([10_000], 2, seed=94)
    dts, _ = build(case)
    hp = z.HParams(step=2)
    r, ws = run_step(dts, hp)
    assert r["status"] == 0
    before = to_np_f32(dts[0].master)
    ws.zero_()  # the caller reuses the workspace for something else
    res = z.new_result()
    z.zero_step(dts, hp, 0.0, ws, res)
    r = z.read_result(res)
    assert r["status"] == z.ZERO_ERR_STALE_WORKSPACE and r["skipped"] == 1
    assert bits_equal(to_np_f32(dts[0].master), before)
    z.zero_workspace_forget(ws)
    z.zero_step(dts, hp, 0.0, ws, res)
    assert z.read_result(res)["status"] == 0
    assert not bits_equal(to_np_f32(dts[0].master), before)


def test_workspace_too_small_raises():
    case = Case([10_000], 2, seed=95)
    dts, _ = build(case)
    hp = z.HParams(step=2, max_grad_norm=1.0)
    need = z.zero_step_workspace_bytes(dts, 2, hp)
    with pytest.raises(z.ZeroError) as e:
        z.zero_step(dts, hp, 0.0, z.workspace(need - 256), z.new_result())
    assert e.value.status == z.ZERO_ERR_WORKSPACE_TOO_SMALL


def test_binding_rejects_host_workspaces_before_any_launch():
    M = 2
    case = Case([4099], M, seed=97)
    dts, hts = build(case)
    hp = z.HParams(step=3)
    res = z.new_result()
    host_ws = torch.empty(z.zero_step_workspace_bytes(dts, M, hp), dtype=torch.uint8)
    with pytest.raises(ValueError, match="ws: must be a device tensor"):
        z.zero_step(dts, hp, 0.0, host_ws, res)
    acc = torch.empty(4099, dtype=torch.float32, device="cuda")
    sh = [z.GradShard(dts[0].grads, acc)]
    with pytest.raises(ValueError, match="ws: must be a device tensor"):
        z.zero_bucket_reduce(sh, z.BUCKET_FINAL, 1.0, 1, z.new_bucket_partials(1), torch.empty(4096, dtype=torch.uint8))
    with pytest.raises(ValueError, match="ws: must be a device tensor"):
        z.BucketReducer(sh, z.new_bucket_partials(1), torch.empty(4096, dtype=torch.uint8))
    ats = [z.AccTensor(acc, dts[0].master, dts[0].exp_avg, dts[0].exp_avg_sq, dts[0].param_out)]
    with pytest.raises(ValueError, match="ws: must be a device tensor"):
        z.zero_step_accumulated(ats, hp, z.new_bucket_partials(1), 1, 1, 0.0, torch.empty(4096, dtype=torch.uint8),
                                res)
    ots = [z.OffloadTensor(dts[0].grads, torch.from_numpy(hts[0].master.copy()), torch.from_numpy(hts[0].exp_avg.copy()),
                           torch.from_numpy(hts[0].exp_avg_sq.copy()), dts[0].param_out)]
    pageable = torch.empty(z.zero_offload_host_workspace_bytes(ots), dtype=torch.uint8)
    with pytest.raises(ValueError, match="pinned"):
        z.zero_offload_step(ots, hp, 0.0, z.workspace(z.zero_offload_workspace_bytes(ots, M)), pageable)
    torch.cuda.synchronize()
    # nothing ran: the state is the one build() wrote
    assert bits_equal(to_np_f32(dts[0].master), hts[0].master)


def test_empty_bucket_writes_the_record():
    res = z.new_result()
    z.zero_step([z.ZeroTensor([torch.empty(0, dtype=torch.bfloat16, device="cuda")] * 2,
                              *[torch.empty(0, device="cuda") for _ in range(3)],
                              torch.empty(0, dtype=torch.bfloat16, device="cuda"))],
                z.HParams(max_grad_norm=1.0), 4.0, None, res)
    r = z.read_result(res)
    assert r["sumsq"] == 4.0 and r["grad_norm"] == 2.0 and r["found_inf"] == 0


@pytest.mark.parametrize("sizes,M,max_norm", [([300_001], 8, 0.0), ([4_000_000], 64, 0.0), ([100_003, 512], 4, 1e-3),
                                               ([5_000_000], 8, 1.0)])
def test_consecutive_steps_on_one_workspace_each_write_their_record(sizes, M, max_norm):
    # The fold pass's last workgroup writes the record and re-arms its arrival
    # counter; every step on the same workspace must report its own values.
    case = Case(sizes, M, seed=96, grad_std=1e-3)
    dts, hts = build(case)
    hp = z.HParams(step=3, max_grad_norm=max_norm)
    ws = z.workspace(z.zero_step_workspace_bytes(dts, M, hp))
    res = z.new_result()
    state = hts
    records = []
    for k, ext in enumerate([0.0, 0.5, 2.0, 0.125, 7.0]):
        hp.step = 3 + k
        z.zero_step(dts, hp, ext, ws, res)
        r = z.read_result(res)
        state, ro = oracle.zero_step(state, hp_oracle(hp), ext)
        records.append((r, ro))
        assert r["status"] == 0 and r["found_inf"] == 0
        # 1e-9: the oracle's left-to-right fp64 sum of 4M squares is itself
        # about 1e-11 from the exact sum; the steps differ by far more.
        assert math.isclose(r["sumsq"], ro.sumsq, rel_tol=1e-9), (k, r, ro)
        assert abs(r["clip_coef"] - ro.clip_coef) <= 1e-9 * ro.clip_coef
    for d, h in zip(dts, state):
        assert_tensor_matches(d, h, "after 5 steps", ulp_max=ulp_gate(*records))


def test_step_runner_equals_the_binding_call_bitwise():
    # the prepared form of zero_step and zero_step_amp (tensor list marshalled
    # once): three steps with changing hyperparameters, bit for bit against
    # the plain binding calls on a copy of the same inputs
    sizes, M = [100_003, 4099, 7], 8
    case = Case(sizes, M, seed=97)
    d1, _ = build(case)
    d2, _ = build(case)
    r1, r2 = z.new_result(), z.new_result()
    ws1 = z.workspace(z.zero_step_workspace_bytes(d1, M, z.HParams(max_grad_norm=1.0)))
    ws2 = z.workspace(z.zero_step_workspace_bytes(d2, M, z.HParams(max_grad_norm=1.0)))
    runner = z.StepRunner(d1, ws1, r1)
    for k, hp in enumerate((z.HParams(step=2), z.HParams(step=3, max_grad_norm=0.01), z.HParams(step=4))):
        runner.step(hp, 0.5 * k)
        z.zero_step(d2, hp, 0.5 * k, ws2, r2)
        assert z.read_result(r1) == z.read_result(r2), k
        for a, b in zip(d1, d2):
            for x, y in ((a.master, b.master), (a.exp_avg, b.exp_avg), (a.exp_avg_sq, b.exp_avg_sq)):
                assert bits_equal(to_np_f32(x), to_np_f32(y)), k
            assert np.array_equal(to_np_u16(a.param_out), to_np_u16(b.param_out)), k
    cfg = z.LossScaleConfig(initial_scale_power=4, window=2, hysteresis=1, min_scale=1.0)
    ls1, ls2 = z.new_loss_scale(), z.new_loss_scale()
    z.zero_loss_scale_init(cfg, ls1)
    z.zero_loss_scale_init(cfg, ls2)
    for k in range(3):
        hp = z.HParams(step=5 + k)
        runner.step_amp(hp, cfg, ls1)
        z.zero_step_amp(d2, hp, cfg, ls2, 0.0, ws2, r2)
        assert z.read_result(r1) == z.read_result(r2) and z.read_loss_scale(ls1) == z.read_loss_scale(ls2), k
        for a, b in zip(d1, d2):
            assert bits_equal(to_np_f32(a.master), to_np_f32(b.master)), k
