"""The C ABI on the CPU: the library loads, exports every function that
include/*.h declares, and rejects bad arguments before touching the GPU.
No call here launches a kernel."""
import ctypes
import glob
import os
import re

import pytest

import sharded_optimizer_step_amd as z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b(zero_\w+)\s*\(", src, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def exported_symbols(path):
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True, check=True).stdout
    return {line.split()[-1] for line in out.splitlines() if line.strip()}


def test_header_declares_the_boundary():
    names = declared_functions()
    assert set(names) == set(z.EXPORTS), names


def test_library_exports_every_declared_symbol():
    syms = exported_symbols(z.LIB_PATH)
    missing = [n for n in declared_functions() if n not in syms]
    assert not missing, missing
    L = z.lib()
    for n in declared_functions():
        assert getattr(L, n) is not None


def test_struct_layouts_match_header(tmp_path):
    """Compile the header with gcc and compare every field offset with the
    ctypes mirrors of the Python binding."""
    import subprocess
    fields = {"zero_adamw_hparams": z._CHparams, "zero_tensor": z._CTensor,
              "zero_loss_scale_config": z._CLossScaleConfig, "zero_grad_shard": z._CGradShard,
              "zero_acc_tensor": z._CAccTensor, "zero_offload_tensor": z._COffloadTensor,
              "zero_result": z._CResult}
    body = []
    for cname, cls in fields.items():
        body.append(f'printf("{cname} %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            body.append(f'printf("{cname}.{f} %zu\\n", offsetof({cname}, {f}));')
    body.append('printf("zero_result %zu\\n", sizeof(zero_result));')
    body.append('printf("zero_loss_scale %zu\\n", sizeof(zero_loss_scale));')
    for f in ("scale", "inv_scale", "good_steps", "overflows"):
        body.append(f'printf("zero_loss_scale.{f} %zu\\n", offsetof(zero_loss_scale, {f}));')
    body.append('printf("zero_bucket_partial %zu\\n", sizeof(zero_bucket_partial));')
    for f in ("sumsq", "stamp", "found_inf", "grad_scale", "reserved"):
        body.append(f'printf("zero_bucket_partial.{f} %zu\\n", offsetof(zero_bucket_partial, {f}));')
    consts = {"ZERO_BUCKET_ACCUMULATE": z.BUCKET_ACCUMULATE, "ZERO_BUCKET_FINAL": z.BUCKET_FINAL,
              "ZERO_BUCKET_STREAM_STORES": z.BUCKET_STREAM_STORES,
              "ZERO_STREAM_STORES_MIN_PARAMS": z.STREAM_STORES_MIN_PARAMS,
              "ZERO_NOALLOC_SCRATCH_BYTES": z.NOALLOC_SCRATCH_BYTES}
    for cname in consts:
        body.append(f'printf("{cname} %lld\\n", (long long)({cname}));')
    src = tmp_path / "layout.c"
    src.write_text("#include <stddef.h>\n#include <stdio.h>\n#include \"zero_step.h\"\nint main(void){" +
                   "".join(body) + "return 0;}\n")
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
                    "-o", str(exe), str(src)], check=True)
    got = dict(l.split() for l in subprocess.run([str(exe)], capture_output=True, text=True,
                                                  check=True).stdout.splitlines())
    for cname, cls in fields.items():
        assert int(got[cname]) == ctypes.sizeof(cls), cname
        for f, _ in cls._fields_:
            assert int(got[f"{cname}.{f}"]) == getattr(cls, f).offset, (cname, f)
    for cname, v in consts.items():
        assert int(got[cname]) == v, cname
    assert int(got["zero_result"]) == z.RESULT_BYTES
    # read_loss_scale unpacks "<ffii"
    assert int(got["zero_loss_scale"]) == z.LOSS_SCALE_BYTES
    assert [int(got[f"zero_loss_scale.{f}"]) for f in ("scale", "inv_scale", "good_steps", "overflows")] == [0, 4, 8, 12]
    # read_bucket_partial unpacks "<dQifq"
    assert int(got["zero_bucket_partial"]) == z.BUCKET_PARTIAL_BYTES
    assert [int(got[f"zero_bucket_partial.{f}"]) for f in ("sumsq", "stamp", "found_inf", "grad_scale",
                                                           "reserved")] == [0, 8, 16, 20, 24]


def test_status_strings():
    assert z.zero_status_string(0) == "ok"
    assert "workspace" in z.zero_status_string(2)
    assert "stale" in z.zero_status_string(4) or "no longer" in z.zero_status_string(4)
    assert z.zero_status_string(99) == "unknown status"


def _hp(**kw):
    return z.HParams(**kw)._c()


@pytest.mark.parametrize("kw", [dict(lr=-1.0), dict(lr=float("nan")), dict(beta1=1.0), dict(beta2=-0.1),
                                dict(eps=-1e-8), dict(step=0), dict(grad_scale=0.0),
                                dict(grad_scale=float("inf")), dict(max_grad_norm=float("nan")),
                                # finite as binary64, but 0, subnormal or +inf once rounded to binary32
                                dict(grad_scale=1e-50), dict(grad_scale=1e-40), dict(grad_scale=1e300),
                                dict(weight_decay=float("inf"))])
def test_bad_hparams_are_rejected_without_launch(kw):
    L = z.lib()
    h = _hp(**kw)
    assert L.zero_adamw_step(None, None, None, None, None, 10, ctypes.byref(h), None, None) == 1
    arr = (z._CTensor * 1)()
    arr[0] = z._CTensor(10, None, None, None, None, None)
    assert L.zero_step_workspace_bytes(arr, 1, 2, ctypes.byref(h)) == 0
    assert L.zero_step(arr, 1, 2, ctypes.byref(h), 0.0, None, 0, ctypes.c_void_p(256), None) == 1


def test_reserved_field_must_be_zero():
    L = z.lib()
    h = _hp()
    h.reserved = 1
    assert L.zero_adamw_step(None, None, None, None, None, 10, ctypes.byref(h), None, None) == 1


def test_shard_reduce_argument_checks():
    L = z.lib()
    fake = (ctypes.c_void_p * 2)(256, 512)
    assert L.zero_shard_reduce(fake, 0, 10, 1.0, 1024, None) == 1          # M < 1
    assert L.zero_shard_reduce(fake, 65537, 10, 1.0, 1024, None) == 1      # M too large
    assert L.zero_shard_reduce(fake, 2, -1, 1.0, 1024, None) == 1          # n < 0
    assert L.zero_shard_reduce(fake, 2, 10, 0.0, 1024, None) == 1          # scale <= 0
    assert L.zero_shard_reduce(fake, 2, 10, float("nan"), 1024, None) == 1
    for bad in (1e-50, 1e-40, 1e300):  # binary32 rounding 0, subnormal, +inf
        assert L.zero_shard_reduce(fake, 2, 10, bad, 1024, None) == 1
    assert L.zero_shard_reduce(None, 2, 10, 1.0, 1024, None) == 1          # no replica array
    assert L.zero_shard_reduce(fake, 2, 10, 1.0, None, None) == 1          # no output
    nul = (ctypes.c_void_p * 2)(256, None)
    assert L.zero_shard_reduce(nul, 2, 10, 1.0, 1024, None) == 1          # a null replica
    assert L.zero_shard_reduce(fake, 2, 0, 1.0, None, None) == 0           # n == 0: no-op


def test_adamw_and_check_argument_checks():
    L = z.lib()
    h = _hp()
    assert L.zero_adamw_step(None, None, None, None, None, 0, ctypes.byref(h), None, None) == 0  # n == 0
    assert L.zero_adamw_step(256, 256, 256, None, 256, 5, ctypes.byref(h), None, None) == 1      # no g
    assert L.zero_adamw_step(256, 256, 256, 256, 256, -1, ctypes.byref(h), None, None) == 1
    assert L.zero_grad_check_norm(256, 10, None, 0.0, None, 1 << 20, None, None) == 1            # no result
    assert L.zero_grad_check_norm(256, 10, None, 0.0, None, 1 << 20, 512, None) == 1             # no ws
    assert L.zero_grad_check_norm(256, 10, None, 0.0, 1024, 16, 512, None) == 2                  # ws short
    assert L.zero_grad_check_norm_workspace_bytes(0) == 0
    assert L.zero_grad_check_norm_workspace_bytes(1) > 0


def test_zero_step_argument_checks():
    L = z.lib()
    h = _hp(max_grad_norm=1.0)
    ptrs = (ctypes.c_void_p * 2)(256, 512)
    arr = (z._CTensor * 1)()
    arr[0] = z._CTensor(100, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), 1024, 2048, 4096, 8192)
    need = L.zero_step_workspace_bytes(arr, 1, 2, ctypes.byref(h))
    assert need > 100 * 4  # two-pass: holds the fp32 reduced gradient
    res = ctypes.c_void_p(1 << 20)
    assert L.zero_step(arr, 1, 2, ctypes.byref(h), 0.0, 1 << 24, need - 1, res, None) == 2   # ws short
    assert L.zero_step(arr, 1, 2, ctypes.byref(h), 0.0, (1 << 24) + 16, need, res, None) == 1  # ws misaligned
    assert L.zero_step(arr, 1, 2, ctypes.byref(h), 0.0, None, need, res, None) == 1          # no ws
    assert L.zero_step(arr, 1, 2, ctypes.byref(h), 0.0, 1 << 24, need, None, None) == 1       # no result
    assert L.zero_step(arr, -1, 2, ctypes.byref(h), 0.0, 1 << 24, need, res, None) == 1
    assert L.zero_step(arr, 1, 0, ctypes.byref(h), 0.0, 1 << 24, need, res, None) == 1
    nul = (ctypes.c_void_p * 2)(256, None)
    arr2 = (z._CTensor * 1)()
    arr2[0] = z._CTensor(100, ctypes.cast(nul, ctypes.POINTER(ctypes.c_void_p)), 1024, 2048, 4096, 8192)
    assert L.zero_step(arr2, 1, 2, ctypes.byref(h), 0.0, 1 << 24, need, res, None) == 1      # null replica
    arr3 = (z._CTensor * 1)()
    arr3[0] = z._CTensor(-5, None, None, None, None, None)
    assert L.zero_step_workspace_bytes(arr3, 1, 2, ctypes.byref(h)) == 0


@pytest.mark.parametrize("ext", [-1.0, -1e-300, float("-inf")])
def test_negative_external_sumsq_is_rejected_without_launch(ext):
    L = z.lib()
    h = _hp(max_grad_norm=1.0)
    ptrs = (ctypes.c_void_p * 2)(256, 512)
    arr = (z._CTensor * 1)()
    arr[0] = z._CTensor(100, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), 1024, 2048, 4096, 8192)
    need = L.zero_step_workspace_bytes(arr, 1, 2, ctypes.byref(h))
    res = ctypes.c_void_p(1 << 20)
    assert L.zero_step(arr, 1, 2, ctypes.byref(h), ext, 1 << 24, need, res, None) == 1
    assert L.zero_step(arr, 0, 2, ctypes.byref(h), ext, 1 << 24, need, res, None) == 1     # empty list too
    cfg = z.LossScaleConfig()._c()
    assert L.zero_step_amp(arr, 1, 2, ctypes.byref(h), ctypes.byref(cfg), ctypes.c_void_p(1 << 22), ext, 1 << 24,
                           need, res, None) == 1
    assert L.zero_grad_check_norm(256, 10, None, ext, 1024, 1 << 20, 512, None) == 1
    assert L.zero_grad_check_norm(None, 0, None, ext, None, 0, 512, None) == 1
    acc = (z._CAccTensor * 1)()
    acc[0] = z._CAccTensor(100, 256, 1024, 2048, 4096, 8192)
    aneed = L.zero_step_accumulated_workspace_bytes(acc, 1)
    assert L.zero_step_accumulated(acc, 1, ctypes.byref(h), ctypes.c_void_p(1 << 21), 1, 0, ext, 1 << 24, aneed,
                                   res, None) == 1
    off, keep = _offload()
    r = z._CResult()
    assert L.zero_offload_step(off, 1, 2, ctypes.byref(h), ext, 1 << 24, L.zero_offload_workspace_bytes(off, 1, 2),
                               1 << 25, L.zero_offload_host_workspace_bytes(off, 1), ctypes.byref(r), 0, None) == 1


@pytest.mark.parametrize("ext", [float("nan"), float("inf"), 0.0, 2.5])
def test_nonnegative_or_nonfinite_external_sumsq_passes_the_checks(ext):
    # NaN and +inf carry another rank's non-finite gradient into the norm: the
    # call gets as far as the workspace check
    L = z.lib()
    h = _hp(max_grad_norm=1.0)
    ptrs = (ctypes.c_void_p * 2)(256, 512)
    arr = (z._CTensor * 1)()
    arr[0] = z._CTensor(100, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), 1024, 2048, 4096, 8192)
    need = L.zero_step_workspace_bytes(arr, 1, 2, ctypes.byref(h))
    assert L.zero_step(arr, 1, 2, ctypes.byref(h), ext, 1 << 24, need - 1, ctypes.c_void_p(1 << 20), None) == 2


def test_a_pass_beyond_the_launch_limit_is_rejected_before_any_launch():
    # 2^43 elements: the update pass would need 2^32 tiles of 2048 elements
    L = z.lib()
    h = _hp(max_grad_norm=1.0)
    ptrs = (ctypes.c_void_p * 2)(256, 512)
    arr = (z._CTensor * 1)()
    arr[0] = z._CTensor(1 << 43, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), 1024, 2048, 4096, 8192)
    need = L.zero_step_workspace_bytes(arr, 1, 2, ctypes.byref(h))
    assert need > 4 << 43
    assert L.zero_step(arr, 1, 2, ctypes.byref(h), 0.0, 1 << 24, need, ctypes.c_void_p(1 << 20), None) == 1


def test_workspace_sizes_follow_the_traffic_plan():
    one = z.zero_step_workspace_bytes_for_sizes([1_000_000], 8, z.HParams())
    two = z.zero_step_workspace_bytes_for_sizes([1_000_000], 8, z.HParams(max_grad_norm=1.0))
    skip = z.zero_step_workspace_bytes_for_sizes([1_000_000], 8, z.HParams(skip_on_nonfinite=1))
    # the single pass keeps no gradient; clip or skip keeps the fp32 reduced gradient once
    assert one < 1_000_000
    assert two - one >= 4 * 1_000_000 and skip == two
    ragged = z.zero_step_workspace_bytes_for_sizes([512, 0, 4099, 11011], 8, z.HParams(max_grad_norm=1.0))
    assert ragged >= 4 * (512 + 4099 + 11011)


def test_forget_needs_a_pointer():
    L = z.lib()
    assert L.zero_workspace_forget(None) == 1
    assert L.zero_workspace_forget(ctypes.c_void_p(4096)) == 0


@pytest.mark.parametrize("kw", [dict(initial_scale_power=128), dict(initial_scale_power=-127), dict(window=0),
                                dict(hysteresis=0), dict(min_scale=0.0), dict(min_scale=-1.0),
                                dict(min_scale=float("inf")), dict(min_scale=float("nan"))])
def test_bad_loss_scale_config_is_rejected_without_launch(kw):
    L = z.lib()
    c = z.LossScaleConfig(**kw)._c()
    ls, res = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21)
    assert L.zero_loss_scale_init(ctypes.byref(c), ls, None) == 1
    assert L.zero_loss_scale_update(ctypes.byref(c), res, ls, None) == 1
    h = _hp()
    ptrs = (ctypes.c_void_p * 2)(256, 512)
    arr = (z._CTensor * 1)()
    arr[0] = z._CTensor(100, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), 1024, 2048, 4096, 8192)
    need = L.zero_step_amp_workspace_bytes(arr, 1, 2, ctypes.byref(h))
    assert L.zero_step_amp(arr, 1, 2, ctypes.byref(h), ctypes.byref(c), ls, 0.0, 1 << 24, need, res, None) == 1


def test_loss_scale_entry_points_need_their_buffers():
    L = z.lib()
    c = z.LossScaleConfig()._c()
    assert L.zero_loss_scale_init(None, ctypes.c_void_p(1 << 20), None) == 1
    assert L.zero_loss_scale_init(ctypes.byref(c), None, None) == 1
    assert L.zero_loss_scale_update(ctypes.byref(c), None, ctypes.c_void_p(1 << 20), None) == 1
    assert L.zero_loss_scale_update(ctypes.byref(c), ctypes.c_void_p(1 << 21), None, None) == 1
    h = _hp()  # no clipping, no skip: zero_step alone would be single-pass
    ptrs = (ctypes.c_void_p * 2)(256, 512)
    arr = (z._CTensor * 1)()
    arr[0] = z._CTensor(100, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), 1024, 2048, 4096, 8192)
    need = L.zero_step_amp_workspace_bytes(arr, 1, 2, ctypes.byref(h))
    assert need == L.zero_step_workspace_bytes(arr, 1, 2, ctypes.byref(_hp(skip_on_nonfinite=1)))
    assert need > L.zero_step_workspace_bytes(arr, 1, 2, ctypes.byref(h))
    res = ctypes.c_void_p(1 << 21)
    assert L.zero_step_amp(arr, 1, 2, ctypes.byref(h), ctypes.byref(c), None, 0.0, 1 << 24, need, res, None) == 1
    assert L.zero_step_amp(arr, 1, 2, ctypes.byref(h), None, ctypes.c_void_p(1 << 20), 0.0, 1 << 24, need, res,
                           None) == 1
    assert L.zero_step_amp(arr, 1, 2, ctypes.byref(h), ctypes.byref(c), ctypes.c_void_p(1 << 20), 0.0, 1 << 24,
                           need - 1, res, None) == 2


def _shards(n=100, M=2, acc=4096):
    ptrs = (ctypes.c_void_p * M)(*[256 * (r + 1) for r in range(M)])
    arr = (z._CGradShard * 1)()
    arr[0] = z._CGradShard(n, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), acc)
    return arr, ptrs


def test_bucket_reduce_argument_checks():
    L = z.lib()
    arr, keep = _shards()
    need = L.zero_bucket_reduce_workspace_bytes(arr, 1, 2)
    assert need > 0
    part, ws = ctypes.c_void_p(1 << 20), 1 << 24
    A, F = z.BUCKET_ACCUMULATE, z.BUCKET_FINAL
    assert L.zero_bucket_reduce(arr, 1, 2, 4, 1.0, 0, part, ws, need, None) == 1           # unknown flag
    assert L.zero_bucket_reduce(arr, 1, 2, F, 1.0, 0, None, ws, need, None) == 1           # final, no partial
    assert L.zero_bucket_reduce(arr, 1, 2, F | A, 0.0, 0, part, ws, need, None) == 1       # final, scale <= 0
    assert L.zero_bucket_reduce(arr, 1, 2, F, float("inf"), 0, part, ws, need, None) == 1
    assert L.zero_bucket_reduce(arr, 1, 2, F, 1e-50, 0, part, ws, need, None) == 1          # binary32 rounding 0
    assert L.zero_bucket_reduce(arr, 1, 2, F, 1e300, 0, part, ws, need, None) == 1          # binary32 rounding inf
    assert L.zero_bucket_reduce(arr, 1, 0, A, 1.0, 0, part, ws, need, None) == 1            # M < 1
    assert L.zero_bucket_reduce(arr, -1, 2, A, 1.0, 0, part, ws, need, None) == 1
    assert L.zero_bucket_reduce(None, 1, 2, A, 1.0, 0, part, ws, need, None) == 1
    assert L.zero_bucket_reduce(arr, 1, 2, A, 1.0, 0, part, ws, need - 1, None) == 2        # ws short
    assert L.zero_bucket_reduce(arr, 1, 2, A, 1.0, 0, part, ws + 16, need, None) == 1       # ws misaligned
    assert L.zero_bucket_reduce(arr, 1, 2, A, 1.0, 0, part, None, need, None) == 1          # no ws
    nacc, k2 = _shards(acc=0)
    assert L.zero_bucket_reduce(nacc, 1, 2, A, 1.0, 0, part, ws, need, None) == 1           # no accumulator
    nul = (ctypes.c_void_p * 2)(256, None)
    arr2 = (z._CGradShard * 1)()
    arr2[0] = z._CGradShard(100, ctypes.cast(nul, ctypes.POINTER(ctypes.c_void_p)), 4096)
    assert L.zero_bucket_reduce(arr2, 1, 2, A, 1.0, 0, part, ws, need, None) == 1           # a null replica
    assert L.zero_bucket_reduce(arr, 0, 2, A, 1.0, 0, None, None, 0, None) == 0             # empty, not final
    neg, k3 = _shards(n=-1)
    assert L.zero_bucket_reduce_workspace_bytes(neg, 1, 2) == 0
    assert L.zero_bucket_reduce_workspace_bytes(arr, 1, 0) == 0


def test_step_accumulated_argument_checks():
    L = z.lib()
    h = _hp(max_grad_norm=1.0)
    arr = (z._CAccTensor * 1)()
    big = (z._CAccTensor * 1)()
    big[0] = z._CAccTensor(1_000_000, 256, 1024, 2048, 4096, 8192)
    # no gradient copy: the step reads the caller's accumulator
    assert 0 < L.zero_step_accumulated_workspace_bytes(big, 1) < 1_000_000 // 100
    arr[0] = z._CAccTensor(100, 256, 1024, 2048, 4096, 8192)
    need = L.zero_step_accumulated_workspace_bytes(arr, 1)
    parts, res, ws = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21), 1 << 24
    assert L.zero_step_accumulated(arr, 1, ctypes.byref(h), parts, 1, 0, 0.0, ws, need, None, None) == 1  # no res
    assert L.zero_step_accumulated(arr, 1, ctypes.byref(h), None, 1, 0, 0.0, ws, need, res, None) == 1   # no partials
    assert L.zero_step_accumulated(arr, 1, ctypes.byref(h), parts, -1, 0, 0.0, ws, need, res, None) == 1
    assert L.zero_step_accumulated(arr, 1, ctypes.byref(h), parts, 1, 0, 0.0, ws, need - 1, res, None) == 2
    assert L.zero_step_accumulated(arr, 1, ctypes.byref(h), parts, 1, 0, 0.0, None, need, res, None) == 1
    bad = _hp(step=0)
    assert L.zero_step_accumulated(arr, 1, ctypes.byref(bad), parts, 1, 0, 0.0, ws, need, res, None) == 1
    arr2 = (z._CAccTensor * 1)()
    arr2[0] = z._CAccTensor(100, None, 1024, 2048, 4096, 8192)
    assert L.zero_step_accumulated(arr2, 1, ctypes.byref(h), parts, 1, 0, 0.0, ws, need, res, None) == 1
    arr3 = (z._CAccTensor * 1)()
    arr3[0] = z._CAccTensor(-1, None, None, None, None, None)
    assert L.zero_step_accumulated_workspace_bytes(arr3, 1) == 0
    assert L.zero_step_accumulated(arr3, 1, ctypes.byref(h), parts, 1, 0, 0.0, ws, need, res, None) == 1


def _offload(n=100, M=2):
    ptrs = (ctypes.c_void_p * M)(*[256 * (r + 1) for r in range(M)])
    arr = (z._COffloadTensor * 1)()
    arr[0] = z._COffloadTensor(n, ctypes.cast(ptrs, ctypes.POINTER(ctypes.c_void_p)), 1024, 2048, 4096, 8192)
    return arr, ptrs


def test_offload_step_argument_checks():
    L = z.lib()
    h = _hp(max_grad_norm=1.0)
    arr, keep = _offload()
    need = L.zero_offload_workspace_bytes(arr, 1, 2)
    hneed = L.zero_offload_host_workspace_bytes(arr, 1)
    assert need > 4 * 100 and hneed >= 6 * 100   # the fp32 gradient on the device; g and bf16 staged on the host
    res = z._CResult()
    ws, hw = 1 << 24, 1 << 25
    call = lambda a=arr, T=1, M=2, hp=h, w=ws, wb=need, hws=hw, hb=hneed, r=ctypes.byref(res), th=0: \
        L.zero_offload_step(a, T, M, ctypes.byref(hp), 0.0, w, wb, hws, hb, r, th, None)
    assert call(r=None) == 1                       # no result
    assert call(th=-1) == 1                        # negative thread count
    assert call(M=0) == 1
    assert call(T=-1) == 1
    assert call(hp=_hp(step=0)) == 1
    assert call(w=None) == 1 and call(w=ws + 16) == 1          # no / misaligned device workspace
    assert call(hws=None) == 1 and call(hws=hw + 8) == 1       # no / misaligned host workspace
    assert call(hb=hneed - 1) == 2                             # host workspace short
    assert call(wb=need - 1) == 2                              # device workspace short
    nul = (ctypes.c_void_p * 2)(256, None)
    arr2 = (z._COffloadTensor * 1)()
    arr2[0] = z._COffloadTensor(100, ctypes.cast(nul, ctypes.POINTER(ctypes.c_void_p)), 1024, 2048, 4096, 8192)
    assert call(a=arr2) == 1                                   # a null replica
    arr3, k3 = _offload()
    arr3[0].exp_avg = None
    assert call(a=arr3) == 1                                   # no host state
    neg, k4 = _offload(n=-1)
    assert L.zero_offload_workspace_bytes(neg, 1, 2) == 0 and L.zero_offload_host_workspace_bytes(neg, 1) == 0


def test_amp_forms_need_their_loss_scale():
    L = z.lib()
    c = z.LossScaleConfig()._c()
    bad = z.LossScaleConfig(window=0)._c()
    h = _hp()
    ls, res, ws, parts = ctypes.c_void_p(1 << 20), ctypes.c_void_p(1 << 21), 1 << 24, ctypes.c_void_p(1 << 22)
    arr, keep = _shards()
    need = L.zero_bucket_reduce_workspace_bytes(arr, 1, 2)
    assert L.zero_bucket_reduce_amp(arr, 1, 2, z.BUCKET_FINAL, 1.0, None, 0, parts, ws, need, None) == 1
    acc = (z._CAccTensor * 1)()
    acc[0] = z._CAccTensor(100, 256, 1024, 2048, 4096, 8192)
    an = L.zero_step_accumulated_workspace_bytes(acc, 1)
    assert L.zero_step_accumulated_amp(acc, 1, ctypes.byref(h), ctypes.byref(c), None, parts, 1, 0, 0.0, ws, an, res,
                                       None) == 1
    assert L.zero_step_accumulated_amp(acc, 1, ctypes.byref(h), ctypes.byref(bad), ls, parts, 1, 0, 0.0, ws, an, res,
                                       None) == 1
    off, k2 = _offload()
    on = L.zero_offload_workspace_bytes(off, 1, 2)
    hn = L.zero_offload_host_workspace_bytes(off, 1)
    r = z._CResult()
    assert L.zero_offload_step_amp(off, 1, 2, ctypes.byref(h), ctypes.byref(c), None, 0.0, ws, on, 1 << 25, hn,
                                   ctypes.byref(r), 0, None) == 1
    assert L.zero_offload_step_amp(off, 1, 2, ctypes.byref(h), None, ls, 0.0, ws, on, 1 << 25, hn, ctypes.byref(r),
                                   0, None) == 1


def test_noalloc_step_rejects_before_any_device_call():
    # zero_step_noalloc checks its arguments and its plan's size against the
    # static scratch on the host; these calls never reach the device (the
    # pointers are fake and there may be no GPU at all)
    L = z.lib()
    M = 4
    fake = (ctypes.c_void_p * M)(*[4096 * (r + 1) for r in range(M)])
    arr = (z._CTensor * 1)()
    clip = _hp(max_grad_norm=1.0)  # two-pass: the plan also holds the fp32 gradient, 4 B per element
    n_big = z.NOALLOC_SCRATCH_BYTES // 4 + 1
    arr[0] = z._CTensor(n_big, ctypes.cast(fake, ctypes.POINTER(ctypes.c_void_p)), 1 << 20, 2 << 20, 3 << 20, 4 << 20)
    assert L.zero_step_workspace_bytes(arr, 1, M, ctypes.byref(clip)) > z.NOALLOC_SCRATCH_BYTES
    assert L.zero_step_noalloc(arr, 1, M, ctypes.byref(clip), 0.0, ctypes.c_void_p(256), None) == \
        z.ZERO_ERR_SCRATCH_TOO_SMALL
    assert "scratch" in z.zero_status_string(z.ZERO_ERR_SCRATCH_TOO_SMALL)
    # argument errors come first
    assert L.zero_step_noalloc(arr, 1, M, ctypes.byref(clip), 0.0, None, None) == 1          # no result record
    assert L.zero_step_noalloc(arr, 1, 0, ctypes.byref(clip), 0.0, ctypes.c_void_p(256), None) == 1   # M < 1
    assert L.zero_step_noalloc(arr, 1, M, ctypes.byref(clip), -1.0, ctypes.c_void_p(256), None) == 1  # external < 0
    bad = _hp(grad_scale=1e-50)
    assert L.zero_step_noalloc(arr, 1, M, ctypes.byref(bad), 0.0, ctypes.c_void_p(256), None) == 1
    arr[0] = z._CTensor(10, ctypes.cast(fake, ctypes.POINTER(ctypes.c_void_p)), None, 2 << 20, 3 << 20, 4 << 20)
    assert L.zero_step_noalloc(arr, 1, M, ctypes.byref(clip), 0.0, ctypes.c_void_p(256), None) == 1  # no master
    # the single-pass plan of the 2e9-element shard (tables only) fits
    assert z.zero_step_workspace_bytes_for_sizes([2_000_000_000], 8, z.HParams()) <= z.NOALLOC_SCRATCH_BYTES
    assert z.zero_step_workspace_bytes_for_sizes([n_big], M, z.HParams(max_grad_norm=1.0)) > z.NOALLOC_SCRATCH_BYTES


def test_bucket_step_argument_checks():
    # zero_bucket_step refuses, before any device call, what it cannot do in
    # one pass (clipping, skipping), unknown flags, a missing partial and an
    # accumulating call without accumulators
    L = z.lib()
    M = 2
    fake = (ctypes.c_void_p * M)(4096, 8192)
    arr = (z._CBucketTensor * 1)()
    arr[0] = z._CBucketTensor(100, ctypes.cast(fake, ctypes.POINTER(ctypes.c_void_p)), None, 1 << 20, 2 << 20,
                              3 << 20, 4 << 20)
    need = L.zero_bucket_step_workspace_bytes(arr, 1, M)
    assert need > 0
    ok = _hp()
    part, ws = ctypes.c_void_p(256), ctypes.c_void_p(1 << 24)
    assert L.zero_bucket_step(arr, 1, M, 0, ctypes.byref(_hp(max_grad_norm=1.0)), 1, part, ws, need, None) == 1
    assert L.zero_bucket_step(arr, 1, M, 0, ctypes.byref(_hp(skip_on_nonfinite=1)), 1, part, ws, need, None) == 1
    assert L.zero_bucket_step(arr, 1, M, z.BUCKET_FINAL, ctypes.byref(ok), 1, part, ws, need, None) == 1
    assert L.zero_bucket_step(arr, 1, M, 8, ctypes.byref(ok), 1, part, ws, need, None) == 1
    assert L.zero_bucket_step(arr, 1, M, z.BUCKET_STREAM_STORES | z.BUCKET_FINAL, ctypes.byref(ok), 1, part, ws, need,
                              None) == 1
    assert L.zero_bucket_step(arr, 1, M, z.BUCKET_ACCUMULATE, ctypes.byref(ok), 1, part, ws, need, None) == 1
    assert L.zero_bucket_step(arr, 1, M, 0, ctypes.byref(ok), 1, None, ws, need, None) == 1
    assert L.zero_bucket_step(arr, 1, 0, 0, ctypes.byref(ok), 1, part, ws, need, None) == 1
    assert L.zero_bucket_step(arr, -1, M, 0, ctypes.byref(ok), 1, part, ws, need, None) == 1
    assert L.zero_bucket_step(arr, 1, M, 0, ctypes.byref(_hp(grad_scale=1e-50)), 1, part, ws, need, None) == 1
    arr[0] = z._CBucketTensor(100, ctypes.cast(fake, ctypes.POINTER(ctypes.c_void_p)), None, None, 2 << 20,
                              3 << 20, 4 << 20)
    assert L.zero_bucket_step(arr, 1, M, 0, ctypes.byref(ok), 1, part, ws, need, None) == 1   # no master
    arr[0] = z._CBucketTensor(-1, None, None, None, None, None, None)
    assert L.zero_bucket_step_workspace_bytes(arr, 1, M) == 0
