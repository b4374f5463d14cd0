"""The seeded input generator (CPU): known-answer vectors of Philox4x32-10,
determinism, gather == fill, and the moments of the synthetic distributions."""
import numpy as np
import pytest

import synth
from synth.workloads import WORKLOADS


@pytest.mark.parametrize("ctr,key,want", [
    # Known-answer vectors of Philox4x32-10 (Salmon et al., SC 2011 reference set)
    ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
    ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
    ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
     [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
])
def test_philox_known_answers(ctr, key, want):
    assert synth.philox4x32_10(ctr, key) == want


def test_fill_is_deterministic_and_gather_matches():
    st = synth.stream_id(synth.KIND_GRAD, 5, 3)
    a = synth.host_bf16(100000, 1001, st, 1e-4, start=12345)
    b = synth.host_bf16(100000, 1001, st, 1e-4, start=12345)
    assert np.array_equal(a, b)
    idx = np.array([12345, 12346, 50000, 112344], np.int64)
    assert np.array_equal(synth.host_bf16_at(idx, 1001, st, 1e-4), a[idx - 12345])
    f = synth.host_f32(1000, 7, st, 0.02, start=99)
    assert np.array_equal(synth.host_f32_at(np.arange(99, 1099), 7, st, 0.02), f)
    # different streams and seeds give different data
    assert not np.array_equal(a, synth.host_bf16(100000, 1001, st + 1, 1e-4, start=12345))
    assert not np.array_equal(a, synth.host_bf16(100000, 1002, st, 1e-4, start=12345))


def test_bf16_codes_are_truncated_float_values():
    st = synth.stream_id(synth.KIND_GRAD, 0, 0)
    f = synth.host_f32(50000, 3, st, 1e-4)
    h = synth.host_bf16(50000, 3, st, 1e-4)
    assert np.array_equal(h, (f.view(np.uint32) >> 16).astype(np.uint16))


def test_moments_of_the_synthetic_distributions():
    n = 1 << 20
    z = synth.host_f32(n, 11, synth.stream_id(synth.KIND_MASTER, 0, 0), 1.0).astype(np.float64)
    assert abs(z.mean()) < 5e-3 and abs(z.std() - 1.0) < 5e-3
    k = ((z - z.mean()) ** 4).mean() / z.var() ** 2
    assert abs(k - (3 - 1.2 / 8)) < 0.03  # Irwin-Hall(8) kurtosis 2.85
    a = synth.host_f32(n, 11, synth.stream_id(synth.KIND_EXP_AVG_SQ, 0, 0), 1e-8, absval=True)
    assert (a >= 0).all() and abs(a.mean() / 1e-8 - 0.7979) < 0.01  # E|z| = sqrt(2/pi)


def test_inject_positions_seeded_and_in_range():
    p1 = synth.inject_positions(1004, 1, 8, 2_000_000_000, 1e-9)
    p2 = synth.inject_positions(1004, 1, 8, 2_000_000_000, 1e-9)
    assert p1 == p2 and 1 <= len(p1) <= 60
    assert all(0 <= r < 8 and 0 <= i < 2_000_000_000 for r, i in p1)
    assert synth.inject_positions(1004, 3, 8, 2_000_000_000, 1e-9) != p1
    assert len(synth.inject_positions(1, 1, 4, 100, 1e-9)) == 1  # at least one


def test_workload_shapes():
    w = WORKLOADS
    assert w[0].n_total == 262_144 and w[0].M == 4
    assert w[1].n_total == 15_554_976 and w[1].tensors[0].start == 46_664_928
    assert w[2].n_total == 117_187_500 and w[2].M == 64
    assert len(w[3].tensors) == 288 and w[3].n_total == 809_533_440
    assert sorted({t.n for t in w[3].tensors}) == [512, 2_097_152, 5_636_096]
    assert w[4].n_total == 2_000_000_000 and w[4].grad_scale == 2.0**-16
    assert [x.bytes_per_param() for x in w] == [34, 50, 154, 42, 50]
