"""The Python binding's own argument checks, on the CPU: the device buffers
the library writes through from kernels must be device tensors, so that a
host address never reaches a kernel."""
import pytest
import torch

import sharded_optimizer_step_amd as z


def test_workspace_check_accepts_none_and_sizes_any_dtype():
    assert z._need_ws(None) == 0


@pytest.mark.parametrize("ws", [torch.empty(64, dtype=torch.uint8), torch.empty(16, dtype=torch.float32)])
def test_host_workspace_is_rejected(ws):
    with pytest.raises(ValueError, match="device tensor"):
        z._need_ws(ws)


def test_non_tensor_workspace_is_rejected():
    with pytest.raises(TypeError):
        z._need_ws(bytearray(64))


def test_device_checks_reject_host_tensors_for_device_arguments():
    with pytest.raises(ValueError, match="device tensor"):
        z._need(torch.empty(8, dtype=torch.float32), torch.float32, "g")
    with pytest.raises(TypeError, match="expected torch.bfloat16"):
        z._need(torch.empty(8, dtype=torch.float32), torch.bfloat16, "grads[0]")


def test_host_checks_reject_wrong_dtype_and_sizes():
    with pytest.raises(TypeError):
        z._need_host(torch.empty(8, dtype=torch.float64), torch.float32, "master")
    with pytest.raises(ValueError, match="expected 9 elements"):
        z._need_host(torch.empty(8, dtype=torch.float32), torch.float32, "master", 9)
    with pytest.raises(ValueError, match="contiguous"):
        z._need_host(torch.empty(8, 2, dtype=torch.float32).t(), torch.float32, "master")
