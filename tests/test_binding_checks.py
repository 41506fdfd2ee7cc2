"""The Python binding refuses, before any launch, arguments whose pointers would not
address device memory of the size the kernels assume.  CPU part: tensors in host memory
are refused (a host address handed to a kernel would be read as a device address); the
GPU part with device tensors of the wrong shape, dtype or layout is in
test_gpu_parity.py."""
import pytest
import torch

from group_gemm_amd import _binding as B


def test_host_tensors_are_refused():
    lhs = torch.zeros(64, 32, dtype=torch.bfloat16)
    rhs = torch.zeros(2, 32, 16, dtype=torch.bfloat16)
    gs = torch.tensor([32, 32], dtype=torch.int32)
    dout = torch.zeros(64, 16, dtype=torch.bfloat16)
    for call in (lambda: B.ragged_dot_m(lhs, rhs, gs),
                 lambda: B.ragged_dot_m(lhs, rhs, gs, beta=1.0),
                 lambda: B.ragged_dot_k(lhs, dout, gs),
                 lambda: B.ragged_dot_m_gated(lhs, rhs, rhs, gs),
                 lambda: B.padded_dot("m", lhs, rhs, gs, 32),
                 lambda: B.padded_dot("k", lhs, dout, gs, 32),
                 lambda: B.moe_permute(lhs, torch.zeros(64, 2, dtype=torch.int32), 4),
                 lambda: B.moe_unpermute(lhs, torch.zeros(64, dtype=torch.int32), torch.zeros(32, 2)),
                 lambda: B.build_schedule(gs, 64, 16, 32, 16),
                 lambda: B.read_device_status(torch.zeros(256, dtype=torch.uint8))):
        with pytest.raises(ValueError, match="CUDA"):
            call()


def test_non_tensors_are_refused():
    with pytest.raises(TypeError):
        B._tensor([1, 2], "x", None)


def test_tensor_check_messages():
    # the checks that do not need device memory: layout, shape and dtype are examined
    # only after the device, so a host tensor reports its device first
    t = torch.zeros(4, 4).t()
    with pytest.raises(ValueError, match="CUDA"):
        B._tensor(t, "t", None, shape=(4, 4), dtype=torch.float32)
