"""ragged_dot_m_noalloc, called through the C ABI, against ragged_dot_m on the same inputs:
two calls in a row on one GPU (the second with a smaller input, so the library's static
scratch keeps the first call's state when the second starts), bf16 on the per-XCD tile
queues, MXFP8 and fp32; the status bits reach the caller's word."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from group_gemm_amd import _binding as B
from group_gemm_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def noalloc(d, out, status=None):
    """The C-ABI call itself (ctypes), no workspace."""
    m, k = d["lhs"].shape
    g, _, n = d["rhs"].shape
    code = B.lib().ragged_dot_m_noalloc(_p(d["lhs"]), _p(d["rhs"]), _p(d["group_sizes"]), _p(out), m, k, n, g,
                                        B.GG_DT[d["lhs"].dtype], B.GG_DT[out.dtype], _p(d.get("lhs_scale")),
                                        _p(d.get("rhs_scale")), _p(status),
                                        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert code == 0, B.status_string(code)
    return out


CASES = [
    # (kind, first (m, k, n, group_sizes), second, smaller)
    ("bf16", (4000, 128, 2304, [0, 17, 300, 1, 256, 129, 700, 5, 0, 64, 128, 127, 257, 33, 90, 200, 11, 0, 40, 60,
                                3, 8, 100, 2, 0, 50, 12, 7, 1, 399]),
     (700, 256, 512, [1, 255, 256, 150, 0, 38])),
    ("mxfp8", (600, 512, 400, [0, 37, 256, 1, 300, 6]), (257, 128, 256, [128, 129])),
    ("f32", (300, 192, 264, [7, 1, 255, 0]), (64, 128, 64, [16, 0, 40, 8])),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_noalloc_matches_ragged_dot_m(case):
    kind, first, second = CASES[case]
    for i, (m, k, n, gs) in enumerate((first, second)):
        say("noalloc", kind, "call", i, m, k, n, len(gs))
        d = {key: v.to(DEV) for key, v in W.small_inputs("m", kind, m, k, n, gs, seed=90 + 2 * case + i).items()}
        out_dtype = torch.float32 if kind == "f32" else torch.bfloat16
        want = B.ragged_dot_m(d["lhs"], d["rhs"], d["group_sizes"], out_dtype=out_dtype,
                              lhs_scale=d.get("lhs_scale"), rhs_scale=d.get("rhs_scale"))
        out = torch.full((m, n), float("nan"), dtype=out_dtype, device=DEV)
        status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
        noalloc(d, out, status)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: bit-identical, and within the oracle's bar
        assert torch.equal(out.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32),
                           want.view(torch.int16 if out_dtype == torch.bfloat16 else torch.int32))
        assert int(status.item()) == 0
        ref = oracle.ragged_dot_m(W.to_numpy_raw(d["lhs"]), W.to_numpy_raw(d["rhs"]), np.array(gs, np.int32),
                                  W.to_numpy_raw(d["lhs_scale"]) if "lhs_scale" in d else None,
                                  W.to_numpy_raw(d["rhs_scale"]) if "rhs_scale" in d else None)
        y = out.double().cpu().numpy()
        if out_dtype == torch.float32:
            assert np.linalg.norm(y - ref) <= 1e-5 * np.linalg.norm(ref)
        else:
            assert np.all(np.abs(y - ref) <= 1e-2 * np.abs(ref) + 1e-2)
        assert torch.all(out[sum(gs):] == 0)


def test_noalloc_status_and_no_status_word():
    say("noalloc status bits")
    m, k, n = 200, 64, 64
    d = {key: v.to(DEV) for key, v in W.small_inputs("m", "bf16", m, k, n, [0, 120, 80, 0], seed=99).items()}
    d["group_sizes"] = torch.tensor([-5, 120, 150, 3], dtype=torch.int32, device=DEV)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    out = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    noalloc(d, out, status)
    want = B.ragged_dot_m(d["lhs"], d["rhs"], d["group_sizes"])
    torch.cuda.synchronize()
    assert int(status.item()) == 3
    assert torch.equal(out.view(torch.int16), want.view(torch.int16))
    # without a status word the bits stay in the library's scratch; the result is the same
    out2 = torch.empty_like(out)
    noalloc(d, out2, None)
    torch.cuda.synchronize()
    assert torch.equal(out2.view(torch.int16), want.view(torch.int16))
