"""Host-side checks of the seeded input generators (CPU only)."""
import numpy as np
import torch

from group_gemm_amd import workloads as W


def test_balanced_rule_examples():
    # "Group-GEMM in XLA", Part 2 "Autotuning" and Part 4 "Fixing group_sizes
    # Deterministically": 1024 rows over 4 groups, and 1002 rows over 4 groups.
    assert W.balanced_group_sizes(1024, 4).tolist() == [256, 256, 256, 256]
    assert W.balanced_group_sizes(1002, 4).tolist() == [251, 251, 250, 250]
    gs = W.balanced_group_sizes(8191, 8)
    assert gs.sum() == 8191 and gs.max() - gs.min() == 1


def test_every_workload_sums_to_m():
    for w in W.WORKLOADS.values():
        gs = W.group_sizes(w)
        assert gs.dtype == np.int32 and gs.shape == (w.g,) and int(gs.sum()) == w.m
        assert np.all(gs >= 0)


def test_workload_shapes_of_routing():
    gs1 = W.group_sizes(W.WORKLOADS["tiny_fp32"])
    assert gs1.tolist() == [16, 0, 40, 8]
    gs2 = W.group_sizes(W.WORKLOADS["mixtral8x7b_up_bf16"])
    assert gs2.min() > 900 and gs2.max() < 1150                 # near-balanced top-2 of 8
    assert np.array_equal(gs2, W.group_sizes(W.WORKLOADS["mixtral8x7b_up_mxfp8"]))
    gs3 = W.group_sizes(W.WORKLOADS["deepseekv3_routed_bf16"])
    assert (gs3 < 16).sum() >= 3 and (gs3 > 1000).sum() >= 3    # skewed: tiny and huge groups
    gz = W.group_sizes(W.WORKLOADS["deepseekv3_routed_bf16_zeros"])
    assert (gz == 0).sum() == 4
    assert np.array_equal(gs2, W.group_sizes(W.WORKLOADS["mixtral8x7b_dgrad_bf16"]))
    gs5 = W.group_sizes(W.WORKLOADS["llama4scout_wgrad_bf16"])
    assert gs5.max() > 2 * gs5.mean()                           # Dirichlet(0.5) is uneven


def test_seeds_reproduce():
    w = W.WORKLOADS["deepseekv3_routed_bf16"]
    assert np.array_equal(W.group_sizes(w, 0), W.group_sizes(w, 0))
    assert not np.array_equal(W.group_sizes(w, 0), W.group_sizes(w, 1))


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.14159], dtype=np.float32)
    ours = W.f32_to_bf16_bits(x)
    lib = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, lib)


def test_mx_quantize_round_trip():
    x = torch.randn(6, 96, generator=torch.Generator().manual_seed(0))
    codes, scales = W.mx_quantize(x, axis=1)
    assert codes.dtype == torch.uint8 and codes.shape == (6, 96) and scales.shape == (6, 3)
    deq = codes.view(torch.float8_e4m3fn).double() * torch.repeat_interleave(
        scales.view(torch.float8_e8m0fnu).double(), 32, dim=1)
    # e4m3 keeps 3 mantissa bits (relative rounding error <= 2^-4); the shared exponent
    # floor(log2 amax) - 8 puts the block maximum in [256, 512) and values above 448 are
    # clipped, so the largest elements of a block may lose up to 1/8
    err = (deq - x.double()).abs()
    xa = x.double().abs()
    assert torch.all(err <= 0.125 * xa + 2 ** -9 * xa.amax())
    assert (err <= 2 ** -4 * xa + 1e-12).double().mean() > 0.9
    # scales along the other axis of a 3-D tensor
    w = torch.randn(2, 64, 5, generator=torch.Generator().manual_seed(1))
    c3, s3 = W.mx_quantize(w, axis=1)
    assert c3.shape == (2, 64, 5) and s3.shape == (2, 2, 5)


def test_small_inputs_layout():
    d = W.small_inputs("m", "bf16", 10, 16, 8, [3, 7])
    assert d["lhs"].dtype == torch.bfloat16 and d["lhs"].shape == (10, 16)
    assert d["rhs"].shape == (2, 16, 8)
    d = W.small_inputs("k", "f32", 10, 16, 8, [3, 7])
    assert d["dout"].shape == (10, 8)
    d = W.small_inputs("m", "mxfp8", 10, 64, 8, [3, 7])
    assert d["lhs_scale"].shape == (10, 2) and d["rhs_scale"].shape == (2, 2, 8)
