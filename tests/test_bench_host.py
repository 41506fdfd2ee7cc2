"""Host-side checks of the benchmark's accounting (no GPU): the useful flops and the
algorithmic bytes it divides by the measured time are the closed forms of each workload,
and a request for more than one GPU is refused with a message."""
import os
import subprocess
import sys

import numpy as np

import bench
from group_gemm_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_headline_flops_and_bytes_closed_form():
    w = W.WORKLOADS["mixtral8x7b_up_bf16"]
    gs = W.group_sizes(w)
    assert int(gs.sum()) == 8192 and int((gs > 0).sum()) == 8
    # useful work: 2 flops per multiply-add of every routed row with its expert's matrix
    assert bench.useful_flops(w, gs) == 2.0 * 8192 * 4096 * 14336
    # bytes: lhs once, the 8 experts' weights once, the bf16 output once
    assert bench.algorithmic_bytes(w, gs) == 8192 * 4096 * 2 + 8 * 4096 * 14336 * 2 + 8192 * 14336 * 2


def test_skewed_routing_counts_only_non_empty_experts():
    w = W.WORKLOADS["deepseekv3_routed_bf16_zeros"]
    gs = W.group_sizes(w)
    nonempty = int((gs > 0).sum())
    assert nonempty < w.g
    assert bench.algorithmic_bytes(w, gs) == (w.m * w.k * 2 + nonempty * w.k * w.n * 2 + w.m * w.n * 2)


def test_mxfp8_bytes_include_scales():
    w = W.WORKLOADS["mixtral8x7b_up_mxfp8"]
    gs = W.group_sizes(w)
    k32 = w.k // 32
    expect = w.m * w.k + 8 * w.k * w.n + w.m * w.n * 2 + w.m * k32 + 8 * k32 * w.n
    assert bench.algorithmic_bytes(w, gs) == expect


def test_contracting_and_gated_accounting():
    w = W.WORKLOADS["llama4scout_wgrad_bf16"]
    gs = W.group_sizes(w)
    S = int(gs.sum())
    assert bench.useful_flops(w, gs) == 2.0 * S * w.k * w.n
    # rows of both operands once, and every [k, n] slab of the fp32 output, empty groups included
    assert bench.algorithmic_bytes(w, gs) == S * w.k * 2 + S * w.n * 2 + w.g * w.k * w.n * 4
    g = W.WORKLOADS["mixtral8x7b_gated_bf16"]
    gsg = W.group_sizes(g)
    assert bench.useful_flops(g, gsg) == 2 * bench.useful_flops(W.WORKLOADS["mixtral8x7b_up_bf16"], gsg)


def test_routing_workloads_are_rated_in_bytes():
    p = W.WORKLOADS["deepseekv3_permute_bf16"]
    u = W.WORKLOADS["deepseekv3_unpermute_bf16"]
    assert bench.useful_flops(p, None) == 0.0
    # permute: token rows and ids read once; sorted rows, both index maps and the sizes written
    assert bench.algorithmic_bytes(p, None) == p.tokens * p.k * 2 + p.m * 4 + p.m * p.k * 2 + 2 * p.m * 4 + p.g * 4
    # un-permute: expert rows, inverse order and weights read once; token rows written
    assert bench.algorithmic_bytes(u, None) == u.m * u.n * 2 + u.m * 4 + u.m * 4 + u.tokens * u.n * 2


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
