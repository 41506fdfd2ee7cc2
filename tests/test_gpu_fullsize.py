"""GPU parity at the full workload sizes, in the call the benchmark times.

The oracle cannot recompute a whole [32768, 2048] or [16, 5120, 8192] result in test
time, so it checks sampled outputs one by one: in the non-contracting form, the first and
last row of every group (group edges are where a wrong offset shows), one row in every
256-row tile of every group and random rows; in the contracting form, both ends of k and
one k-index in every 256-wide k-tile of every group.  Every
element of the result is also checked for properties that hold at any size: finite, and
exactly zero past sum(group_sizes).
"""
import numpy as np
import pytest
import torch

import oracle
from group_gemm_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)


def raw(t):
    return W.to_numpy_raw(t)


def sample_rows(gs, rng, extra=64, tile=256):
    """The first and last row of every non-empty group, one random row in every 256-row
    m-tile of every group (so every output tile the kernel computes is compared on at
    least one row, over all of its columns), plus `extra` random rows."""
    starts = np.concatenate([[0], np.cumsum(gs)[:-1]])
    rows = []
    for h in np.nonzero(gs)[0]:
        st, s = int(starts[h]), int(gs[h])
        rows += [st, st + s - 1]
        for t0 in range(0, s, tile):
            rows.append(st + t0 + int(rng.integers(0, min(tile, s - t0))))
    rows += rng.integers(0, int(gs.sum()), extra).tolist()
    return np.unique(np.array(rows, dtype=np.int64))


@pytest.mark.parametrize("name", ["mixtral8x7b_up_bf16", "deepseekv3_routed_bf16", "deepseekv3_routed_bf16_zeros",
                                  "mixtral8x7b_up_mxfp8"])
def test_full_size_ragged_m(name):
    import group_gemm_amd as G
    w = W.WORKLOADS[name]
    say("full size", name)
    gs = W.group_sizes(w)
    d = W.make_inputs(w, device=DEV, gs=gs)
    out = torch.full((w.m, w.n), float("nan"), dtype=torch.bfloat16, device=DEV)
    G.ragged_dot_m(d["lhs"], d["rhs"], d["group_sizes"], out=out, lhs_scale=d.get("lhs_scale"),
                   rhs_scale=d.get("rhs_scale"))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite output"
    S = int(gs.sum())
    if S < w.m:
        assert bool((out[S:] == 0).all())
    rng = np.random.default_rng(w.wid)
    # the MXFP8 oracle decodes two scales per product: fewer extra rows for it
    rows = sample_rows(gs, rng, extra=8 if w.in_dtype == "mxfp8" else 64)
    ref = oracle.ragged_dot_m(raw(d["lhs"]), raw(d["rhs"]), gs, raw(d["lhs_scale"]) if "lhs_scale" in d else None,
                              raw(d["rhs_scale"]) if "rhs_scale" in d else None, rows=rows)
    y = out[torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
    bad = np.abs(y - ref) > 1e-2 * np.abs(ref) + 1e-2
    assert not bad.any(), f"{name}: {int(bad.sum())} of {bad.size} sampled elements outside the bf16 bar"


def test_full_size_ragged_m_nk():
    """The data-gradient workload: [g,n,k] weights as stored, sampled rows against the oracle."""
    import group_gemm_amd as G
    w = W.WORKLOADS["mixtral8x7b_dgrad_bf16"]
    say("full size", w.name)
    gs = W.group_sizes(w)
    d = W.make_inputs(w, device=DEV, gs=gs)
    out = torch.full((w.m, w.n), float("nan"), dtype=torch.bfloat16, device=DEV)
    G.ragged_dot_m(d["lhs"], d["rhs"], d["group_sizes"], out=out, rhs_layout="nk")
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite output"
    rows = sample_rows(gs, np.random.default_rng(w.wid))
    ref = oracle.ragged_dot_m_nk(raw(d["lhs"]), raw(d["rhs"]), gs, rows=rows)
    y = out[torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
    bad = np.abs(y - ref) > 1e-2 * np.abs(ref) + 1e-2
    assert not bad.any(), f"{w.name}: {int(bad.sum())} of {bad.size} sampled elements outside the bf16 bar"


def test_full_size_ragged_m_gated():
    """The fused gate/up workload (SiLU), sampled rows against the oracle."""
    import group_gemm_amd as G
    w = W.WORKLOADS["mixtral8x7b_gated_bf16"]
    say("full size", w.name)
    gs = W.group_sizes(w)
    d = W.make_inputs(w, device=DEV, gs=gs)
    out = torch.full((w.m, w.n), float("nan"), dtype=torch.bfloat16, device=DEV)
    G.ragged_dot_m_gated(d["lhs"], d["w0"], d["w1"], d["group_sizes"], act="silu", out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite output"
    rows = sample_rows(gs, np.random.default_rng(w.wid))
    ref = oracle.ragged_dot_m_gated(raw(d["lhs"]), raw(d["w0"]), raw(d["w1"]), gs, act="silu", rows=rows)
    y = out[torch.from_numpy(rows).to(DEV)].double().cpu().numpy()
    bad = np.abs(y - ref) > 1e-2 * np.abs(ref) + 1e-2
    assert not bad.any(), f"{w.name}: {int(bad.sum())} of {bad.size} sampled elements outside the bf16 bar"


def test_full_size_ragged_k():
    import group_gemm_amd as G
    w = W.WORKLOADS["llama4scout_wgrad_bf16"]
    say("full size", w.name)
    gs = W.group_sizes(w)
    d = W.make_inputs(w, device=DEV, gs=gs)
    out = torch.full((w.g, w.k, w.n), float("nan"), dtype=torch.float32, device=DEV)
    G.ragged_dot_k(d["lhs"], d["dout"], d["group_sizes"], out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite output"
    # both ends of k and one k-index in every 256-wide k-tile, for every group
    rng = np.random.default_rng(5)
    pairs = []
    for h in range(w.g):
        ks = {0, w.k - 1} | {t0 + int(rng.integers(0, min(256, w.k - t0))) for t0 in range(0, w.k, 256)}
        pairs += [(h, i) for i in sorted(ks)]
    pairs = np.array(pairs, dtype=np.int64)
    ref = oracle.ragged_dot_k(raw(d["lhs"]), raw(d["dout"]), gs, pairs=pairs)
    y = out[torch.from_numpy(pairs[:, 0]).to(DEV), torch.from_numpy(pairs[:, 1]).to(DEV)].double().cpu().numpy()
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel <= 1e-5, f"normwise relative error {rel:.3e} over the sampled rows"
    for h in np.nonzero(gs == 0)[0]:
        assert bool((out[h] == 0).all())


def test_ragged_k_group_over_2gib():
    """A group whose dout rows span more than 2 GiB: the ring loads address one 32-row slice at
    a time, so the vectorised kernel covers it (k = 64, n = 16384, 68000 rows in one group)."""
    import group_gemm_amd as G
    m, k, n = 70000, 64, 16384
    gs = np.array([68000, 0, 2000], dtype=np.int32)
    assert m * n * 2 > 2 ** 31
    say("ragged_dot_k, dout over 2 GiB", m, k, n, gs.tolist())
    gen = torch.Generator(device=DEV).manual_seed(11)
    lhs = torch.randn((m, k), generator=gen, device=DEV).to(torch.bfloat16)
    dout = torch.randn((m, n), generator=gen, device=DEV).to(torch.bfloat16)
    out = torch.full((3, k, n), float("nan"), dtype=torch.float32, device=DEV)
    G.ragged_dot_k(lhs, dout, torch.from_numpy(gs).to(DEV), out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), "non-finite output"
    assert bool((out[1] == 0).all())
    pairs = np.array([(0, 0), (0, 37), (0, k - 1), (2, 0), (2, 21), (2, k - 1)], dtype=np.int64)
    ref = oracle.ragged_dot_k(raw(lhs), raw(dout), gs, pairs=pairs)
    y = out[torch.from_numpy(pairs[:, 0]).to(DEV), torch.from_numpy(pairs[:, 1]).to(DEV)].double().cpu().numpy()
    rel = np.linalg.norm(y - ref) / np.linalg.norm(ref)
    assert rel <= 1e-5, f"normwise relative error {rel:.3e} over the sampled rows"


def test_full_size_padded_matches_ragged():
    """The padded baseline, at the size the benchmark times it, gives the ragged result."""
    import group_gemm_amd as G
    w = W.WORKLOADS["mixtral8x7b_up_bf16"]
    say("full size padded", w.name)
    gs = W.group_sizes(w)
    d = W.make_inputs(w, device=DEV, gs=gs)
    cap = int(np.ceil(gs.max() / 256) * 256)
    y_pad = G.padded_dot("m", d["lhs"], d["rhs"], d["group_sizes"], cap)
    y_rag = G.ragged_dot_m(d["lhs"], d["rhs"], d["group_sizes"])
    torch.cuda.synchronize()
    # same kernel family, same k order per element: the two results agree to bf16 rounding
    diff = (y_pad.float() - y_rag.float()).abs()
    assert float(diff.max()) <= 1e-2 + 1e-2 * float(y_rag.float().abs().max())
