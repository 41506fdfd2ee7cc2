"""GPU parity of the MoE permute / un-permute calls through the C ABI against the oracle.

Permute is index and byte work, so every output is compared bit-exactly: sorted rows,
scale rows, group_sizes, both index maps.  Un-permute is a weighted sum: fp32 outputs
normwise within 1e-5 of the fp64 oracle, bf16 outputs every element within
1e-2 |ref| + 1e-2.  Outputs start out as garbage (NaN / -7) so that an element the call
fails to write shows.
("Group-GEMM in XLA", Part 4 "The Three MoE Compute Paths in MaxText", Path 1.)
"""
import numpy as np
import pytest
import torch

import oracle
from group_gemm_amd import workloads as W

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def gg():
    import group_gemm_amd
    return group_gemm_amd


def say(*a):
    print("[case]", *a, flush=True)


def raw(t):
    return W.to_numpy_raw(t)


def draw_experts(r, tokens, top_k, g, distinct=True):
    if distinct and top_k <= g:
        return W.topk_indices(r.standard_normal((tokens, g)), top_k).astype(np.int32)
    return r.integers(0, g, size=(tokens, top_k)).astype(np.int32)


def make_x(r, tokens, k, dtype):
    x = r.standard_normal((tokens, k)).astype(np.float32)
    if dtype == "f32":
        return torch.from_numpy(x).to(DEV), None
    if dtype == "bf16":
        return torch.from_numpy(W.f32_to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).to(DEV), None
    codes, scales = W.mx_quantize(torch.from_numpy(x), axis=1)
    return codes.to(DEV), scales.to(DEV)


def run_permute(x, experts_np, g, x_scale=None, ws=None):
    """moe_permute with outputs and workspace that start out as garbage."""
    G = gg()
    e = torch.from_numpy(experts_np).to(DEV)
    tokens, k = x.shape
    M = experts_np.size
    if ws is None:
        ws = torch.empty(G.workspace_bytes("permute", M, k, 0, g, 0, x.dtype), dtype=torch.uint8, device=DEV)
        ws.fill_(0xAB)
    k32 = None if x_scale is None else x_scale.shape[1]
    out = (torch.full((M, k), float("nan"), device=DEV).to(x.dtype) if x.dtype != torch.uint8
           else torch.full((M, k), 0x7F, dtype=torch.uint8, device=DEV),
           None if x_scale is None else torch.full((M, k32), 0xEE, dtype=torch.uint8, device=DEV),
           torch.full((g,), -7, dtype=torch.int32, device=DEV),
           torch.full((M,), -7, dtype=torch.int32, device=DEV),
           torch.full((M,), -7, dtype=torch.int32, device=DEV))
    outs = G.moe_permute(x, e, g, x_scale=x_scale, workspace=ws, out=out)
    torch.cuda.synchronize()
    return outs, ws


PERMUTE_CASES = [
    # tokens, top_k, k, g, dtype, note
    (1, 1, 8, 1, "bf16", "one copy"),
    (37, 2, 64, 8, "bf16", "Mixtral-like top-2 of 8"),
    (301, 8, 128, 256, "bf16", "DeepSeek-like top-8 of 256"),
    (200, 4, 96, 1024, "bf16", "g at its maximum"),
    (129, 3, 40, 5, "f32", "fp32 rows"),
    (64, 2, 13, 6, "bf16", "rows not a multiple of 16 bytes"),
    (90, 2, 256, 8, "e4m3", "e4m3 rows with E8M0 scale rows"),
    (9000, 8, 16, 64, "bf16", "72000 copies: several chunks of several 1024-copy steps"),
    (20000, 8, 8, 256, "bf16", "160000 copies"),
]


@pytest.mark.parametrize("tokens,top_k,k,g,dtype,note", PERMUTE_CASES)
def test_permute_matches_oracle(tokens, top_k, k, g, dtype, note):
    say("permute", tokens, top_k, k, g, dtype, note)
    r = np.random.default_rng([tokens, top_k, k, g])
    x, xs = make_x(r, tokens, k, dtype)
    experts = draw_experts(r, tokens, top_k, g)
    (sx, ss, gs, s2c, c2s), ws = run_permute(x, experts, g, xs)
    want = oracle.moe_permute(raw(x), experts, g, None if xs is None else raw(xs))
    assert np.array_equal(raw(gs), want[2])
    assert np.array_equal(raw(s2c), want[3])
    assert np.array_equal(raw(c2s), want[4])
    assert np.array_equal(raw(sx), want[0])
    if xs is not None:
        assert np.array_equal(raw(ss), want[1])
    assert gg().read_device_status(ws) == 0


def test_permute_unrouted_ids_and_status():
    say("permute: ids outside [0, g) are not routed and flagged")
    r = np.random.default_rng(5)
    tokens, top_k, k, g = 500, 4, 32, 16
    x, _ = make_x(r, tokens, k, "bf16")
    experts = draw_experts(r, tokens, top_k, g)
    experts[3, 0], experts[77, 2], experts[499, 3] = -1, g, 1 << 20
    (sx, _, gs, s2c, c2s), ws = run_permute(x, experts, g)
    want = oracle.moe_permute(raw(x), experts, g)
    for got, ref in zip((sx, gs, s2c, c2s), (want[0], want[2], want[3], want[4])):
        assert np.array_equal(raw(got), ref)
    assert int(raw(gs).sum()) == tokens * top_k - 3
    assert (raw(sx)[-3:] == 0).all() and (raw(s2c)[-3:] == -1).all()
    assert gg().read_device_status(ws) & 0x8
    # a clean call on the same workspace clears the flag
    run_permute(x, draw_experts(r, tokens, top_k, g), g, ws=ws)
    assert gg().read_device_status(ws) == 0


def test_permute_empty():
    say("permute: zero tokens")
    G = gg()
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    e = torch.empty((0, 2), dtype=torch.int32, device=DEV)
    sx, _, gs, s2c, c2s = G.moe_permute(x, e, 8)
    torch.cuda.synchronize()
    assert sx.shape == (0, 64) and raw(gs).tolist() == [0] * 8
    out = G.moe_unpermute(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV), c2s,
                          torch.empty((0, 2), dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    assert out.shape == (0, 64)


def test_permute_all_to_one_expert():
    say("permute: every copy to one expert (the order must stay the copy order)")
    r = np.random.default_rng(6)
    tokens, top_k, k, g = 3000, 2, 16, 32
    x, _ = make_x(r, tokens, k, "bf16")
    experts = np.full((tokens, top_k), 17, dtype=np.int32)
    (sx, _, gs, s2c, c2s), _ = run_permute(x, experts, g)
    assert raw(s2c).tolist() == list(range(tokens * top_k))
    assert raw(gs)[17] == tokens * top_k and raw(gs).sum() == tokens * top_k
    assert np.array_equal(raw(sx), np.repeat(raw(x), top_k, axis=0))


UNPERMUTE_CASES = [
    # tokens, top_k, n, in, out
    (1, 1, 8, "bf16", "bf16"),
    (37, 2, 520, "bf16", "bf16"),
    (301, 8, 1024, "bf16", "f32"),
    (129, 3, 72, "f32", "f32"),
    (64, 2, 13, "bf16", "bf16"),
    (50, 4, 777, "f32", "bf16"),
]


def _to(t_np, dtype):
    if dtype == "f32":
        return torch.from_numpy(t_np.astype(np.float32)).to(DEV)
    return torch.from_numpy(W.f32_to_bf16_bits(t_np).view(np.int16)).view(torch.bfloat16).to(DEV)


@pytest.mark.parametrize("tokens,top_k,n,ind,outd", UNPERMUTE_CASES)
def test_unpermute_matches_oracle(tokens, top_k, n, ind, outd):
    say("unpermute", tokens, top_k, n, ind, outd)
    r = np.random.default_rng([tokens, top_k, n, 1])
    M = tokens * top_k
    y = _to(r.standard_normal((M, n)).astype(np.float32), ind)
    experts = draw_experts(r, tokens, top_k, 8, distinct=False)
    experts[0, 0] = -1   # one unrouted copy
    c2s = oracle.moe_permute(np.zeros((tokens, 1), np.float32), experts, 8)[4]
    w = r.random((tokens, top_k)).astype(np.float32)
    out_dtype = torch.float32 if outd == "f32" else torch.bfloat16
    out = torch.full((tokens, n), float("nan"), dtype=out_dtype, device=DEV)
    gg().moe_unpermute(y, torch.from_numpy(c2s).to(DEV), torch.from_numpy(w).to(DEV), out=out)
    torch.cuda.synchronize()
    ref = oracle.moe_unpermute(raw(y), c2s, w)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    if outd == "f32":
        assert np.linalg.norm(got - ref) <= 1e-5 * np.linalg.norm(ref)
    else:
        assert not (np.abs(got - ref) > 1e-2 * np.abs(ref) + 1e-2).any()


def test_moe_layer_permute_gemm_unpermute():
    """The sparse path end to end on the device (permute, ragged_dot_m, un-permute) against
    the same three steps in the oracle."""
    say("moe layer: permute -> ragged_dot_m -> unpermute")
    G = gg()
    r = np.random.default_rng(11)
    tokens, top_k, k, n, g = 700, 2, 256, 384, 8
    x, _ = make_x(r, tokens, k, "bf16")
    experts = draw_experts(r, tokens, top_k, g)
    wts = _to((r.standard_normal((g, k, n)) / np.sqrt(k)).astype(np.float32), "bf16")
    w = r.random((tokens, top_k)).astype(np.float32)
    sx, _, gs, _, c2s = G.moe_permute(x, torch.from_numpy(experts).to(DEV), g)
    y = G.ragged_dot_m(sx, wts, gs, out_dtype=torch.float32)
    out = G.moe_unpermute(y, c2s, torch.from_numpy(w).to(DEV), out_dtype=torch.float32)
    torch.cuda.synchronize()
    osx, _, ogs, _, oc2s = oracle.moe_permute(raw(x), experts, g)
    ref = oracle.moe_unpermute(oracle.ragged_dot_m(osx, raw(wts), ogs), oc2s, w)
    got = out.double().cpu().numpy()
    assert np.linalg.norm(got - ref) <= 1e-5 * np.linalg.norm(ref)


def test_full_size_permute_unpermute():
    """The DeepSeek-like pre/post-processing at its full size, as the benchmark times it:
    index maps and group_sizes bit-exact; sampled sorted rows and tokens against the oracle."""
    G = gg()
    w = W.WORKLOADS["deepseekv3_permute_bf16"]
    say("full size permute", w.name)
    d = W.make_inputs(w, device=DEV)
    sx, _, gs, s2c, c2s = G.moe_permute(d["x"], d["experts"], w.g)
    torch.cuda.synchronize()
    experts = raw(d["experts"])
    tok = np.arange(w.tokens, dtype=np.float32)[:, None]        # rows = their token index
    _, _, ogs, os2c, oc2s = oracle.moe_permute(tok, experts, w.g)
    assert np.array_equal(raw(gs), ogs) and np.array_equal(raw(gs), W.group_sizes(w))
    assert np.array_equal(raw(s2c), os2c) and np.array_equal(raw(c2s), oc2s)
    rng = np.random.default_rng(9)
    rows = np.unique(np.concatenate([[0, w.m - 1], np.cumsum(ogs)[:-1], rng.integers(0, w.m, 256)]))
    rows = rows[rows < w.m]
    xs = raw(d["x"])
    want_rows = xs[os2c[rows] // w.top_k]
    assert np.array_equal(raw(sx[torch.from_numpy(rows).to(DEV)]), want_rows)

    u = W.WORKLOADS["deepseekv3_unpermute_bf16"]
    say("full size unpermute", u.name)
    du = W.make_inputs(u, device=DEV)
    out = torch.full((u.tokens, u.n), float("nan"), dtype=torch.bfloat16, device=DEV)
    G.moe_unpermute(du["y"], c2s, du["weights"], out=out)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all())
    toks = np.unique(np.concatenate([[0, u.tokens - 1], rng.integers(0, u.tokens, 64)]))
    sel = np.concatenate([oc2s[t * u.top_k:(t + 1) * u.top_k] for t in toks])
    ysub = raw(du["y"][torch.from_numpy(sel.astype(np.int64)).to(DEV)])
    # the selected rows, re-indexed so copy j of sampled token q sits at row q * top_k + j
    ref = oracle.moe_unpermute(ysub, np.arange(sel.size, dtype=np.int32), raw(du["weights"])[toks])
    got = out[torch.from_numpy(toks).to(DEV)].double().cpu().numpy()
    assert not (np.abs(got - ref) > 1e-2 * np.abs(ref) + 1e-2).any()


def test_moe_layer_graph_capture():
    """permute -> ragged_dot_m -> un-permute captured in one HIP graph: nothing is read back
    on the host, so replays follow new routing written into the same expert-id buffer.
    Every replay is checked against the eager calls, with eager work between replays."""
    say("moe layer in a captured graph, replayed over new routing")
    G = gg()
    r = np.random.default_rng(13)
    tokens, top_k, k, n, g = 500, 2, 128, 256, 8
    x, _ = make_x(r, tokens, k, "bf16")
    wts = _to((r.standard_normal((g, k, n)) / np.sqrt(k)).astype(np.float32), "bf16")
    w = torch.from_numpy(r.random((tokens, top_k)).astype(np.float32)).to(DEV)
    experts = torch.from_numpy(draw_experts(r, tokens, top_k, g)).to(DEV)
    M = tokens * top_k
    pws = torch.empty(G.workspace_bytes("permute", M, k, 0, g), dtype=torch.uint8, device=DEV)
    mws = torch.empty(G.workspace_bytes("ragged_m", M, k, n, g), dtype=torch.uint8, device=DEV)
    bufs = (torch.empty((M, k), dtype=torch.bfloat16, device=DEV), None,
            torch.empty((g,), dtype=torch.int32, device=DEV), torch.empty((M,), dtype=torch.int32, device=DEV),
            torch.empty((M,), dtype=torch.int32, device=DEV))
    y = torch.empty((M, n), dtype=torch.bfloat16, device=DEV)
    out = torch.empty((tokens, n), dtype=torch.bfloat16, device=DEV)

    def layer():
        sx, _, gs, _, c2s = G.moe_permute(x, experts, g, workspace=pws, out=bufs)
        G.ragged_dot_m(sx, wts, gs, out=y, workspace=mws)
        G.moe_unpermute(y, c2s, w, out=out)

    def eager():
        sx, _, gs, _, c2s = G.moe_permute(x, experts, g)
        return G.moe_unpermute(G.ragged_dot_m(sx, wts, gs), c2s, w).clone()

    layer()   # warm-up outside the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            layer()
    for rep in range(4):
        experts.copy_(torch.from_numpy(draw_experts(r, tokens, top_k, g)))
        want = eager()
        out.fill_(float("nan"))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {rep}"
