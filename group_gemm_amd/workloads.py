"""Seeded synthetic inputs for ragged-dot: routing -> group_sizes, operand values, and the
MXFP8 quantisation of operands.

This module feeds both the GPU library's tests/benchmark and the CPU oracle.  It holds
none of the ragged-dot arithmetic (no products, no sums over k): it only draws inputs.

Structure follows the pages' MoE pipeline ("Group-GEMM in XLA: Making Mixture-of-Experts
Fast and Memory-Efficient", Part 4 "Path 1 -- Sparse / Ragged-Dot (Dropless)"): a router
picks the top-k experts of every token, tokens are sorted by expert, and a bincount gives
group_sizes.  The sorted rows are drawn i.i.d. directly in sorted order (the permutation
does not change any product).  Balanced sizes follow the same page, Part 4 "Fixing
group_sizes Deterministically" (the first M mod E experts get one extra row).

Draws: numpy ``default_rng([workload_id, stream, seed])`` for routing (stream 0) and for
small host-side operands; torch generators (CPU or GPU) seeded from the same triple for
large operands, so a workload of several GiB is drawn on the device in milliseconds.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch

# ---------------------------------------------------------------------------------------
# workload catalogue


@dataclasses.dataclass(frozen=True)
class Workload:
    wid: int            # numeric id, part of every seed
    name: str
    op: str             # "m" (ragged_dot_m) or "k" (ragged_dot_k)
    in_dtype: str       # "f32" | "bf16" | "mxfp8"
    out_dtype: str      # "f32" | "bf16"
    m: int
    k: int
    n: int
    g: int
    routing: str        # recipe name, see group_sizes()
    tokens: int = 0
    top_k: int = 0


WORKLOADS = {
    w.name: w
    for w in [
        Workload(1, "tiny_fp32", "m", "f32", "f32", 64, 128, 64, 4, "fixed"),
        Workload(2, "mixtral8x7b_up_bf16", "m", "bf16", "bf16", 8192, 4096, 14336, 8,
                 "topk_normal_logits", tokens=4096, top_k=2),
        Workload(3, "deepseekv3_routed_bf16", "m", "bf16", "bf16", 32768, 7168, 2048, 256,
                 "rank_zipf_gumbel", tokens=4096, top_k=8),
        Workload(4, "mixtral8x7b_up_mxfp8", "m", "mxfp8", "bf16", 8192, 4096, 14336, 8,
                 "topk_normal_logits", tokens=4096, top_k=2),
        Workload(5, "llama4scout_wgrad_bf16", "k", "bf16", "f32", 16384, 5120, 8192, 16,
                 "dirichlet_multinomial", tokens=16384, top_k=1),
        # correctness-only variant of the skewed workload with exactly-empty experts
        Workload(6, "deepseekv3_routed_bf16_zeros", "m", "bf16", "bf16", 32768, 7168, 2048,
                 256, "rank_zipf_gumbel_zeros", tokens=4096, top_k=8),
        # data gradient of the Mixtral-like up-projection (Table 7 class dgrad_wi): the
        # output gradient [8192, 14336] times each expert's stored weights [4096, 14336]^T
        Workload(7, "mixtral8x7b_dgrad_bf16", "m_nk", "bf16", "bf16", 8192, 14336, 4096, 8,
                 "topk_normal_logits", tokens=4096, top_k=2),
        # the same up-projection as a fused gate/up pair with SiLU: two [8, 4096, 14336]
        # weight tensors, one [8192, 14336] intermediate
        Workload(8, "mixtral8x7b_gated_bf16", "m_gated", "bf16", "bf16", 8192, 4096, 14336, 8,
                 "topk_normal_logits", tokens=4096, top_k=2),
        # MoE pre/post-processing around the DeepSeek-like routed block: permute 4096 tokens
        # of width 7168 to their top-8 of 256 experts (m = 32768 copies), and un-permute
        # [32768, 7168] expert outputs back into 4096 tokens with the router weights
        Workload(9, "deepseekv3_permute_bf16", "permute", "bf16", "bf16", 32768, 7168, 0, 256,
                 "rank_zipf_gumbel", tokens=4096, top_k=8),
        Workload(10, "deepseekv3_unpermute_bf16", "unpermute", "bf16", "bf16", 32768, 0, 7168, 256,
                 "rank_zipf_gumbel", tokens=4096, top_k=8),
    ]
}

# the MXFP8, data-gradient and gated workloads reuse the bf16 forward one's routing stream,
# so all see the same sizes; the permute workloads reuse the DeepSeek-like routing
_ROUTING_WID = {4: 2, 7: 2, 8: 2, 9: 3, 10: 3}


def rng(wid: int, stream: int, seed: int = 0) -> np.random.Generator:
    return np.random.default_rng([wid, stream, seed])


def torch_seed(wid: int, stream: int, seed: int = 0) -> int:
    return (wid * 1_000_003 + stream * 10_007 + seed) & 0x7FFFFFFF


# ---------------------------------------------------------------------------------------
# group sizes


def balanced_group_sizes(M: int, E: int) -> np.ndarray:
    """M // E rows per expert, the remainder spread one row each over the first experts."""
    base = M // E
    gs = np.full((E,), base, dtype=np.int32)
    gs[: M - base * E] += 1
    return gs


def topk_indices(scores: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores per row (ties: lower index first)."""
    order = np.argsort(-scores, axis=1, kind="stable")
    return order[:, :k]


_TOPK_ROUTINGS = ("topk_normal_logits", "rank_zipf_gumbel", "rank_zipf_gumbel_zeros")


def routing_experts(w: Workload, seed: int = 0) -> np.ndarray:
    """int32 [tokens, top_k]: the experts the router picks for every token (top-k
    routings only), the draws group_sizes() counts."""
    r = rng(_ROUTING_WID.get(w.wid, w.wid), 0, seed)
    if w.routing == "topk_normal_logits":
        logits = r.standard_normal((w.tokens, w.g))
        experts = topk_indices(logits, w.top_k)
    elif w.routing in ("rank_zipf_gumbel", "rank_zipf_gumbel_zeros"):
        rank = r.permutation(w.g) + 1                      # popularity rank of each expert
        p = rank.astype(np.float64) ** -1.1                # Zipf(s = 1.1) over ranks
        if w.routing.endswith("zeros"):
            p[np.argsort(rank)[-4:]] = 0.0                 # four least popular never chosen
        p /= p.sum()
        with np.errstate(divide="ignore"):
            logp = np.log(p)
        gumbel = r.gumbel(size=(w.tokens, w.g))
        experts = topk_indices(logp[None, :] + gumbel, w.top_k)   # k distinct experts ~ p
    else:
        raise ValueError(f"{w.routing} draws no per-token experts")
    return np.ascontiguousarray(experts, dtype=np.int32)


def router_weights(w: Workload, seed: int = 0) -> np.ndarray:
    """float32 [tokens, top_k] combine weights: a softmax over N(0,1) scores of the
    selected experts (positive, each token's weights sum to 1)."""
    s = rng(w.wid, 3, seed).standard_normal((w.tokens, w.top_k))
    e = np.exp(s - s.max(axis=1, keepdims=True))
    return (e / e.sum(axis=1, keepdims=True)).astype(np.float32)


def group_sizes(w: Workload, seed: int = 0) -> np.ndarray:
    """Realised int32[g] group sizes of a workload (host-side, seeded)."""
    r = rng(_ROUTING_WID.get(w.wid, w.wid), 0, seed)
    if w.routing == "fixed":
        gs = np.array([16, 0, 40, 8], dtype=np.int32)
    elif w.routing in _TOPK_ROUTINGS:
        gs = np.bincount(routing_experts(w, seed).ravel(), minlength=w.g).astype(np.int32)
    elif w.routing == "dirichlet_multinomial":
        p = r.dirichlet(np.full(w.g, 0.5))
        gs = r.multinomial(w.tokens * w.top_k, p).astype(np.int32)
    else:
        raise ValueError(w.routing)
    assert gs.sum() == w.m, (w.name, int(gs.sum()), w.m)
    return gs


# ---------------------------------------------------------------------------------------
# element formats (input preparation only)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round-to-nearest-even float32 -> bfloat16 bit patterns (uint16); inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def mx_quantize(x: torch.Tensor, axis: int):
    """OCP-MX style quantisation of float32 ``x`` to e4m3 codes + E8M0 scales, one scale
    per 32 contiguous elements along ``axis``.  Shared exponent e = floor(log2(amax)) - 8
    (8 = largest e4m3 exponent), clamped to [-127, 127]; elements x / 2^e rounded to
    nearest-even e4m3 and saturated at +-448; an all-zero block gets scale byte 0.
    Returns (codes uint8 same shape as x, scales uint8 with that axis divided by 32)."""
    x = x.to(torch.float32)
    xm = x.movedim(axis, -1)
    L = xm.shape[-1]
    assert L % 32 == 0, "MX blocks need the blocked axis to be a multiple of 32"
    blk = xm.reshape(*xm.shape[:-1], L // 32, 32)
    amax = blk.abs().amax(dim=-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 8, torch.full_like(amax, -127.0))
    e = e.clamp(-127, 127)
    q = torch.ldexp(blk, -e.unsqueeze(-1)).clamp(-448.0, 448.0)
    codes = q.to(torch.float8_e4m3fn).view(torch.uint8).reshape(xm.shape).movedim(-1, axis)
    scales = (e + 127).to(torch.uint8).movedim(-1, axis)
    return codes.contiguous(), scales.contiguous()


# ---------------------------------------------------------------------------------------
# operand values


def _randn(shape, wid, stream, seed, device, std=1.0):
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(wid, stream, seed))
    t = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t


def _uniform(shape, wid, stream, seed, device):
    gen = torch.Generator(device=device)
    gen.manual_seed(torch_seed(wid, stream, seed))
    return torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * 2 - 1


def make_inputs(w: Workload, device="cpu", seed: int = 0, gs: np.ndarray | None = None):
    """Operands of a workload as torch tensors on ``device``.

    Returns a dict with ``group_sizes`` (int32), and for op "permute": ``x`` [tokens,k] and
    ``experts`` int32 [tokens,top_k]; for op "unpermute": ``y`` [m,n] (expert outputs in
    sorted order), ``experts`` and ``weights`` float32 [tokens,top_k]; for op "m": ``lhs`` [m,k], ``rhs``
    [g,k,n]; for op "m_nk": ``lhs`` [m,k], ``rhs`` [g,n,k] (k contiguous); for op "k":
    ``lhs`` [m,k], ``dout`` [m,n].  bf16 operands are torch.bfloat16;
    MXFP8 operands are uint8 e4m3 codes plus ``lhs_scale`` [m,k/32] and ``rhs_scale``
    [g,k/32,n] (uint8 E8M0)."""
    if gs is None:
        gs = group_sizes(w, seed)
    out = {"group_sizes": torch.from_numpy(np.ascontiguousarray(gs, dtype=np.int32)).to(device)}
    m, k, n, g = w.m, w.k, w.n, w.g
    if w.op == "permute":
        out["x"] = _randn((w.tokens, k), w.wid, 1, seed, device).to(torch.bfloat16)
        out["experts"] = torch.from_numpy(routing_experts(w, seed)).to(device)
    elif w.op == "unpermute":
        out["y"] = _randn((m, n), w.wid, 1, seed, device).to(torch.bfloat16)
        out["experts"] = torch.from_numpy(routing_experts(w, seed)).to(device)
        out["weights"] = torch.from_numpy(router_weights(w, seed)).to(device)
    elif w.in_dtype == "f32":
        out["lhs"] = _uniform((m, k), w.wid, 1, seed, device)
        out["rhs"] = _uniform((g, k, n), w.wid, 2, seed, device)
    elif w.op == "k":
        out["lhs"] = _randn((m, k), w.wid, 1, seed, device).to(torch.bfloat16)
        out["dout"] = _randn((m, n), w.wid, 2, seed, device).to(torch.bfloat16)
    elif w.op == "m_gated":
        out["lhs"] = _randn((m, k), w.wid, 1, seed, device).to(torch.bfloat16)
        for key, stream in (("w0", 2), ("w1", 3)):
            wt = torch.empty((g, k, n), device=device, dtype=torch.bfloat16)
            for h in range(g):
                wt[h] = _randn((k, n), w.wid, stream, seed * 65536 + h, device, std=1 / math.sqrt(k)).to(torch.bfloat16)
            out[key] = wt
    elif w.op == "m_nk":
        out["lhs"] = _randn((m, k), w.wid, 1, seed, device).to(torch.bfloat16)
        rhs = torch.empty((g, n, k), device=device, dtype=torch.bfloat16)
        for h in range(g):
            rhs[h] = _randn((n, k), w.wid, 2, seed * 65536 + h, device, std=1 / math.sqrt(k)).to(torch.bfloat16)
        out["rhs"] = rhs
    elif w.in_dtype == "bf16":
        out["lhs"] = _randn((m, k), w.wid, 1, seed, device).to(torch.bfloat16)
        rhs = torch.empty((g, k, n), device=device, dtype=torch.bfloat16)
        for h in range(g):   # per expert, so peak float32 scratch is one expert's matrix
            rhs[h] = _randn((k, n), w.wid, 2, seed * 65536 + h, device, std=1 / math.sqrt(k)).to(torch.bfloat16)
        out["rhs"] = rhs
    elif w.in_dtype == "mxfp8":
        x = _randn((m, k), w.wid, 1, seed, device)
        out["lhs"], out["lhs_scale"] = mx_quantize(x, axis=1)
        rc = torch.empty((g, k, n), device=device, dtype=torch.uint8)
        rs = torch.empty((g, k // 32, n), device=device, dtype=torch.uint8)
        for h in range(g):
            wmat = _randn((k, n), w.wid, 2, seed * 65536 + h, device, std=1 / math.sqrt(k))
            rc[h], rs[h] = mx_quantize(wmat, axis=0)
        out["rhs"], out["rhs_scale"] = rc, rs
    else:
        raise ValueError(w.in_dtype)
    return out


def small_inputs(op: str, in_dtype: str, m: int, k: int, n: int, gs, seed: int = 0,
                 device="cpu"):
    """Small seeded operands for parity tests at any shape (N(0,1) lhs, N(0,1/k) rhs or
    N(0,1) dout).  Same dict layout as make_inputs."""
    gs = np.ascontiguousarray(gs, dtype=np.int32)
    g = gs.shape[0]
    r = rng(900 + seed, 1, seed)
    lhs = r.standard_normal((m, k)).astype(np.float32)
    if op == "m":
        second = (r.standard_normal((g, k, n)) / math.sqrt(max(k, 1))).astype(np.float32)
    else:
        second = r.standard_normal((m, n)).astype(np.float32)
    out = {"group_sizes": torch.from_numpy(gs).to(device)}
    key = "rhs" if op == "m" else "dout"
    if in_dtype == "f32":
        out["lhs"] = torch.from_numpy(lhs).to(device)
        out[key] = torch.from_numpy(second).to(device)
    elif in_dtype == "bf16":
        out["lhs"] = torch.from_numpy(f32_to_bf16_bits(lhs).view(np.int16)).view(torch.bfloat16).to(device)
        out[key] = torch.from_numpy(f32_to_bf16_bits(second).view(np.int16)).view(torch.bfloat16).to(device)
    elif in_dtype == "mxfp8":
        assert op == "m"
        out["lhs"], out["lhs_scale"] = [t.to(device) for t in mx_quantize(torch.from_numpy(lhs), 1)]
        out["rhs"], out["rhs_scale"] = [t.to(device) for t in mx_quantize(torch.from_numpy(second), 1)]
    else:
        raise ValueError(in_dtype)
    return out


def to_numpy_raw(t: torch.Tensor) -> np.ndarray:
    """Host copy of a tensor in the oracle's raw form: float32 stays float32, bfloat16
    becomes uint16 bit patterns, uint8 stays uint8 (e4m3 codes / E8M0 scales)."""
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    if t.dtype in (torch.float32, torch.uint8, torch.int32, torch.int64):
        return t.cpu().numpy()
    raise TypeError(t.dtype)


def useful_flops(w: Workload, gs) -> float:
    """2 * sum(m_g) * k * n, the only work credited to the ragged dot (twice that for the
    fused gate/up pair, which computes two products)."""
    f = 2.0 * float(np.sum(np.maximum(gs, 0))) * w.k * w.n
    return 2.0 * f if w.op == "m_gated" else f
