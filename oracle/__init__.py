"""CPU oracle for ragged-dot.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, the smoke check and the benchmark's CPU-baseline leg may import this
package.  It shares no code with the GPU library (``group_gemm_amd``) and never imports
it.  The arithmetic lives in ``oracle.c`` (fp64 accumulation); this module marshals
numpy arrays into it and adds the padded-dot procedure, written with numpy in fp64.

Sources: "Group-GEMM in XLA: Making Mixture-of-Experts Fast and Memory-Efficient"
(AMD ROCm blog) -- Part 1 "The Ragged-Dot Operation" and "The Naive Support, and Why It
Hurts: Padded-Dot"; Part 3 "Non-Contracting (the MoE Case)" and "Contracting"; Part 4
"The Three MoE Compute Paths in MaxText" (permute / un-permute, in numpy).
"""
import ctypes
import os

import math

import numpy as np

from . import build as _build

F32, BF16, E4M3 = 0, 1, 2          # the oracle's own element codes (see oracle.c)

_lib = None


def lib():
    """Load liboracle.so, compiling it first if it is not there yet."""
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        L.oracle_ragged_dot_m.argtypes = [ctypes.c_int, vp, vp, vp, vp, vp, i64, i64, i64, i32,
                                          vp, i64, vp]
        L.oracle_ragged_dot_m.restype = ctypes.c_int
        L.oracle_ragged_dot_k.argtypes = [ctypes.c_int, vp, vp, vp, i64, i64, i64, i32, vp, i64,
                                          vp]
        L.oracle_ragged_dot_k.restype = ctypes.c_int
        for name in ("orc_decode_bf16", "orc_decode_e4m3", "orc_decode_e8m0"):
            getattr(L, name).restype = ctypes.c_double
        L.orc_decode_bf16.argtypes = [ctypes.c_uint16]
        L.orc_decode_e4m3.argtypes = [ctypes.c_uint8]
        L.orc_decode_e8m0.argtypes = [ctypes.c_uint8]
        L.oracle_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _dtype_code(a):
    """Element code of a raw input array: float32 -> F32, uint16 (bf16 bits) -> BF16,
    uint8 (e4m3 codes) -> E4M3."""
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError(f"unsupported oracle input dtype {a.dtype}")


def ragged_dot_m(lhs, rhs, group_sizes, lhs_scale=None, rhs_scale=None, rows=None):
    """fp64 result of the non-contracting ragged dot: [m, n], or only the listed rows.

    lhs [m, k] and rhs [g, k, n] are float32, uint16 (bfloat16 bit patterns) or uint8 (OCP
    e4m3 codes, then with E8M0 ``lhs_scale`` [m, k/32] and ``rhs_scale`` [g, k/32, n]).
    """
    lhs = np.ascontiguousarray(lhs)
    rhs = np.ascontiguousarray(rhs)
    gs = np.ascontiguousarray(group_sizes, dtype=np.int32)
    m, k = lhs.shape
    g, k2, n = rhs.shape
    assert k2 == k and gs.shape == (g,) and lhs.dtype == rhs.dtype
    code = _dtype_code(lhs)
    if code == E4M3:
        lhs_scale = np.ascontiguousarray(lhs_scale, dtype=np.uint8)
        rhs_scale = np.ascontiguousarray(rhs_scale, dtype=np.uint8)
        assert lhs_scale.shape == (m, k // 32) and rhs_scale.shape == (g, k // 32, n)
    if rows is not None:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
    nrows = m if rows is None else rows.shape[0]
    out = np.empty((nrows, n), dtype=np.float64)
    rc = lib().oracle_ragged_dot_m(code, _ptr(lhs), _ptr(rhs), _ptr(lhs_scale), _ptr(rhs_scale),
                                   _ptr(gs), m, k, n, g, _ptr(rows), nrows, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_ragged_dot_m rejected its arguments")
    return out


def ragged_dot_m_nk(lhs, rhs_nk, group_sizes, rows=None):
    """fp64 result of the ragged dot whose weights are contracted on their last axis
    ("Group-GEMM in XLA", Part 4 Table 7, classes dgrad_wi / dgrad_wo: rhs contracting
    dimension 2): out[r, :] = lhs[r, :] . rhs_nk[h]^T for the rows r of group h, with
    rhs_nk [g, n, k].  The same sum as ragged_dot_m over the transposed weights."""
    rhs_nk = np.asarray(rhs_nk)
    return ragged_dot_m(lhs, np.swapaxes(rhs_nk, 1, 2), group_sizes, rows=rows)


def ragged_dot_m_epilogue(lhs, rhs, group_sizes, bias=None, alpha=1.0, beta=0.0, c=None, lhs_scale=None,
                          rhs_scale=None):
    """fp64 out[r, :] = alpha * (lhs[r, :] . rhs[h]) + bias[h, :n] + beta * c[r, :] for the rows r
    of group h (the grouped-GEMM alpha / beta of "Group-GEMM in XLA" Part 2 and the
    per-expert bias of the aiter MXFP8 MoE GEMM); rows past the groups' total are 0.
    bias [g, >=n] and c [m, n] are float arrays (c already decoded to its values)."""
    base = ragged_dot_m(lhs, rhs, group_sizes, lhs_scale, rhs_scale)
    m, n = base.shape
    out = alpha * base
    if c is not None and beta != 0.0:
        out = out + beta * np.asarray(c, dtype=np.float64)
    start = 0
    for h, s in enumerate(np.asarray(group_sizes)):
        s = max(int(s), 0)
        s = min(s, m - start)
        if bias is not None:
            out[start:start + s] += np.asarray(bias, dtype=np.float64)[h, :n]
        start += s
    out[start:] = 0.0
    return out


def ragged_dot_k_epilogue(lhs, dout, group_sizes, alpha=1.0, beta=0.0, c=None):
    """fp64 out[h] = alpha * (lhs_h^T . dout_h) + beta * c[h] (c [g, k, n] float values)."""
    out = alpha * ragged_dot_k(lhs, dout, group_sizes)
    if c is not None and beta != 0.0:
        out = out + beta * np.asarray(c, dtype=np.float64)
    return out


def silu(x):
    """x * sigmoid(x) = x / (1 + e^-x), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def gelu_tanh(x):
    """The tanh form of GELU: 0.5 x (1 + tanh(sqrt(2/pi) (x + 0.044715 x^3))), in fp64."""
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (x + 0.044715 * x ** 3)))


ACTIVATIONS = {"silu": silu, "gelu_tanh": gelu_tanh}


def ragged_dot_m_gated(lhs, w0, w1, group_sizes, act="silu", bias0=None, bias1=None, rows=None):
    """fp64 gated projection of an MoE expert block ("Group-GEMM in XLA", Part 1: the gate and
    up einsums over w0 and w1, then activation(layer_w0) * layer_w1; Part 4: gmm_up with both
    weights and biases, then the FFN activation):
    out[r, :] = act(lhs[r, :] . w0[h] + bias0[h, :n]) * (lhs[r, :] . w1[h] + bias1[h, :n]),
    rows past the groups' total 0; `rows` selects output rows as in ragged_dot_m."""
    gate = ragged_dot_m(lhs, w0, group_sizes, rows=rows)
    up = ragged_dot_m(lhs, w1, group_sizes, rows=rows)
    m = np.asarray(lhs).shape[0]
    n = gate.shape[1]
    gs = np.asarray(group_sizes)
    # the group of every output row under the clamping reading (-1: past the total)
    grp = np.full(m, -1, dtype=np.int64)
    start = 0
    for h, s in enumerate(gs):
        s = min(max(int(s), 0), m - start)
        grp[start:start + s] = h
        start += s
    sel = grp if rows is None else grp[np.asarray(rows, dtype=np.int64)]
    if bias0 is not None:
        gate = gate + np.where(sel[:, None] >= 0, np.asarray(bias0, dtype=np.float64)[np.maximum(sel, 0), :n], 0.0)
    if bias1 is not None:
        up = up + np.where(sel[:, None] >= 0, np.asarray(bias1, dtype=np.float64)[np.maximum(sel, 0), :n], 0.0)
    out = ACTIVATIONS[act](gate) * up
    out[sel < 0] = 0.0
    return out


def ragged_dot_k(lhs, dout, group_sizes, pairs=None):
    """fp64 result of the contracting ragged dot: [g, k, n], or the rows out[g_q, i_q, :]
    for the (g, i) pairs given as an int array of shape [npairs, 2]."""
    lhs = np.ascontiguousarray(lhs)
    dout = np.ascontiguousarray(dout)
    gs = np.ascontiguousarray(group_sizes, dtype=np.int32)
    m, k = lhs.shape
    m2, n = dout.shape
    assert m2 == m and lhs.dtype == dout.dtype
    g = gs.shape[0]
    code = _dtype_code(lhs)
    if pairs is not None:
        pairs = np.ascontiguousarray(pairs, dtype=np.int64).reshape(-1, 2)
    npairs = g * k if pairs is None else pairs.shape[0]
    out = np.empty((npairs, n), dtype=np.float64)
    rc = lib().oracle_ragged_dot_k(code, _ptr(lhs), _ptr(dout), _ptr(gs), m, k, n, g,
                                   _ptr(pairs), npairs, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_ragged_dot_k rejected its arguments")
    return out.reshape(g, k, n) if pairs is None else out


def decode(a, scale=None, scale_axis=None):
    """fp64 values of raw inputs via the oracle's own decoders (elementwise calls; meant
    for small arrays).  For e4m3 codes pass the E8M0 ``scale`` array and the axis along
    which one scale covers 32 elements."""
    L = lib()
    a = np.asarray(a)
    code = _dtype_code(a)
    if code == F32:
        v = a.astype(np.float64)
    elif code == BF16:
        v = np.vectorize(L.orc_decode_bf16, otypes=[np.float64])(a)
    else:
        v = np.vectorize(L.orc_decode_e4m3, otypes=[np.float64])(a)
    if scale is not None:
        s = np.vectorize(L.orc_decode_e8m0, otypes=[np.float64])(np.asarray(scale))
        v = v * np.repeat(s, 32, axis=scale_axis)
    return v


def padded_dot_m(lhs, rhs, group_sizes, capacity, lhs_scale=None, rhs_scale=None):
    """The padded-dot baseline written as its three steps, in fp64 numpy:
    (1) scatter group g's rows into slab P[g, 0:m_g] of a zeroed [g, C, k] buffer;
    (2) one batched matmul P[g] @ rhs[g] -> [g, C, n];
    (3) gather rows 0:m_g of every slab back into the [m, n] output.
    Rows past a group's capacity are dropped (they read as 0), as are rows past
    sum(group_sizes) -- the same clamping reading as the ragged oracle.
    ("Group-GEMM in XLA", Part 1 "The Naive Support, and Why It Hurts: Padded-Dot".)"""
    gs = np.asarray(group_sizes, dtype=np.int64)
    m, k = lhs.shape
    g, _, n = rhs.shape
    A = decode(lhs, lhs_scale, 1) if lhs_scale is not None else decode(lhs)
    B = decode(rhs, rhs_scale, 1) if rhs_scale is not None else decode(rhs)
    P = np.zeros((g, capacity, k))
    start, covered = [], 0
    for h in range(g):
        s = min(max(int(gs[h]), 0), m - covered)
        start.append((covered, s))
        c = min(s, capacity)
        P[h, :c] = A[covered:covered + c]
        covered += s
    Q = np.matmul(P, B)                      # step 2: uniform batched GEMM
    out = np.zeros((m, n))
    for h, (st, s) in enumerate(start):
        c = min(s, capacity)
        out[st:st + c] = Q[h, :c]
    return out


def padded_dot_k(lhs, dout, group_sizes, capacity):
    """The padded contracting form written as its steps, in fp64 numpy:
    (1) scatter the rows of group g of lhs and of dout into slabs P[g, 0:m_g] of zeroed
    [g, C, k] and [g, C, n] buffers;
    (2) one batched product P_lhs[g]^T @ P_dout[g] -> [g, k, n].
    Rows past a group's capacity are dropped (only the first C rows of the group are
    scattered), as are rows past sum(group_sizes) -- the clamping reading of the ragged
    oracle.  ("Group-GEMM in XLA", Part 1 "The Naive Support, and Why It Hurts:
    Padded-Dot", applied to the contracting variant of Part 3 "Contracting".)"""
    gs = np.asarray(group_sizes, dtype=np.int64)
    m, k = lhs.shape
    n = dout.shape[1]
    g = gs.shape[0]
    A, D = decode(lhs), decode(dout)
    PA = np.zeros((g, capacity, k))
    PD = np.zeros((g, capacity, n))
    covered = 0
    for h in range(g):
        s = min(max(int(gs[h]), 0), m - covered)
        c = min(s, capacity)
        PA[h, :c] = A[covered:covered + c]
        PD[h, :c] = D[covered:covered + c]
        covered += s
    return np.matmul(np.swapaxes(PA, 1, 2), PD)   # step 2: uniform batched contraction


def bf16_values(a):
    """fp64 values of bfloat16 bit patterns (uint16): a bfloat16 is the upper half of an
    IEEE binary32, so the pattern shifted up 16 bits is that binary32 exactly."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    with np.errstate(invalid="ignore"):   # signalling-NaN patterns stay NaN
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def moe_permute(x, experts, g, x_scale=None):
    """The MoE pre-processing of the sparse path ("Group-GEMM in XLA", Part 4 "The Three MoE
    Compute Paths in MaxText", Path 1, permute; and "Router to expert and back"): every
    token is repeated top_k times (copy i is token i // top_k), the copies are ordered by
    a stable argsort of the flattened expert ids, the repeated rows are taken in that
    order, and a bincount of the ids gives group_sizes.

    Reading for ids outside [0, g): such a copy is not routed -- it sorts after every
    routed copy, gets no row (sorted rows past the routed total are zero, their index -1)
    and is not counted.  Rows are moved as raw elements (any dtype); `x_scale` rows (the
    E8M0 scales of e4m3 rows) are moved the same way.

    Returns (sorted_x [M, k], sorted_scale or None, group_sizes int32 [g],
    sorted_to_copy int32 [M], copy_to_sorted int32 [M]), M = tokens * top_k."""
    experts = np.asarray(experts)
    T, K = experts.shape
    M = T * K
    flat = experts.reshape(-1).astype(np.int64)
    routed = (flat >= 0) & (flat < g)
    order = np.argsort(np.where(routed, flat, g), kind="stable")
    S = int(routed.sum())
    sorted_to_copy = np.full(M, -1, dtype=np.int32)
    sorted_to_copy[:S] = order[:S]
    copy_to_sorted = np.full(M, -1, dtype=np.int32)
    copy_to_sorted[order[:S]] = np.arange(S, dtype=np.int32)
    group_sizes = np.bincount(flat[routed], minlength=g).astype(np.int32)

    def take(a):
        replicated = np.repeat(np.asarray(a), K, axis=0)
        out = np.zeros_like(replicated)
        out[:S] = replicated[order[:S]]
        return out

    return (take(x), None if x_scale is None else take(x_scale), group_sizes, sorted_to_copy,
            copy_to_sorted)


def moe_unpermute(y, copy_to_sorted, weights):
    """The MoE post-processing of the sparse path (same page and section, un-permute):
    the expert outputs y [M, n] (sorted order) are put back in copy order with the inverse
    permutation, viewed as [tokens, top_k, n], and summed over top_k with the router
    weights [tokens, top_k], in fp64.  A copy whose entry lies outside [0, M) (-1: not
    routed) adds nothing.  y is float32 or bfloat16 bit patterns (uint16)."""
    y = np.asarray(y)
    yv = bf16_values(y) if y.dtype == np.uint16 else y.astype(np.float64)
    w = np.asarray(weights, dtype=np.float64)
    T, K = w.shape
    M, n = yv.shape
    assert M == T * K
    c2s = np.asarray(copy_to_sorted, dtype=np.int64)
    ok = (c2s >= 0) & (c2s < M)
    unsorted = np.zeros((M, n))
    unsorted[ok] = yv[c2s[ok]]
    return np.einsum("tkn,tk->tn", unsorted.reshape(T, K, n), w)


def num_threads():
    return lib().oracle_num_threads()


def set_num_threads(n):
    """Thread count of the C oracle's later calls (OpenMP)."""
    L = lib()
    L.oracle_set_num_threads.argtypes = [ctypes.c_int]
    L.oracle_set_num_threads(int(n))
