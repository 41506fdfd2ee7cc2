"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Every test here runs on the CPU.  Each pin is chosen so that a plausible slip in the
oracle (a dropped term, a wrong group index, a transposed operand, a misplaced scale)
fails at least one of them.  Sources: "Group-GEMM in XLA: Making Mixture-of-Experts Fast
and Memory-Efficient" (AMD ROCm blog) and "[Triton/Gluon] Merge MoE MXFP8 GEMM into
existing _moe_gemm_a8w8 kernel" (ROCm/aiter pull request 5658).
"""
import math

import numpy as np
import pytest
import torch

import golden
import oracle
from group_gemm_amd import workloads as W


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _bf16_bits(a):
    return W.f32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def _bf16_values(bits):
    """Library decode (torch) of bfloat16 bit patterns, independent of the oracle."""
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()


def _e4m3_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).double().numpy()


def _e8m0_values(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e8m0fnu).double().numpy()


def _blocks(gs, m):
    """(start, size) of every group under the clamping reading, written out plainly."""
    out, run = [], 0
    for s in gs:
        s = max(int(s), 0)
        s = min(s, m - run)
        out.append((run, s))
        run += s
    return out


# ---- P1: the pages' worked example (inputs printed; outputs worked by hand) ---------------

def test_worked_example_m():
    fx = golden.load("worked_example.txt")
    out = oracle.ragged_dot_m(_f32(fx["lhs"]), _f32(fx["rhs"]), fx["group_sizes"].astype(np.int32))
    # inputs are decimal fractions rounded to float32; the hand result is exact decimal
    np.testing.assert_allclose(out, fx["out_m"], rtol=0, atol=1e-6)


def test_worked_example_k():
    fx = golden.load("worked_example.txt")
    out = oracle.ragged_dot_k(_f32(fx["lhs"]), _f32(fx["dout"]), fx["group_sizes"].astype(np.int32))
    np.testing.assert_allclose(out, fx["out_k"], rtol=0, atol=1e-6)
    # the two slabs add up to the full contraction lhs^T . dout
    np.testing.assert_allclose(out.sum(axis=0), _f32(fx["lhs"]).astype(np.float64).T @ fx["dout"], atol=1e-6)


# ---- P2 / P3 / P5: independent definitions and special cases ------------------------------

@pytest.mark.parametrize("gs", [[5, 0, 7, 4], [0, 0, 16, 0], [1, 2, 3, 4], [16, 0, 0, 0]])
def test_m_matches_per_group_matmul(gs):
    m, k, n = 16, 12, 7
    r = np.random.default_rng(1)
    lhs, rhs = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((len(gs), k, n)))
    out = oracle.ragged_dot_m(lhs, rhs, gs)
    ref = np.zeros((m, n))
    for h, (st, s) in enumerate(_blocks(gs, m)):
        ref[st:st + s] = lhs[st:st + s].astype(np.float64) @ rhs[h].astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)


def test_m_matches_dense_masked_formula():
    """out = sum_g diag(1[r in g]) . lhs . rhs[g]: every expert evaluated on every row, then
    masked -- the dense-masked choice of "Memory and Kernel Optimizations", "Why MoE
    requires grouped GEMM", which performs E/k times the routed work for the same result."""
    m, k, n, gs = 20, 9, 6, [4, 0, 9, 5, 2]
    r = np.random.default_rng(2)
    lhs, rhs = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((len(gs), k, n)))
    ref = np.zeros((m, n))
    for h, (st, s) in enumerate(_blocks(gs, m)):
        mask = np.zeros(m)
        mask[st:st + s] = 1.0
        ref += np.diag(mask) @ lhs.astype(np.float64) @ rhs[h].astype(np.float64)
    np.testing.assert_allclose(oracle.ragged_dot_m(lhs, rhs, gs), ref, rtol=1e-13, atol=1e-13)


def test_single_group_is_plain_matmul():
    r = np.random.default_rng(3)
    lhs, rhs = _f32(r.standard_normal((11, 8))), _f32(r.standard_normal((1, 8, 5)))
    np.testing.assert_allclose(oracle.ragged_dot_m(lhs, rhs, [11]),
                               lhs.astype(np.float64) @ rhs[0].astype(np.float64), rtol=1e-13, atol=1e-13)
    dout = _f32(r.standard_normal((11, 5)))
    np.testing.assert_allclose(oracle.ragged_dot_k(lhs, dout, [11])[0],
                               lhs.astype(np.float64).T @ dout.astype(np.float64), rtol=1e-13, atol=1e-13)


def test_equal_groups_are_batched_matmul():
    r = np.random.default_rng(4)
    g, c, k, n = 3, 4, 6, 5
    lhs, rhs = _f32(r.standard_normal((g * c, k))), _f32(r.standard_normal((g, k, n)))
    ref = np.matmul(lhs.astype(np.float64).reshape(g, c, k), rhs.astype(np.float64)).reshape(g * c, n)
    np.testing.assert_allclose(oracle.ragged_dot_m(lhs, rhs, [c] * g), ref, rtol=1e-13, atol=1e-13)


# ---- P4: padded-dot equivalence -----------------------------------------------------------

@pytest.mark.parametrize("capacity", ["max", "m"])
def test_padded_equals_ragged(capacity):
    m, k, n, gs = 24, 10, 7, [6, 0, 11, 3, 4]
    r = np.random.default_rng(5)
    lhs, rhs = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((len(gs), k, n)))
    C = max(gs) if capacity == "max" else m
    ragged = oracle.ragged_dot_m(lhs, rhs, gs)
    padded = oracle.padded_dot_m(lhs, rhs, gs, C)
    # padding rows add exact zeros, but numpy's batched matmul may sum in another order
    np.testing.assert_allclose(padded, ragged, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gs,m,cap", [([5, 0, 4], 9, 3), ([2, 6, 1], 10, 4), ([7], 7, 1), ([0, 3, 3], 8, 3)])
def test_padded_m_over_capacity_brute_force(gs, m, cap):
    """Rows past a group's capacity are dropped: the first min(m_g, C) rows of every group
    get their product, the rest of the group and rows past sum(group_sizes) are 0 (written
    out with plain loops; keeping any other C rows of a group fails here)."""
    k, n = 3, 4
    r = np.random.default_rng(16)
    lhs, rhs = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((len(gs), k, n)))
    out = oracle.padded_dot_m(lhs, rhs, gs, cap)
    expect = np.zeros((m, n))
    row = 0
    for h, s in enumerate(gs):
        for i in range(s):
            if i < cap:
                for j in range(n):
                    expect[row, j] = sum(float(lhs[row, t]) * float(rhs[h, t, j]) for t in range(k))
            row += 1
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=1e-14)
    assert np.count_nonzero(np.any(out != 0, axis=1)) == sum(min(s, cap) for s in gs)


@pytest.mark.parametrize("capacity", ["max", "m"])
def test_padded_k_equals_ragged(capacity):
    m, k, n, gs = 24, 6, 5, [6, 0, 11, 3, 4]
    r = np.random.default_rng(17)
    lhs, dout = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((m, n)))
    C = max(gs) if capacity == "max" else m
    np.testing.assert_allclose(oracle.padded_dot_k(lhs, dout, gs, C), oracle.ragged_dot_k(lhs, dout, gs),
                               rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("gs,m,cap", [([5, 0, 4], 9, 3), ([2, 6, 1], 10, 4)])
def test_padded_k_over_capacity_brute_force(gs, m, cap):
    """The contracting padded form over capacity: group h sums over its first min(m_h, C)
    rows only (plain loops)."""
    k, n = 3, 4
    r = np.random.default_rng(18)
    lhs, dout = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((m, n)))
    out = oracle.padded_dot_k(lhs, dout, gs, cap)
    expect = np.zeros((len(gs), k, n))
    start = 0
    for h, s in enumerate(gs):
        for i in range(k):
            for j in range(n):
                expect[h, i, j] = sum(float(lhs[start + q, i]) * float(dout[start + q, j]) for q in range(min(s, cap)))
        start += s
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=1e-14)


# ---- P6: brute force on tiny shapes, boundary cases ---------------------------------------

@pytest.mark.parametrize("gs,m", [([0, 0, 0], 5), ([5, 0, 0], 5), ([0, 5, 0], 5), ([0, 0, 5], 5),
                                  ([2, 1, 1], 6), ([3, 0, 2], 5), ([1, 1, 1, 1, 1], 5)])
def test_m_brute_force(gs, m):
    k, n = 3, 4
    r = np.random.default_rng(6)
    lhs, rhs = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((len(gs), k, n)))
    out = oracle.ragged_dot_m(lhs, rhs, gs)
    expect = [[0.0] * n for _ in range(m)]
    row = 0
    for h, s in enumerate(gs):
        for _ in range(s):
            for j in range(n):
                acc = 0.0
                for t in range(k):
                    acc += float(lhs[row, t]) * float(rhs[h, t, j])
                expect[row][j] = acc
            row += 1
    np.testing.assert_allclose(out, np.array(expect), rtol=1e-14, atol=1e-14)
    assert np.all(out[sum(gs):] == 0.0)


def test_invalid_sizes_follow_clamping_reading():
    """Negative sizes count as 0; a group is cut at row m (reading of a silence)."""
    m, k, n = 10, 4, 3
    r = np.random.default_rng(7)
    lhs, rhs = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((4, k, n)))
    gs = [-3, 4, 9, 2]           # effective: 0, 4, 6 (cut), 0
    out = oracle.ragged_dot_m(lhs, rhs, gs)
    ref = np.zeros((m, n))
    ref[0:4] = lhs[0:4].astype(np.float64) @ rhs[1].astype(np.float64)
    ref[4:10] = lhs[4:10].astype(np.float64) @ rhs[2].astype(np.float64)
    np.testing.assert_allclose(out, ref, rtol=1e-13, atol=1e-13)
    dout = _f32(r.standard_normal((m, n)))
    outk = oracle.ragged_dot_k(lhs, dout, gs)
    assert np.all(outk[0] == 0) and np.all(outk[3] == 0)
    np.testing.assert_allclose(outk[2], lhs[4:10].astype(np.float64).T @ dout[4:10].astype(np.float64),
                               rtol=1e-13, atol=1e-13)


def test_degenerate_sizes():
    r = np.random.default_rng(8)
    # k = 0: every covered row is an empty sum
    out = oracle.ragged_dot_m(np.zeros((4, 0), np.float32), np.zeros((2, 0, 3), np.float32), [1, 3])
    assert out.shape == (4, 3) and np.all(out == 0)
    # m = 0, n = 0
    assert oracle.ragged_dot_m(np.zeros((0, 4), np.float32), _f32(r.standard_normal((2, 4, 3))), [0, 0]).shape == (0, 3)
    assert oracle.ragged_dot_m(_f32(r.standard_normal((3, 4))), np.zeros((1, 4, 0), np.float32), [3]).shape == (3, 0)


# ---- P7 / P8 / P9: contracting-form invariants --------------------------------------------

def test_k_slabs_sum_to_full_contraction():
    m, k, n, gs = 30, 7, 5, [4, 9, 0, 17]
    r = np.random.default_rng(9)
    lhs, dout = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((m, n)))
    out = oracle.ragged_dot_k(lhs, dout, gs)
    np.testing.assert_allclose(out.sum(axis=0), lhs.astype(np.float64).T @ dout.astype(np.float64),
                               rtol=1e-12, atol=1e-12)
    assert np.all(out[2] == 0.0)                  # empty group: exactly zero


def test_k_is_the_weight_gradient_of_m():
    """<dout, ragged_dot_m(lhs, W)> = sum_g <ragged_dot_k(lhs, dout)[g], W[g]> for any W:
    the contracting form is the weight gradient of the forward form (Table 7 pairs fwd_wi
    with wgrad_wi)."""
    m, k, n, gs = 25, 6, 4, [7, 0, 12, 6]
    r = np.random.default_rng(10)
    lhs, dout = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((m, n)))
    Wt = _f32(r.standard_normal((len(gs), k, n)))
    lhs_side = float(np.sum(dout.astype(np.float64) * oracle.ragged_dot_m(lhs, Wt, gs)))
    rhs_side = float(np.sum(oracle.ragged_dot_k(lhs, dout, gs) * Wt.astype(np.float64)))
    assert math.isclose(lhs_side, rhs_side, rel_tol=1e-12, abs_tol=1e-12)


@pytest.mark.parametrize("gs,m", [([0, 0, 0], 5), ([2, 0, 3], 5), ([1, 1, 1, 1], 6), ([0, 4, 0], 4)])
def test_m_nk_brute_force(gs, m):
    """rhs contracted on its last axis (Table 7, dgrad classes): triple loop over rhs[h, j, t]."""
    k, n = 3, 5
    r = np.random.default_rng(11)
    lhs, rhs_nk = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((len(gs), n, k)))
    out = oracle.ragged_dot_m_nk(lhs, rhs_nk, gs)
    expect = np.zeros((m, n))
    row = 0
    for h, s in enumerate(gs):
        for _ in range(s):
            for j in range(n):
                expect[row, j] = sum(float(lhs[row, t]) * float(rhs_nk[h, j, t]) for t in range(k))
            row += 1
    np.testing.assert_allclose(out, expect, rtol=1e-14, atol=1e-14)


def test_m_nk_is_the_data_gradient_of_m():
    """<dY, ragged_dot_m(X, W)> = <ragged_dot_m_nk(dY, W), X> for any X, with W [g, K, N] as
    stored: the dgrad class is the data gradient of the forward class it is paired with
    (Table 7: fwd_wi [M,K] x [E,K,N] -> [M,N]; dgrad_wi [M,N] x [E,K,N] -> [M,K])."""
    m, K, N, gs = 21, 5, 7, [6, 0, 9, 6]
    r = np.random.default_rng(12)
    X, dY = _f32(r.standard_normal((m, K))), _f32(r.standard_normal((m, N)))
    Wt = _f32(r.standard_normal((len(gs), K, N)))
    lhs_side = float(np.sum(dY.astype(np.float64) * oracle.ragged_dot_m(X, Wt, gs)))
    rhs_side = float(np.sum(oracle.ragged_dot_m_nk(dY, Wt, gs) * X.astype(np.float64)))
    assert math.isclose(lhs_side, rhs_side, rel_tol=1e-12, abs_tol=1e-12)


def test_m_epilogue_bias_alpha_brute_force():
    """bias[h] is added to every row of group h, alpha scales the product; rows past the
    groups' total stay 0 (written out plainly)."""
    m, k, n, gs = 9, 3, 4, [3, 0, 4]
    r = np.random.default_rng(13)
    lhs, rhs = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((len(gs), k, n)))
    bias = _f32(r.standard_normal((len(gs), n + 2)))   # row stride n + 2: only the first n used
    out = oracle.ragged_dot_m_epilogue(lhs, rhs, gs, bias=bias, alpha=-0.5)
    row = 0
    for h, s in enumerate(gs):
        for _ in range(s):
            for j in range(n):
                acc = sum(float(lhs[row, t]) * float(rhs[h, t, j]) for t in range(k))
                assert math.isclose(out[row, j], -0.5 * acc + float(bias[h, j]), rel_tol=1e-13, abs_tol=1e-13)
            row += 1
    assert np.all(out[sum(gs):] == 0.0)


def test_m_epilogue_beta_accumulates_split_k():
    """beta = 1 on a first partial product gives the whole product: the sum over k split in
    two parts equals the sum over all of k."""
    m, k, n, gs = 17, 10, 6, [5, 0, 12]
    r = np.random.default_rng(14)
    lhs, rhs = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((len(gs), k, n)))
    first = oracle.ragged_dot_m(lhs[:, :4], rhs[:, :4], gs)
    both = oracle.ragged_dot_m_epilogue(lhs[:, 4:], rhs[:, 4:], gs, beta=1.0, c=first)
    np.testing.assert_allclose(both, oracle.ragged_dot_m(lhs, rhs, gs), rtol=1e-12, atol=1e-12)


def test_k_epilogue_beta_is_gradient_accumulation():
    """Two micro-batches accumulated with beta = 1 give the weight gradient of their union,
    each group's rows of both batches taken together."""
    k, n = 4, 5
    gs1, gs2 = [3, 0, 2], [1, 4, 0]
    r = np.random.default_rng(15)
    a1, d1 = _f32(r.standard_normal((sum(gs1), k))), _f32(r.standard_normal((sum(gs1), n)))
    a2, d2 = _f32(r.standard_normal((sum(gs2), k))), _f32(r.standard_normal((sum(gs2), n)))
    acc = oracle.ragged_dot_k_epilogue(a2, d2, gs2, beta=1.0, c=oracle.ragged_dot_k(a1, d1, gs1))
    rows_a, rows_d, s1, s2 = [], [], 0, 0
    for h in range(3):
        rows_a += [a1[s1:s1 + gs1[h]], a2[s2:s2 + gs2[h]]]
        rows_d += [d1[s1:s1 + gs1[h]], d2[s2:s2 + gs2[h]]]
        s1 += gs1[h]; s2 += gs2[h]
    union = oracle.ragged_dot_k(np.concatenate(rows_a), np.concatenate(rows_d), [a + b for a, b in zip(gs1, gs2)])
    np.testing.assert_allclose(acc, union, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("alpha,beta", [(-2.0, 0.25), (0.5, 1.0), (3.0, 0.0), (1.0, -0.5)])
def test_k_epilogue_alpha_beta_brute_force(alpha, beta):
    """out[h] = alpha * (sum over the rows of h of lhs^T dout) + beta * c[h], written out with
    plain loops; an empty group gives exactly beta * c[h].  alpha scales the product only:
    alpha * (acc + beta * c) fails here whenever alpha != 1 and beta != 0."""
    m, k, n, gs = 8, 3, 4, [3, 0, 5]
    r = np.random.default_rng(19)
    lhs, dout = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((m, n)))
    c = r.standard_normal((len(gs), k, n))
    out = oracle.ragged_dot_k_epilogue(lhs, dout, gs, alpha=alpha, beta=beta, c=c)
    start = 0
    for h, s in enumerate(gs):
        for i in range(k):
            for j in range(n):
                acc = sum(float(lhs[start + q, i]) * float(dout[start + q, j]) for q in range(s))
                assert math.isclose(out[h, i, j], alpha * acc + beta * c[h, i, j], rel_tol=1e-13, abs_tol=1e-13)
        start += s
    assert np.array_equal(out[1], beta * c[1])


def test_activations_match_library_routines():
    """silu against x * expit(x) (scipy) and the tanh GELU against torch's, over a wide range;
    silu(0) = 0 and silu(x) -> x, 0 at the ends."""
    from scipy.special import expit
    x = np.linspace(-30.0, 30.0, 2001)
    np.testing.assert_allclose(oracle.silu(x), x * expit(x), rtol=1e-14, atol=1e-300)
    ref = torch.nn.functional.gelu(torch.from_numpy(x), approximate="tanh").numpy()
    np.testing.assert_allclose(oracle.gelu_tanh(x), ref, rtol=1e-13, atol=1e-15)
    assert oracle.silu(0.0) == 0.0 and abs(oracle.silu(40.0) - 40.0) < 1e-12 and abs(oracle.silu(-40.0)) < 1e-12


@pytest.mark.parametrize("act", ["silu", "gelu_tanh"])
def test_gated_brute_force(act):
    """act(x . w0[h] + b0[h]) * (x . w1[h] + b1[h]) written out with loops; rows past the
    total are 0."""
    m, k, n, gs = 8, 3, 4, [2, 0, 5]
    r = np.random.default_rng(16)
    lhs = _f32(r.standard_normal((m, k)))
    w0, w1 = _f32(r.standard_normal((3, k, n))), _f32(r.standard_normal((3, k, n)))
    b0, b1 = _f32(r.standard_normal((3, n + 1))), _f32(r.standard_normal((3, n + 1)))
    out = oracle.ragged_dot_m_gated(lhs, w0, w1, gs, act=act, bias0=b0, bias1=b1)
    f = {"silu": lambda v: v / (1.0 + math.exp(-v)),
         "gelu_tanh": lambda v: 0.5 * v * (1.0 + math.tanh(math.sqrt(2.0 / math.pi) * (v + 0.044715 * v ** 3)))}[act]
    row = 0
    for h, s in enumerate(gs):
        for _ in range(s):
            for j in range(n):
                gate = sum(float(lhs[row, t]) * float(w0[h, t, j]) for t in range(k)) + float(b0[h, j])
                up = sum(float(lhs[row, t]) * float(w1[h, t, j]) for t in range(k)) + float(b1[h, j])
                assert math.isclose(out[row, j], f(gate) * up, rel_tol=1e-12, abs_tol=1e-12)
            row += 1
    assert np.all(out[sum(gs):] == 0.0)
    rows = np.array([7, 0, 3])
    np.testing.assert_array_equal(oracle.ragged_dot_m_gated(lhs, w0, w1, gs, act=act, bias0=b0, bias1=b1, rows=rows),
                                  out[rows])


def test_k_pairs_select_rows_of_the_full_result():
    m, k, n, gs = 14, 5, 3, [3, 0, 11]
    r = np.random.default_rng(11)
    lhs, dout = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((m, n)))
    full = oracle.ragged_dot_k(lhs, dout, gs)
    pairs = np.array([[2, 4], [0, 0], [1, 3], [2, 1]])
    sel = oracle.ragged_dot_k(lhs, dout, gs, pairs=pairs)
    for q, (h, i) in enumerate(pairs):
        assert np.array_equal(sel[q], full[h, i])
    rows = np.array([13, 0, 2, 3])
    fm = oracle.ragged_dot_m(lhs, _f32(r.standard_normal((3, k, n))), gs)
    assert fm.shape == (m, n)


# ---- element decoding: bf16, OCP e4m3, E8M0 -----------------------------------------------

def test_bf16_decode_matches_library():
    bits = np.arange(0, 1 << 16, 7, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]          # finite patterns only
    ours = oracle.decode(bits)
    np.testing.assert_array_equal(ours, _bf16_values(bits))


def test_e4m3_decode_table():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.decode(codes)
    lib = _e4m3_values(codes)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(ours[ok], lib[ok])
    # values the OCP FP8 specification fixes
    assert ours[0x7E] == 448.0 and ours[0xFE] == -448.0
    assert ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6 and ours[0x38] == 1.0
    assert ours[0x00] == 0.0 and np.signbit(ours[0x80])
    assert np.isnan(ours[0x7F]) and np.isnan(ours[0xFF]) and np.isnan(ours).sum() == 2


def test_e8m0_decode_table():
    L = oracle.lib()
    ours = np.array([L.orc_decode_e8m0(s) for s in range(256)])
    lib = _e8m0_values(np.arange(256, dtype=np.uint8))
    assert np.isnan(ours[255]) and np.isnan(lib[255])
    np.testing.assert_array_equal(ours[:255], lib[:255])
    assert ours[127] == 1.0 and ours[0] == 2.0 ** -127 and ours[254] == 2.0 ** 127


# ---- P10-P12: MXFP8 scale placement -------------------------------------------------------

def _mx_case(m=12, k=64, n=5, g=3, seed=12):
    r = np.random.default_rng(seed)
    lhs = r.integers(0, 256, (m, k), dtype=np.uint8)
    rhs = r.integers(0, 256, (g, k, n), dtype=np.uint8)
    lhs[(lhs & 0x7F) == 0x7F] = 0x38                    # no NaN codes
    rhs[(rhs & 0x7F) == 0x7F] = 0x38
    ls = r.integers(120, 135, (m, k // 32), dtype=np.uint8)      # varies along both axes
    rs = r.integers(118, 137, (g, k // 32, n), dtype=np.uint8)   # varies along all three
    return lhs, rhs, ls, rs


def _mx_reference(lhs, rhs, ls, rs, gs):
    """Dequantise with library decoders, then per-group fp64 matmul."""
    A = _e4m3_values(lhs) * np.repeat(_e8m0_values(ls), 32, axis=1)
    B = _e4m3_values(rhs) * np.repeat(_e8m0_values(rs), 32, axis=1)
    out = np.zeros((A.shape[0], B.shape[2]))
    for h, (st, s) in enumerate(_blocks(gs, A.shape[0])):
        out[st:st + s] = A[st:st + s] @ B[h]
    return out


def test_mx_matches_dequantised_reference():
    lhs, rhs, ls, rs = _mx_case()
    gs = [5, 0, 7]
    ours = oracle.ragged_dot_m(lhs, rhs, gs, ls, rs)
    np.testing.assert_allclose(ours, _mx_reference(lhs, rhs, ls, rs, gs), rtol=1e-12, atol=1e-12)


def test_mx_scale_identity_and_mutants():
    """With one scale per operand per 32-element k block, the block's dot product times
    2^(sa + sb - 254) equals the dot product of the scaled operands (the identity the aiter
    follow-up commits rest on).  A swapped rhs-scale axis or a dropped rhs scale must be
    caught by the bf16 tolerance used for parity."""
    lhs, rhs, ls, rs = _mx_case()
    gs = [5, 0, 7]
    m, k = lhs.shape
    n = rhs.shape[2]
    ours = oracle.ragged_dot_m(lhs, rhs, gs, ls, rs)
    unit_l, unit_r = np.full_like(ls, 127), np.full_like(rs, 127)
    by_blocks = np.zeros((m, n))
    for b in range(k // 32):
        sl = slice(32 * b, 32 * b + 32)
        part = oracle.ragged_dot_m(np.ascontiguousarray(lhs[:, sl]), np.ascontiguousarray(rhs[:, sl, :]), gs,
                                   unit_l[:, :1], unit_r[:, :1, :])
        grp = np.full(m, -1)
        for h, (st, s) in enumerate(_blocks(gs, m)):
            grp[st:st + s] = h
        for r_ in range(m):
            if grp[r_] >= 0:
                by_blocks[r_] += part[r_] * 2.0 ** (ls[r_, b].astype(int) + rs[grp[r_], b, :].astype(int) - 254)
    np.testing.assert_allclose(ours, by_blocks, rtol=1e-12, atol=1e-12)

    def within_bf16_bar(y, ref):
        return bool(np.all(np.abs(y - ref) <= 1e-2 * np.abs(ref) + 1e-2))

    ref = _mx_reference(lhs, rhs, ls, rs, gs)
    assert within_bf16_bar(ours, ref)
    g = rhs.shape[0]
    swapped = np.ascontiguousarray(rs.transpose(0, 2, 1)).reshape(g, k // 32, n)
    assert not within_bf16_bar(oracle.ragged_dot_m(lhs, rhs, gs, ls, swapped), ref)
    assert not within_bf16_bar(oracle.ragged_dot_m(lhs, rhs, gs, ls, unit_r), ref)


def test_mx_unit_scales_is_plain_fp8_gemm():
    lhs, rhs, ls, rs = _mx_case(seed=13)
    gs = [4, 4, 4]
    ones_l, ones_r = np.full_like(ls, 127), np.full_like(rs, 127)
    ours = oracle.ragged_dot_m(lhs, rhs, gs, ones_l, ones_r)
    A, B = _e4m3_values(lhs), _e4m3_values(rhs)
    ref = np.concatenate([A[4 * h:4 * h + 4] @ B[h] for h in range(3)])
    np.testing.assert_allclose(ours, ref, rtol=1e-13, atol=1e-13)


# ---- bf16 inputs --------------------------------------------------------------------------

def test_bf16_inputs_decode_exactly():
    r = np.random.default_rng(14)
    m, k, n, gs = 9, 16, 6, [2, 7]
    lhs, rhs = _bf16_bits(r.standard_normal((m, k))), _bf16_bits(r.standard_normal((2, k, n)))
    ours = oracle.ragged_dot_m(lhs, rhs, gs)
    A, B = _bf16_values(lhs), _bf16_values(rhs)
    ref = np.concatenate([A[:2] @ B[0], A[2:] @ B[1]])
    np.testing.assert_allclose(ours, ref, rtol=1e-13, atol=1e-13)
    dout = _bf16_bits(r.standard_normal((m, n)))
    outk = oracle.ragged_dot_k(lhs, dout, gs)
    D = _bf16_values(dout)
    np.testing.assert_allclose(outk[1], A[2:].T @ D[2:], rtol=1e-13, atol=1e-13)


def test_row_selection_matches_full_result():
    r = np.random.default_rng(15)
    m, k, n, gs = 17, 8, 5, [3, 0, 9, 2]
    lhs, rhs = _f32(r.standard_normal((m, k))), _f32(r.standard_normal((4, k, n)))
    full = oracle.ragged_dot_m(lhs, rhs, gs)
    rows = np.array([16, 0, 14, 3, 11])
    np.testing.assert_array_equal(oracle.ragged_dot_m(lhs, rhs, gs, rows=rows), full[rows])


# ---------------------------------------------------------------------------------------
# permute / un-permute ("Group-GEMM in XLA", Part 4 "The Three MoE Compute Paths in MaxText")


def _brute_permute(experts, g):
    """Counting loops: for each expert in turn, its copies in index order."""
    flat = [int(e) for e in np.asarray(experts).reshape(-1)]
    s2c = []
    for e in range(g):
        for i, x in enumerate(flat):
            if x == e:
                s2c.append(i)
    sizes = [sum(1 for x in flat if x == e) for e in range(g)]
    return s2c, sizes


@pytest.mark.parametrize("g,top_k,tokens,bad", [(4, 2, 9, False), (5, 3, 7, True), (1, 1, 5, False),
                                                (16, 4, 11, True)])
def test_permute_brute_force(g, top_k, tokens, bad):
    r = np.random.default_rng([g, top_k, tokens])
    experts = r.integers(0, g, size=(tokens, top_k)).astype(np.int32)
    if bad:
        experts[0, 0] = g          # one past the last expert
        experts[-1, -1] = -1
    x = r.standard_normal((tokens, 6)).astype(np.float32)
    sx, ss, gs, s2c, c2s = oracle.moe_permute(x, experts, g)
    want_s2c, want_gs = _brute_permute(experts, g)
    S = len(want_s2c)
    M = tokens * top_k
    assert ss is None
    assert gs.tolist() == want_gs
    assert s2c[:S].tolist() == want_s2c and (s2c[S:] == -1).all()
    for p, i in enumerate(want_s2c):
        assert np.array_equal(sx[p], x[i // top_k])
        assert c2s[i] == p
    assert (sx[S:] == 0).all()
    routed = set(want_s2c)
    assert all(c2s[i] == -1 for i in range(M) if i not in routed)


def test_permute_worked_example():
    """Worked by hand: three tokens, top-2 of three experts, ids [[2, 0], [1, 2], [0, 0]]
    flatten to [2, 0, 1, 2, 0, 0]; the stable argsort is [1, 4, 5, 2, 0, 3], the bincount
    [3, 1, 2] and the inverse order [4, 0, 3, 5, 1, 2]."""
    x = np.array([[10.0], [20.0], [30.0]], dtype=np.float32)
    sx, _, gs, s2c, c2s = oracle.moe_permute(x, np.array([[2, 0], [1, 2], [0, 0]], np.int32), 3)
    assert s2c.tolist() == [1, 4, 5, 2, 0, 3]
    assert gs.tolist() == [3, 1, 2]
    assert sx[:, 0].tolist() == [10.0, 30.0, 30.0, 20.0, 10.0, 20.0]
    assert c2s.tolist() == [4, 0, 3, 5, 1, 2]


def test_unpermute_of_permuted_rows_is_weighted_identity():
    """With the expert block replaced by the identity, un-permute(permute(x)) is
    x[t] * (sum of the weights of t's routed copies)."""
    r = np.random.default_rng(7)
    T, K, g, k = 40, 3, 6, 10
    experts = r.integers(0, g, size=(T, K)).astype(np.int32)
    experts[3, 1] = -1                      # an unrouted copy adds nothing
    w = r.random((T, K)).astype(np.float32)
    x = r.standard_normal((T, k)).astype(np.float32)
    sx, _, _, _, c2s = oracle.moe_permute(x, experts, g)
    out = oracle.moe_unpermute(sx, c2s, w)
    wsum = np.where(experts >= 0, w.astype(np.float64), 0.0).sum(axis=1)
    np.testing.assert_allclose(out, x.astype(np.float64) * wsum[:, None], rtol=1e-15, atol=0)


def test_unpermute_brute_force_bf16():
    r = np.random.default_rng(8)
    T, K, n = 5, 2, 7
    y = _bf16_bits(r.standard_normal((T * K, n)))
    c2s = r.permutation(T * K).astype(np.int32)
    c2s[4] = -1
    w = r.random((T, K)).astype(np.float32)
    yv = _bf16_values(y)
    want = np.zeros((T, n))
    for t in range(T):
        for j in range(K):
            p = c2s[t * K + j]
            if p >= 0:
                want[t] += float(w[t, j]) * yv[p]
    np.testing.assert_allclose(oracle.moe_unpermute(y, c2s, w), want, rtol=1e-15, atol=0)


def test_sparse_path_equals_dense_path():
    """Path 1 (permute, ragged dot, un-permute) computes the same layer output as Path 2
    (every token through every expert, combined with weights that are zero off the
    token's selection) -- the pages' comparison of the two dropless paths."""
    r = np.random.default_rng(9)
    T, K, g, k, n = 24, 2, 5, 16, 12
    logits = r.standard_normal((T, g))
    experts = W.topk_indices(logits, K).astype(np.int32)
    w = r.random((T, K)).astype(np.float32)
    x = r.standard_normal((T, k)).astype(np.float32)
    wts = r.standard_normal((g, k, n)).astype(np.float32)
    sx, _, gs, _, c2s = oracle.moe_permute(x, experts, g)
    y = oracle.ragged_dot_m(sx, wts, gs)
    sparse = oracle.moe_unpermute(y.astype(np.float32), c2s, w)
    dense_w = np.zeros((T, g))
    for t in range(T):
        for j in range(K):
            dense_w[t, experts[t, j]] += w[t, j]
    per_expert = np.einsum("tk,ekn->ten", x.astype(np.float64), wts.astype(np.float64))
    dense = np.einsum("ten,te->tn", per_expert, dense_w)
    np.testing.assert_allclose(sparse, dense, rtol=1e-6, atol=1e-6)   # y rounded to fp32 once


def test_bf16_values_match_library():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    a, b = oracle.bf16_values(bits), _bf16_values(bits)
    same = (a == b) | (np.isnan(a) & np.isnan(b))
    assert same.all()
