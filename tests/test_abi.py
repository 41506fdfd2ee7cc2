"""The C-ABI library loads, exports every symbol its header declares, and rejects bad
arguments on the host before touching the GPU.  CPU only: every call below fails host
validation, so no pointer passed here is ever dereferenced."""
import ctypes
import os
import re

import pytest

from group_gemm_amd import _binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "groupgemm.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([A-Za-z_][A-Za-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("ragged_dot_m", "ragged_dot_m_nk", "ragged_dot_m_epilogue", "ragged_dot_k_epilogue", "ragged_dot_m_gated",
                     "ragged_dot_k", "moe_permute", "moe_unpermute",
                     "padded_dot", "gg_workspace_bytes", "gg_schedule",
                     "gg_read_device_status", "gg_status_string", "gg_abi_version"):
        assert required in names


def test_library_exports_every_declared_symbol():
    L = B.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_abi_version_and_strings():
    assert B.abi_version() == 5
    for code in range(8):
        assert B.status_string(code)


# fake, aligned, never-dereferenced addresses
P = ctypes.c_void_p(0x10000)
NULL = None
WS_SMALL = 8


def _m(lhs=P, rhs=P, gs=P, out=P, m=64, k=64, n=64, g=4, ind=1, outd=1, ls=NULL, rs=NULL, ws=P, wsb=4096):
    return B.lib().ragged_dot_m(lhs, rhs, gs, out, m, k, n, g, ind, outd, ls, rs, ws, wsb, None)


def test_ragged_m_host_validation():
    assert _m(gs=NULL) == 1                      # GG_ERR_NULL_PTR
    assert _m(lhs=NULL) == 1
    assert _m(ws=NULL) == 1
    assert _m(g=0) == 2                          # GG_ERR_BAD_SHAPE
    assert _m(g=1025) == 2
    assert _m(m=-1) == 2
    assert _m(k=1 << 31) == 2
    assert _m(ind=0, outd=1) == 3                # fp32 in -> bf16 out: GG_ERR_BAD_DTYPE
    assert _m(ind=7) == 3
    assert _m(ws=ctypes.c_void_p(0x10004)) == 4  # workspace not 16-byte aligned
    assert _m(lhs=ctypes.c_void_p(0x10001)) == 4 # bf16 operand on an odd address
    assert _m(wsb=WS_SMALL) == 5                 # GG_ERR_WORKSPACE_TOO_SMALL
    assert _m(ind=2, k=48, ls=P, rs=P) == 6      # e4m3 needs k % 32 == 0
    assert _m(ind=2, k=64, ls=NULL, rs=P) == 1   # e4m3 needs scales


def test_ragged_m_nk_host_validation():
    def nk(lhs=P, rhs=P, gs=P, out=P, m=64, k=64, n=64, g=4, ind=1, outd=1, ws=P, wsb=4096):
        return B.lib().ragged_dot_m_nk(lhs, rhs, gs, out, m, k, n, g, ind, outd, ws, wsb, None)
    assert nk(gs=NULL) == 1
    assert nk(rhs=NULL) == 1
    assert nk(g=0) == 2
    assert nk(ind=0, outd=0) == 6                # fp32 [g,n,k] weights: not offered
    assert nk(ind=2) == 6                        # nor e4m3
    assert nk(outd=2) == 3                       # e4m3 output
    assert nk(rhs=ctypes.c_void_p(0x10008)) == 4 # the ring path needs 16-byte alignment
    assert nk(k=60) == 6                         # k % 8
    assert nk(n=12) == 6                         # n % 8
    assert nk(wsb=WS_SMALL) == 5


def test_epilogue_host_validation():
    L = B.lib()
    def me(bias=NULL, stride=0, alpha=1.0, beta=0.0, ind=1, outd=1, gs=P, g=4, k=64):
        return L.ragged_dot_m_epilogue(P, P, gs, P, 64, k, 64, g, ind, outd, NULL, NULL, bias, stride, alpha, beta, P, 4096,
                                       None)
    assert me(bias=P, stride=32) == 2                          # bias row stride below n
    assert me(bias=ctypes.c_void_p(0x10002), stride=64) == 4   # bias not 4-byte aligned
    assert me(gs=NULL, alpha=2.0) == 1
    assert me(g=0, beta=1.0) == 2
    assert me(ind=0, outd=1, alpha=2.0) == 3                   # fp32 in -> bf16 out
    assert me(ind=2, k=48, alpha=2.0) == 6
    def ke(alpha=1.0, beta=0.0, ind=1, outd=0, gs=P, wsb=4096):
        return L.ragged_dot_k_epilogue(P, P, gs, P, 64, 64, 64, 4, ind, outd, alpha, beta, P, wsb, None)
    assert ke(gs=NULL, beta=1.0) == 1
    assert ke(ind=2, beta=1.0) == 3
    assert ke(beta=1.0, wsb=WS_SMALL) == 5


def test_gated_host_validation():
    L = B.lib()
    def gt(w1=P, act=0, ind=1, outd=1, b0=NULL, stride=0, k=64, gs=P):
        return L.ragged_dot_m_gated(P, P, w1, gs, P, 64, k, 64, 4, ind, outd, act, b0, NULL, stride, P, 4096, None)
    assert gt(gs=NULL) == 1
    assert gt(w1=NULL) == 1
    assert gt(ind=0, outd=0) == 6            # fp32 not offered
    assert gt(act=7) == 6
    assert gt(b0=P, stride=8) == 2           # bias stride below n
    assert gt(w1=ctypes.c_void_p(0x10008)) == 4
    assert gt(k=60) == 6


def test_ragged_k_host_validation():
    L = B.lib()
    assert L.ragged_dot_k(P, P, NULL, P, 64, 64, 64, 4, 1, 0, P, 4096, None) == 1
    assert L.ragged_dot_k(P, P, P, P, 64, 64, 64, 0, 1, 0, P, 4096, None) == 2
    assert L.ragged_dot_k(P, P, P, P, 64, 64, 64, 4, 2, 0, P, 4096, None) == 3   # e4m3 not offered
    assert L.ragged_dot_k(P, P, P, P, 64, 64, 64, 4, 1, 0, P, 8, None) == 5


def test_padded_host_validation():
    L = B.lib()
    assert L.padded_dot(0, P, P, P, P, 64, 64, 64, 4, 16, 1, 1, NULL, NULL, P, 1 << 30, None) == 6   # bad mode
    assert L.padded_dot(2, P, P, P, P, 64, 64, 64, 4, 0, 1, 1, NULL, NULL, P, 1 << 30, None) == 2   # capacity 0
    need = B.workspace_bytes("padded_m", 64, 64, 64, 4, 16)
    assert need > 256
    assert L.padded_dot(2, P, P, P, P, 64, 64, 64, 4, 16, 1, 1, NULL, NULL, P, need - 1, None) == 5
    assert L.padded_dot(3, P, P, P, P, 64, 64, 64, 4, 16, 2, 0, P, P, P, 1 << 30, None) == 3        # e4m3 k-mode


def test_workspace_sizes():
    assert B.workspace_bytes("ragged_m", 8192, 4096, 14336, 8) == 256
    assert B.workspace_bytes("ragged_k", 16384, 5120, 8192, 16) == 256
    # padded lhs [g,C,k] bf16 + padded result room [g,C,n] fp32
    g, C, k, n = 8, 1280, 4096, 14336
    assert B.workspace_bytes("padded_m", 8192, k, n, g, C) >= g * C * (2 * k + 4 * n)
    assert B.lib().gg_workspace_bytes(0, 1, 1, 1, 0, 0, 1) == 0


def test_schedule_host_validation():
    L = B.lib()
    assert L.gg_schedule(P, 9, 1, 3, 0, 1, P, P, P, None) == 2
    assert L.gg_schedule(NULL, 9, 1, 3, 3, 1, P, P, P, None) == 1


def test_permute_host_validation():
    L = B.lib()
    need = B.workspace_bytes("permute", 64 * 2, 64, 0, 8)
    def pm(x=P, xs=NULL, e=P, sx=P, ss=NULL, gs=P, s2c=P, c2s=P, tokens=64, top_k=2, k=64, g=8, dt=1, ws=P, wsb=need):
        return L.moe_permute(x, xs, e, sx, ss, gs, s2c, c2s, tokens, top_k, k, g, dt, ws, wsb, None)
    assert pm(e=NULL) == 1
    assert pm(c2s=NULL) == 1
    assert pm(ws=NULL) == 1
    assert pm(x=NULL) == 1
    assert pm(top_k=0) == 2
    assert pm(g=0) == 2 and pm(g=1025) == 2
    assert pm(tokens=-1) == 2
    assert pm(tokens=1 << 29, top_k=4) == 2      # more than 2^30 copies
    assert pm(dt=5) == 3
    assert pm(xs=P) == 3                         # scales only with e4m3
    assert pm(dt=2) == 1                         # e4m3 without scales
    assert pm(dt=2, k=48, xs=P, ss=P) == 6       # e4m3 needs k % 32 == 0
    assert pm(e=ctypes.c_void_p(0x10002)) == 4
    assert pm(x=ctypes.c_void_p(0x10001)) == 4   # bf16 rows on an odd address
    assert pm(ws=ctypes.c_void_p(0x10008)) == 4
    assert pm(wsb=need - 1) == 5


def test_unpermute_host_validation():
    L = B.lib()
    def up(y=P, c2s=P, w=P, out=P, tokens=64, top_k=2, n=64, ind=1, outd=1):
        return L.moe_unpermute(y, c2s, w, out, tokens, top_k, n, ind, outd, None)
    assert up(c2s=NULL) == 1 and up(w=NULL) == 1 and up(y=NULL) == 1
    assert up(tokens=-1) == 2
    assert up(top_k=0) == 2 and up(n=-1) == 2
    assert up(ind=2) == 3 and up(outd=2) == 3
    assert up(w=ctypes.c_void_p(0x10002)) == 4


def test_permute_workspace_size():
    # header + counts [chunks, g] + one flag per chunk; chunks of at least 1024 copies, at most 64
    assert B.workspace_bytes("permute", 32768, 7168, 0, 256) == 256 + 32 * 256 * 4 + 256
    assert B.workspace_bytes("permute", 0, 7168, 0, 256) == 256
    assert B.workspace_bytes("permute", 1 << 24, 16, 0, 1024) == 256 + 64 * 1024 * 4 + 256
    assert B.workspace_bytes("permute", (1 << 30) + 1, 16, 0, 8) == 0
