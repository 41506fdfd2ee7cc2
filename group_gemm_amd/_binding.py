"""ctypes binding of libgroupgemm.so: argument marshalling only.

Every computation happens in the library's HIP kernels.  torch supplies device memory
and the current stream; there is no CPU fallback: if the library is missing or a call
fails, an exception is raised.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgroupgemm.so")

GG_DT = {torch.float32: 0, torch.bfloat16: 1, torch.uint8: 2, torch.float8_e4m3fn: 2}
OP = {"ragged_m": 0, "ragged_k": 1, "padded_m": 2, "padded_k": 3, "permute": 4}
DEV_NEGATIVE_SIZE, DEV_SUM_EXCEEDS_M, DEV_OVER_CAPACITY, DEV_BAD_EXPERT = 0x1, 0x2, 0x4, 0x8

_lib = None


class GGError(RuntimeError):
    def __init__(self, code, what):
        super().__init__(f"{what}: {status_string(code)} (code {code})")
        self.code = code


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m group_gemm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        L.gg_workspace_bytes.argtypes = [ctypes.c_int, i64, i64, i64, i32, i64, ctypes.c_int]
        L.gg_workspace_bytes.restype = sz
        L.ragged_dot_m.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp, sz, vp]
        L.ragged_dot_m_noalloc.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                                           vp]
        L.ragged_dot_k.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_int, ctypes.c_int, vp, sz, vp]
        L.ragged_dot_m_nk.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_int, ctypes.c_int, vp, sz, vp]
        f32 = ctypes.c_float
        L.ragged_dot_m_epilogue.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_int, ctypes.c_int, vp, vp, vp,
                                            i64, f32, f32, vp, sz, vp]
        L.ragged_dot_k_epilogue.argtypes = [vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_int, ctypes.c_int, f32, f32, vp,
                                            sz, vp]
        L.ragged_dot_m_gated.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i32, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                         vp, vp, i64, vp, sz, vp]
        L.padded_dot.argtypes = [ctypes.c_int, vp, vp, vp, vp, i64, i64, i64, i32, i64, ctypes.c_int, ctypes.c_int,
                                 vp, vp, vp, sz, vp]
        L.moe_permute.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i32, i64, i32, ctypes.c_int, vp, sz, vp]
        L.moe_unpermute.argtypes = [vp, vp, vp, vp, i64, i32, i64, ctypes.c_int, ctypes.c_int, vp]
        L.gg_schedule.argtypes = [vp, i64, i64, i32, i32, i32, vp, vp, vp, vp]
        L.gg_read_device_status.argtypes = [vp, ctypes.POINTER(ctypes.c_uint32), vp]
        L.gg_status_string.argtypes = [ctypes.c_int]
        L.gg_status_string.restype = ctypes.c_char_p
        L.gg_abi_version.restype = ctypes.c_int
        for f in ("ragged_dot_m", "ragged_dot_m_noalloc", "ragged_dot_m_nk", "ragged_dot_m_epilogue", "ragged_dot_m_gated", "ragged_dot_k",
                  "ragged_dot_k_epilogue",
                  "padded_dot", "moe_permute", "moe_unpermute", "gg_schedule", "gg_read_device_status"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(code):
    return lib().gg_status_string(code).decode()


def abi_version():
    return lib().gg_abi_version()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(code, what):
    if code != 0:
        raise GGError(code, what)


def workspace_bytes(op, m, k, n, g, capacity=0, in_dtype=torch.bfloat16):
    return int(lib().gg_workspace_bytes(OP[op], m, k, n, g, capacity, GG_DT[in_dtype]))


def _workspace(op, m, k, n, g, capacity, in_dtype, device, workspace):
    need = workspace_bytes(op, m, k, n, g, capacity, in_dtype)
    if need == 0:
        raise ValueError("bad arguments for the workspace size")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    else:
        _tensor(workspace, "workspace", device, dtype=torch.uint8)
        if workspace.numel() < need:
            raise ValueError(f"workspace holds {workspace.numel()} bytes, the call needs {need}")
    return workspace


# Every pointer handed to the library must address device memory of the right size: the
# kernels trust the shapes they are given.  These checks run before any launch.
_IN_DTYPES = (torch.float32, torch.bfloat16, torch.uint8, torch.float8_e4m3fn)


def _tensor(t, name, device, shape=None, dtype=None, dtypes=None, contiguous=True):
    if not torch.is_tensor(t):
        raise TypeError(f"{name} must be a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a CUDA (HIP) device, not {t.device}")
    if device is not None and t.device != torch.device(device):
        raise ValueError(f"{name} is on {t.device}, the call runs on {device}")
    if contiguous and not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if dtypes is not None and t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")


def _is_e4m3(t):
    return t.dtype in (torch.uint8, torch.float8_e4m3fn)


def _scales(lhs, lhs_scale, rhs_scale, m, k, n, g, device):
    """E8M0 scales: required (uint8 [m, k/32] and [g, k/32, n]) for e4m3 inputs, else absent."""
    if _is_e4m3(lhs):
        if lhs_scale is None or rhs_scale is None:
            raise ValueError("e4m3 inputs need lhs_scale and rhs_scale")
        if k % 32:
            raise ValueError("e4m3 inputs need k % 32 == 0")
        _tensor(lhs_scale, "lhs_scale", device, (m, k // 32), torch.uint8)
        _tensor(rhs_scale, "rhs_scale", device, (g, k // 32, n), torch.uint8)
    elif lhs_scale is not None or rhs_scale is not None:
        raise ValueError("scales are taken only with e4m3 inputs")


def _out(out, name, device, shape, out_dtype):
    if out is not None:
        _tensor(out, name, device, shape, dtypes=(torch.float32, torch.bfloat16))
        if out_dtype is not None and out.dtype != out_dtype:
            raise ValueError(f"{name} has dtype {out.dtype}, but out_dtype is {out_dtype}")
        return out
    return torch.empty(shape, dtype=out_dtype, device=device)


def _bias(b, name, g, n, device):
    if b is None:
        return 0
    _tensor(b, name, device, dtype=torch.float32, contiguous=False)
    if b.dim() != 2 or b.shape[0] != g or b.shape[1] < n or b.stride(1) != 1 or b.stride(0) < n:
        raise ValueError(f"{name} must be float32 [g, >=n] with unit column stride")
    return b.stride(0)


def ragged_dot_m(lhs, rhs, group_sizes, out=None, out_dtype=None, lhs_scale=None, rhs_scale=None, workspace=None,
                 rhs_layout="kn", bias=None, alpha=1.0, beta=0.0):
    """out[m,n]: row block of group h of lhs [m,k] times rhs[h] [k,n]; rows past
    sum(group_sizes) are 0.  e4m3 inputs (uint8 codes) need E8M0 lhs_scale [m,k/32] and
    rhs_scale [g,k/32,n].  rhs_layout="nk" takes rhs as [g,n,k] (k contiguous) and
    multiplies by rhs[h]^T: the data-gradient classes, bf16 only (ragged_dot_m_nk).
    bias (fp32 [g, >=n], unit column stride), alpha, beta: out = alpha * (lhs . rhs[h]) +
    bias[h] + beta * out, in place (ragged_dot_m_epilogue; beta != 0 reads `out`, which
    must then be given)."""
    dev = lhs.device
    _tensor(lhs, "lhs", None, dtypes=_IN_DTYPES)
    if lhs.dim() != 2 or rhs.dim() != 3:
        raise ValueError("lhs must be [m,k] and rhs [g,k,n] (or [g,n,k])")
    m, k = lhs.shape
    if rhs_layout == "nk":
        g, n, k2 = rhs.shape
    elif rhs_layout == "kn":
        g, k2, n = rhs.shape
    else:
        raise ValueError(f"rhs_layout must be 'kn' or 'nk', not {rhs_layout!r}")
    _tensor(rhs, "rhs", dev, dtype=lhs.dtype)
    _tensor(group_sizes, "group_sizes", dev, (g,), torch.int32)
    if k2 != k:
        raise ValueError(f"lhs has k = {k}, rhs has {k2}")
    _scales(lhs, lhs_scale, rhs_scale, m, k, n, g, dev)
    epilogue = bias is not None or alpha != 1.0 or beta != 0.0
    if epilogue and rhs_layout != "kn":
        raise ValueError("the epilogue takes [g,k,n] weights")
    if beta != 0.0 and out is None:
        raise ValueError("beta != 0 accumulates into `out`, which must be given")
    if rhs_layout == "nk" and (lhs_scale is not None or rhs_scale is not None):
        raise ValueError("rhs_layout='nk' takes no scales")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else (torch.float32 if lhs.dtype == torch.float32 else torch.bfloat16)
    stride = _bias(bias, "bias", g, n, dev)
    out = _out(out, "out", dev, (m, n), out_dtype)
    ws = _workspace("ragged_m", m, k, n, g, 0, lhs.dtype, dev, workspace)
    if epilogue:
        code = lib().ragged_dot_m_epilogue(_p(lhs), _p(rhs), _p(group_sizes), _p(out), m, k, n, g, GG_DT[lhs.dtype],
                                           GG_DT[out.dtype], _p(lhs_scale), _p(rhs_scale), _p(bias), stride,
                                           float(alpha), float(beta), _p(ws), ws.numel(), _stream(dev))
        _check(code, "ragged_dot_m_epilogue")
        return out
    if rhs_layout == "nk":
        code = lib().ragged_dot_m_nk(_p(lhs), _p(rhs), _p(group_sizes), _p(out), m, k, n, g, GG_DT[lhs.dtype],
                                     GG_DT[out.dtype], _p(ws), ws.numel(), _stream(dev))
        _check(code, "ragged_dot_m_nk")
        return out
    code = lib().ragged_dot_m(_p(lhs), _p(rhs), _p(group_sizes), _p(out), m, k, n, g, GG_DT[lhs.dtype],
                              GG_DT[out.dtype], _p(lhs_scale), _p(rhs_scale), _p(ws), ws.numel(), _stream(dev))
    _check(code, "ragged_dot_m")
    return out


def ragged_dot_m_noalloc(lhs, rhs, group_sizes, out, lhs_scale=None, rhs_scale=None, status=None):
    """ragged_dot_m into a caller-given `out` with no workspace: the library keeps the per-call
    state in its own static device array (one per GPU; calls on one GPU must not overlap).
    `status`: optional device int32 [1] that receives the GG_DEV_* bits.  Allocates nothing."""
    dev = lhs.device
    _tensor(lhs, "lhs", None, dtypes=_IN_DTYPES)
    if lhs.dim() != 2 or rhs.dim() != 3:
        raise ValueError("lhs must be [m,k] and rhs [g,k,n]")
    m, k = lhs.shape
    g, k2, n = rhs.shape
    _tensor(rhs, "rhs", dev, dtype=lhs.dtype)
    _tensor(group_sizes, "group_sizes", dev, (g,), torch.int32)
    if k2 != k:
        raise ValueError(f"lhs has k = {k}, rhs has {k2}")
    _scales(lhs, lhs_scale, rhs_scale, m, k, n, g, dev)
    if out is None:
        raise ValueError("out must be given (the call allocates nothing)")
    _out(out, "out", dev, (m, n), None)
    if status is not None:
        _tensor(status, "status", dev, (1,), dtypes=(torch.int32, torch.uint32))
    code = lib().ragged_dot_m_noalloc(_p(lhs), _p(rhs), _p(group_sizes), _p(out), m, k, n, g, GG_DT[lhs.dtype],
                                      GG_DT[out.dtype], _p(lhs_scale), _p(rhs_scale), _p(status), _stream(dev))
    _check(code, "ragged_dot_m_noalloc")
    return out


ACT = {"silu": 0, "gelu_tanh": 1}


def ragged_dot_m_gated(lhs, w0, w1, group_sizes, act="silu", out=None, out_dtype=None, bias0=None, bias1=None,
                       workspace=None):
    """out[m,n] = act(lhs . w0[h] + bias0[h]) * (lhs . w1[h] + bias1[h]) for the rows of group h
    (the fused gate/up projection); rows past sum(group_sizes) are 0.  bf16 lhs [m,k] and
    w0 / w1 [g,k,n]; biases fp32 [g, >=n] sharing one row stride, or None."""
    dev = lhs.device
    _tensor(lhs, "lhs", None, dtype=torch.bfloat16)
    if lhs.dim() != 2 or w0.dim() != 3:
        raise ValueError("lhs must be [m,k] and w0, w1 [g,k,n]")
    m, k = lhs.shape
    g, k2, n = w0.shape
    _tensor(w0, "w0", dev, dtype=lhs.dtype)
    _tensor(w1, "w1", dev, tuple(w0.shape), lhs.dtype)
    _tensor(group_sizes, "group_sizes", dev, (g,), torch.int32)
    if k2 != k:
        raise ValueError(f"lhs has k = {k}, w0 has {k2}")
    if act not in ACT:
        raise ValueError(f"act must be one of {sorted(ACT)}")
    s0, s1 = _bias(bias0, "bias0", g, n, dev), _bias(bias1, "bias1", g, n, dev)
    if s0 and s1 and s0 != s1:
        raise ValueError("bias0 and bias1 must share one row stride")
    stride = s0 or s1
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    out = _out(out, "out", dev, (m, n), out_dtype)
    ws = _workspace("ragged_m", m, k, n, g, 0, lhs.dtype, dev, workspace)
    code = lib().ragged_dot_m_gated(_p(lhs), _p(w0), _p(w1), _p(group_sizes), _p(out), m, k, n, g, GG_DT[lhs.dtype],
                                    GG_DT[out.dtype], ACT[act], _p(bias0), _p(bias1), stride, _p(ws), ws.numel(),
                                    _stream(dev))
    _check(code, "ragged_dot_m_gated")
    return out


def ragged_dot_k(lhs, dout, group_sizes, out=None, out_dtype=None, workspace=None, alpha=1.0, beta=0.0):
    """out[g,k,n]: out[h] = lhs[rows of h]^T . dout[rows of h]; empty groups give 0.
    alpha, beta: out[h] = alpha * (...) + beta * out[h], in place (ragged_dot_k_epilogue;
    beta = 1 accumulates over micro-steps; beta != 0 needs `out`)."""
    dev = lhs.device
    _tensor(lhs, "lhs", None, dtypes=(torch.float32, torch.bfloat16))
    if lhs.dim() != 2 or dout.dim() != 2 or group_sizes.dim() != 1:
        raise ValueError("lhs must be [m,k], dout [m,n] and group_sizes [g]")
    m, k = lhs.shape
    m2, n = dout.shape
    g = group_sizes.shape[0]
    _tensor(dout, "dout", dev, dtype=lhs.dtype)
    _tensor(group_sizes, "group_sizes", dev, (g,), torch.int32)
    if m2 != m:
        raise ValueError(f"lhs has {m} rows, dout {m2}")
    if beta != 0.0 and out is None:
        raise ValueError("beta != 0 accumulates into `out`, which must be given")
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.float32
    out = _out(out, "out", dev, (g, k, n), out_dtype)
    ws = _workspace("ragged_k", m, k, n, g, 0, lhs.dtype, dev, workspace)
    if alpha != 1.0 or beta != 0.0:
        code = lib().ragged_dot_k_epilogue(_p(lhs), _p(dout), _p(group_sizes), _p(out), m, k, n, g, GG_DT[lhs.dtype],
                                           GG_DT[out.dtype], float(alpha), float(beta), _p(ws), ws.numel(),
                                           _stream(dev))
        _check(code, "ragged_dot_k_epilogue")
        return out
    code = lib().ragged_dot_k(_p(lhs), _p(dout), _p(group_sizes), _p(out), m, k, n, g, GG_DT[lhs.dtype],
                              GG_DT[out.dtype], _p(ws), ws.numel(), _stream(dev))
    _check(code, "ragged_dot_k")
    return out


def padded_dot(mode, a, b, group_sizes, capacity, out=None, out_dtype=None, a_scale=None, b_scale=None,
               workspace=None):
    """The capacity-padded baseline: mode "m" (a = lhs [m,k], b = rhs [g,k,n]) or "k"
    (a = lhs [m,k], b = dout [m,n])."""
    dev = a.device
    _tensor(a, "a", None, dtypes=_IN_DTYPES)
    if mode not in ("m", "k"):
        raise ValueError(f"mode must be 'm' or 'k', not {mode!r}")
    if a.dim() != 2 or group_sizes.dim() != 1:
        raise ValueError("a must be [m,k] and group_sizes [g]")
    g = group_sizes.shape[0]
    m, k = a.shape
    _tensor(b, "b", dev, dtype=a.dtype)
    _tensor(group_sizes, "group_sizes", dev, (g,), torch.int32)
    if mode == "m":
        if b.dim() != 3 or b.shape[0] != g or b.shape[1] != k:
            raise ValueError(f"b must be [g={g}, k={k}, n]")
        n = b.shape[2]
        shape = (m, n)
        _scales(a, a_scale, b_scale, m, k, n, g, dev)
        default = torch.float32 if a.dtype == torch.float32 else torch.bfloat16
    else:
        if b.dim() != 2 or b.shape[0] != m:
            raise ValueError(f"b must be [m={m}, n]")
        if a_scale is not None or b_scale is not None:
            raise ValueError("the contracting form takes no scales")
        n = b.shape[1]
        shape = (g, k, n)
        default = torch.float32
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else default
    out = _out(out, "out", dev, shape, out_dtype)
    op = "padded_" + mode
    ws = _workspace(op, m, k, n, g, capacity, a.dtype, dev, workspace)
    code = lib().padded_dot(OP[op], _p(a), _p(b), _p(group_sizes), _p(out), m, k, n, g, capacity, GG_DT[a.dtype],
                            GG_DT[out.dtype], _p(a_scale), _p(b_scale), _p(ws), ws.numel(), _stream(dev))
    _check(code, "padded_dot")
    return out


def moe_permute(x, experts, g, x_scale=None, workspace=None, out=None):
    """Sort the top-k copies of the tokens of x [tokens, k] by expert (experts: int32
    [tokens, top_k]); returns (sorted_x [M, k], sorted_scale [M, k/32] or None, group_sizes
    int32 [g], sorted_to_copy int32 [M], copy_to_sorted int32 [M]) with M = tokens * top_k.
    e4m3 inputs (uint8 codes) need their E8M0 x_scale [tokens, k/32].  `out` may supply
    that tuple of output tensors (an entry None is allocated)."""
    dev = x.device
    _tensor(x, "x", None, dtypes=_IN_DTYPES)
    if x.dim() != 2:
        raise ValueError("x must be [tokens, k]")
    tokens, k = x.shape
    _tensor(experts, "experts", dev, dtype=torch.int32)
    if experts.dim() != 2 or experts.shape[0] != tokens:
        raise ValueError("experts must be int32 [tokens, top_k]")
    top_k = experts.shape[1]
    M = tokens * top_k
    if _is_e4m3(x):
        if x_scale is None or k % 32:
            raise ValueError("e4m3 rows need x_scale [tokens, k/32] (k % 32 == 0)")
        _tensor(x_scale, "x_scale", dev, (tokens, k // 32), torch.uint8)
    elif x_scale is not None:
        raise ValueError("x_scale is taken only with e4m3 rows")
    sorted_x, sorted_scale, group_sizes, s2c, c2s = out if out is not None else (None,) * 5
    if sorted_x is None:
        sorted_x = torch.empty((M, k), dtype=x.dtype, device=dev)
    if x_scale is not None and sorted_scale is None:
        sorted_scale = torch.empty((M, k // 32), dtype=torch.uint8, device=dev)
    if group_sizes is None:
        group_sizes = torch.empty((g,), dtype=torch.int32, device=dev)
    if s2c is None:
        s2c = torch.empty((M,), dtype=torch.int32, device=dev)
    if c2s is None:
        c2s = torch.empty((M,), dtype=torch.int32, device=dev)
    _tensor(sorted_x, "sorted_x", dev, (M, k), x.dtype)
    if x_scale is not None:
        _tensor(sorted_scale, "sorted_scale", dev, (M, k // 32), torch.uint8)
    elif sorted_scale is not None:
        raise ValueError("sorted_scale is taken only with e4m3 rows")
    _tensor(group_sizes, "group_sizes", dev, (g,), torch.int32)
    _tensor(s2c, "sorted_to_copy", dev, (M,), torch.int32)
    _tensor(c2s, "copy_to_sorted", dev, (M,), torch.int32)
    ws = _workspace("permute", M, k, 0, g, 0, x.dtype, dev, workspace)
    code = lib().moe_permute(_p(x), _p(x_scale), _p(experts), _p(sorted_x), _p(sorted_scale), _p(group_sizes), _p(s2c),
                             _p(c2s), tokens, top_k, k, g, GG_DT[x.dtype], _p(ws), ws.numel(), _stream(dev))
    _check(code, "moe_permute")
    return sorted_x, sorted_scale, group_sizes, s2c, c2s


def moe_unpermute(y, copy_to_sorted, weights, out=None, out_dtype=None):
    """out[t, :] = sum_j weights[t, j] * y[copy_to_sorted[t * top_k + j], :] for y
    [tokens * top_k, n] in sorted order and fp32 weights [tokens, top_k]."""
    dev = y.device
    _tensor(y, "y", None, dtypes=(torch.float32, torch.bfloat16))
    if y.dim() != 2 or weights.dim() != 2:
        raise ValueError("y must be [tokens * top_k, n] and weights [tokens, top_k]")
    tokens, top_k = weights.shape
    M, n = y.shape
    if M != tokens * top_k:
        raise ValueError(f"y has {M} rows, weights give {tokens} x {top_k}")
    _tensor(weights, "weights", dev, dtype=torch.float32)
    _tensor(copy_to_sorted, "copy_to_sorted", dev, (M,), torch.int32)
    if out_dtype is None:
        out_dtype = out.dtype if out is not None else torch.bfloat16
    out = _out(out, "out", dev, (tokens, n), out_dtype)
    code = lib().moe_unpermute(_p(y), _p(copy_to_sorted), _p(weights), _p(out), tokens, top_k, n, GG_DT[y.dtype],
                               GG_DT[out.dtype], _stream(dev))
    _check(code, "moe_unpermute")
    return out


def build_schedule(group_sizes, m, n, block_m, block_n):
    """Run the scan alone; returns (row_off int32[g+1], tile_off int32[g+1], status) on
    the device."""
    dev = group_sizes.device
    _tensor(group_sizes, "group_sizes", None, dtype=torch.int32)
    if group_sizes.dim() != 1:
        raise ValueError("group_sizes must be int32 [g]")
    g = group_sizes.shape[0]
    row_off = torch.empty(g + 1, dtype=torch.int32, device=dev)
    tile_off = torch.empty(g + 1, dtype=torch.int32, device=dev)
    status = torch.empty(1, dtype=torch.int32, device=dev)
    code = lib().gg_schedule(_p(group_sizes), m, n, g, block_m, block_n, _p(row_off), _p(tile_off), _p(status),
                             _stream(dev))
    _check(code, "gg_schedule")
    return row_off, tile_off, status


def read_device_status(workspace):
    _tensor(workspace, "workspace", None, dtype=torch.uint8)
    if workspace.numel() < 4:
        raise ValueError("workspace too small to hold the status word")
    flags = ctypes.c_uint32(0)
    _check(lib().gg_read_device_status(_p(workspace), ctypes.byref(flags), _stream(workspace.device)),
           "gg_read_device_status")
    return flags.value
