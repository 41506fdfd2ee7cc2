"""MI355X (gfx950) ragged-dot Group-GEMM: Python binding over the C-ABI library.

The calls are imported lazily so that ``group_gemm_amd.workloads`` can be used without
loading the GPU library.
"""
_API = ("ragged_dot_m", "ragged_dot_m_noalloc", "ragged_dot_m_gated", "ragged_dot_k", "padded_dot", "moe_permute", "moe_unpermute",
        "workspace_bytes", "read_device_status",
        "build_schedule", "abi_version", "status_string", "lib", "GGError")


def __getattr__(name):
    if name in _API:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
