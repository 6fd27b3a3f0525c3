"""MI355X-native forward pass of one Beam-style Mixture-of-Experts block.

The compute path is the C-ABI library ``libmoe.so`` (hand-written HIP for
gfx950).  ``group_limited_routing_router_amd.moe`` is a thin ctypes binding to
it; the binding is loaded lazily so that ``inputs`` (shapes and seeded draws)
can be imported without a GPU or a built library.
"""

_BINDING_NAMES = (
    "moe_route", "moe_permute", "moe_expert_ffn", "moe_expert_gate_up", "moe_expert_down",
    "moe_combine", "moe_combine_residual", "moe_dense_mlp", "moe_expert_ffn_fp8", "moe_forward",
    "moe_forward_fp8", "moe_forward_noalloc", "moe_peak_stream_read", "moe_peak_mfma_bf16",
    "moe_peak_mfma_stream",
    "moe_workspace_bytes", "MoEProblem", "MoEError", "DTYPE_F32", "DTYPE_BF16",
    "load_library", "library_path",
)


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import moe
        return getattr(moe, name)
    raise AttributeError(name)
