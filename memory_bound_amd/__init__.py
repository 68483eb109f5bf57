"""libfuse for MI355X (gfx950): single-pass fused row kernels behind a C ABI.

The package holds the HIP sources and the C-ABI library (``csrc/``, built into ``libfuse.so`` by
``memory_bound_amd.build``), the Python binding (``api``: one function per C entry point, same
names), the seeded synthetic inputs (``synth``) and the roofline arithmetic (``roofline``).
"""
from .api import (  # noqa: F401
    FuseError,
    fuse_add_layernorm,
    fuse_bias_gelu_residual,
    fuse_copy,
    fuse_softmax_rows,
    fuse_swiglu_dualgemm,
    fuse_unfused_add_layernorm,
    fuse_unfused_bias_gelu_residual,
    fuse_unfused_softmax_rows,
    fuse_unfused_swiglu,
    fuse_unfused_workspace_bytes,
    fuse_version,
)
