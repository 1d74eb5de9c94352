"""Monarch block-diagonal multiply for MI355X (gfx950).

The library computes Y = X · (Qout·L·P·R)ᵀ and its backward pass, and the
projection of a dense matrix onto Monarch factors, in HIP kernels behind the
C ABI of include/monarch.h (libmonarch.so, built in-tree
by build_lib.py). This package holds the ctypes binding (binding.py),
tensor-level helpers (torch_api.py, imports torch) and the seeded synthetic
input generator (synthetic.py).
"""
from .binding import (  # noqa: F401
    ACT_NONE, ACT_RELU, BF16, F32, LIB_PATH, MonarchError, load_library, monarch_abi_version,
    monarch_bwd, monarch_bwd_workspace_bytes, monarch_describe, monarch_fwd, monarch_project,
    monarch_status_string, monarch_linear_mid, monarch_fwd_ex, monarch_bwd_ex,
    monarch_bwd_ex_workspace_bytes, monarch_describe_ex, monarch_hyper_saved_elems,
    monarch_hyper_fwd, monarch_hyper_bwd_workspace_bytes, monarch_hyper_bwd,
    monarch_hyper_describe, monarch_dyad_fwd_workspace_bytes, monarch_dyad_fwd,
    monarch_dyad_bwd_workspace_bytes, monarch_dyad_bwd, monarch_dyad_describe,
    monarch_bwd_noalloc, monarch_stream_copy,
)
