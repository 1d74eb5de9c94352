"""fp64 CPU oracle for the Monarch multiply. TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import anything from this package. It shares no code with the GPU library.
"""
from .monarch_oracle import (  # noqa: F401
    derive_sizes, param_count, block_diag_dense, stride_permutation, output_permutation,
    dense_factors, monarch_matrix, forward, backward, mlp_forward, mlp_backward,
    forward_rows, backward_dx_rows, weight_grad_entries, rel_frobenius,
    max_row_rel_error, parity_error,
)
from . import monarch_projection  # noqa: F401,E402
from . import monarch_linear  # noqa: F401,E402
from . import monarch_hypercube  # noqa: F401,E402
from . import dyad  # noqa: F401,E402
