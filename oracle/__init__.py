"""fp64 CPU oracle for the fused chunked forward-KL loss.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything in this package: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP library
(``chunked_kl_loss_amd``) and imports nothing from it.

See ``oracle.kl_dense`` for what is computed and which passage each step
follows.
"""
from .kl_dense import (  # noqa: F401
    teacher_probs,
    dense_teacher,
    row_scale,
    kl_dense,
    kl_rows,
    kl_sparse_loss,
    lse_rows,
    dw_rows,
)
