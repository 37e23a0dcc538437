"""fp64 CPU oracle for Token Sparse Attention (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg import this
package.  The HIP library and its Python binding never do.
"""
from . import tsa_oracle  # noqa: F401
