"""fp64 CPU oracle of the SparsePR operator (test infrastructure only).

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this package; the product path never does.
"""
from . import sparsepr_oracle  # noqa: F401
