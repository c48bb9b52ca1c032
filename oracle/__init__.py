"""CPU oracle for the multi-round LSH-attention forward (test infrastructure only)."""
from . import lsh_oracle  # noqa: F401
