"""CPU oracle for the Pyramid Sparse Attention forward pass.

TEST INFRASTRUCTURE ONLY: imported by tests/, the smoke check and the benchmark's
CPU-baseline leg. The product path never imports it."""
from . import psa_oracle  # noqa: F401
