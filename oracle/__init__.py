"""CPU oracle of the DSA sparse-attention path (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg use it; the
product path never imports it.
"""
from . import dsa_oracle  # noqa: F401
