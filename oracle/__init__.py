"""Float64 CPU oracle for the MSA hot path.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.
"""
from . import msa_oracle  # noqa: F401
