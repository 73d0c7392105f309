"""fp64 CPU oracle for the MSA hot path (test infrastructure only)."""
from .msa_oracle import *  # noqa: F401,F403
