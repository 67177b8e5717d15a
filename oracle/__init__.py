"""fp64 CPU oracle for paged MLA (test infrastructure only; see mla_oracle)."""
from .mla_oracle import *  # noqa: F401,F403
