"""fp64 CPU oracle (test infrastructure only; never imported by the library)."""
from . import opr_oracle  # noqa: F401
