"""CPU oracle (test infrastructure only): see oracle.moe_oracle."""
from . import moe_oracle  # noqa: F401
