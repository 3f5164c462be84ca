"""fp64 CPU oracle for the group-wise fake-quant linear (test infrastructure only)."""
from .qat_oracle import *  # noqa: F401,F403
from . import qat_oracle  # noqa: F401
