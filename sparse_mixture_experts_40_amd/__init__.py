"""MI355X (gfx950) sparse mixture-of-experts block forward.

The compute path is the HIP library ``libmoe.so`` (C ABI in ``include/moe.h``);
``binding`` is its thin ctypes wrapper. Importing the package does not load the
library; ``binding`` raises if it is missing.
"""
from .configs import MoEConfig, WORKLOADS  # noqa: F401

__all__ = ["MoEConfig", "WORKLOADS"]
