"""CSA2 layer step on MI355X (gfx950): HIP kernels behind a C ABI (include/csa2.h),
with a thin torch-facing binding (``csa2``) and the layer-mode driver (``layer``)."""
from . import csa2  # noqa: F401

__all__ = ["csa2"]
