"""DFlash block-diffusion drafter step on AMD Instinct MI355X (gfx950).

The compute lives in ``libdflash.so`` (hand-written HIP kernels behind the C
ABI declared in ``include/dflash.h``).  ``_lib`` is the ctypes binding with the
ABI's entry-point names; ``runtime`` keeps weights, the paged context cache and
the workspace in device memory.  Build with
``python -m block_diffusion_drafter_gemm_amd.build``.
"""
from ._lib import LIB_PATH, DflashError, load  # noqa: F401
