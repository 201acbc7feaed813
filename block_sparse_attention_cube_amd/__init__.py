"""Video sparse attention (VSA) for MI355X (gfx950): HIP kernels behind a C ABI.

The computation lives in libvsa.so (include/vsa.h); this package is its
PyTorch binding.  Importing it does not load the library; the first call does,
and fails loudly if the library is missing.
"""
from .binding import (BackwardPlan, ForwardFp8Plan, ForwardPlan, VSAFunction, backward,
                      backward_cube, check_problem, coarse, cube_counts, dense, fine, fine_fp8,
                      fine_raster, forward, forward_cube, forward_fp8, forward_static,
                      make_problem, quantize_fp8, reorder, vsa_attention, workspace_bytes)
from ._lib import VSAError, LIB_PATH

__all__ = ["BackwardPlan", "ForwardFp8Plan", "ForwardPlan", "VSAFunction", "VSAError", "LIB_PATH",
           "backward", "backward_cube", "check_problem", "coarse", "cube_counts", "dense", "fine",
           "fine_fp8", "fine_raster", "forward", "forward_cube", "forward_fp8", "forward_static",
           "make_problem", "quantize_fp8", "reorder", "vsa_attention", "workspace_bytes"]
