"""Parallel constrained decoding on AMD Instinct MI355X (gfx950).

The decoding path is the C ABI in include/pcd.h, implemented by the HIP
kernels under csrc/ and built into libpcd.so; `binding` marshals Python
arguments to it.  Build with `python -m constrained_decoding_pcd_amd.build`.
"""
from .binding import (DTYPE_BF16, DTYPE_F32, EXPORTS, KERNEL_CLASSES, LIB_PATH, MAX_PENDING, PcdError, PcdModel, PcdState,  # noqa: F401
                      config_of, debug_plan, limits_for, load_library, upload_weights)
