"""HiLS (Hierarchical Landmark Sparse) attention for AMD Instinct MI355X (gfx950).

The compute path is the C-ABI library ``libhils.so`` (hand-written HIP
kernels); ``hils`` is its thin ctypes binding.
"""
from .hils import (  # noqa: F401
    hils_forward, hils_decode, hils_decode_noalloc, hils_backward, hils_landmarks,
    hils_landmarks_backward,
    hils_workspace_size, make_params,
    hils_profile_kernel, hils_profile_count, KERNEL_IDS,
    load_library, HilsError, HilsParams, EXPORTS, LIB_PATH,
    HILS_F32, HILS_BF16, HILS_OP_FORWARD, HILS_OP_DECODE, HILS_OP_BACKWARD,
)
