"""Video Delta Attention (VDA) forward for AMD Instinct MI355X (gfx950).

The computation lives in hand-written HIP kernels in libvda.so (csrc/); this
package is its ctypes binding (argument marshalling only) and its build step.
"""
from .binding import (  # noqa: F401
    EXPORTED, LIB_PATH, VDA_DTYPE_BF16, VDA_DTYPE_F32, VDA_ERR_BAD_DTYPE, VDA_ERR_HIP,
    VDA_ERR_INVALID_ARG, VDA_ERR_MISALIGNED, VDA_ERR_NOT_SPD, VDA_ERR_SCRATCH_TOO_SMALL, VDA_ERR_WORKSPACE_TOO_SMALL,
    VDA_NOALLOC_MAX_BYTES, VDA_OK, VdaDesc,
    VdaError, VdaPrepDesc, desc_from_tensors, forward, load_library, make_desc, make_prep_desc,
    vda_check_desc, vda_prep, vda_prep_check_desc,
    vda_debug_chunks, vda_debug_chunks_decay, vda_debug_frame_maps, vda_debug_solve, vda_debug_stats,
    vda_debug_states, vda_debug_states_decay, vda_forward, vda_forward_decay, vda_forward_noalloc, vda_forward_timed,
    vda_status_string, vda_workspace_bytes,
)
