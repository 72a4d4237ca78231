"""KDA (Kimi Delta Attention) for MI355X: hand-written HIP kernels behind a
C ABI (include/kda.h), with a ctypes binding of the same names."""
from .kda import (  # noqa: F401
    KDA_BF16, KDA_F32, KDA_F_RAW_GATES, KDA_F_SCALAR_G, KDA_F_SKIP_CONV, KDA_F_SKIP_L2,
    KDA_NOALLOC_SCRATCH_BYTES, KDAError, KDAState, kda_backward_workspace_bytes, kda_chunk_backward,
    kda_backward_workspace_min_bytes,
    kda_chunk_prefill, kda_chunk_prefill_noalloc, kda_conv_prologue, kda_decode_step,
    kda_stream_rmw,
    kda_decode_step_gated, kda_prologue_backward, kda_prologue_backward_workspace_bytes,
    kda_gated_rmsnorm, kda_prefill_workspace_bytes, kda_state_alloc, kda_state_bytes,
    kda_state_free, kda_state_get_dims, kda_state_reset, kda_state_ring, kda_state_S,
    kda_version, last_error, lib, make_dims,
)
