"""MI355X-native (gfx950) Gated DeltaNet core.

The hot path (gate preparation, chunk-local WY auxiliaries, inter-chunk state
scan, recurrent decode step, the Gated DeltaNet-2 chunked prefill and its
gradient) is
hand-written HIP in ``csrc/`` behind the C ABI
of ``include/gdn.h``; ``binding`` is its thin ctypes wrapper for torch tensors.
"""
from .binding import (  # noqa: F401
    BWD2_STAGE_NAMES, GDN2_CHUNK_BWD_STAGES, GDN_BF16, GDN_CHUNK_FWD_STAGES, GDN_F32, GDNError, STAGE_NAMES, StageEvents, alloc_workspace,
    alloc_workspace_gdn2, gdn2_chunk_bwd, gdn2_chunk_bwd_workspace_bytes, gdn2_chunk_fwd_workspace_bytes,
    gdn2_chunk_fwd, gdn2_recurrent_step, gdn_causal_conv1d, gdn_chunk_fwd, gdn_chunk_fwd_noalloc, gdn_gated_rmsnorm, gdn_chunk_fwd_workspace_bytes, gdn_dims, gdn_recurrent_step, lib,
    make_dims,
)
