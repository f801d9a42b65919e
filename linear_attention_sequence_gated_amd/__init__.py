"""MI355X-native gated delta rule: chunkwise forward, its gradients and single-token decode.

The compute path is libgdn.so (hand-written HIP kernels for gfx950 behind the C
ABI of include/gdn.h); this package is its thin ctypes binding.
"""
from .gdn import (GDN_BF16, GDN_C64, GDN_F32, GDN_NOALLOC_MAX_WORKSPACE, GdnError, chunk_bwd, chunk_fwd, chunk_fwd_prologue,  # noqa: F401
                  fwd_channel_decay, gdn_chunk_bwd, gdn_chunk_bwd_workspace_bytes, gdn_chunk_fwd,
                  gdn_chunk_fwd_noalloc, gdn_chunk_fwd_prologue, gdn_chunk_fwd_prologue_workspace_bytes,
                  gdn_chunk_fwd_workspace_bytes, gdn_fwd_channel_decay, gdn_recurrent_step,
                  gdn_status_str, load, recurrent_step)
