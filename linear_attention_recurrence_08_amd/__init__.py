"""MI355X-native KDA (Kimi Delta Attention) token mixer: chunkwise prefill (optionally saving state
snapshots), single-token decode, the input stage and the gated output stage, as hand-written HIP
kernels for gfx950 behind the C ABI in include/kda.h.

The binding (kda.py) loads libkda.so built in-tree by build.py; it has no CPU fallback.
"""
from .kda import (KDA_BF16, KDA_F32, KDAError, kda_chunk_fwd, kda_chunk_fwd_chunk64,
                  kda_chunk_fwd_gated, kda_chunk_fwd_gated_fuses, kda_chunk_fwd_snapshots,
                  kda_chunk_fwd_split, kda_chunk_fwd_split_noalloc, kda_chunk_fwd_split_segments,
                  kda_chunk_fwd_split_workspace_bytes, kda_decode_step, kda_decode_step_gated,
                  kda_decode_step_layer, kda_frontend, kda_output_gate, kda_status_string,
                  load_library)

__all__ = ["KDA_BF16", "KDA_F32", "KDAError", "kda_chunk_fwd", "kda_chunk_fwd_chunk64",
           "kda_chunk_fwd_gated", "kda_chunk_fwd_gated_fuses", "kda_chunk_fwd_snapshots",
           "kda_chunk_fwd_split", "kda_chunk_fwd_split_noalloc", "kda_chunk_fwd_split_segments",
           "kda_chunk_fwd_split_workspace_bytes", "kda_decode_step", "kda_decode_step_gated",
           "kda_decode_step_layer", "kda_frontend", "kda_output_gate", "kda_status_string",
           "load_library"]
