"""MI355X (gfx950) chunkwise Kimi Delta Attention: HIP kernels behind a C ABI.

The Python surface mirrors the C ABI names in include/kda.h:
``kda_chunk_fwd``, ``kda_segment_summary``, ``kda_summary_merge``,
``kda_recurrent_fwd``, ``kda_chunk_bwd``, ``kda_segment_summary_bwd``,
``kda_summary_merge_bwd``, ``kda_chunk_fwd_noalloc``.
"""
from .kda import (KdaError, kda_chunk_bwd, kda_chunk_fwd, kda_chunk_fwd_noalloc,  # noqa: F401
                  kda_chunk_offsets_host, kda_recurrent_fwd, kda_segment_summary, kda_segment_summary_bwd,
                  kda_summary_merge, kda_summary_merge_bwd, load)
