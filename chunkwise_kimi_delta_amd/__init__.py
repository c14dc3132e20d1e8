"""MI355X (gfx950) chunkwise Kimi Delta Attention: HIP kernels behind a C ABI.

The Python surface mirrors the C ABI names in include/kda.h:
``kda_chunk_fwd``, ``kda_segment_summary``, ``kda_summary_merge``,
``kda_recurrent_fwd``.
"""
from .kda import (KdaError, kda_chunk_fwd, kda_chunk_offsets_host, kda_recurrent_fwd,  # noqa: F401
                  kda_segment_summary, kda_summary_merge, load)
