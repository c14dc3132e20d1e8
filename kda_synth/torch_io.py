"""Move a ``kda_synth.Problem`` onto a torch device (no arithmetic of the method).

bf16 workloads hold bf16-exact float32 arrays, so the cast to torch.bfloat16
is lossless and the device sees exactly the values the oracle reads.
"""
from __future__ import annotations

import numpy as np
import torch


def to_torch(p, device="cuda") -> dict:
    dt = torch.bfloat16 if p.dtype == "bf16" else torch.float32

    def tok(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x)).to(device=device, dtype=dt)

    def f32(x):
        return None if x is None else torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)

    t = dict(q=tok(p.q), k=tok(p.k), v=tok(p.v), g=tok(p.g), beta=tok(p.beta),
             A_log=f32(p.A_log), dt_bias=f32(p.dt_bias), h0=f32(p.h0))
    if p.cu_seqlens is not None:
        t["cu_host"] = torch.from_numpy(np.ascontiguousarray(p.cu_seqlens, dtype=np.int32))
        t["cu"] = t["cu_host"].to(device)
    else:
        t["cu_host"] = t["cu"] = None
    t["state_indices"] = (None if p.state_indices is None else
                          torch.from_numpy(np.ascontiguousarray(p.state_indices, dtype=np.int32)).to(device))
    return t


def flag_kwargs(p) -> dict:
    """The problem's in-kernel preprocessing switches as binding keyword arguments."""
    return dict(gate_in_kernel=p.gate_in_kernel, safe_gate=p.safe_gate, lower_bound=p.lower_bound,
                qk_l2norm=p.l2norm, beta_sigmoid=p.beta_sigmoid, eps=p.eps)
