"""kda_chunk_fwd_noalloc (fixed device scratch, no allocation) against
kda_chunk_fwd (caller workspace), through the C ABI: two calls in a row, the
second smaller, each compared bit for bit (the same kernels on the same
inputs)."""
import numpy as np
import pytest
import torch

import kda_synth as ks
from kda_synth.torch_io import flag_kwargs, to_torch

pytestmark = pytest.mark.gpu


def _pair(kda, p):
    t = to_torch(p)
    kw = flag_kwargs(p)
    args = (t["q"], t["k"], t["v"], t["g"], t["beta"])
    common = dict(scale=p.scale, A_log=t["A_log"], dt_bias=t["dt_bias"], cu_seqlens=t["cu"],
                  cu_seqlens_host=t["cu_host"], state_indices=t["state_indices"], **kw)
    cache = p.state_indices is not None
    h0a = t["h0"].clone() if t["h0"] is not None else None
    h0b = t["h0"].clone() if t["h0"] is not None else None
    o_ref, f_ref = kda.kda_chunk_fwd(*args, initial_state=h0a, **common)
    o = torch.empty_like(t["v"])
    f = None if cache else torch.empty_like(f_ref)
    o_na, f_na = kda.kda_chunk_fwd_noalloc(*args, o=o, final_state=f, initial_state=h0b, **common)
    torch.cuda.synchronize()
    assert o_na.data_ptr() == o.data_ptr()
    assert torch.equal(o_na, o_ref), (o_na.float() - o_ref.float()).abs().max()
    assert torch.equal(f_na, f_ref), (f_na - f_ref).abs().max()
    assert torch.isfinite(o_na.float()).all() and o_na.float().abs().max() > 0


def test_noalloc_matches_workspace_call_twice(gpu_lib):
    # first call: packed sequences with a state cache updated in place
    _pair(gpu_lib, ks.make("varlen", lens=[300, 70, 513, 1], H=4, cache_rows=6, n_invalid=1))
    # second, smaller call on the same scratch: one short BSND sequence
    _pair(gpu_lib, ks.make("layer", T=130, H=2))


def test_noalloc_rejects_oversize_problem(gpu_lib):
    p = ks.make("layer", T=64, H=1)
    t = to_torch(p)
    big = torch.empty((1, 8192, 32, 128), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.KdaError, match="fixed scratch"):
        gpu_lib.kda_chunk_fwd_noalloc(big, big, big, big, torch.empty((1, 8192, 32), dtype=torch.bfloat16,
                                      device="cuda"), o=torch.empty_like(big),
                                      A_log=torch.zeros(32, device="cuda"), gate_in_kernel=True)
    del t
