"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before launching anything."""
import ctypes
import os
import re

import pytest
import torch

from chunkwise_kimi_delta_amd import kda

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return kda.load()


def _declared():
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kda_[a-z_]+)\s*\(", src)))


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"kda_chunk_fwd", "kda_segment_summary", "kda_summary_merge"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(kda.EXPORTS)
    assert lib.kda_abi_version() == 1


def _problem(**kw):
    d = dict(layout=0, dtype=1, B=1, T=8192, Hk=32, Hv=32, K=128, V=128, chunk_size=64, flags=15,
             scale=128 ** -0.5, eps=1e-6, lower_bound=-5.0, num_seqs=1, cu_seqlens_host=None,
             state_rows=0)
    d.update(kw)
    return kda.KdaProblem(*[d[f] for f, _ in kda.KdaProblem._fields_])


def _ws(lib, p, summary=False):
    sz = ctypes.c_size_t()
    fn = lib.kda_segment_summary_workspace_size if summary else lib.kda_chunk_fwd_workspace_size
    st = fn(ctypes.byref(p), ctypes.byref(sz))
    return st, sz.value


def test_workspace_size_layer_and_monotone(lib):
    st, b = _ws(lib, _problem())
    assert st == 0
    # One record per (head, chunk): w, qg (bf16 64x128), kg^T hi (bf16 128x64) and lo
    # (e4m3 128x64), Aqk (bf16 64x64), the chunk decay (fp32 128) and u (fp32 64x128).
    per = 64 * 128 * 2 * 2 + 128 * 64 * 2 + 128 * 64 + 64 * 64 * 2 + 128 * 4 + 128 * 64 * 4
    assert b >= 32 * 128 * per and b < 32 * 128 * per + 8 * 256
    prev = 0
    for T in (0, 1, 64, 65, 1000, 8192):
        st, b = _ws(lib, _problem(T=T))
        assert st == 0 and b >= prev
        prev = b
    st, bs = _ws(lib, _problem(), summary=True)
    assert st == 0 and bs < _ws(lib, _problem())[1]


@pytest.mark.parametrize("kw,status", [
    (dict(chunk_size=32), kda.KDA_ERR_UNSUPPORTED),
    (dict(K=96), kda.KDA_ERR_UNSUPPORTED),
    (dict(V=256), kda.KDA_ERR_UNSUPPORTED),
    (dict(dtype=0), kda.KDA_ERR_UNSUPPORTED),            # fp32 with K=128
    (dict(dtype=7), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(layout=3), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(Hk=3), kda.KDA_ERR_INVALID_ARGUMENT),          # 32 % 3 != 0
    (dict(Hk=0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(flags=64), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(scale=float("nan")), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(eps=-1.0), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(num_seqs=2), kda.KDA_ERR_INVALID_ARGUMENT),    # BSND needs num_seqs == B
    (dict(T=-1), kda.KDA_ERR_INVALID_ARGUMENT),
    (dict(state_rows=-2), kda.KDA_ERR_INVALID_ARGUMENT),
])
def test_bad_descriptors_are_rejected(lib, kw, status):
    st, _ = _ws(lib, _problem(**kw))
    assert st == status, lib.kda_last_error()
    assert lib.kda_last_error()


def _tnd(cu):
    arr = (ctypes.c_int32 * len(cu))(*cu)
    p = _problem(layout=1, T=cu[-1], num_seqs=len(cu) - 1,
                 cu_seqlens_host=ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
    return p, arr


def test_tnd_cu_seqlens_validation(lib):
    p, keep = _tnd([0, 100, 100, 300])
    assert _ws(lib, p)[0] == 0                    # empty sequence allowed
    p, keep = _tnd([0, 100, 50, 300])
    assert _ws(lib, p)[0] == kda.KDA_ERR_INVALID_ARGUMENT
    p, keep = _tnd([1, 100])
    assert _ws(lib, p)[0] == kda.KDA_ERR_INVALID_ARGUMENT
    p, keep = _tnd([0, 100])
    p.T = 99
    assert _ws(lib, p)[0] == kda.KDA_ERR_INVALID_ARGUMENT


def test_chunk_map_matches_worked_example():
    """Two sequences of lengths 8 and 4 at chunk size 4 give chunks owned by
    sequences [1, 1, 2] ("KDA Chunk Backward — TPU/Pallas Kernel Design",
    section 3.8 worked example)."""
    off = kda.kda_chunk_offsets_host(torch.tensor([0, 8, 12], dtype=torch.int32), 4).tolist()
    assert off == [0, 2, 3]
    owner = [n + 1 for n in range(2) for _ in range(off[n + 1] - off[n])]
    assert owner == [1, 1, 2]
    # partial last chunk and empty sequences
    off = kda.kda_chunk_offsets_host(torch.tensor([0, 65, 65, 129, 130], dtype=torch.int32)).tolist()
    assert off == [0, 2, 2, 3, 4]


def test_calls_fail_closed_without_launching(lib):
    p = _problem(T=128)
    st = lib.kda_chunk_fwd(ctypes.byref(p), *([None] * 13), 0, None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT            # q/k/v... are NULL
    # misaligned pointers are rejected before any device access
    fake = 0x1000
    st = lib.kda_chunk_fwd(ctypes.byref(p), fake + 2, fake, fake, fake, fake, fake, None, None,
                           None, None, fake, None, fake, 1 << 40, None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT and b"aligned" in lib.kda_last_error()
    st = lib.kda_chunk_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None,
                           None, None, fake, None, fake, 10, None)
    assert st == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    assert lib.kda_summary_merge(1, 32, 128, 96, fake, fake, fake, None) == kda.KDA_ERR_UNSUPPORTED
    assert lib.kda_summary_merge(-1, 32, 128, 128, fake, fake, fake, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_summary_merge(0, 32, 128, 128, None, None, fake, None) == 0   # P = 0: nothing to do
    for s in range(5):
        assert lib.kda_status_string(s)
