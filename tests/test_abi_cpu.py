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
    assert lib.kda_abi_version() == kda.ABI_VERSION == 2


def test_binding_argument_counts_match_the_header(lib):
    """Every function the header declares is bound with exactly as many
    argument types as it has parameters (a missing one makes ctypes pass the
    trailing arguments with the wrong width)."""
    src = open(os.path.join(ROOT, "include", "kda.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    decls = re.findall(r"\b(kda_[a-z_]+)\s*\(([^;{]*?)\)\s*;", src, flags=re.S)
    assert len(decls) == len(kda.EXPORTS)
    for name, params in decls:
        params = params.strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        bound = getattr(lib, name).argtypes
        assert bound is not None and len(bound) == n, (name, n, bound)


def _problem(**kw):
    d = dict(layout=0, dtype=1, B=1, T=8192, Hk=32, Hv=32, K=128, V=128, chunk_size=64, flags=15,
             scale=128 ** -0.5, eps=1e-6, lower_bound=-5.0, num_seqs=1, cu_seqlens_host=None,
             state_rows=0, scan_segments=0)
    d.update(kw)
    return kda.KdaProblem(*[d[f] for f, _ in kda.KdaProblem._fields_])


def test_segment_plan_grows_the_workspace_only_when_it_splits(lib):
    """The layer (32 heads x 8 tiles = 256 scans) fills the GPU: no split, the
    plain workspace.  Few heads on a long sequence: the library splits (the
    summaries, their prefixes and the incoming states join the workspace);
    scan_segments = 1 turns that off and n > 1 forces it."""
    _, plain = _ws(lib, _problem())
    assert _ws(lib, _problem(scan_segments=1))[1] == plain
    _, few = _ws(lib, _problem(Hk=2, Hv=2, T=65536))
    _, few_off = _ws(lib, _problem(Hk=2, Hv=2, T=65536, scan_segments=1))
    assert few > few_off
    seg_bytes = 2 * 16 * 128 * (128 + 2 * 128) * 4          # 16 segments x 2 heads
    assert few - few_off >= seg_bytes
    _, forced = _ws(lib, _problem(scan_segments=3))
    assert forced > plain


def test_noalloc_rejects_problems_beyond_its_scratch_before_any_device_access(lib):
    """The layer problem needs ~395 MB of workspace, beyond the 64 MiB scratch:
    the call fails closed on the host (fake pointers are never touched)."""
    p = _problem()
    fake = 0x1000
    st = lib.kda_chunk_fwd_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None,
                                   None, None, fake, None, None)
    assert st == kda.KDA_ERR_UNSUPPORTED and b"fixed scratch" in lib.kda_last_error()
    assert kda.NOALLOC_SCRATCH_BYTES == 64 << 20


def test_fp32_tokens_at_k128_are_in_the_envelope(lib):
    st, b = _ws(lib, _problem(dtype=0))
    assert st == 0 and b > 0
    st, _ = _ws(lib, _problem(dtype=0, flags=15 | 2, lower_bound=0.0))   # floor 0 is allowed
    assert st == 0


def _ws(lib, p, summary=False):
    sz = ctypes.c_size_t()
    fn = lib.kda_segment_summary_workspace_size if summary else lib.kda_chunk_fwd_workspace_size
    st = fn(ctypes.byref(p), ctypes.byref(sz))
    return st, sz.value


def test_workspace_size_layer_and_monotone(lib):
    st, b = _ws(lib, _problem())
    assert st == 0
    # One record per (head, chunk): w, qg (bf16 64x128), kg^T (fp16 128x64), Aqk (fp16
    # 64x64), the chunk decay (fp32 128) and u (fp16 64x128).
    per = 64 * 128 * 2 * 2 + 128 * 64 * 2 + 64 * 64 * 2 + 128 * 4 + 128 * 64 * 2
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
    (dict(dtype=0, K=96), kda.KDA_ERR_UNSUPPORTED),      # fp32 with an unbuilt K
    (dict(flags=15 | 2, lower_bound=0.5), kda.KDA_ERR_INVALID_ARGUMENT),   # safe-gate floor > 0
    (dict(flags=15 | 2, lower_bound=float("-inf")), kda.KDA_ERR_INVALID_ARGUMENT),
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
    (dict(scan_segments=-1), kda.KDA_ERR_INVALID_ARGUMENT),
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
    st = lib.kda_chunk_fwd(ctypes.byref(p), *([None] * 13), 0, None, None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT            # q/k/v... are NULL
    # misaligned pointers are rejected before any device access
    fake = 0x1000
    st = lib.kda_chunk_fwd(ctypes.byref(p), fake + 2, fake, fake, fake, fake, fake, None, None,
                           None, None, fake, None, fake, 1 << 40, None, None)
    assert st == kda.KDA_ERR_INVALID_ARGUMENT and b"aligned" in lib.kda_last_error()
    st = lib.kda_chunk_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None,
                           None, None, fake, None, fake, 10, None, None)
    assert st == kda.KDA_ERR_WORKSPACE_TOO_SMALL
    # the gate bias is read 16 bytes at a time: a misaligned one is rejected
    for fn in (lambda: lib.kda_chunk_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake + 4, None,
                                         None, None, fake, None, fake, 1 << 40, None, None),
               lambda: lib.kda_recurrent_fwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, fake + 4,
                                             None, None, None, fake, None, None)):
        assert fn() == kda.KDA_ERR_INVALID_ARGUMENT and b"dt_bias" in lib.kda_last_error()
    # the backward writes dq, dk and dg 16 bytes at a time: misaligned ones are rejected
    for bad in range(3):
        outs = [fake] * 5
        outs[(0, 1, 3)[bad]] = fake + 4
        st = lib.kda_chunk_bwd(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None, None, None, fake, None,
                               *outs, None, None, None, fake, 1 << 40, None)
        assert st == kda.KDA_ERR_INVALID_ARGUMENT and (b"dq", b"dk", b"dg")[bad] in lib.kda_last_error()
    # an empty selection (N = 0) launches nothing and succeeds
    p0, keep = _tnd([0])
    sz = ctypes.c_size_t()
    assert lib.kda_chunk_fwd_workspace_size(ctypes.byref(p0), ctypes.byref(sz)) == 0
    st = lib.kda_chunk_fwd(ctypes.byref(p0), None, None, None, None, None, fake, None, None,
                           fake, None, None, None, fake, sz.value, None, None)
    assert st == 0, lib.kda_last_error()
    assert lib.kda_summary_merge(1, 32, 128, 96, fake, fake, fake, None) == kda.KDA_ERR_UNSUPPORTED
    assert lib.kda_summary_merge(-1, 32, 128, 128, fake, fake, fake, None) == kda.KDA_ERR_INVALID_ARGUMENT
    assert lib.kda_summary_merge(0, 32, 128, 128, None, None, fake, None) == 0   # P = 0: nothing to do
    for s in range(5):
        assert lib.kda_status_string(s)


# ------------------------------------------------- binding argument checks
def _cpu_layer(B=1, T=70, Hk=2, Hv=4, K=64, V=64, dtype=torch.bfloat16):
    z = lambda *s: torch.zeros(*s, dtype=dtype)
    return dict(q=z(B, T, Hk, K), k=z(B, T, Hk, K), v=z(B, T, Hv, V), g=z(B, T, Hv, K),
                beta=z(B, T, Hv), A_log=torch.zeros(Hv), dt_bias=torch.zeros(Hv, K))


def _fwd(t, **kw):
    return kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], A_log=t["A_log"],
                             dt_bias=t["dt_bias"], gate_in_kernel=True, **kw)


@pytest.mark.parametrize("name,bad,err", [
    ("k", torch.zeros(1, 70, 1, 64, dtype=torch.bfloat16), ValueError),    # fewer q/k heads than q
    ("v", torch.zeros(1, 70, 4, 64, dtype=torch.bfloat16)[:, :69], ValueError),
    ("g", torch.zeros(1, 70, 4, 32, dtype=torch.bfloat16), ValueError),
    ("beta", torch.zeros(1, 70, 2, dtype=torch.bfloat16), ValueError),
    ("A_log", torch.zeros(3), ValueError),
    ("dt_bias", torch.zeros(4, 64, dtype=torch.float64), TypeError),
    ("g", torch.zeros(1, 70, 4, 64, dtype=torch.float32), TypeError),       # dtype differs from v
])
def test_binding_rejects_wrong_shapes_and_dtypes(lib, name, bad, err):
    t = _cpu_layer()
    t[name] = bad
    with pytest.raises(err):
        _fwd(t)


def test_binding_rejects_wrong_state_shapes(lib):
    t = _cpu_layer()
    with pytest.raises(ValueError, match="initial_state"):
        _fwd(t, initial_state=torch.zeros(2, 4, 64, 64))                    # N = 1, not 2
    with pytest.raises(ValueError, match="final_state"):
        _fwd(t, final_state=torch.zeros(1, 2, 64, 64))
    with pytest.raises(ValueError, match="o has shape"):
        _fwd(t, o=torch.zeros(1, 70, 4, 32, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="state_indices"):
        _fwd(t, initial_state=torch.zeros(5, 4, 64, 64), state_indices=torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match="cu_seqlens"):
        _fwd(t, cu_seqlens=torch.tensor([0, 70], dtype=torch.int32))         # BSND takes none


def test_binding_rejects_host_tensors_before_the_library_call(lib):
    """Well-shaped CPU tensors fail on the device check: no pointer reaches the library."""
    t = _cpu_layer()
    with pytest.raises(ValueError, match="GPU device"):
        _fwd(t)
    with pytest.raises(ValueError, match="GPU device"):
        kda.kda_segment_summary(t["k"], t["v"], t["g"], t["beta"], A_log=t["A_log"], gate_in_kernel=True)
    with pytest.raises(ValueError, match="GPU device"):
        kda.kda_summary_merge(torch.zeros(2, 4, 64, 64), torch.zeros(2, 4, 64, 64), torch.zeros(4, 64, 64))
    with pytest.raises(ValueError, match="M has shape"):
        kda.kda_summary_merge(torch.zeros(2, 4, 64, 32), torch.zeros(2, 4, 64, 64), torch.zeros(4, 64, 64))


def test_binding_tnd_needs_matching_cu_seqlens(lib):
    z = lambda *s: torch.zeros(*s, dtype=torch.bfloat16)
    t = dict(q=z(70, 2, 64), k=z(70, 2, 64), v=z(70, 2, 64), g=z(70, 2, 64), beta=z(70, 2),
             A_log=torch.zeros(2), dt_bias=None)
    with pytest.raises(ValueError, match="cu_seqlens"):
        _fwd(t)
    with pytest.raises(ValueError, match="same length"):
        _fwd(t, cu_seqlens=torch.tensor([0, 70], dtype=torch.int32),
             cu_seqlens_host=torch.tensor([0, 30, 70], dtype=torch.int32))
