"""ctypes binding of the KDA C ABI (include/kda.h).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libkda_mi355x.so``.  PyTorch provides device memory and the
current stream.  If the library is missing the calls raise; there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

# KDA_LIBRARY selects another build of the same ABI (the host sanitizer build
# of the validation code is one).
LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                         "libkda_mi355x.so")

KDA_OK, KDA_ERR_INVALID_ARGUMENT, KDA_ERR_UNSUPPORTED, KDA_ERR_WORKSPACE_TOO_SMALL, KDA_ERR_HIP = range(5)
KDA_F32, KDA_BF16 = 0, 1
KDA_LAYOUT_BSND, KDA_LAYOUT_TND = 0, 1
KDA_GATE_IN_KERNEL, KDA_SAFE_GATE, KDA_QK_L2NORM, KDA_BETA_SIGMOID = 1, 2, 4, 8
CHUNK = 64


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"KDA status {status}: {message}")
        self.status = status


class KdaProblem(ctypes.Structure):
    _fields_ = [("layout", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("B", ctypes.c_int32), ("T", ctypes.c_int32),
                ("Hk", ctypes.c_int32), ("Hv", ctypes.c_int32),
                ("K", ctypes.c_int32), ("V", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("flags", ctypes.c_uint32),
                ("scale", ctypes.c_float), ("eps", ctypes.c_float), ("lower_bound", ctypes.c_float),
                ("num_seqs", ctypes.c_int32),
                ("cu_seqlens_host", ctypes.POINTER(ctypes.c_int32)),
                ("state_rows", ctypes.c_int32), ("scan_segments", ctypes.c_int32)]


_lib = None
EXPORTS = ("kda_chunk_fwd_workspace_size", "kda_chunk_fwd", "kda_chunk_bwd_workspace_size", "kda_chunk_bwd",
           "kda_segment_summary_bwd_workspace_size", "kda_segment_summary_bwd", "kda_summary_merge_bwd",
           "kda_segment_summary_workspace_size",
           "kda_segment_summary", "kda_summary_merge", "kda_recurrent_fwd", "kda_chunk_fwd_noalloc",
           "kda_chunk_offsets_host",
           "kda_status_string", "kda_last_error", "kda_abi_version")
ABI_VERSION = 2
STAGE_EVENTS = 3


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (once); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m chunkwise_kimi_delta_amd.build`")
    lib = ctypes.CDLL(path)
    P, VP, SZ, I32 = ctypes.POINTER(KdaProblem), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    lib.kda_chunk_fwd_workspace_size.argtypes = [P, ctypes.POINTER(SZ)]
    lib.kda_segment_summary_workspace_size.argtypes = [P, ctypes.POINTER(SZ)]
    lib.kda_chunk_fwd.argtypes = [P] + [VP] * 13 + [SZ, VP, VP]
    lib.kda_segment_summary.argtypes = [P] + [VP] * 10 + [SZ, VP, VP]
    lib.kda_summary_merge.argtypes = [I32, I32, I32, I32, VP, VP, VP, VP]
    lib.kda_recurrent_fwd.argtypes = [P] + [VP] * 12 + [VP]
    lib.kda_chunk_fwd_noalloc.argtypes = [P] + [VP] * 12 + [VP]
    lib.kda_chunk_bwd_workspace_size.argtypes = [P, ctypes.POINTER(SZ)]
    lib.kda_chunk_bwd.argtypes = [P] + [VP] * 20 + [SZ, VP]
    lib.kda_segment_summary_bwd_workspace_size.argtypes = [P, ctypes.POINTER(SZ)]
    lib.kda_segment_summary_bwd.argtypes = [P] + [VP] * 11 + [SZ, VP]
    lib.kda_summary_merge_bwd.argtypes = [I32, I32, I32, I32, VP, VP, VP, VP]
    lib.kda_chunk_offsets_host.argtypes = [VP, I32, I32, VP]
    lib.kda_status_string.argtypes = [I32]
    lib.kda_status_string.restype = ctypes.c_char_p
    lib.kda_last_error.argtypes = []
    lib.kda_last_error.restype = ctypes.c_char_p
    lib.kda_abi_version.argtypes = []
    lib.kda_abi_version.restype = I32
    for name in ("kda_chunk_fwd_workspace_size", "kda_chunk_fwd", "kda_chunk_bwd_workspace_size",
                 "kda_chunk_bwd", "kda_segment_summary_bwd_workspace_size", "kda_segment_summary_bwd",
                 "kda_summary_merge_bwd", "kda_segment_summary_workspace_size",
                 "kda_segment_summary", "kda_summary_merge", "kda_recurrent_fwd", "kda_chunk_fwd_noalloc",
                 "kda_chunk_offsets_host"):
        getattr(lib, name).restype = I32
    if lib.kda_abi_version() != ABI_VERSION:
        raise RuntimeError(f"{path} has ABI version {lib.kda_abi_version()}, expected {ABI_VERSION}: rebuild it")
    _lib = lib
    return lib


def _check(status: int):
    if status != KDA_OK:
        lib = load()
        raise KdaError(status, f"{lib.kda_status_string(status).decode()}: {lib.kda_last_error().decode()}")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise TypeError(f"token tensors must be bf16 or fp32, got {t.dtype}")


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _need(t: Optional[torch.Tensor], name: str, dtype=None, shape=None, device=None):
    """Shape, dtype, layout and device of one tensor argument: the C ABI sees
    only pointers, so a wrong size here would become an out-of-bounds access."""
    if t is None:
        return
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _gpu_device(v: torch.Tensor) -> torch.device:
    if v.device.type != "cuda":
        raise ValueError(f"tensors must be on a GPU device, got {v.device}")
    return v.device


def _events(stage_events):
    if stage_events is None:
        return None
    ev = list(stage_events)
    if len(ev) != STAGE_EVENTS:
        raise ValueError(f"stage_events needs {STAGE_EVENTS} entries")
    return (ctypes.c_void_p * STAGE_EVENTS)(*ev)


def make_problem(q_or_k: torch.Tensor, v: torch.Tensor, *, scale: float, flags: int, eps: float,
                 lower_bound: float, cu_host: Optional[torch.Tensor], state_rows: int = 0,
                 scan_segments: int = 0):
    """Fill the C problem descriptor from tensor shapes (BSND if 4-D, TND if 3-D)."""
    if q_or_k.dim() == 4:
        B, T, Hk, K = q_or_k.shape
        layout, N, cu_ptr = KDA_LAYOUT_BSND, B, None
    elif q_or_k.dim() == 3:
        if cu_host is None:
            raise ValueError("3-D (TND) token tensors need cu_seqlens")
        T, Hk, K = q_or_k.shape
        B, layout, N = 1, KDA_LAYOUT_TND, cu_host.numel() - 1
        cu_ptr = ctypes.cast(cu_host.data_ptr(), ctypes.POINTER(ctypes.c_int32))
    else:
        raise ValueError("token tensors are [B,T,H,D] or [T,H,D]")
    Hv, V = v.shape[-2], v.shape[-1]
    p = KdaProblem(layout, _dtype_code(v), B, T, Hk, Hv, K, V, CHUNK, flags, scale, eps, lower_bound,
                   N, cu_ptr, state_rows, scan_segments)
    return p, N


def _cu_pair(cu_seqlens, cu_seqlens_host, device, tokens: torch.Tensor):
    """Device and host copies of cu_seqlens (int32); only 3-D (TND) token
    tensors take them."""
    if tokens.dim() == 4:
        if cu_seqlens is not None or cu_seqlens_host is not None:
            raise ValueError("4-D (BSND) token tensors take no cu_seqlens")
        return None, None
    if cu_seqlens is None:
        raise ValueError("3-D (TND) token tensors need cu_seqlens")
    cu_h = cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens.detach().to("cpu")
    cu_h = cu_h.to(torch.int32).contiguous()
    if cu_h.device.type != "cpu":
        raise ValueError("cu_seqlens_host must be a CPU tensor")
    if cu_seqlens.dim() != 1 or cu_h.dim() != 1 or cu_seqlens.numel() != cu_h.numel() or cu_h.numel() < 1:
        raise ValueError("cu_seqlens and its host copy must be 1-D of the same length N+1 >= 1")
    cu_d = cu_seqlens if cu_seqlens.device == device else cu_h.to(device)
    cu_d = cu_d.to(torch.int32).contiguous()
    return cu_d, cu_h


def _forward_args(q, k, v, g, beta, *, scale, A_log, dt_bias, initial_state, cu_seqlens,
                  cu_seqlens_host, state_indices, output_final_state, gate_in_kernel, safe_gate,
                  lower_bound, qk_l2norm, beta_sigmoid, eps, o, final_state, scan_segments=0,
                  alloc_o=True):
    """Checks and marshalling shared by the forward calls: every tensor's shape,
    dtype, layout and device, then the problem descriptor and the outputs."""
    if q.dim() not in (3, 4) or v.dim() != q.dim():
        raise ValueError("token tensors are [B,T,H,D] or [T,H,D], q and v alike")
    lead, Hk, K = tuple(q.shape[:-2]), q.shape[-2], q.shape[-1]
    Hv, V = v.shape[-2], v.shape[-1]
    cache = state_indices is not None
    _need(k, "k", None, q.shape)
    _need(v, "v", None, lead + (Hv, V))
    _need(g, "g", None, lead + (Hv, K))
    _need(beta, "beta", None, lead + (Hv,))
    _need(A_log, "A_log", torch.float32, (Hv,))
    _need(dt_bias, "dt_bias", torch.float32, (Hv, K))
    if gate_in_kernel and A_log is None:
        raise ValueError("gate_in_kernel needs A_log")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta")):
        _need(t, n, v.dtype)
    if q.dim() == 4:
        if cu_seqlens is not None or cu_seqlens_host is not None:
            raise ValueError("4-D (BSND) token tensors take no cu_seqlens")
        N = q.shape[0]
    else:
        if cu_seqlens is None:
            raise ValueError("3-D (TND) token tensors need cu_seqlens")
        if cu_seqlens_host is not None and cu_seqlens_host.numel() != cu_seqlens.numel():
            raise ValueError("cu_seqlens and its host copy must be 1-D of the same length N+1 >= 1")
        N = cu_seqlens.numel() - 1
    if cache:
        if initial_state is None or initial_state.dim() != 4 or initial_state.shape[0] < 1:
            raise ValueError("state_indices needs the state cache [rows,Hv,K,V] as initial_state")
        rows = initial_state.shape[0]
        _need(initial_state, "initial_state", torch.float32, (rows, Hv, K, V))
        _need(state_indices, "state_indices", None, (N,))
        _need(final_state, "final_state", torch.float32, (rows, Hv, K, V))
    else:
        rows = 0
        _need(initial_state, "initial_state", torch.float32, (N, Hv, K, V))
        _need(final_state, "final_state", torch.float32, (N, Hv, K, V))
    _need(o, "o", v.dtype, v.shape)
    dev = _gpu_device(v)
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (g, "g"), (beta, "beta"), (A_log, "A_log"),
                 (dt_bias, "dt_bias"), (initial_state, "initial_state"), (final_state, "final_state"),
                 (o, "o")):
        _need(t, n, device=dev)
    cu_d, cu_h = _cu_pair(cu_seqlens, cu_seqlens_host, dev, q)
    if scale is None:
        scale = K ** -0.5
    flags = ((KDA_GATE_IN_KERNEL if gate_in_kernel else 0) | (KDA_SAFE_GATE if safe_gate else 0)
             | (KDA_QK_L2NORM if qk_l2norm else 0) | (KDA_BETA_SIGMOID if beta_sigmoid else 0))
    p, N = make_problem(q, v, scale=scale, flags=flags, eps=eps, lower_bound=lower_bound,
                        cu_host=cu_h, state_rows=rows, scan_segments=scan_segments)
    if o is None and alloc_o:
        o = torch.empty(v.shape, dtype=v.dtype, device=dev)
    if cache:
        si = state_indices.to(device=dev, dtype=torch.int32).contiguous()
        if final_state is None and output_final_state:
            final_state = initial_state
    else:
        si = None
        if final_state is None and output_final_state:
            final_state = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev)
    return p, dev, cu_d, si, o, final_state


def kda_chunk_fwd(q, k, v, g, beta, *, scale: Optional[float] = None, A_log=None, dt_bias=None,
                  initial_state=None, cu_seqlens=None, cu_seqlens_host=None, state_indices=None,
                  output_final_state: bool = True, gate_in_kernel: bool = False,
                  safe_gate: bool = False, lower_bound: float = -5.0, qk_l2norm: bool = False,
                  beta_sigmoid: bool = False, eps: float = 1e-6, o=None, final_state=None,
                  workspace=None, stage_events=None, scan_segments: int = 0
                  ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunkwise KDA forward.  Returns (o, final_state).

    With ``state_indices`` the ``initial_state`` is a state cache
    [rows,Hv,K,V]; final states are scattered into ``final_state`` (default:
    the same cache, in place) and that cache is returned.  ``stage_events``:
    three raw hipEvent_t handles the call records at its stage boundaries.
    ``scan_segments``: 0 lets the library choose the segment-parallel scan,
    1 turns it off, n > 1 cuts each sequence into at most n segments.
    """
    lib = load()
    p, dev, cu_d, si, o, final_state = _forward_args(
        q, k, v, g, beta, scale=scale, A_log=A_log, dt_bias=dt_bias, initial_state=initial_state,
        cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, state_indices=state_indices,
        output_final_state=output_final_state, gate_in_kernel=gate_in_kernel, safe_gate=safe_gate,
        lower_bound=lower_bound, qk_l2norm=qk_l2norm, beta_sigmoid=beta_sigmoid, eps=eps, o=o,
        final_state=final_state, scan_segments=scan_segments)
    ws_bytes = ctypes.c_size_t()
    _check(lib.kda_chunk_fwd_workspace_size(ctypes.byref(p), ctypes.byref(ws_bytes)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes.value, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check(lib.kda_chunk_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(cu_d), _ptr(si),
                             _ptr(o), _ptr(final_state), _ptr(workspace), workspace.numel(),
                             _stream(dev), _events(stage_events)))
    return o, final_state


NOALLOC_SCRATCH_BYTES = 64 << 20


def kda_chunk_fwd_noalloc(q, k, v, g, beta, *, o, final_state=None, scale: Optional[float] = None,
                          A_log=None, dt_bias=None, initial_state=None, cu_seqlens=None,
                          cu_seqlens_host=None, state_indices=None, gate_in_kernel: bool = False,
                          safe_gate: bool = False, lower_bound: float = -5.0, qk_l2norm: bool = False,
                          beta_sigmoid: bool = False, eps: float = 1e-6, scan_segments: int = 0):
    """``kda_chunk_fwd`` without a workspace: the library's fixed device scratch
    serves instead (problems needing more than NOALLOC_SCRATCH_BYTES are
    rejected).  The outputs are the caller's (``o`` required; ``final_state``
    optional, or the cache itself in cache mode), so nothing is allocated.
    Calls that overlap on one GPU share the scratch and race."""
    lib = load()
    p, dev, cu_d, si, o, final_state = _forward_args(
        q, k, v, g, beta, scale=scale, A_log=A_log, dt_bias=dt_bias, initial_state=initial_state,
        cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, state_indices=state_indices,
        output_final_state=state_indices is not None, gate_in_kernel=gate_in_kernel,
        safe_gate=safe_gate, lower_bound=lower_bound, qk_l2norm=qk_l2norm, beta_sigmoid=beta_sigmoid,
        eps=eps, o=o, final_state=final_state, scan_segments=scan_segments)
    _check(lib.kda_chunk_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                     _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(cu_d),
                                     _ptr(si), _ptr(o), _ptr(final_state), _stream(dev)))
    return o, final_state


def kda_chunk_bwd(q, k, v, g, beta, do, *, dht=None, scale: Optional[float] = None, A_log=None,
                  dt_bias=None, initial_state=None, cu_seqlens=None, cu_seqlens_host=None,
                  gate_in_kernel: bool = False, safe_gate: bool = False, lower_bound: float = -5.0,
                  qk_l2norm: bool = False, beta_sigmoid: bool = False, eps: float = 1e-6,
                  workspace=None) -> dict:
    """Gradients of sum(do * o) + sum(dht * final_state) for the forward with
    the same arguments (dense initial states).  Returns fp32 tensors: dq, dk
    (shape of q / k), dv, dg (w.r.t. g as passed), dbeta (w.r.t. beta as
    passed), and dA_log / ddt_bias (with the in-kernel gate) and dh0 (with an
    initial state)."""
    lib = load()
    p, dev, cu_d, _, _, _ = _forward_args(
        q, k, v, g, beta, scale=scale, A_log=A_log, dt_bias=dt_bias, initial_state=initial_state,
        cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, state_indices=None,
        output_final_state=False, gate_in_kernel=gate_in_kernel, safe_gate=safe_gate,
        lower_bound=lower_bound, qk_l2norm=qk_l2norm, beta_sigmoid=beta_sigmoid, eps=eps, o=None,
        final_state=None, alloc_o=False)
    N, Hv, K, V = p.num_seqs, v.shape[-2], q.shape[-1], v.shape[-1]
    _need(do, "do", v.dtype, v.shape, dev)
    _need(dht, "dht", torch.float32, (N, Hv, K, V), dev)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty(q.shape, **f32), dk=torch.empty(k.shape, **f32), dv=torch.empty(v.shape, **f32),
               dg=torch.empty(g.shape, **f32), dbeta=torch.empty(beta.shape, **f32))
    if gate_in_kernel:
        out["dA_log"] = torch.empty((Hv,), **f32)
        if dt_bias is not None:
            out["ddt_bias"] = torch.empty((Hv, K), **f32)
    if initial_state is not None:
        out["dh0"] = torch.empty((N, Hv, K, V), **f32)
    ws_bytes = ctypes.c_size_t()
    _check(lib.kda_chunk_bwd_workspace_size(ctypes.byref(p), ctypes.byref(ws_bytes)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes.value, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check(lib.kda_chunk_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(A_log),
                             _ptr(dt_bias), _ptr(initial_state), _ptr(cu_d), _ptr(do), _ptr(dht),
                             _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                             _ptr(out["dbeta"]), _ptr(out.get("dA_log")), _ptr(out.get("ddt_bias")),
                             _ptr(out.get("dh0")), _ptr(workspace), workspace.numel(), _stream(dev)))
    return out


def kda_segment_summary_bwd(q, k, v, g, beta, do, *, scale: Optional[float] = None, A_log=None,
                            dt_bias=None, cu_seqlens=None, cu_seqlens_host=None,
                            gate_in_kernel: bool = False, safe_gate: bool = False, lower_bound: float = -5.0,
                            qk_l2norm: bool = False, beta_sigmoid: bool = False, eps: float = 1e-6,
                            local=None, workspace=None) -> torch.Tensor:
    """Backward summary: the gradient of sum(do * o) with respect to each
    sequence's initial state when nothing flows in from its final state
    (fp32 [N,Hv,K,V])."""
    lib = load()
    p, dev, cu_d, _, _, _ = _forward_args(
        q, k, v, g, beta, scale=scale, A_log=A_log, dt_bias=dt_bias, initial_state=None,
        cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, state_indices=None,
        output_final_state=False, gate_in_kernel=gate_in_kernel, safe_gate=safe_gate,
        lower_bound=lower_bound, qk_l2norm=qk_l2norm, beta_sigmoid=beta_sigmoid, eps=eps, o=None,
        final_state=None, alloc_o=False)
    N, Hv, K, V = p.num_seqs, v.shape[-2], q.shape[-1], v.shape[-1]
    _need(do, "do", v.dtype, v.shape, dev)
    _need(local, "local", torch.float32, (N, Hv, K, V), dev)
    if local is None:
        local = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev)
    ws_bytes = ctypes.c_size_t()
    _check(lib.kda_segment_summary_bwd_workspace_size(ctypes.byref(p), ctypes.byref(ws_bytes)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes.value, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check(lib.kda_segment_summary_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                       _ptr(A_log), _ptr(dt_bias), _ptr(cu_d), _ptr(do), _ptr(local),
                                       _ptr(workspace), workspace.numel(), _stream(dev)))
    return local


def kda_summary_merge_bwd(M: torch.Tensor, local: torch.Tensor, state: torch.Tensor) -> torch.Tensor:
    """In place: state <- M[j]^T state + local[j] for j from the last to the first.  Returns ``state``."""
    lib = load()
    if state.dim() != 3 or local.dim() != 4:
        raise ValueError("state is [Hv,K,V] and local [P,Hv,K,V]")
    Hv, K, V = state.shape
    P = local.shape[0]
    _need(local, "local", torch.float32, (P, Hv, K, V))
    _need(M, "M", torch.float32, (P, Hv, K, K))
    dev = _gpu_device(state)
    for t, n in ((M, "M"), (local, "local"), (state, "state")):
        _need(t, n, torch.float32, device=dev)
    _check(lib.kda_summary_merge_bwd(P, Hv, K, V, _ptr(M), _ptr(local), _ptr(state), _stream(state.device)))
    return state


def kda_recurrent_fwd(q, k, v, g, beta, *, scale: Optional[float] = None, A_log=None, dt_bias=None,
                      initial_state=None, cu_seqlens=None, cu_seqlens_host=None, state_indices=None,
                      output_final_state: bool = True, gate_in_kernel: bool = False,
                      safe_gate: bool = False, lower_bound: float = -5.0, qk_l2norm: bool = False,
                      beta_sigmoid: bool = False, eps: float = 1e-6, o=None, final_state=None
                      ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Token-by-token KDA forward (decode: a few tokens per sequence, the state
    cache updated in place).  Same arguments and results as ``kda_chunk_fwd``;
    no workspace."""
    lib = load()
    p, dev, cu_d, si, o, final_state = _forward_args(
        q, k, v, g, beta, scale=scale, A_log=A_log, dt_bias=dt_bias, initial_state=initial_state,
        cu_seqlens=cu_seqlens, cu_seqlens_host=cu_seqlens_host, state_indices=state_indices,
        output_final_state=output_final_state, gate_in_kernel=gate_in_kernel, safe_gate=safe_gate,
        lower_bound=lower_bound, qk_l2norm=qk_l2norm, beta_sigmoid=beta_sigmoid, eps=eps, o=o,
        final_state=final_state)
    _check(lib.kda_recurrent_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                 _ptr(A_log), _ptr(dt_bias), _ptr(initial_state), _ptr(cu_d), _ptr(si),
                                 _ptr(o), _ptr(final_state), _stream(dev)))
    return o, final_state


def kda_segment_summary(k, v, g, beta, *, A_log=None, dt_bias=None, cu_seqlens=None,
                        cu_seqlens_host=None, gate_in_kernel: bool = False, safe_gate: bool = False,
                        lower_bound: float = -5.0, qk_l2norm: bool = False,
                        beta_sigmoid: bool = False, eps: float = 1e-6, M=None, S_tilde=None,
                        workspace=None, stage_events=None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Per-sequence affine summary (M [N,Hv,K,K], S~ [N,Hv,K,V]), fp32."""
    lib = load()
    if k.dim() not in (3, 4) or v.dim() != k.dim():
        raise ValueError("token tensors are [B,T,H,D] or [T,H,D], k and v alike")
    lead, K = tuple(k.shape[:-2]), k.shape[-1]
    Hv, V = v.shape[-2], v.shape[-1]
    _need(v, "v", None, lead + (Hv, V))
    _need(g, "g", None, lead + (Hv, K))
    _need(beta, "beta", None, lead + (Hv,))
    _need(A_log, "A_log", torch.float32, (Hv,))
    _need(dt_bias, "dt_bias", torch.float32, (Hv, K))
    if gate_in_kernel and A_log is None:
        raise ValueError("gate_in_kernel needs A_log")
    for t, n in ((k, "k"), (v, "v"), (g, "g"), (beta, "beta")):
        _need(t, n, v.dtype)
    dev = _gpu_device(v)
    for t, n in ((k, "k"), (v, "v"), (g, "g"), (beta, "beta")):
        _need(t, n, device=dev)
    _need(A_log, "A_log", device=dev)
    _need(dt_bias, "dt_bias", device=dev)
    cu_d, cu_h = _cu_pair(cu_seqlens, cu_seqlens_host, dev, k)
    flags = ((KDA_GATE_IN_KERNEL if gate_in_kernel else 0) | (KDA_SAFE_GATE if safe_gate else 0)
             | (KDA_QK_L2NORM if qk_l2norm else 0) | (KDA_BETA_SIGMOID if beta_sigmoid else 0))
    p, N = make_problem(k, v, scale=1.0, flags=flags, eps=eps, lower_bound=lower_bound, cu_host=cu_h)
    K, V, Hv = k.shape[-1], v.shape[-1], v.shape[-2]
    _need(M, "M", torch.float32, (N, Hv, K, K), dev)
    _need(S_tilde, "S_tilde", torch.float32, (N, Hv, K, V), dev)
    if M is None:
        M = torch.empty((N, Hv, K, K), dtype=torch.float32, device=dev)
    if S_tilde is None:
        S_tilde = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev)
    ws_bytes = ctypes.c_size_t()
    _check(lib.kda_segment_summary_workspace_size(ctypes.byref(p), ctypes.byref(ws_bytes)))
    if workspace is None:
        workspace = torch.empty(max(ws_bytes.value, 256), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, None, dev)
    _check(lib.kda_segment_summary(ctypes.byref(p), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                   _ptr(A_log), _ptr(dt_bias), _ptr(cu_d), _ptr(M), _ptr(S_tilde),
                                   _ptr(workspace), workspace.numel(), _stream(dev),
                                   _events(stage_events)))
    return M, S_tilde


def kda_summary_merge(M: torch.Tensor, S_tilde: torch.Tensor, state: torch.Tensor) -> torch.Tensor:
    """In place: state <- M[j] state + S_tilde[j] for j in order.  Returns ``state``."""
    lib = load()
    if state.dim() != 3 or S_tilde.dim() != 4:
        raise ValueError("state is [Hv,K,V] and S_tilde [P,Hv,K,V]")
    Hv, K, V = state.shape
    P = S_tilde.shape[0]
    _need(S_tilde, "S_tilde", torch.float32, (P, Hv, K, V))
    _need(M, "M", torch.float32, (P, Hv, K, K))
    dev = _gpu_device(state)
    for t, n in ((M, "M"), (S_tilde, "S_tilde"), (state, "state")):
        _need(t, n, torch.float32, device=dev)
    _check(lib.kda_summary_merge(P, Hv, K, V, _ptr(M), _ptr(S_tilde), _ptr(state),
                                 _stream(state.device)))
    return state


def kda_chunk_offsets_host(cu_seqlens_host: torch.Tensor, chunk: int = CHUNK) -> torch.Tensor:
    """First chunk index of each packed sequence, plus the total, computed by the library."""
    lib = load()
    cu = cu_seqlens_host.to(torch.int32).contiguous()
    out = torch.empty(cu.numel(), dtype=torch.int32)
    _check(lib.kda_chunk_offsets_host(cu.data_ptr(), cu.numel() - 1, chunk, out.data_ptr()))
    return out


def workspace_bytes(q_or_k: torch.Tensor, v: torch.Tensor, cu_seqlens_host=None, summary: bool = False,
                    scan_segments: int = 0) -> int:
    """Device workspace bytes a forward (or summary) call needs for these shapes."""
    lib = load()
    cu = None if cu_seqlens_host is None else cu_seqlens_host.to(torch.int32).contiguous()
    p, _ = make_problem(q_or_k, v, scale=1.0, flags=0, eps=0.0, lower_bound=0.0, cu_host=cu,
                        scan_segments=scan_segments)
    sz = ctypes.c_size_t()
    fn = lib.kda_segment_summary_workspace_size if summary else lib.kda_chunk_fwd_workspace_size
    _check(fn(ctypes.byref(p), ctypes.byref(sz)))
    return sz.value
