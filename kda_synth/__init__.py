"""Seeded synthetic inputs for chunkwise Kimi Delta Attention (KDA).

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the method's arithmetic: no gate activation, no L2Norm, no
sigmoid, no recurrence.  Both the fp64 CPU oracle (through the tests) and the
GPU library (through the tests and the benchmark) receive the very same
arrays from here.

Every workload is drawn from one ``numpy.random.Generator(PCG64(seed))``, in
a fixed order (q, k, v, gate input, beta input, A_log, dt_bias, states,
indices, lengths, extras).  Values are drawn in float32 and rounded to bf16
(round-to-nearest-even) on the CPU where the workload stores bf16, so the
float32 arrays returned hold exactly the bits the GPU receives.

The five workloads mirror the shapes the KDA pages discuss: a tiny fp32
check, a Kimi-Linear-shaped layer (H=32, d=128, T=8192), a packed varlen
prefill with a state cache, one segment of a 1M-token sequence split eight
ways, and a GQA long batch.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = ["Problem", "bf16_round", "make", "WORKLOADS", "preceding_summary_inputs"]


def bf16_round(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32.

    NaN stays NaN.  The result is exactly representable in bf16, so a later
    ``torch.tensor(..., dtype=torch.bfloat16)`` conversion is lossless.
    """
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32).copy()
    nan = np.isnan(a)
    if nan.any():
        out[nan] = np.float32("nan")
    return out.reshape(a.shape)


@dataclass
class Problem:
    """One KDA forward problem.  Arrays are float32 (bf16-exact when dtype=='bf16').

    Layout ``bsnd``: q,k [B,T,Hk,K]; v [B,T,Hv,V]; g [B,T,Hv,K]; beta [B,T,Hv].
    Layout ``tnd``: the same without the B axis, with ``cu_seqlens`` [N+1].
    ``g`` holds the raw gate input when ``gate_in_kernel`` is set, else the
    natural-log decay itself.  ``beta`` holds the raw logit when
    ``beta_sigmoid`` is set, else beta itself.
    """
    name: str
    layout: str
    dtype: str
    B: int
    T: int
    Hk: int
    Hv: int
    K: int
    V: int
    q: Optional[np.ndarray]
    k: np.ndarray
    v: np.ndarray
    g: np.ndarray
    beta: np.ndarray
    scale: float
    gate_in_kernel: bool = False
    safe_gate: bool = False
    lower_bound: float = -5.0
    l2norm: bool = False
    beta_sigmoid: bool = False
    eps: float = 1e-6
    A_log: Optional[np.ndarray] = None
    dt_bias: Optional[np.ndarray] = None
    h0: Optional[np.ndarray] = None          # [N,Hv,K,V] or cache [rows,Hv,K,V]
    cu_seqlens: Optional[np.ndarray] = None  # int32 [N+1] (tnd)
    state_indices: Optional[np.ndarray] = None  # int32 [N] (cache mode)
    extras: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.cu_seqlens) - 1 if self.layout == "tnd" else self.B

    @property
    def cache_mode(self) -> bool:
        return self.state_indices is not None

    def seq_bounds(self):
        """(batch index, token start, token end) per sequence."""
        if self.layout == "tnd":
            cu = self.cu_seqlens
            return [(0, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
        return [(b, 0, self.T) for b in range(self.B)]


def _normal(rng, shape, std=1.0):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)).astype(np.float32)


def _store(x, dtype):
    return bf16_round(x) if dtype == "bf16" else np.ascontiguousarray(x, dtype=np.float32)


def _kimi_gate_params(rng, Hv, K):
    # A_log uniform in log space on [log 1, log 16]; dt_bias ~ N(0, 0.1^2).
    A_log = rng.uniform(0.0, math.log(16.0), size=(Hv,)).astype(np.float32)
    dt_bias = _normal(rng, (Hv, K), 0.1)
    return A_log, dt_bias


def make_tiny(seed=1000, T=256, K=64, V=64, normalized_qk=True, preactivated_beta=True) -> Problem:
    """B=1, H=1, T=256, dk=dv=64, fp32; precomputed natural-log gate; zero h0.

    ``normalized_qk``: q,k are L2-normalised per token by the harness and the
    in-kernel L2Norm is off; otherwise raw q,k with in-kernel L2Norm.
    ``preactivated_beta``: beta = sigmoid(N(0,1)) given directly; otherwise
    the raw logit with in-kernel sigmoid.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    shp = (1, T, 1)
    q = _normal(rng, shp + (K,))
    k = _normal(rng, shp + (K,))
    v = _normal(rng, shp + (V,))
    graw = _normal(rng, shp + (K,))
    braw = _normal(rng, shp)
    # Input recipe (not the method's gate): g = -softplus(x) * 0.1.
    g = (-np.logaddexp(0.0, graw.astype(np.float64)) * 0.1).astype(np.float32)
    if normalized_qk:
        q = (q / np.sqrt((q.astype(np.float64) ** 2).sum(-1, keepdims=True))).astype(np.float32)
        k = (k / np.sqrt((k.astype(np.float64) ** 2).sum(-1, keepdims=True))).astype(np.float32)
    if preactivated_beta:
        beta = (1.0 / (1.0 + np.exp(-braw.astype(np.float64)))).astype(np.float32)
    else:
        beta = braw
    return Problem(name="tiny", layout="bsnd", dtype="f32", B=1, T=T, Hk=1, Hv=1, K=K, V=V,
                   q=q, k=k, v=v, g=g, beta=beta, scale=1.0 / math.sqrt(K),
                   l2norm=not normalized_qk, beta_sigmoid=not preactivated_beta)


def make_layer(seed=1001, B=1, T=8192, H=32, K=128, V=128, dtype="bf16", h0_std=0.02) -> Problem:
    """Kimi-Linear-shaped layer: in-kernel gate, L2Norm and sigmoid; fp32 h0."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _store(_normal(rng, (B, T, H, K)), dtype)
    k = _store(_normal(rng, (B, T, H, K)), dtype)
    v = _store(_normal(rng, (B, T, H, V)), dtype)
    g = _store(_normal(rng, (B, T, H, K)), dtype)
    b = _store(_normal(rng, (B, T, H)), dtype)
    A_log, dt_bias = _kimi_gate_params(rng, H, K)
    h0 = _normal(rng, (B, H, K, V), h0_std) if h0_std else None
    return Problem(name="layer", layout="bsnd", dtype=dtype, B=B, T=T, Hk=H, Hv=H, K=K, V=V,
                   q=q, k=k, v=v, g=g, beta=b, scale=1.0 / math.sqrt(K),
                   gate_in_kernel=True, l2norm=True, beta_sigmoid=True,
                   A_log=A_log, dt_bias=dt_bias, h0=h0)


def make_varlen(seed=1002, n_seqs=16, min_len=512, max_len=8192, H=32, K=128, V=128,
                dtype="bf16", cache_rows=64, n_invalid=2, lens=None) -> Problem:
    """Packed TND prefill with a state cache gathered/scattered by index.

    ``lens`` overrides the drawn sequence lengths (zero-length sequences allowed).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    if lens is None:
        lens = rng.integers(min_len, max_len + 1, size=n_seqs)
    else:
        lens = np.asarray(lens, dtype=np.int64)
        n_seqs = len(lens)
    cu = np.zeros(n_seqs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    q = _store(_normal(rng, (T, H, K)), dtype)
    k = _store(_normal(rng, (T, H, K)), dtype)
    v = _store(_normal(rng, (T, H, V)), dtype)
    g = _store(_normal(rng, (T, H, K)), dtype)
    b = _store(_normal(rng, (T, H)), dtype)
    A_log, dt_bias = _kimi_gate_params(rng, H, K)
    cache = _normal(rng, (cache_rows, H, K, V), 0.02)
    idx = rng.permutation(cache_rows)[:n_seqs].astype(np.int32)
    if n_invalid:
        bad = rng.choice(n_seqs, size=n_invalid, replace=False)
        idx[bad] = -1
    return Problem(name="varlen", layout="tnd", dtype=dtype, B=1, T=T, Hk=H, Hv=H, K=K, V=V,
                   q=q, k=k, v=v, g=g, beta=b, scale=1.0 / math.sqrt(K),
                   gate_in_kernel=True, l2norm=True, beta_sigmoid=True,
                   A_log=A_log, dt_bias=dt_bias, h0=cache, cu_seqlens=cu, state_indices=idx)


def make_segment(seed=1003, T=131072, H=32, K=128, V=128, dtype="bf16", n_prev=7,
                 factors_per_prev=16) -> Problem:
    """One segment of a long sequence: its own tokens plus the raw draws for the
    preceding segments' summaries (see ``preceding_summary_inputs``)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _store(_normal(rng, (1, T, H, K)), dtype)
    k = _store(_normal(rng, (1, T, H, K)), dtype)
    v = _store(_normal(rng, (1, T, H, V)), dtype)
    g = _store(_normal(rng, (1, T, H, K)), dtype)
    b = _store(_normal(rng, (1, T, H)), dtype)
    A_log, dt_bias = _kimi_gate_params(rng, H, K)
    # Preceding summaries: the transition of each is the product of
    # `factors_per_prev` delta-rule factors drawn here (raw keys, raw beta
    # logits and natural-log decays -softplus(N(0,1))*0.1); S~ ~ N(0, 0.02^2).
    n_f = n_prev * factors_per_prev
    pk = _store(_normal(rng, (n_f, H, K)), dtype)
    pb = _store(_normal(rng, (n_f, H)), dtype)
    pg = _store((-np.logaddexp(0.0, _normal(rng, (n_f, H, K)).astype(np.float64)) * 0.1)
                .astype(np.float32), dtype)
    pS = _normal(rng, (n_prev, H, K, V), 0.02)
    extras = dict(prev_k=pk, prev_beta=pb, prev_g=pg, prev_S=pS, n_prev=n_prev,
                  factors_per_prev=factors_per_prev)
    return Problem(name="segment", layout="bsnd", dtype=dtype, B=1, T=T, Hk=H, Hv=H, K=K, V=V,
                   q=q, k=k, v=v, g=g, beta=b, scale=1.0 / math.sqrt(K),
                   gate_in_kernel=True, l2norm=True, beta_sigmoid=True,
                   A_log=A_log, dt_bias=dt_bias, h0=None, extras=extras)


def preceding_summary_inputs(p: Problem) -> Problem:
    """The preceding segments' factor draws as a packed problem (v = 0).

    Each preceding segment j is a sequence of ``factors_per_prev`` tokens
    whose zero-value summary transition is the ordered product of its
    delta-rule factors.  Returned in TND layout with the segment's dtype, precomputed gate,
    raw keys with L2Norm on and raw beta logits with sigmoid on.
    """
    ex = p.extras
    n, f = ex["n_prev"], ex["factors_per_prev"]
    H, K, V = p.Hv, p.K, p.V
    cu = (np.arange(n + 1, dtype=np.int32) * f).astype(np.int32)
    z = np.zeros((n * f, H, V), dtype=np.float32)
    return Problem(name="segment-prev", layout="tnd", dtype=p.dtype, B=1, T=n * f, Hk=H, Hv=H,
                   K=K, V=V, q=None, k=ex["prev_k"], v=z, g=ex["prev_g"], beta=ex["prev_beta"],
                   scale=p.scale, l2norm=True, beta_sigmoid=True, cu_seqlens=cu)


def make_gqa(seed=1004, B=4, T=16384, Hk=16, Hv=64, K=128, V=128, dtype="bf16") -> Problem:
    """GQA long batch: Hk q/k heads shared by Hv/Hk value heads; safe gate on."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = _store(_normal(rng, (B, T, Hk, K)), dtype)
    k = _store(_normal(rng, (B, T, Hk, K)), dtype)
    v = _store(_normal(rng, (B, T, Hv, V)), dtype)
    g = _store(_normal(rng, (B, T, Hv, K)), dtype)
    b = _store(_normal(rng, (B, T, Hv)), dtype)
    A_log, dt_bias = _kimi_gate_params(rng, Hv, K)
    h0 = _normal(rng, (B, Hv, K, V), 0.02)
    return Problem(name="gqa", layout="bsnd", dtype=dtype, B=B, T=T, Hk=Hk, Hv=Hv, K=K, V=V,
                   q=q, k=k, v=v, g=g, beta=b, scale=1.0 / math.sqrt(K),
                   gate_in_kernel=True, safe_gate=True, l2norm=True, beta_sigmoid=True,
                   A_log=A_log, dt_bias=dt_bias, h0=h0)


def make_decode(seed=1005, n_seqs=64, tokens=1, H=32, K=128, V=128, dtype="bf16", cache_rows=128,
                n_invalid=2, lens=None) -> Problem:
    """Decode step after a prefill: ``tokens`` new tokens for each of ``n_seqs``
    sequences (TND), initial states gathered from a state cache by index and
    final states scattered back in place; the layer's gate, L2Norm and sigmoid.
    ``lens`` overrides the per-sequence token counts."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens = np.full(n_seqs, tokens, dtype=np.int64) if lens is None else np.asarray(lens, dtype=np.int64)
    n_seqs = len(lens)
    cu = np.zeros(n_seqs + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lens)
    T = int(cu[-1])
    q = _store(_normal(rng, (T, H, K)), dtype)
    k = _store(_normal(rng, (T, H, K)), dtype)
    v = _store(_normal(rng, (T, H, V)), dtype)
    g = _store(_normal(rng, (T, H, K)), dtype)
    b = _store(_normal(rng, (T, H)), dtype)
    A_log, dt_bias = _kimi_gate_params(rng, H, K)
    cache = _normal(rng, (cache_rows, H, K, V), 0.02)
    idx = rng.permutation(cache_rows)[:n_seqs].astype(np.int32)
    if n_invalid:
        bad = rng.choice(n_seqs, size=n_invalid, replace=False)
        idx[bad] = -1
    return Problem(name="decode", layout="tnd", dtype=dtype, B=1, T=T, Hk=H, Hv=H, K=K, V=V,
                   q=q, k=k, v=v, g=g, beta=b, scale=1.0 / math.sqrt(K),
                   gate_in_kernel=True, l2norm=True, beta_sigmoid=True,
                   A_log=A_log, dt_bias=dt_bias, h0=cache, cu_seqlens=cu, state_indices=idx)


def make_longseq(seed=1006, T=65536, H=4, **kw) -> Problem:
    """A long sequence over few heads (the layer's recipe): too few (head,
    column-tile) scans to occupy the GPU, the case for the segment-parallel scan."""
    p = make_layer(seed=seed, T=T, H=H, **kw)
    p.name = "longseq"
    return p


WORKLOADS = {
    "tiny": make_tiny,
    "layer": make_layer,
    "varlen": make_varlen,
    "segment": make_segment,
    "gqa": make_gqa,
    "decode": make_decode,
    "longseq": make_longseq,
}


def make(name: str, **kw) -> Problem:
    """Build a named workload; keyword overrides shrink it for quick tests."""
    return WORKLOADS[name](**kw)
