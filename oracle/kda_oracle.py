"""fp64 CPU oracle for the Kimi Delta Attention (KDA) forward, summary and merge.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the graft smoke check and the
benchmark's CPU-baseline leg may import this module.  The product library
never calls it, links it or falls back to it.

It computes the plain definition, not the chunked algorithm:

* KDA is a gated delta rule with a per-channel decay.  Per token t, with the
  state S (K x V), decay alpha_t = exp(g_t) (one factor per key channel),
  write strength beta_t, key k_t and value v_t:
      S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T,
      o_t = scale * S_t^T q_t.
  The chunked form (64-token chunks with WY factors) reaches exactly this
  result ("KDA Chunk Backward — TPU/Pallas Kernel Design", section 1 and 1.2;
  "Hyper-Parallel Chunk KDA", section 7, which tests every stage against a CPU
  recurrence).  The oracle therefore runs the token recurrence, written as
  "decay, then correct the value the decayed state predicts, then write":
      S' = Diag(alpha_t) S;  S = S' + beta_t k_t (v_t - S'^T k_t)^T.
* Gate, L2Norm and beta activation follow the fused-interface parameters of
  "Hyper-Parallel Chunk KDA", section 4 and 4.1: g = -exp(A_log[h]) *
  softplus(g_raw + dt_bias[h, :]), optionally clamped below at lower_bound
  (safe gate); q and k divided by sqrt(sum x^2 + eps); beta = sigmoid(b).
* Grouped heads: value head h reads query/key head h // (Hv / Hk)
  ("Hyper-Parallel Chunk KDA", section 4.2).
* Packed sequences reset the state at every sequence start ("Hyper-Parallel
  Chunk KDA", section 6.5).  In cache mode the initial state of sequence n is
  cache row idx[n] when 0 <= idx[n] < rows, else zero; its final state is
  written back to that row only when the index is valid (vllm-ascend KDA
  prefill state copy page, numeric-contract and addressing sections).
* Segment summary: S~ is the state reached from a zero state; M is the
  ordered product of the per-token transitions (I - beta k k^T) Diag(alpha),
  later tokens on the left, i.e. the same recurrence with v = 0 started from
  the identity.  Then any incoming state X leaves the segment as M X + S~
  ("KDA Context Parallelism (KCP)", notation and composition sections;
  "Hyper-Parallel 支持 Gated DeltaNet Context Parallel", section 6.4).
* Merge: S <- M_j S + S~_j for the preceding segments j in time order,
  starting from zero or from a given state ("KDA Context Parallelism (KCP)",
  algorithm step 4).

Pins (what ties these functions to the pages and to mathematics rather than
to themselves) live in ``tests/test_oracle_pins.py``: closed forms for beta=0
and for linear attention with orthonormal keys, last-write-wins, a scalar
closed form, brute-force matrix products at tiny sizes, linearity, L2Norm
scale invariance, gate closed forms, packed == separate runs, grouped heads ==
repeated heads, the summary identities (affinity, split invariance,
non-commutativity, M not droppable); the in-kernel preprocessing route of
``forward`` and ``segment_summary`` (gate, safe-gate clamp, sigmoid, L2Norm,
per-head parameters, grouped heads) against the bare recurrence fed inputs
prepared element by element with the scalar math library; and the ``heads=``
and ``t_max=`` subsets against slices of the full run.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

F64 = np.float64


# ---------------------------------------------------------------- activations
def softplus(x: np.ndarray) -> np.ndarray:
    """log(1 + e^x) in fp64, evaluated without overflow."""
    x = np.asarray(x, dtype=F64)
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def sigmoid(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=F64)
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def kimi_gate(g_raw: np.ndarray, A_log: np.ndarray, dt_bias: Optional[np.ndarray],
              safe_gate: bool = False, lower_bound: float = -5.0) -> np.ndarray:
    """Natural-log decay from the raw gate: -exp(A_log[h]) * softplus(g_raw + dt_bias[h]).

    ``g_raw`` has shape [..., H, K]; A_log [H]; dt_bias [H, K] or None (zero).
    With the safe gate the result is clamped below at ``lower_bound``.
    ("Hyper-Parallel Chunk KDA", section 4: use_gate_in_kernel, a_log,
    dt_bias, safe_gate, lower_bound.)
    """
    x = np.asarray(g_raw, dtype=F64)
    if dt_bias is not None:
        x = x + np.asarray(dt_bias, dtype=F64)
    g = -np.exp(np.asarray(A_log, dtype=F64))[:, None] * softplus(x)
    if safe_gate:
        g = np.maximum(g, lower_bound)
    return g


def l2norm(x: np.ndarray, eps: float = 1e-6) -> np.ndarray:
    """x / sqrt(sum(x^2) + eps) over the last axis ("Hyper-Parallel Chunk KDA", 4.1)."""
    x = np.asarray(x, dtype=F64)
    return x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


# ------------------------------------------------------------------ recurrence
def recurrence(k: np.ndarray, v: np.ndarray, g: np.ndarray, beta: np.ndarray,
               S0: np.ndarray, q: Optional[np.ndarray] = None, scale: float = 1.0
               ) -> Tuple[Optional[np.ndarray], np.ndarray]:
    """Token-by-token KDA recurrence for one sequence, all heads at once.

    k [T,H,K], v [T,H,V], g [T,H,K] (natural log), beta [T,H], S0 [H,K,V],
    q [T,H,K] or None.  Returns (o [T,H,V] or None, S_T [H,K,V]), fp64.
    """
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    alpha = np.exp(np.asarray(g, F64))
    beta = np.asarray(beta, F64)
    S = np.array(S0, dtype=F64, copy=True)
    T = k.shape[0]
    o = None if q is None else np.zeros(v.shape, F64)
    qq = None if q is None else np.asarray(q, F64)
    for t in range(T):
        S *= alpha[t][:, :, None]                                   # Diag(alpha_t) S
        pred = np.einsum("hkv,hk->hv", S, k[t])                      # S'^T k_t
        S += beta[t][:, None, None] * k[t][:, :, None] * (v[t] - pred)[:, None, :]
        if o is not None:
            o[t] = scale * np.einsum("hkv,hk->hv", S, qq[t])          # scale S_t^T q_t
    return o, S


# ------------------------------------------------------------- full problems
def _prepared(q, k, g, beta, *, Hv, gate_in_kernel, safe_gate, lower_bound, l2norm_on,
              beta_sigmoid, eps, A_log, dt_bias):
    """Apply the in-kernel preprocessing the flags ask for and expand grouped heads."""
    Hk = k.shape[-2]
    rep = Hv // Hk
    kk = l2norm(k, eps) if l2norm_on else np.asarray(k, F64)
    qq = None
    if q is not None:
        qq = l2norm(q, eps) if l2norm_on else np.asarray(q, F64)
    if rep > 1:
        kk = np.repeat(kk, rep, axis=-2)
        if qq is not None:
            qq = np.repeat(qq, rep, axis=-2)
    if gate_in_kernel:
        gg = kimi_gate(g, A_log, dt_bias, safe_gate, lower_bound)
    else:
        gg = np.asarray(g, F64)
        if safe_gate:
            gg = np.maximum(gg, lower_bound)
    bb = sigmoid(beta) if beta_sigmoid else np.asarray(beta, F64)
    return qq, kk, gg, bb


def _seq_slices(layout, B, T, cu_seqlens):
    if layout == "tnd":
        cu = np.asarray(cu_seqlens)
        return [(None, int(cu[n]), int(cu[n + 1])) for n in range(len(cu) - 1)]
    return [(b, 0, T) for b in range(B)]


def forward(p, heads: Optional[Sequence[int]] = None, t_max: Optional[int] = None):
    """KDA forward of a whole problem (attributes as in ``kda_synth.Problem``).

    Returns (o, final) in fp64: o has the problem's v layout with Hv heads;
    final is [N,Hv,K,V] (or the updated cache [rows,Hv,K,V] in cache mode).
    ``heads`` restricts the computation to a subset of value heads (o and
    final keep full shape, other heads stay zero / cache-unchanged); ``t_max``
    stops each sequence after that many tokens (sampled checks of long runs).
    """
    Hv, K, V = p.Hv, p.K, p.V
    hs = list(range(Hv)) if heads is None else list(heads)
    rep = Hv // p.Hk
    kh_idx = [h // rep for h in hs]
    o = np.zeros(p.v.shape, F64)
    seqs = _seq_slices(p.layout, p.B, p.T, p.cu_seqlens)
    cache = p.state_indices is not None
    if cache:
        final = np.array(p.h0, dtype=F64, copy=True)
    else:
        final = np.zeros((len(seqs), Hv, K, V), F64)
    for n, (b, t0, t1) in enumerate(seqs):
        if t_max is not None:
            t1 = min(t1, t0 + t_max)
        sl = (b, slice(t0, t1)) if b is not None else (slice(t0, t1),)
        q = None if p.q is None else p.q[sl][:, kh_idx]
        k = p.k[sl][:, kh_idx]
        v = p.v[sl][:, hs]
        g = p.g[sl][:, hs]
        beta = p.beta[sl][:, hs]
        A_log = None if p.A_log is None else p.A_log[hs]
        dt_bias = None if p.dt_bias is None else p.dt_bias[hs]
        qq, kk, gg, bb = _prepared(q, k, g, beta, Hv=len(hs) * 1, gate_in_kernel=p.gate_in_kernel,
                                   safe_gate=p.safe_gate, lower_bound=p.lower_bound,
                                   l2norm_on=p.l2norm, beta_sigmoid=p.beta_sigmoid, eps=p.eps,
                                   A_log=A_log, dt_bias=dt_bias)
        if cache:
            r = int(p.state_indices[n])
            valid = 0 <= r < p.h0.shape[0]
            S0 = np.array(p.h0[r][hs], F64) if valid else np.zeros((len(hs), K, V), F64)
        else:
            valid = True
            S0 = np.zeros((len(hs), K, V), F64) if p.h0 is None else np.array(p.h0[n][hs], F64)
        oo, S = recurrence(kk, v, gg, bb, S0, q=qq, scale=p.scale)
        if oo is not None:
            if b is not None:
                o[b, t0:t1][:, hs] = oo
            else:
                o[t0:t1][:, hs] = oo
        if cache:
            if valid:
                final[r][hs] = S
        else:
            final[n][hs] = S
    return o, final


def segment_summary(p, heads: Optional[Sequence[int]] = None):
    """Per-sequence affine summary (M [N,Hv,K,K], S~ [N,Hv,K,V]) of a problem.

    S~ is the state reached from zero; M is the transition product, computed
    by running the recurrence with v = 0 from the identity.
    """
    Hv, K, V = p.Hv, p.K, p.V
    hs = list(range(Hv)) if heads is None else list(heads)
    rep = Hv // p.Hk
    kh_idx = [h // rep for h in hs]
    seqs = _seq_slices(p.layout, p.B, p.T, p.cu_seqlens)
    M = np.zeros((len(seqs), Hv, K, K), F64)
    St = np.zeros((len(seqs), Hv, K, V), F64)
    for n, (b, t0, t1) in enumerate(seqs):
        sl = (b, slice(t0, t1)) if b is not None else (slice(t0, t1),)
        k = p.k[sl][:, kh_idx]
        v = p.v[sl][:, hs]
        g = p.g[sl][:, hs]
        beta = p.beta[sl][:, hs]
        A_log = None if p.A_log is None else p.A_log[hs]
        dt_bias = None if p.dt_bias is None else p.dt_bias[hs]
        _, kk, gg, bb = _prepared(None, k, g, beta, Hv=len(hs), gate_in_kernel=p.gate_in_kernel,
                                  safe_gate=p.safe_gate, lower_bound=p.lower_bound,
                                  l2norm_on=p.l2norm, beta_sigmoid=p.beta_sigmoid, eps=p.eps,
                                  A_log=A_log, dt_bias=dt_bias)
        _, S = recurrence(kk, v, gg, bb, np.zeros((len(hs), K, V), F64))
        eye = np.broadcast_to(np.eye(K, dtype=F64), (len(hs), K, K)).copy()
        _, Mn = recurrence(kk, np.zeros((kk.shape[0], len(hs), K), F64), gg, bb, eye)
        St[n][hs] = S
        M[n][hs] = Mn
    return M, St


def summary_merge(M: np.ndarray, S_tilde: np.ndarray, state: Optional[np.ndarray] = None
                  ) -> np.ndarray:
    """S <- M_j S + S~_j for j = 0..P-1 in time order (M [P,H,K,K], S~ [P,H,K,V])."""
    M = np.asarray(M, F64)
    S_tilde = np.asarray(S_tilde, F64)
    S = np.zeros(S_tilde.shape[1:], F64) if state is None else np.array(state, F64)
    for j in range(M.shape[0]):
        S = np.matmul(M[j], S) + S_tilde[j]
    return S


# ------------------------------------------------------------------ compare
def compare(x: np.ndarray, ref: np.ndarray) -> dict:
    """err_max = max|x - ref| / max|ref|, rel_l2 and the non-finite count."""
    x = np.asarray(x, F64)
    ref = np.asarray(ref, F64)
    den = max(float(np.max(np.abs(ref))) if ref.size else 0.0, 1e-30)
    d = np.abs(x - ref)
    nrm = float(np.linalg.norm(ref))
    return dict(err_max=float(np.max(d)) / den if d.size else 0.0,
                rel_l2=float(np.linalg.norm(x - ref)) / max(nrm, 1e-30),
                nonfinite=int((~np.isfinite(x)).sum()))


# ------------------------------------------------------------------ backward
def recurrence_bwd(k, v, g, beta, S0, q, scale, do, dST, ckpt=64):
    """Adjoint of ``recurrence`` for one sequence, all heads at once, fp64.

    Forward per token (decay, correct the decayed state's prediction, write,
    read):  S' = Diag(alpha) S;  e = v - S'^T k;  S = S' + beta k e^T;
    o = scale S^T q,  alpha = exp(g).  Given do [T,H,V] = dL/do and
    dST [H,K,V] = dL/dS_T (None = 0), walks the tokens backwards and returns
    (dq [T,H,K], dk [T,H,K], dv [T,H,V], dg [T,H,K], dbeta [T,H], dS0 [H,K,V]),
    the gradients with respect to the recurrence's own inputs (g natural-log
    decay, beta the write strength, q and k as used).  States are kept every
    ``ckpt`` tokens and the ones in between recomputed ("KDA Chunk Backward —
    TPU/Pallas Kernel Design", section 1.1: the backward recomputes forward
    quantities instead of storing them).
    """
    k = np.asarray(k, F64)
    v = np.asarray(v, F64)
    q = np.asarray(q, F64)
    g = np.asarray(g, F64)
    alpha = np.exp(g)
    beta = np.asarray(beta, F64)
    do = np.asarray(do, F64)
    T, H, K = k.shape
    V = v.shape[-1]
    # forward pass keeping the state at every checkpoint
    marks = {}
    S = np.array(S0, dtype=F64, copy=True)
    for t in range(T):
        if t % ckpt == 0:
            marks[t] = S.copy()
        S = _step(S, k[t], v[t], alpha[t], beta[t])
    dS = np.zeros((H, K, V), F64) if dST is None else np.array(dST, dtype=F64, copy=True)
    dq = np.zeros((T, H, K), F64)
    dk = np.zeros((T, H, K), F64)
    dv = np.zeros((T, H, V), F64)
    dg = np.zeros((T, H, K), F64)
    db = np.zeros((T, H), F64)
    for c0 in reversed(range(0, T, ckpt)):
        c1 = min(T, c0 + ckpt)
        states = [marks[c0]]                         # states[i] = S before token c0 + i
        for t in range(c0, c1):
            states.append(_step(states[-1], k[t], v[t], alpha[t], beta[t]))
        for t in reversed(range(c0, c1)):
            Sp = states[t - c0]                       # S_{t-1}
            Sd = alpha[t][:, :, None] * Sp            # S' = Diag(alpha) S_{t-1}
            pred = np.einsum("hkv,hk->hv", Sd, k[t])
            e = v[t] - pred
            St = states[t - c0 + 1]
            # o_t = scale S_t^T q_t
            dq[t] = scale * np.einsum("hkv,hv->hk", St, do[t])
            dS = dS + scale * q[t][:, :, None] * do[t][:, None, :]
            # S_t = S' + beta k e^T
            db[t] = np.einsum("hk,hkv,hv->h", k[t], dS, e)
            de = beta[t][:, None] * np.einsum("hkv,hk->hv", dS, k[t])
            dk[t] = beta[t][:, None] * np.einsum("hkv,hv->hk", dS, e)
            # e = v - S'^T k
            dv[t] = de
            dSd = dS - k[t][:, :, None] * de[:, None, :]
            dk[t] -= np.einsum("hkv,hv->hk", Sd, de)
            # S' = Diag(alpha) S_{t-1}, alpha = exp(g)
            dg[t] = np.einsum("hkv,hkv->hk", dSd, Sp) * alpha[t]
            dS = alpha[t][:, :, None] * dSd
    return dq, dk, dv, dg, db, dS


def _step(S, k, v, alpha, beta):
    Sd = alpha[:, :, None] * S
    e = v - np.einsum("hkv,hk->hv", Sd, k)
    return Sd + beta[:, None, None] * k[:, :, None] * e[:, None, :]


def _l2norm_bwd(x, dy, eps):
    """Gradient of x / sqrt(sum x^2 + eps) (last axis) given dy."""
    x = np.asarray(x, F64)
    r = 1.0 / np.sqrt((x * x).sum(-1, keepdims=True) + eps)
    y = x * r
    return r * (dy - y * (y * dy).sum(-1, keepdims=True))


def backward(p, do, dht=None, heads: Optional[Sequence[int]] = None):
    """Gradients of a whole problem's forward (dense initial states; BSND or
    TND), fp64: dict with dq, dk (shape of p.q / p.k: grouped heads summed over
    their value heads), dv, dg (w.r.t. p.g: the raw gate with the in-kernel
    gate, else the natural-log decay), dbeta (w.r.t. p.beta: the logit with the
    in-kernel sigmoid), dA_log [Hv], ddt_bias [Hv, K] (in-kernel gate), dh0
    [N, Hv, K, V].  The loss is sum(do * o) + sum(dht * final_state).

    Per token the adjoint of the recurrence (``recurrence_bwd``); then the
    preprocessing of "Hyper-Parallel Chunk KDA", section 4: sigmoid'(b) =
    s(1 - s); the gate -exp(A_log) softplus(g + dt_bias) has derivative
    -exp(A_log) sigmoid(g + dt_bias) in g and dt_bias and itself in A_log, zero
    where the safe-gate clamp is active; L2Norm's derivative is
    r (dy - y (y . dy)).  ``heads`` restricts the work to those value heads
    (the other heads' gradients stay zero, and dq/dk receive only their share).
    """
    if p.state_indices is not None:
        raise ValueError("the backward takes dense initial states")
    Hv, K, V = p.Hv, p.K, p.V
    hs = list(range(Hv)) if heads is None else list(heads)
    rep = Hv // p.Hk
    kh_idx = [h // rep for h in hs]
    do = np.asarray(do, F64)
    seqs = _seq_slices(p.layout, p.B, p.T, p.cu_seqlens)
    out = dict(dq=np.zeros(p.q.shape, F64), dk=np.zeros(p.k.shape, F64), dv=np.zeros(p.v.shape, F64),
               dg=np.zeros(p.g.shape, F64), dbeta=np.zeros(p.beta.shape, F64),
               dA_log=np.zeros(Hv, F64), ddt_bias=np.zeros((Hv, K), F64),
               dh0=np.zeros((len(seqs), Hv, K, V), F64))
    for n, (b, t0, t1) in enumerate(seqs):
        sl = (b, slice(t0, t1)) if b is not None else (slice(t0, t1),)
        qr = np.asarray(p.q[sl][:, kh_idx], F64)
        kr = np.asarray(p.k[sl][:, kh_idx], F64)
        v = p.v[sl][:, hs]
        graw = np.asarray(p.g[sl][:, hs], F64)
        braw = np.asarray(p.beta[sl][:, hs], F64)
        qq = l2norm(qr, p.eps) if p.l2norm else qr
        kk = l2norm(kr, p.eps) if p.l2norm else kr
        bb = sigmoid(braw) if p.beta_sigmoid else braw
        if p.gate_in_kernel:
            z = graw + (0.0 if p.dt_bias is None else np.asarray(p.dt_bias, F64)[hs])
            g_act = -np.exp(np.asarray(p.A_log, F64)[hs])[:, None] * softplus(z)
        else:
            g_act = graw
        clamped = (g_act < p.lower_bound) if p.safe_gate else np.zeros(g_act.shape, bool)
        gg = np.where(clamped, p.lower_bound, g_act)
        S0 = np.zeros((len(hs), K, V), F64) if p.h0 is None else np.array(p.h0[n][hs], F64)
        dST = None if dht is None else np.asarray(dht, F64)[n][hs]
        dq, dk, dv, dgg, db, dS0 = recurrence_bwd(kk, v, gg, bb, S0, qq, p.scale, do[sl][:, hs], dST)
        if p.l2norm:
            dq = _l2norm_bwd(qr, dq, p.eps)
            dk = _l2norm_bwd(kr, dk, p.eps)
        dgg = np.where(clamped, 0.0, dgg)
        if p.gate_in_kernel:
            dz = dgg * -np.exp(np.asarray(p.A_log, F64)[hs])[:, None] * sigmoid(z)
            out["dA_log"][hs] += (dgg * g_act).sum(axis=(0, 2))
            if p.dt_bias is not None:
                out["ddt_bias"][hs] += dz.sum(axis=0)
            dgraw = dz
        else:
            dgraw = dgg
        dbraw = db * bb * (1.0 - bb) if p.beta_sigmoid else db
        tgt = (lambda name: out[name][b]) if b is not None else (lambda name: out[name])
        for j, h in enumerate(hs):
            tgt("dq")[t0:t1, kh_idx[j]] += dq[:, j]
            tgt("dk")[t0:t1, kh_idx[j]] += dk[:, j]
            tgt("dv")[t0:t1, h] = dv[:, j]
            tgt("dg")[t0:t1, h] = dgraw[:, j]
            tgt("dbeta")[t0:t1, h] = dbraw[:, j]
        out["dh0"][n][hs] = dS0
    return out


def segment_summary_bwd(p, do, heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Backward summary of each sequence: ``local`` [N, Hv, K, V], the gradient
    of sum(do * o) with respect to the sequence's initial state when nothing
    flows in from its final state.  The state gradient's recursion does not
    involve the states themselves, so the full gradient with respect to the
    initial state is affine in the final state's gradient dS_T:
        dS_0 = M^T dS_T + local,
    with M the forward summary's transition ("Hyper-Parallel Chunk KDA",
    sections 5.2 and 6.4: the backward pre-process and the reverse merge;
    "KDA Chunk Backward — TPU/Pallas Kernel Design", section 2.4)."""
    return backward(p, do, None, heads=heads)["dh0"]


def summary_merge_bwd(M: np.ndarray, local: np.ndarray, dstate: Optional[np.ndarray] = None
                      ) -> np.ndarray:
    """Reverse merge: S <- M_j^T S + local_j for j = P-1 down to 0, from the
    gradient of the last segment's final state (zero if None); the result is
    the gradient with respect to the first segment's initial state, and each
    intermediate value is the gradient a preceding segment receives for its
    final state (M [P,H,K,K], local [P,H,K,V])."""
    M = np.asarray(M, F64)
    local = np.asarray(local, F64)
    S = np.zeros(local.shape[1:], F64) if dstate is None else np.array(dstate, F64)
    for j in reversed(range(M.shape[0])):
        S = np.matmul(np.swapaxes(M[j], -1, -2), S) + local[j]
    return S
