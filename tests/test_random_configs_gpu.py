"""GPU parity over seeded random problem configurations.

Each case draws one combination of what the boundary accepts -- token dtype,
head dims, grouped heads, dense or packed layout with ragged and empty
sequences, in-kernel or precomputed gate (with and without the safe-gate
clamp, from slow to strong decay), in-kernel or given L2Norm and sigmoid,
no / dense / cached initial states, automatic or forced scan segments -- and
compares the forward (and, for dense states, the backward) with the fp64
oracle at the bars of the other parity tests.  The draws are printed before
each call, so a failing case names itself.
"""
import dataclasses
import math

import numpy as np
import pytest

import kda_synth as ks
from oracle import kda_oracle as orc
from test_backward_gpu import bwd_case
from test_parity_gpu import TOL_BF16_OUT, TOL_F32, TOL_STATE, check, np64, run_fwd, say

pytestmark = pytest.mark.gpu

N_FWD = 24
N_BWD = 10


def _rows(rng, shape, dtype, unit=False):
    x = rng.standard_normal(size=shape).astype(np.float32)
    if unit:
        x /= np.sqrt((x * x).sum(-1, keepdims=True) + 1e-6)
    return ks.bf16_round(x) if dtype == "bf16" else x


def random_problem(seed: int, dense_states: bool = False) -> ks.Problem:
    rng = np.random.default_rng(9000 + seed)
    dtype = "f32" if rng.random() < 0.3 else "bf16"
    K = int(rng.choice([64, 128]))
    V = int(rng.choice([64, 128]))
    Hk = int(rng.integers(1, 3))
    Hv = Hk * int(rng.choice([1, 2, 4]))
    packed = rng.random() < 0.5
    if packed:
        n = int(rng.integers(1, 5))
        lens = rng.integers(0, 151, size=n)
        if lens.sum() == 0:
            lens[0] = 1
        cu = np.zeros(n + 1, dtype=np.int32)
        cu[1:] = np.cumsum(lens)
        B, T, lead = 1, int(cu[-1]), (int(cu[-1]),)
    else:
        n = B = int(rng.integers(1, 3))
        T = int(rng.integers(1, 201))
        cu, lead = None, (B, T)
    l2 = bool(rng.random() < 0.5)
    q = _rows(rng, lead + (Hk, K), dtype, unit=not l2)
    k = _rows(rng, lead + (Hk, K), dtype, unit=not l2)
    v = _rows(rng, lead + (Hv, V), dtype)
    gate_in_kernel = bool(rng.random() < 0.6)
    A_log = dt_bias = None
    if gate_in_kernel:
        g = _rows(rng, lead + (Hv, K), dtype)
        lo = -3.0 if rng.random() < 0.3 else 0.0        # slow decays (A_log < 0) now and then
        A_log = rng.uniform(lo, math.log(16.0), size=(Hv,)).astype(np.float32)
        if rng.random() < 0.7:
            dt_bias = (rng.standard_normal(size=(Hv, K)) * 0.1).astype(np.float32)
    else:
        s = float(rng.choice([0.02, 0.3, 3.0]))           # per-token decay from slow to strong
        x = rng.standard_normal(size=lead + (Hv, K))
        g = (-np.logaddexp(0.0, x) * s).astype(np.float32)
        g = ks.bf16_round(g) if dtype == "bf16" else g
    safe_gate = bool(rng.random() < 0.3)
    lower_bound = float(rng.choice([-5.0, -2.0]))
    beta_sigmoid = bool(rng.random() < 0.5)
    if beta_sigmoid:
        beta = _rows(rng, lead + (Hv,), dtype)
    else:
        beta = rng.uniform(0.05, 0.95, size=lead + (Hv,)).astype(np.float32)
        beta = ks.bf16_round(beta) if dtype == "bf16" else beta
    h0, idx = None, None
    r = rng.random()
    if packed and not dense_states and r < 0.35:
        rows = n + 2
        h0 = (rng.standard_normal(size=(rows, Hv, K, V)) * 0.02).astype(np.float32)
        idx = rng.permutation(rows)[:n].astype(np.int32)
        if n > 1 and rng.random() < 0.5:
            idx[int(rng.integers(0, n))] = -1
    elif r < 0.75:
        h0 = (rng.standard_normal(size=(n, Hv, K, V)) * 0.02).astype(np.float32)
    return ks.Problem(name=f"random{seed}", layout="tnd" if packed else "bsnd", dtype=dtype, B=B, T=T,
                      Hk=Hk, Hv=Hv, K=K, V=V, q=q, k=k, v=v, g=g, beta=beta, scale=1.0 / math.sqrt(K),
                      gate_in_kernel=gate_in_kernel, safe_gate=safe_gate, lower_bound=lower_bound,
                      l2norm=l2, beta_sigmoid=beta_sigmoid, A_log=A_log, dt_bias=dt_bias, h0=h0,
                      cu_seqlens=cu, state_indices=idx)


def describe(p, **extra):
    lens = None if p.cu_seqlens is None else np.diff(p.cu_seqlens).tolist()
    return (f"case {p.name}: {p.layout} {p.dtype} B={p.B} T={p.T} lens={lens} Hk={p.Hk} Hv={p.Hv} "
            f"K={p.K} V={p.V} gate_in_kernel={p.gate_in_kernel} safe_gate={p.safe_gate} "
            f"lower_bound={p.lower_bound} l2norm={p.l2norm} beta_sigmoid={p.beta_sigmoid} "
            f"dt_bias={p.dt_bias is not None} h0={None if p.h0 is None else p.h0.shape[0]} "
            f"cache={p.state_indices is not None} {extra}")


@pytest.mark.parametrize("seed", range(N_FWD))
def test_random_forward(gpu_lib, seed):
    p = random_problem(seed)
    segs = int(np.random.default_rng(500 + seed).choice([0, 0, 2, 3]))
    say(describe(p, scan_segments=segs))
    o, f = run_fwd(gpu_lib, p, scan_segments=segs)
    ro, rf = orc.forward(p)
    f32 = p.dtype == "f32"
    check("o", np64(o), ro, TOL_F32 if f32 else TOL_BF16_OUT)
    check("final_state", np64(f), rf, TOL_F32 if f32 else TOL_STATE)


@pytest.mark.parametrize("seed", range(N_BWD))
def test_random_backward(gpu_lib, seed):
    p = random_problem(100 + seed, dense_states=True)
    say(describe(p))
    bwd_case(gpu_lib, p)
