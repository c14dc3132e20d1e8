"""Pins for the oracle's backward: central finite differences of the forward
oracle's loss sum(do * o) + sum(dht * final_state) for every input element,
at tiny sizes, on the in-kernel route (gate, safe-gate clamp, sigmoid,
L2Norm), with grouped heads, packed sequences and initial states.  A dropped
term, a sign, a wrong index or a missing head-sum in the adjoint fails here.
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import kda_oracle as orc

RNG = np.random.default_rng


def _problem(layout, seed, safe=True, gate=True, Hk=2, Hv=4, T=9, K=4, V=3):
    r = RNG(seed)
    lens = [4, 5] if layout == "tnd" else None
    B = 1 if layout == "tnd" else 2
    shp = (T,) if layout == "tnd" else (B, T)
    N = len(lens) if lens else B
    p = SimpleNamespace(
        name="t", layout=layout, dtype="f32", B=B, T=T, Hk=Hk, Hv=Hv, K=K, V=V,
        q=r.standard_normal(shp + (Hk, K)), k=r.standard_normal(shp + (Hk, K)),
        v=r.standard_normal(shp + (Hv, V)),
        g=(r.standard_normal(shp + (Hv, K)) if gate else -np.abs(r.standard_normal(shp + (Hv, K)))),
        beta=r.standard_normal(shp + (Hv,)) if True else None, scale=0.6,
        gate_in_kernel=gate, safe_gate=safe, lower_bound=-1.0, l2norm=True, beta_sigmoid=True,
        eps=1e-3, A_log=np.log(r.uniform(0.3, 2.0, Hv)), dt_bias=r.standard_normal((Hv, K)) * 0.3,
        h0=r.standard_normal((N, Hv, K, V)) * 0.5,
        cu_seqlens=np.array([0, 4, 9], dtype=np.int32) if lens else None, state_indices=None)
    if not gate:
        p.A_log, p.dt_bias = None, None
    return p


def _loss(p, do, dht):
    o, f = orc.forward(p)
    return float((do * o).sum() + (dht * f).sum())


def _fd(p, name, do, dht, h=1e-6):
    base = getattr(p, name)
    grad = np.zeros(base.shape)
    for idx in np.ndindex(*base.shape):
        x = base.copy()
        x[idx] += h
        setattr(p, name, x)
        lp = _loss(p, do, dht)
        x[idx] -= 2 * h
        lm = _loss(p, do, dht)
        grad[idx] = (lp - lm) / (2 * h)
    setattr(p, name, base)
    return grad


def _away_from_clamp(p):
    """Move gate inputs whose activated decay sits within 1e-3 of the clamp, so
    that the finite-difference step never crosses it."""
    z = p.g + p.dt_bias if p.gate_in_kernel else p.g
    for _ in range(50):
        z = p.g + (p.dt_bias if p.gate_in_kernel else 0)
        act = -np.exp(p.A_log)[:, None] * orc.softplus(z) if p.gate_in_kernel else p.g
        near = np.abs(act - p.lower_bound) < 1e-3
        if not near.any():
            return
        p.g = np.where(near, p.g + 0.01, p.g)


@pytest.mark.parametrize("layout,safe,gate", [("bsnd", True, True), ("tnd", True, True),
                                              ("bsnd", False, False)])
def test_backward_matches_finite_differences(layout, safe, gate):
    p = _problem(layout, seed=50 + safe + 2 * gate, safe=safe, gate=gate)
    _away_from_clamp(p)
    r = RNG(60)
    do = r.standard_normal(p.v.shape)
    dht = r.standard_normal(p.h0.shape)
    grads = orc.backward(p, do, dht)
    if safe and gate:
        act = -np.exp(p.A_log)[:, None] * orc.softplus(p.g + p.dt_bias)
        assert (act < p.lower_bound).any() and (act > p.lower_bound).any()
    names = [("q", "dq"), ("k", "dk"), ("v", "dv"), ("g", "dg"), ("beta", "dbeta"), ("h0", "dh0")]
    if gate:
        names += [("A_log", "dA_log"), ("dt_bias", "ddt_bias")]
    for name, gname in names:
        fd = _fd(p, name, do, dht)
        np.testing.assert_allclose(grads[gname], fd, rtol=2e-6, atol=2e-7, err_msg=gname)


def test_backward_recurrence_scalar_closed_form():
    """K = V = 1, no output: s_T = prod(a) s_0 + sum_j prod_{r>j} a_r b_j with
    a_t = (1 - beta k^2) e^g, b_t = beta k v; the gradient of s_T in s_0 is
    prod(a), in v_j it is prod_{r>j} a_r * beta_j k_j."""
    r = RNG(61)
    T = 7
    k = r.uniform(-1, 1, T)
    v = r.standard_normal(T)
    g = -r.uniform(0, 1, T)
    beta = r.uniform(0, 1, T)
    a = (1 - beta * k * k) * np.exp(g)
    _, dk, dv, dg, db, dS0 = orc.recurrence_bwd(k[:, None, None], v[:, None, None], g[:, None, None],
                                                beta[:, None], np.full((1, 1, 1), 0.3),
                                                np.zeros((T, 1, 1)), 1.0, np.zeros((T, 1, 1)),
                                                np.ones((1, 1, 1)), ckpt=3)
    assert abs(dS0[0, 0, 0] - np.prod(a)) < 1e-13
    for j in range(T):
        assert abs(dv[j, 0, 0] - np.prod(a[j + 1:]) * beta[j] * k[j]) < 1e-13


def test_backward_head_subset_equals_slice():
    p = _problem("bsnd", seed=62)
    r = RNG(63)
    do = r.standard_normal(p.v.shape)
    dht = r.standard_normal(p.h0.shape)
    full = orc.backward(p, do, dht)
    part = orc.backward(p, do, dht, heads=[1, 2])      # value heads 1, 2: q/k heads 0 and 1
    for name in ("dv", "dg", "dbeta"):
        np.testing.assert_array_equal(part[name][..., [1, 2], :] if part[name].ndim == 4 else part[name][..., [1, 2]],
                                      full[name][..., [1, 2], :] if full[name].ndim == 4 else full[name][..., [1, 2]])
    np.testing.assert_array_equal(part["dh0"][:, [1, 2]], full["dh0"][:, [1, 2]])
    # a q/k head receives only the selected value heads' share: value heads 0
    # and 1 share q/k head 0, so the two partial runs add up to the full one
    np.testing.assert_allclose(part["dq"][..., 0, :] + orc.backward(p, do, dht, heads=[0])["dq"][..., 0, :],
                               full["dq"][..., 0, :], rtol=1e-12, atol=1e-13)


def test_initial_state_gradient_is_affine_in_the_final_one():
    """dS_0 = M^T dS_T + local, with M the forward summary's transition: the
    backward's state gradient is the forward transition transposed."""
    p = _problem("bsnd", seed=64)
    p = SimpleNamespace(**{**vars(p), "B": 1, "q": p.q[:1], "k": p.k[:1], "v": p.v[:1], "g": p.g[:1],
                           "beta": p.beta[:1], "h0": p.h0[:1]})
    r = RNG(65)
    do = r.standard_normal(p.v.shape)
    dht = r.standard_normal(p.h0.shape)
    M, _ = orc.segment_summary(p)
    local = orc.segment_summary_bwd(p, do)
    full = orc.backward(p, do, dht)["dh0"]
    np.testing.assert_allclose(full[0], np.matmul(np.swapaxes(M[0], -1, -2), dht[0]) + local[0],
                               rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("cuts", [[4], [2, 7], [1, 3, 6]])
def test_reverse_merge_of_split_summaries_equals_full_backward(cuts):
    """A sequence cut into segments: the reverse merge of the segments'
    (M, local) from dS_T equals the full backward's dS_0, and its intermediate
    values equal the full backward's gradient at each cut (the backward's
    composition order is the reverse of the forward's)."""
    p = _problem("bsnd", seed=66)
    p = SimpleNamespace(**{**vars(p), "B": 1, "q": p.q[:1], "k": p.k[:1], "v": p.v[:1], "g": p.g[:1],
                           "beta": p.beta[:1], "h0": p.h0[:1]})
    r = RNG(67)
    do = r.standard_normal(p.v.shape)
    dht = r.standard_normal(p.h0.shape)
    bounds = [0] + cuts + [p.T]
    Ms, locs = [], []
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        seg = SimpleNamespace(**{**vars(p), "T": t1 - t0, "q": p.q[:, t0:t1], "k": p.k[:, t0:t1],
                                 "v": p.v[:, t0:t1], "g": p.g[:, t0:t1], "beta": p.beta[:, t0:t1]})
        Ms.append(orc.segment_summary(seg)[0][0])
        locs.append(orc.segment_summary_bwd(seg, do[:, t0:t1])[0])
    full = orc.backward(p, do, dht)["dh0"][0]
    np.testing.assert_allclose(orc.summary_merge_bwd(np.stack(Ms), np.stack(locs), dht[0]), full,
                               rtol=1e-10, atol=1e-11)
    # gradient arriving at the first cut = backward of the tail from dht
    tail = SimpleNamespace(**{**vars(p), "T": p.T - cuts[0], "q": p.q[:, cuts[0]:], "k": p.k[:, cuts[0]:],
                              "v": p.v[:, cuts[0]:], "g": p.g[:, cuts[0]:], "beta": p.beta[:, cuts[0]:]})
    at_cut = orc.backward(tail, do[:, cuts[0]:], dht)["dh0"][0]
    np.testing.assert_allclose(orc.summary_merge_bwd(np.stack(Ms[1:]), np.stack(locs[1:]), dht[0]), at_cut,
                               rtol=1e-10, atol=1e-11)
    # the forward order gives something else
    S = dht[0].copy()
    for j in range(len(Ms)):
        S = np.matmul(np.swapaxes(Ms[j], -1, -2), S) + locs[j]
    assert np.abs(S - full).max() > 1e-3
