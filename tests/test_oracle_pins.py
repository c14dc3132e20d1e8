"""Pins for the fp64 oracle: each test ties it to mathematics or to a fact the
KDA pages fix, independently of the oracle's own loop.

A plausible slip in the oracle (a dropped term, a wrong sign or index, a
transposed operand, a decay applied after instead of before the write, a
wrong grouped-head map, a summary product in the wrong order) fails at least
one test here.
"""
import math
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import kda_oracle as orc

RNG = np.random.default_rng


def _unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def _prob(T=7, H=2, K=4, V=3, seed=0, layout="bsnd", B=1, **kw):
    r = RNG(seed)
    shp = (B, T) if layout == "bsnd" else (T,)
    d = dict(name="t", layout=layout, dtype="f32", B=B, T=T, Hk=H, Hv=H, K=K, V=V,
             q=r.standard_normal(shp + (H, K)), k=_unit(r.standard_normal(shp + (H, K))),
             v=r.standard_normal(shp + (H, V)),
             g=-np.abs(r.standard_normal(shp + (H, K))) * 0.3,
             beta=r.uniform(0.1, 0.9, shp + (H,)), scale=0.7, gate_in_kernel=False,
             safe_gate=False, lower_bound=-5.0, l2norm=False, beta_sigmoid=False, eps=1e-6,
             A_log=None, dt_bias=None, h0=None, cu_seqlens=None, state_indices=None)
    d.update(kw)
    return SimpleNamespace(**d)


# ------------------------------------------------------------ token recurrence
def test_beta_zero_is_pure_per_channel_decay():
    """beta = 0: the delta rule never writes, so S_T = Diag(e^{sum g}) S_0 and
    o_t = scale * sum_c q_tc e^{G_tc} S_0[c, :] with G_t the inclusive cumsum."""
    r = RNG(1)
    T, H, K, V = 9, 3, 5, 4
    k = _unit(r.standard_normal((T, H, K)))
    q = r.standard_normal((T, H, K))
    v = r.standard_normal((T, H, V))
    g = -r.uniform(0, 0.5, (T, H, K))
    S0 = r.standard_normal((H, K, V))
    o, S = orc.recurrence(k, v, g, np.zeros((T, H)), S0, q=q, scale=0.5)
    G = np.cumsum(g, axis=0)
    np.testing.assert_allclose(S, np.exp(G[-1])[:, :, None] * S0, rtol=1e-13, atol=1e-14)
    for t in range(T):
        for h in range(H):
            expect = 0.5 * sum(q[t, h, c] * math.exp(G[t, h, c]) * S0[h, c] for c in range(K))
            np.testing.assert_allclose(o[t, h], expect, rtol=1e-12, atol=1e-13)


def test_orthonormal_keys_no_decay_is_causal_linear_attention():
    """g = 0, S_0 = 0, orthonormal keys (T <= K): the prediction S^T k_t is zero,
    so o = scale * tril(Q K^T) (beta * V) -- masked linear attention."""
    r = RNG(2)
    T, K, V = 6, 8, 5
    Qm, _ = np.linalg.qr(r.standard_normal((K, K)))
    keys = Qm[:T]                                      # orthonormal rows
    q = r.standard_normal((T, K))
    v = r.standard_normal((T, V))
    beta = r.uniform(0.2, 1.0, T)
    o, S = orc.recurrence(keys[:, None], v[:, None], np.zeros((T, 1, K)), beta[:, None],
                          np.zeros((1, K, V)), q=q[:, None], scale=0.3)
    expect = 0.3 * np.tril(q @ keys.T) @ (beta[:, None] * v)
    np.testing.assert_allclose(o[:, 0], expect, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(S[0], keys.T @ (beta[:, None] * v), rtol=1e-12, atol=1e-12)


def test_last_write_wins_with_unit_beta():
    """beta = 1, no decay, unit key u: after writing (u, v) the state returns
    exactly v for key u, whatever it held before (the delta rule's exactness)."""
    r = RNG(3)
    K, V = 6, 4
    u = _unit(r.standard_normal(K))
    other = _unit(r.standard_normal(K))
    S0 = r.standard_normal((1, K, V))
    ks = np.stack([u, other, u])[:, None]
    vs = r.standard_normal((3, 1, V))
    _, S = orc.recurrence(ks, vs, np.zeros((3, 1, K)), np.ones((3, 1)), S0)
    np.testing.assert_allclose(S[0].T @ u, vs[2, 0], rtol=1e-12, atol=1e-12)


def test_scalar_case_closed_form():
    """K = V = 1: s_t = a_t s_{t-1} + b_t with a_t = (1 - beta k^2) e^{g},
    b_t = beta k v, whose solution is s_T = (prod a) s_0 + sum_j (prod_{r>j} a_r) b_j."""
    r = RNG(4)
    T = 12
    k = r.uniform(-1, 1, T)
    v = r.standard_normal(T)
    g = -r.uniform(0, 1, T)
    beta = r.uniform(0, 1, T)
    s0 = 0.37
    a = (1 - beta * k * k) * np.exp(g)
    b = beta * k * v
    expect = np.prod(a) * s0 + sum(np.prod(a[j + 1:]) * b[j] for j in range(T))
    _, S = orc.recurrence(k[:, None, None], v[:, None, None], g[:, None, None], beta[:, None],
                          np.full((1, 1, 1), s0))
    assert abs(S[0, 0, 0] - expect) < 1e-13


def _brute_force(q, k, v, g, beta, S0, scale):
    """Non-recursive form: S_t = M^{t<-1} S_0 + sum_{j<=t} M^{t<-j+1} beta_j k_j v_j^T,
    M_t = (I - beta_t k_t k_t^T) Diag(alpha_t), later factors on the left."""
    T, K = k.shape
    Ms = [(np.eye(K) - beta[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t])) for t in range(T)]

    def prod(lo, hi):  # M_hi ... M_lo (1-based inclusive), identity if empty
        P = np.eye(K)
        for t in range(lo, hi + 1):
            P = Ms[t - 1] @ P
        return P
    outs, S = [], None
    for t in range(1, T + 1):
        S = prod(1, t) @ S0
        for j in range(1, t + 1):
            S = S + prod(j + 1, t) @ (beta[j - 1] * np.outer(k[j - 1], v[j - 1]))
        outs.append(scale * S.T @ q[t - 1])
    return np.array(outs), S


@pytest.mark.parametrize("seed", [5, 6, 7])
def test_brute_force_matrix_products(seed):
    r = RNG(seed)
    T, K, V = 7, 5, 3
    q = r.standard_normal((T, K))
    k = _unit(r.standard_normal((T, K)))
    v = r.standard_normal((T, V))
    g = -r.uniform(0, 0.8, (T, K))
    beta = r.uniform(0, 1, T)
    S0 = r.standard_normal((K, V))
    o_bf, S_bf = _brute_force(q, k, v, g, beta, S0, 0.6)
    o, S = orc.recurrence(k[:, None], v[:, None], g[:, None], beta[:, None], S0[None],
                          q=q[:, None], scale=0.6)
    np.testing.assert_allclose(o[:, 0], o_bf, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(S[0], S_bf, rtol=1e-11, atol=1e-12)


def test_linear_in_values_and_affine_in_initial_state():
    p = _prob(seed=8)
    r = RNG(9)
    X1 = r.standard_normal((1, p.Hv, p.K, p.V))
    X2 = r.standard_normal((1, p.Hv, p.K, p.V))
    run = lambda v, h0: orc.forward(SimpleNamespace(**{**vars(p), "v": v, "h0": h0}))
    o_a, f_a = run(p.v * 2.5, X1 * 2.5)
    o_1, f_1 = run(p.v, X1)
    np.testing.assert_allclose(o_a, 2.5 * o_1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f_a, 2.5 * f_1, rtol=1e-12, atol=1e-12)
    o12, f12 = run(p.v, X1 + X2)
    o2, f2 = run(p.v, X2)
    o0, f0 = run(p.v, np.zeros_like(X1))
    np.testing.assert_allclose(o12 - o2, o_1 - o0, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(f12 - f2, f_1 - f0, rtol=1e-10, atol=1e-12)


def test_l2norm_makes_output_invariant_to_qk_scale():
    p = _prob(seed=10, l2norm=True, eps=0.0)
    o1, f1 = orc.forward(p)
    o2, f2 = orc.forward(SimpleNamespace(**{**vars(p), "q": p.q * 3.7, "k": p.k * 0.21}))
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(f2, f1, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------- gate / activations
def test_gate_special_values():
    # softplus(0) = ln 2; A_log = 0 -> factor 1; A_log = ln 16 -> factor 16.
    g = orc.kimi_gate(np.zeros((1, 2, 3)), np.array([0.0, math.log(16.0)]), None)
    np.testing.assert_allclose(g[0, 0], -math.log(2.0), rtol=1e-15)
    np.testing.assert_allclose(g[0, 1], -16 * math.log(2.0), rtol=1e-15)
    # dt_bias shifts the argument: softplus(-1 + 1) = ln 2.
    g = orc.kimi_gate(np.full((1, 1, 2), -1.0), np.zeros(1), np.ones((1, 2)))
    np.testing.assert_allclose(g, -math.log(2.0), rtol=1e-15)
    # Large arguments: softplus(x) -> x; very negative: -> e^x (no overflow).
    g = orc.kimi_gate(np.array([[[800.0, -800.0, 30.0]]]), np.zeros(1), None)
    assert g[0, 0, 0] == -800.0 and g[0, 0, 1] == -0.0 or abs(g[0, 0, 1]) < 1e-300
    np.testing.assert_allclose(g[0, 0, 2], -(30.0 + math.exp(-30.0)), rtol=1e-15)
    # Safe gate clamps at the lower bound.
    g = orc.kimi_gate(np.full((1, 1, 1), 3.0), np.array([math.log(16.0)]), None, True, -5.0)
    assert g[0, 0, 0] == -5.0


def test_sigmoid_and_l2norm_special_values():
    np.testing.assert_allclose(orc.sigmoid(np.array([0.0, math.log(3.0)])), [0.5, 0.75], rtol=1e-15)
    np.testing.assert_allclose(orc.l2norm(np.array([3.0, 4.0]), 0.0), [0.6, 0.8], rtol=1e-15)
    # eps sits inside the square root.
    np.testing.assert_allclose(orc.l2norm(np.array([0.0, 1e-3]), 1e-6),
                               [0.0, 1e-3 / math.sqrt(2e-6)], rtol=1e-14)


# ---------------------------------------------------------------- layouts
def test_packed_sequences_equal_separate_runs():
    r = RNG(11)
    lens = [5, 1, 9, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    p = _prob(T=int(cu[-1]), layout="tnd", cu_seqlens=cu, seed=12,
              h0=r.standard_normal((4, 2, 4, 3)))
    o, f = orc.forward(p)
    for n in range(4):
        t0, t1 = cu[n], cu[n + 1]
        sub = SimpleNamespace(**{**vars(p), "layout": "bsnd", "B": 1, "T": t1 - t0,
                                 "q": p.q[None, t0:t1], "k": p.k[None, t0:t1],
                                 "v": p.v[None, t0:t1], "g": p.g[None, t0:t1],
                                 "beta": p.beta[None, t0:t1], "h0": p.h0[n:n + 1],
                                 "cu_seqlens": None})
        os_, fs = orc.forward(sub)
        np.testing.assert_allclose(o[t0:t1], os_[0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(f[n], fs[0], rtol=1e-13, atol=1e-14)


def test_grouped_heads_read_contiguous_qk_groups():
    """Hv = 4 value heads over Hk = 2 q/k heads: value head h reads q/k head h // 2."""
    r = RNG(13)
    T, K, V = 6, 4, 3
    q = r.standard_normal((1, T, 2, K))
    k = _unit(r.standard_normal((1, T, 2, K)))
    p = _prob(T=T, H=4, K=K, V=V, seed=14)
    pg = SimpleNamespace(**{**vars(p), "Hk": 2, "q": q, "k": k})
    o, f = orc.forward(pg)
    for h in range(4):
        oh, sh = orc.recurrence(k[0, :, [h // 2]].transpose(1, 0, 2), p.v[0, :, [h]].transpose(1, 0, 2),
                                p.g[0, :, [h]].transpose(1, 0, 2), p.beta[0, :, [h]].T,
                                np.zeros((1, K, V)), q=q[0, :, [h // 2]].transpose(1, 0, 2),
                                scale=p.scale)
        np.testing.assert_allclose(o[0, :, h], oh[:, 0], rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(f[0, h], sh[0], rtol=1e-13, atol=1e-14)


def test_state_cache_contract():
    """Invalid indices (-1, out of range) start from zero and are not written;
    rows no sequence selects stay bit-identical."""
    r = RNG(15)
    lens = [4, 6, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cache = r.standard_normal((5, 2, 4, 3))
    idx = np.array([3, -1, 7], dtype=np.int32)
    p = _prob(T=int(cu[-1]), layout="tnd", cu_seqlens=cu, seed=16, h0=cache, state_indices=idx)
    o, newcache = orc.forward(p)
    for row in (0, 1, 2, 4):
        assert np.array_equal(newcache[row], cache[row])
    pz = SimpleNamespace(**{**vars(p), "h0": np.stack([cache[3], np.zeros_like(cache[0]),
                                                       np.zeros_like(cache[0])]),
                            "state_indices": None})
    oz, fz = orc.forward(pz)
    np.testing.assert_allclose(o, oz, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(newcache[3], fz[0], rtol=1e-14, atol=1e-15)


# --------------------------------------------------------------- summaries
def _split(p, t_cut):
    a = SimpleNamespace(**{**vars(p), "T": t_cut, "q": p.q[:, :t_cut], "k": p.k[:, :t_cut],
                           "v": p.v[:, :t_cut], "g": p.g[:, :t_cut], "beta": p.beta[:, :t_cut]})
    b = SimpleNamespace(**{**vars(p), "T": p.T - t_cut, "q": p.q[:, t_cut:],
                           "k": p.k[:, t_cut:], "v": p.v[:, t_cut:], "g": p.g[:, t_cut:],
                           "beta": p.beta[:, t_cut:]})
    return a, b


def test_summary_is_affine_map_of_incoming_state():
    p = _prob(T=11, seed=17)
    M, St = orc.segment_summary(p)
    X = RNG(18).standard_normal((1, p.Hv, p.K, p.V))
    _, f = orc.forward(SimpleNamespace(**{**vars(p), "h0": X}))
    np.testing.assert_allclose(np.matmul(M[0], X[0]) + St[0], f[0], rtol=1e-12, atol=1e-13)


def test_summary_transition_is_ordered_factor_product():
    p = _prob(T=5, H=1, K=4, V=2, seed=19)
    M, _ = orc.segment_summary(p)
    k, g, b = p.k[0, :, 0], p.g[0, :, 0], p.beta[0, :, 0]
    P = np.eye(4)
    for t in range(5):
        P = (np.eye(4) - b[t] * np.outer(k[t], k[t])) @ np.diag(np.exp(g[t])) @ P
    np.testing.assert_allclose(M[0, 0], P, rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("cuts", [[3], [1, 6], [2, 4, 9]])
def test_merge_of_split_summaries_equals_full_scan(cuts):
    p = _prob(T=12, seed=20)
    X = RNG(21).standard_normal((p.Hv, p.K, p.V))
    bounds = [0] + cuts + [p.T]
    Ms, Ss = [], []
    for t0, t1 in zip(bounds[:-1], bounds[1:]):
        seg = SimpleNamespace(**{**vars(p), "T": t1 - t0, "q": p.q[:, t0:t1], "k": p.k[:, t0:t1],
                                 "v": p.v[:, t0:t1], "g": p.g[:, t0:t1], "beta": p.beta[:, t0:t1]})
        M, S = orc.segment_summary(seg)
        Ms.append(M[0])
        Ss.append(S[0])
    _, f = orc.forward(SimpleNamespace(**{**vars(p), "h0": X[None]}))
    np.testing.assert_allclose(orc.summary_merge(np.stack(Ms), np.stack(Ss), X), f[0],
                               rtol=1e-11, atol=1e-12)
    _, f0 = orc.forward(p)
    np.testing.assert_allclose(orc.summary_merge(np.stack(Ms), np.stack(Ss)), f0[0],
                               rtol=1e-11, atol=1e-12)


def test_merge_order_matters_and_transition_cannot_be_dropped():
    p = _prob(T=10, seed=22)
    a, b = _split(p, 4)
    Ma, Sa = orc.segment_summary(a)
    Mb, Sb = orc.segment_summary(b)
    right = orc.summary_merge(np.stack([Ma[0], Mb[0]]), np.stack([Sa[0], Sb[0]]))
    swapped = orc.summary_merge(np.stack([Mb[0], Ma[0]]), np.stack([Sb[0], Sa[0]]))
    assert np.max(np.abs(right - swapped)) > 1e-3
    summed = Sa[0] + Sb[0]            # additive (LASP-style) summing
    assert np.max(np.abs(right - summed)) > 1e-3
    _, f0 = orc.forward(p)
    np.testing.assert_allclose(right, f0[0], rtol=1e-11, atol=1e-12)


def test_compare_metric():
    c = orc.compare(np.array([1.0, 2.1]), np.array([1.0, 2.0]))
    assert abs(c["err_max"] - 0.05) < 1e-12 and c["nonfinite"] == 0


# ------------------------------------------- in-kernel preprocessing routes
def _hand_gate(g_raw, A_log, dt_bias, safe, lb):
    """-exp(A_log[h]) * softplus(g_raw + dt_bias[h, c]) element by element with
    the scalar math library (softplus(x) = log(1 + e^x)), then the optional
    clamp at lb ("Hyper-Parallel Chunk KDA", section 4: use_gate_in_kernel,
    a_log, dt_bias, safe_gate, lower_bound)."""
    out = np.empty(g_raw.shape)
    for idx in np.ndindex(*g_raw.shape):
        h, c = idx[-2], idx[-1]
        x = float(g_raw[idx]) + (0.0 if dt_bias is None else float(dt_bias[h, c]))
        sp = x + math.log1p(math.exp(-x)) if x > 0 else math.log1p(math.exp(x))
        val = -math.exp(float(A_log[h])) * sp
        out[idx] = max(val, lb) if safe else val
    return out


def _hand_sigmoid(b):
    return np.vectorize(lambda x: 1.0 / (1.0 + math.exp(-float(x))))(b)


def _hand_l2(x, eps):
    out = np.empty(x.shape)
    for idx in np.ndindex(*x.shape[:-1]):
        row = [float(e) for e in x[idx]]
        r = 1.0 / math.sqrt(sum(e * e for e in row) + eps)
        out[idx] = [e * r for e in row]
    return out


def _gate_prob(safe, seed=30, H=3, Hk=None, T=11, K=4, V=3, layout="bsnd", **kw):
    """A problem on the in-kernel route: raw gate, raw beta logits, raw q/k.
    Every head has its own A_log and dt_bias, so a mis-indexed head fails."""
    r = RNG(seed)
    Hk = Hk or H
    shp = (1, T) if layout == "bsnd" else (T,)
    return _prob(T=T, H=H, K=K, V=V, seed=seed, layout=layout,
                 Hk=Hk, q=r.standard_normal(shp + (Hk, K)) * 2.0,
                 k=r.standard_normal(shp + (Hk, K)) * 0.7,
                 g=r.standard_normal(shp + (H, K)) * 1.5,
                 beta=r.standard_normal(shp + (H,)) * 2.0,
                 A_log=np.log(np.array([0.3, 1.7, 9.0, 2.2, 5.5, 0.8][:H])),
                 dt_bias=r.standard_normal((H, K)) * 0.5,
                 gate_in_kernel=True, safe_gate=safe, lower_bound=-1.2, l2norm=True,
                 beta_sigmoid=True, eps=1e-6, **kw)


@pytest.mark.parametrize("safe", [False, True])
def test_forward_in_kernel_route_equals_hand_prepared_recurrence(safe):
    """forward() on raw inputs with the gate, sigmoid, L2Norm (and clamp) flags
    equals the bare recurrence fed inputs prepared by hand, head by head."""
    p = _gate_prob(safe)
    X = RNG(31).standard_normal((1, p.Hv, p.K, p.V))
    p.h0 = X
    o, f = orc.forward(p)
    g = _hand_gate(p.g[0], p.A_log, p.dt_bias, safe, p.lower_bound)
    if safe:
        assert (g == p.lower_bound).any() and (g > p.lower_bound).any()
    b = _hand_sigmoid(p.beta[0])
    q = _hand_l2(p.q[0], p.eps)
    k = _hand_l2(p.k[0], p.eps)
    for h in range(p.Hv):
        oh, sh = orc.recurrence(k[:, [h]], p.v[0][:, [h]], g[:, [h]], b[:, [h]], X[0][[h]],
                                q=q[:, [h]], scale=p.scale)
        np.testing.assert_allclose(o[0, :, h], oh[:, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(f[0, h], sh[0], rtol=1e-12, atol=1e-13)


def test_precomputed_gate_clamp_and_sigmoid_route():
    """Without the in-kernel gate, the safe gate still clamps the given
    natural-log decay, and the sigmoid flag still activates beta."""
    p = _prob(T=9, H=2, seed=32, safe_gate=True, lower_bound=-0.2, beta_sigmoid=True,
              g=-np.abs(RNG(33).standard_normal((1, 9, 2, 4))) * 0.5,
              beta=RNG(34).standard_normal((1, 9, 2)))
    o, f = orc.forward(p)
    g = np.maximum(p.g[0], -0.2)
    assert (p.g[0] < -0.2).any()
    b = _hand_sigmoid(p.beta[0])
    oh, sh = orc.recurrence(p.k[0], p.v[0], g, b, np.zeros((2, 4, 3)), q=p.q[0], scale=p.scale)
    np.testing.assert_allclose(o[0], oh, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(f[0], sh, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("safe", [False, True])
def test_summary_in_kernel_route_equals_hand_prepared_recurrence(safe):
    p = _gate_prob(safe, seed=35)
    M, St = orc.segment_summary(p)
    g = _hand_gate(p.g[0], p.A_log, p.dt_bias, safe, p.lower_bound)
    b = _hand_sigmoid(p.beta[0])
    k = _hand_l2(p.k[0], p.eps)
    for h in range(p.Hv):
        _, sh = orc.recurrence(k[:, [h]], p.v[0][:, [h]], g[:, [h]], b[:, [h]],
                               np.zeros((1, p.K, p.V)))
        P = np.eye(p.K)
        for t in range(p.T):
            P = (np.eye(p.K) - b[t, h] * np.outer(k[t, h], k[t, h])) @ np.diag(np.exp(g[t, h])) @ P
        np.testing.assert_allclose(St[0, h], sh[0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(M[0, h], P, rtol=1e-11, atol=1e-13)


def test_grouped_heads_on_the_in_kernel_route():
    """Hv = 4 over Hk = 2 with the gate/sigmoid/L2Norm flags: value head h
    reads q/k head h // 2 but its own A_log[h], dt_bias[h] and beta."""
    p = _gate_prob(False, seed=36, H=4, Hk=2)
    o, f = orc.forward(p)
    g = _hand_gate(p.g[0], p.A_log, p.dt_bias, False, 0.0)
    b = _hand_sigmoid(p.beta[0])
    q = _hand_l2(p.q[0], p.eps)
    k = _hand_l2(p.k[0], p.eps)
    for h in range(4):
        oh, sh = orc.recurrence(k[:, [h // 2]], p.v[0][:, [h]], g[:, [h]], b[:, [h]],
                                np.zeros((1, p.K, p.V)), q=q[:, [h // 2]], scale=p.scale)
        np.testing.assert_allclose(o[0, :, h], oh[:, 0], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(f[0, h], sh[0], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("heads", [[2], [3, 0], [1, 2, 3]])
def test_head_subset_equals_slice_of_full_run(heads):
    """forward(heads=...) and segment_summary(heads=...) reproduce the full
    run on those heads (grouped heads, in-kernel route) and leave the rest zero."""
    p = _gate_prob(True, seed=37, H=4, Hk=2)
    p.h0 = RNG(38).standard_normal((1, 4, p.K, p.V))
    o, f = orc.forward(p)
    os_, fs = orc.forward(p, heads=heads)
    rest = [h for h in range(4) if h not in heads]
    np.testing.assert_array_equal(os_[..., heads, :], o[..., heads, :])
    np.testing.assert_array_equal(fs[:, heads], f[:, heads])
    assert not os_[..., rest, :].any() and not fs[:, rest].any()
    M, S = orc.segment_summary(p)
    Ms, Ss = orc.segment_summary(p, heads=heads)
    np.testing.assert_array_equal(Ms[:, heads], M[:, heads])
    np.testing.assert_array_equal(Ss[:, heads], S[:, heads])


def test_head_subset_in_cache_mode_keeps_other_heads():
    lens = [4, 7]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cache = RNG(39).standard_normal((3, 3, 4, 3))
    p = _gate_prob(False, seed=40, T=int(cu[-1]), layout="tnd", cu_seqlens=cu, h0=cache,
                   state_indices=np.array([2, 0], dtype=np.int32))
    _, full = orc.forward(p)
    _, part = orc.forward(p, heads=[1])
    np.testing.assert_array_equal(part[:, 1], full[:, 1])
    np.testing.assert_array_equal(part[:, [0, 2]], cache[:, [0, 2]])


def test_token_limit_equals_truncated_problem():
    """forward(t_max=n) equals the run of each sequence's first n tokens."""
    lens = [9, 3, 12]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    p = _gate_prob(True, seed=41, T=int(cu[-1]), layout="tnd", cu_seqlens=cu,
                   h0=RNG(42).standard_normal((3, 3, 4, 3)))
    o, f = orc.forward(p, t_max=5)
    keep = np.concatenate([np.arange(cu[n], min(cu[n + 1], cu[n] + 5)) for n in range(3)])
    cut = np.concatenate([[0], np.cumsum([min(L, 5) for L in lens])]).astype(np.int32)
    sub = SimpleNamespace(**{**vars(p), "T": int(cut[-1]), "cu_seqlens": cut, "q": p.q[keep],
                             "k": p.k[keep], "v": p.v[keep], "g": p.g[keep], "beta": p.beta[keep]})
    os_, fs = orc.forward(sub)
    np.testing.assert_array_equal(o[keep], os_)
    np.testing.assert_array_equal(f, fs)
    drop = np.setdiff1d(np.arange(p.T), keep)
    assert not o[drop].any()
