"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Bars: bf16 outputs err_max <= 2e-2; fp32 states, summaries and merged states
<= 5e-3; fp32-input runs <= 5e-3 everywhere.  err_max = max|x - ref| / max|ref|.
Small cases span several 64-token chunks with a ragged tail; full-size cases
compare sampled heads (every token and state entry of those heads).
"""
import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import kda_synth as ks
from kda_synth.torch_io import flag_kwargs, to_torch
from oracle import kda_oracle as orc

pytestmark = pytest.mark.gpu

TOL_BF16_OUT = 2e-2
TOL_STATE = 5e-3
TOL_F32 = 5e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check(name, x, ref, tol):
    c = orc.compare(x, ref)
    say(f"  {name}: err_max={c['err_max']:.3e} rel_l2={c['rel_l2']:.3e} nonfinite={c['nonfinite']}")
    assert c["nonfinite"] == 0, name
    assert c["err_max"] <= tol, (name, c)
    return c


def run_fwd(kda, p, t=None, **over):
    t = t or to_torch(p)
    kw = flag_kwargs(p)
    kw.update(over)
    o, f = kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=p.scale,
                             A_log=t["A_log"], dt_bias=t["dt_bias"],
                             initial_state=None if p.h0 is None else t["h0"],
                             cu_seqlens=t["cu"], cu_seqlens_host=t["cu_host"],
                             state_indices=t["state_indices"], **kw)
    torch.cuda.synchronize()
    return o, f


def fwd_case(kda, p, heads=None, o_tol=None, f_tol=TOL_STATE):
    say(f"case {p.name}: layout={p.layout} dtype={p.dtype} B={p.B} T={p.T} Hk={p.Hk} Hv={p.Hv} "
        f"K={p.K} V={p.V} heads={heads}")
    o, f = run_fwd(kda, p)
    ro, rf = orc.forward(p, heads=heads)
    o_tol = o_tol or (TOL_F32 if p.dtype == "f32" else TOL_BF16_OUT)
    go, gf = np64(o), np64(f)
    if heads is not None:
        go, ro = go[..., heads, :], ro[..., heads, :]
        if p.state_indices is None:
            gf, rf = gf[:, heads], rf[:, heads]
        else:
            gf, rf = gf[:, heads], rf[:, heads]
    check("o", go, ro, o_tol)
    check("final_state", gf, rf, f_tol if p.dtype != "f32" else TOL_F32)
    return o, f


# ------------------------------------------------------------------ small cases
def test_tiny_fp32_prenormalised(gpu_lib):
    fwd_case(gpu_lib, ks.make("tiny"))


def test_tiny_fp32_in_kernel_l2norm_and_sigmoid(gpu_lib):
    fwd_case(gpu_lib, ks.make("tiny", normalized_qk=False, preactivated_beta=False))


def test_tiny_flag_paths_agree(gpu_lib):
    """Raw q/k with in-kernel L2Norm equals pre-normalised q/k with it off."""
    a = ks.make("tiny", normalized_qk=False)
    b = ks.make("tiny", normalized_qk=True)
    oa, fa = run_fwd(gpu_lib, a)
    ob, fb = run_fwd(gpu_lib, b)
    check("o(raw+l2) vs o(pre)", np64(oa), np64(ob), 1e-4)


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_layer_small_ragged(gpu_lib, T):
    fwd_case(gpu_lib, ks.make("layer", T=T, H=4))


def test_layer_batch2_no_h0(gpu_lib):
    fwd_case(gpu_lib, ks.make("layer", B=2, T=130, H=3, h0_std=0.0))


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64)])
def test_layer_head_dims_bf16(gpu_lib, K, V):
    fwd_case(gpu_lib, ks.make("layer", T=150, H=2, K=K, V=V))


def test_fp32_k64_v128(gpu_lib):
    fwd_case(gpu_lib, ks.make("layer", T=150, H=2, K=64, V=128, dtype="f32"))


def test_beta_zero_is_pure_decay(gpu_lib):
    """beta = 0 (sigmoid off): the state only decays; o reads the decayed h0."""
    p = ks.make("layer", T=100, H=2)
    p.beta_sigmoid = False
    p.beta = np.zeros_like(p.beta)
    fwd_case(gpu_lib, p)


@pytest.mark.parametrize("vscale", [1e-3, 1e3])
def test_value_scale_far_from_unit(gpu_lib, vscale):
    """With bf16 tokens the workspace keeps u = (I+L)^-1 (beta v) and the scan
    v_new = u - w h in fp16 (normal from 6.1e-5 to 65504).  v scaled by 1e-3 and
    by 1e3 (|v| up to about 4e3) both match the oracle to the usual bars, the
    errors being relative to the outputs' size."""
    p = ks.make("layer", T=200, H=2, h0_std=0.0)
    p.v = ks.bf16_round(p.v * np.float32(vscale))
    fwd_case(gpu_lib, p)


def test_state_keeps_kg_at_fp16_precision(gpu_lib):
    """With bf16 tokens kg^T reaches the state in fp16 (11 significant bits)
    against v_new as an fp16 hi/lo pair; this case's final state measures
    4.5e-4 from the oracle.  A CPU emulation with kg^T carried to bf16's 8 bits
    only puts it at 2.4e-3, so the bound (between the two, well inside the
    5e-3 bar) fails when the kg^T path loses precision."""
    fwd_case(gpu_lib, ks.make("layer", T=1280, H=2), f_tol=8e-4)


def test_small_and_large_decay_heads(gpu_lib):
    """Head 0 decays slowly (every 16-token tile within the single-reference
    range of the diagonal tiles), head 1 fast (per-token decays of tens in log2
    units: the binary split everywhere); both against the oracle."""
    p = ks.make("layer", T=300, H=2)
    p.A_log = np.array([math.log(0.05), math.log(64.0)], dtype=np.float32)
    o, f = fwd_case(gpu_lib, p)
    assert np.isfinite(np64(o)).all() and np.isfinite(np64(f)).all()


def test_varlen_small_with_cache(gpu_lib):
    p = ks.make("varlen", lens=[70, 0, 1, 130, 64, 5], H=3, cache_rows=9, n_invalid=2)
    cache_before = p.h0.copy()
    t = to_torch(p)
    o, cache = run_fwd(gpu_lib, p, t)
    ro, rcache = orc.forward(p)
    check("o", np64(o), ro, TOL_BF16_OUT)
    check("cache", np64(cache), rcache, TOL_STATE)
    touched = set(int(i) for i in p.state_indices if i >= 0)
    got = cache.cpu().numpy()
    for r in range(p.h0.shape[0]):
        if r not in touched:
            assert np.array_equal(got[r], cache_before[r]), f"row {r} changed"


def test_varlen_leading_and_trailing_empty_sequences(gpu_lib):
    """Empty sequences first and last: they own no chunks, so no workgroup of
    theirs may address a record (the first one's would lie before the workspace)."""
    p = ks.make("varlen", lens=[0, 70, 0, 129, 0], H=2, cache_rows=6, n_invalid=0)
    t = to_torch(p)
    o, cache = run_fwd(gpu_lib, p, t)
    ro, rcache = orc.forward(p)
    check("o", np64(o), ro, TOL_BF16_OUT)
    check("cache", np64(cache), rcache, TOL_STATE)


def test_varlen_cache_out_of_range_index_reads_zero(gpu_lib):
    p = ks.make("varlen", lens=[40, 90], H=2, cache_rows=4, n_invalid=0)
    p.state_indices = np.array([7, 2], dtype=np.int32)     # 7 >= rows: invalid
    t = to_torch(p)
    o, cache = run_fwd(gpu_lib, p, t)
    ro, rcache = orc.forward(p)
    check("o", np64(o), ro, TOL_BF16_OUT)
    check("cache", np64(cache), rcache, TOL_STATE)


def test_eps_zero_ragged_tail(gpu_lib):
    """eps = 0 with the in-kernel L2Norm and T % 64 != 0: the rows past the
    sequence end carry zero norms and must stay inert (no 0 * inf)."""
    p = ks.make("layer", T=65, H=2)
    p.eps = 0.0
    fwd_case(gpu_lib, p)


def test_fp32_k128(gpu_lib):
    fwd_case(gpu_lib, ks.make("layer", T=150, H=2, K=128, V=128, dtype="f32"))


def test_varlen_duplicate_gather_indices(gpu_lib):
    """Two sequences may start from the same cache row when nothing is written
    back (vllm-ascend KDA prefill state copy page, numeric contract)."""
    p = ks.make("varlen", lens=[70, 33, 130], H=2, cache_rows=4, n_invalid=0)
    p.state_indices = np.array([1, 3, 1], dtype=np.int32)
    t = to_torch(p)
    before = t["h0"].clone()
    o, fin = gpu_lib.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=p.scale,
                                   A_log=t["A_log"], dt_bias=t["dt_bias"], initial_state=t["h0"],
                                   cu_seqlens=t["cu"], cu_seqlens_host=t["cu_host"],
                                   state_indices=t["state_indices"], output_final_state=False,
                                   **flag_kwargs(p))
    torch.cuda.synchronize()
    assert fin is None and torch.equal(t["h0"], before)
    ro, _ = orc.forward(p)
    check("o", np64(o), ro, TOL_BF16_OUT)


def test_nan_input_propagates(gpu_lib):
    """A NaN in one value row: every output the oracle makes NaN is NaN on the
    GPU too, the chunks before it are unaffected and nothing faults."""
    p = ks.make("layer", T=200, H=2)
    p.v = p.v.copy()
    p.v[0, 100, 1, 7] = np.nan
    o, f = run_fwd(gpu_lib, p)
    ro, rf = orc.forward(p)
    go, gf = np64(o), np64(f)
    assert np.isnan(go[np.isnan(ro)]).all() and np.isnan(gf[np.isnan(rf)]).all()
    assert np.isnan(rf).any()
    check("o before the NaN chunk", go[:, :64], ro[:, :64], TOL_BF16_OUT)
    check("head 0", go[:, :, 0], ro[:, :, 0], TOL_BF16_OUT)


def test_empty_selection(gpu_lib):
    """N = 0 sequences: nothing is launched and nothing is written."""
    z = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    cu = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, f = gpu_lib.kda_chunk_fwd(z, z, z, z, torch.zeros((0, 2), dtype=torch.bfloat16, device="cuda"),
                                 cu_seqlens=cu, cu_seqlens_host=cu.cpu())
    torch.cuda.synchronize()
    assert o.shape == (0, 2, 128) and f.shape == (0, 2, 128, 128)


def test_state_cache_beyond_4GiB(gpu_lib):
    """Cache rows whose byte offsets exceed 2^32: gather and scatter use 64-bit
    addresses (a 32-bit offset would touch row r - 32768 instead)."""
    p = ks.make("varlen", lens=[90, 40], H=2, cache_rows=2, n_invalid=0)
    rows = 33000                                        # 128 KiB per row: 4.3 GB
    cache = torch.zeros((rows, 2, 128, 128), dtype=torch.float32, device="cuda")
    cache[32990] = torch.from_numpy(p.h0[0]).cuda()
    t = to_torch(p)
    si = torch.tensor([32990, 32999], dtype=torch.int32, device="cuda")
    o, cache = gpu_lib.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=p.scale,
                                     A_log=t["A_log"], dt_bias=t["dt_bias"], initial_state=cache,
                                     cu_seqlens=t["cu"], cu_seqlens_host=t["cu_host"],
                                     state_indices=si, **flag_kwargs(p))
    torch.cuda.synchronize()
    # the same problem on a two-row cache [row 32990, zeros] with indices [0, 1]
    ref = dataclasses.replace(p, h0=np.stack([p.h0[0], np.zeros_like(p.h0[0])]),
                              state_indices=np.array([0, 1], dtype=np.int32))
    ro, rcache = orc.forward(ref)
    check("o", np64(o), ro, TOL_BF16_OUT)
    check("row 32990", np64(cache[32990]), rcache[0], TOL_STATE)
    check("row 32999", np64(cache[32999]), rcache[1], TOL_STATE)
    assert not cache[32990 - 32768].any() and not cache[32999 - 32768].any()
    del cache


def test_gqa_small_safe_gate(gpu_lib):
    fwd_case(gpu_lib, ks.make("gqa", B=2, T=150, Hk=2, Hv=8))


def test_two_calls_carry_state(gpu_lib):
    """Running T in two calls (final -> initial) equals one call."""
    p = ks.make("layer", T=200, H=2)
    a = ks.make("layer", T=200, H=2)
    o_full, f_full = run_fwd(gpu_lib, p)
    cut = 96
    for name in ("q", "k", "v", "g", "beta"):
        setattr(a, name, getattr(p, name)[:, :cut])
    a.T = cut
    o1, f1 = run_fwd(gpu_lib, a)
    b = ks.make("layer", T=200, H=2)
    for name in ("q", "k", "v", "g", "beta"):
        setattr(b, name, getattr(p, name)[:, cut:])
    b.T = 200 - cut
    b.h0 = f1.cpu().numpy()
    o2, f2 = run_fwd(gpu_lib, b)
    check("o split", np64(torch.cat([o1, o2], dim=1)), np64(o_full), 1e-2)
    check("final split", np64(f2), np64(f_full), 1e-3)


def test_deterministic(gpu_lib):
    p = ks.make("layer", T=300, H=4)
    t = to_torch(p)
    o1, f1 = run_fwd(gpu_lib, p, t)
    o2, f2 = run_fwd(gpu_lib, p, t)
    assert torch.equal(o1, o2) and torch.equal(f1, f2)


def test_graph_capture_replays_match_eager(gpu_lib):
    """The forward call allocates nothing and never synchronises when its
    outputs and workspace are given, so a caller can capture it in a HIP graph.
    Each replay, with new inputs copied into the captured buffers and eager
    work in between, equals the eager call on the same inputs bit for bit."""
    p = ks.make("layer", T=300, H=4)
    t = to_torch(p)
    kw = flag_kwargs(p)
    names = ("q", "k", "v", "g", "beta")
    static = {n: t[n].clone() for n in names}
    o = torch.empty_like(t["v"])
    f = torch.empty((p.B, p.Hv, p.K, p.V), dtype=torch.float32, device="cuda")
    ws = torch.empty(gpu_lib.workspace_bytes(t["q"], t["v"]), dtype=torch.uint8, device="cuda")

    def call(x, out, fin):
        gpu_lib.kda_chunk_fwd(x["q"], x["k"], x["v"], x["g"], x["beta"], scale=p.scale, A_log=t["A_log"],
                              dt_bias=t["dt_bias"], initial_state=t["h0"], o=out, final_state=fin,
                              workspace=ws, **kw)

    call(static, o, f)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(static, o, f)
    torch.cuda.synchronize()
    for r in range(3):
        gen = torch.Generator(device="cuda").manual_seed(100 + r)
        for n in names:
            static[n].copy_(t[n] * (1 + 0.25 * torch.rand(t[n].shape, generator=gen, device="cuda")).to(t[n].dtype))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        og, fg = o.clone(), f.clone()
        oe, fe = torch.empty_like(o), torch.empty_like(f)
        call({n: static[n].clone() for n in names}, oe, fe)
        torch.cuda.synchronize()
        say(f"  replay {r}: o equal {torch.equal(og, oe)}, final equal {torch.equal(fg, fe)}")
        assert torch.equal(og, oe) and torch.equal(fg, fe)
        assert not torch.equal(og, torch.zeros_like(og))


# ------------------------------------------- segment-parallel state scan
@pytest.mark.parametrize("S", [2, 3, 5, 16])
def test_segmented_scan_matches_oracle(gpu_lib, S):
    """The forward with each sequence cut into S segments (summaries in
    parallel, prefix merge, rescans in parallel) against the oracle and
    against the one-scan forward."""
    p = ks.make("layer", T=1000, H=2)
    t = to_torch(p)
    o1, f1 = run_fwd(gpu_lib, p, t, scan_segments=1)
    oS, fS = run_fwd(gpu_lib, p, t, scan_segments=S)
    ro, rf = orc.forward(p)
    check("o", np64(oS), ro, TOL_BF16_OUT)
    check("final_state", np64(fS), rf, TOL_STATE)
    check("o vs one scan", np64(oS), np64(o1), TOL_BF16_OUT)
    check("final vs one scan", np64(fS), np64(f1), TOL_STATE)


def test_segmented_scan_carries_state_across_segments(gpu_lib):
    """Slow decay (small A_log): the state entering each segment matters, so a
    wrong transition product or merge order shows in o and the final state."""
    p = ks.make("layer", T=2048, H=2)
    p.A_log = np.log(np.array([1e-3, 3e-3], dtype=np.float32))
    p.dt_bias = np.full_like(p.dt_bias, -4.0)
    t = to_torch(p)
    o, f = run_fwd(gpu_lib, p, t, scan_segments=4)
    ro, rf = orc.forward(p)
    say(f"  max|final| = {np.abs(rf).max():.3f}")
    check("o", np64(o), ro, TOL_BF16_OUT)
    check("final_state", np64(f), rf, TOL_STATE)
    # dropping the incoming states (zero start per segment) must be far off
    pz = ks.make("layer", T=512, H=2)
    pz.A_log, pz.dt_bias, pz.h0 = p.A_log, p.dt_bias, None
    for name in ("q", "k", "v", "g", "beta"):
        setattr(pz, name, getattr(p, name)[:, 1536:])
    roz, _ = orc.forward(pz)
    assert np.abs(roz - ro[:, 1536:]).max() > 10 * TOL_BF16_OUT * np.abs(ro).max()


def test_segmented_scan_varlen_with_cache(gpu_lib):
    p = ks.make("varlen", lens=[300, 70, 513, 1, 0, 260], H=3, cache_rows=9, n_invalid=1)
    before = p.h0.copy()
    o, cache = run_fwd(gpu_lib, p, scan_segments=4)
    ro, rcache = orc.forward(p)
    check("o", np64(o), ro, TOL_BF16_OUT)
    check("cache", np64(cache), rcache, TOL_STATE)
    got = cache.cpu().numpy()
    touched = set(int(i) for i in p.state_indices if i >= 0)
    for r in range(p.h0.shape[0]):
        if r not in touched:
            assert np.array_equal(got[r], before[r]), f"row {r} changed"


def test_segmented_scan_automatic_on_few_heads(gpu_lib):
    """Two heads over 16,384 tokens: 16 column-tile scans, so the library splits
    each sequence by itself; every token and state entry against the oracle."""
    p = ks.make("longseq", T=16384, H=2)
    fwd_case(gpu_lib, p)


# ------------------------------------------------------ recurrent (decode)
def run_rec(kda, p, t=None, **over):
    t = t or to_torch(p)
    kw = flag_kwargs(p)
    kw.update(over)
    o, f = kda.kda_recurrent_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=p.scale,
                                 A_log=t["A_log"], dt_bias=t["dt_bias"],
                                 initial_state=None if p.h0 is None else t["h0"],
                                 cu_seqlens=t["cu"], cu_seqlens_host=t["cu_host"],
                                 state_indices=t["state_indices"], **kw)
    torch.cuda.synchronize()
    return o, f


def test_recurrent_decode_step(gpu_lib):
    """One token for each of 64 sequences, states gathered from and scattered
    back into the cache in place; rows no valid index selects stay untouched."""
    p = ks.make("decode")
    before = p.h0.copy()
    o, cache = run_rec(gpu_lib, p)
    ro, rcache = orc.forward(p)
    check("o", np64(o), ro, TOL_BF16_OUT)
    check("cache", np64(cache), rcache, 1e-5)
    got = cache.cpu().numpy()
    touched = set(int(i) for i in p.state_indices if i >= 0)
    for r in range(p.h0.shape[0]):
        if r not in touched:
            assert np.array_equal(got[r], before[r]), f"row {r} changed"


def test_recurrent_multi_token_and_empty_sequences(gpu_lib):
    p = ks.make("decode", lens=[1, 3, 0, 7, 2, 0], H=3, cache_rows=9, n_invalid=1)
    o, cache = run_rec(gpu_lib, p)
    ro, rcache = orc.forward(p)
    check("o", np64(o), ro, TOL_BF16_OUT)
    check("cache", np64(cache), rcache, 1e-5)


@pytest.mark.parametrize("K,V", [(64, 64), (64, 128), (128, 64)])
def test_recurrent_head_dims_fp32_dense_states(gpu_lib, K, V):
    """fp32 tokens, dense initial/final states, BSND, grouped heads, safe gate."""
    p = ks.make("gqa", B=2, T=5, Hk=2, Hv=4, K=K, V=V, dtype="f32")
    o, f = run_rec(gpu_lib, p)
    ro, rf = orc.forward(p)
    check("o", np64(o), ro, 1e-5)
    check("final_state", np64(f), rf, 1e-5)


def test_recurrent_equals_chunked_forward(gpu_lib):
    """Both forms of the method on the same 200-token layer problem."""
    p = ks.make("layer", T=200, H=2)
    t = to_torch(p)
    oc, fc = run_fwd(gpu_lib, p, t)
    orr, fr = run_rec(gpu_lib, p, t)
    check("o recurrent vs chunked", np64(orr), np64(oc), TOL_BF16_OUT)
    check("final recurrent vs chunked", np64(fr), np64(fc), TOL_STATE)
    ro, rf = orc.forward(p)
    check("o recurrent vs oracle", np64(orr), ro, TOL_BF16_OUT)
    check("final recurrent vs oracle", np64(fr), rf, 1e-5)


# ---------------------------------------------------------- summary and merge
def _summary_gpu(kda, p, t=None):
    t = t or to_torch(p)
    kw = flag_kwargs(p)
    M, S = kda.kda_segment_summary(t["k"], t["v"], t["g"], t["beta"], A_log=t["A_log"],
                                   dt_bias=t["dt_bias"], cu_seqlens=t["cu"],
                                   cu_seqlens_host=t["cu_host"], **kw)
    torch.cuda.synchronize()
    return M, S


def test_summary_small_matches_oracle(gpu_lib):
    p = ks.make("layer", T=150, H=2, h0_std=0.0)
    # a gentler gate keeps the transition product away from zero
    p.gate_in_kernel = False
    rng = np.random.default_rng(5)
    p.g = ks.bf16_round((-0.05 * rng.random(p.g.shape)).astype(np.float32))
    M, S = _summary_gpu(gpu_lib, p)
    rM, rS = orc.segment_summary(p)
    check("M", np64(M), rM, TOL_STATE)
    check("S~", np64(S), rS, TOL_STATE)


def test_wide_scan_tiles_forward(gpu_lib):
    """64 heads x 8 column tiles of 16 = 512 tile scans, two rounds per CU: the
    scan runs 32-column tiles (a workgroup loads each chunk's shared operands
    once for two tiles)."""
    fwd_case(gpu_lib, ks.make("layer", T=200, H=64))


def test_many_tile_summary(gpu_lib):
    """32 heads x (V + K) / 16 = 512 summary tile scans (16-column tiles; the
    summary scan runs several workgroups per CU)."""
    p = ks.make("layer", T=150, H=32, h0_std=0.0)
    p.gate_in_kernel = False
    rng = np.random.default_rng(7)
    p.g = ks.bf16_round((-0.05 * rng.random(p.g.shape)).astype(np.float32))
    M, S = _summary_gpu(gpu_lib, p)
    rM, rS = orc.segment_summary(p)
    check("M", np64(M), rM, TOL_STATE)
    check("S~", np64(S), rS, TOL_STATE)


@pytest.mark.parametrize("route", ["precomputed", "in_kernel"])
def test_summary_deep_transition(gpu_lib, route):
    """M over 64 chunks in a regime where it stays O(0.1-1): a near-zero
    precomputed gate with small beta, or the in-kernel gate with small A_log
    (every chunk's transition passes the kg^T lo part of the scan)."""
    p = ks.make("layer", T=4096, H=4, h0_std=0.0)
    rng = np.random.default_rng(11)
    if route == "precomputed":
        p.gate_in_kernel = False
        p.g = ks.bf16_round((-2e-4 * rng.random(p.g.shape)).astype(np.float32))
        p.beta = ks.bf16_round((rng.standard_normal(p.beta.shape) - 5.0).astype(np.float32))
    else:
        p.A_log = np.log(np.array([1e-4, 3e-4, 1e-3, 2e-4], dtype=np.float32))
        p.dt_bias = np.full_like(p.dt_bias, -6.0)
        p.beta = ks.bf16_round((rng.standard_normal(p.beta.shape) - 5.0).astype(np.float32))
    M, S = _summary_gpu(gpu_lib, p)
    rM, rS = orc.segment_summary(p)
    say(f"  max|M| = {np.abs(rM).max():.3f}, max|M - I| = {np.abs(rM - np.eye(p.K)).max():.3f}")
    assert 0.1 < np.abs(rM).max() and np.abs(rM - np.eye(p.K)).max() > 0.05
    check("M", np64(M), rM, TOL_STATE)
    check("S~", np64(S), rS, TOL_STATE)


def test_summary_varlen_matches_oracle(gpu_lib):
    p = ks.make("varlen", lens=[20, 0, 129], H=2, cache_rows=3, n_invalid=0)
    p.state_indices, p.h0 = None, None
    M, S = _summary_gpu(gpu_lib, p)
    rM, rS = orc.segment_summary(p)
    check("M", np64(M), rM, TOL_STATE)
    check("S~", np64(S), rS, TOL_STATE)


def test_merge_matches_oracle(gpu_lib):
    rng = np.random.default_rng(7)
    P, H, K, V = 5, 3, 128, 128
    M = (rng.standard_normal((P, H, K, K)) / math.sqrt(K)).astype(np.float32)
    S = (rng.standard_normal((P, H, K, V)) * 0.02).astype(np.float32)
    X = (rng.standard_normal((H, K, V)) * 0.02).astype(np.float32)
    st = torch.from_numpy(X.copy()).cuda()
    gpu_lib.kda_summary_merge(torch.from_numpy(M).cuda(), torch.from_numpy(S).cuda(), st)
    torch.cuda.synchronize()
    check("merged", np64(st), orc.summary_merge(M, S, X), 1e-5)


def _segment_case(kda, p, heads):
    """Summaries of the preceding segments -> merge -> this segment's summary and fwd."""
    say(f"case segment T={p.T} H={p.Hv} heads={heads}")
    prev = ks.preceding_summary_inputs(p)
    Mp, Sp_unused = _summary_gpu(kda, prev)
    rMp, _ = orc.segment_summary(prev, heads=heads)
    check("preceding M", np64(Mp)[:, heads], rMp[:, heads], TOL_STATE)
    S_prev = p.extras["prev_S"]
    state = torch.zeros((p.Hv, p.K, p.V), dtype=torch.float32, device="cuda")
    kda.kda_summary_merge(Mp, torch.from_numpy(S_prev).cuda(), state)
    torch.cuda.synchronize()
    r_state = orc.summary_merge(rMp[:, heads], S_prev[:, heads])
    check("rebuilt state", np64(state)[heads], r_state, TOL_STATE)
    t = to_torch(p)
    M, S = _summary_gpu(kda, p, t)
    rM, rS = orc.segment_summary(p, heads=heads)
    if np.abs(rM[:, heads]).max() == 0.0:
        # The layer gate (A_log up to ln 16) decays the transition to exact
        # zeros over a segment of this length: the check is then that the GPU
        # returns exact zeros too.  Non-trivial M over many chunks is checked
        # by test_summary_deep_transition.
        say("  segment M: the oracle's transition is exactly zero; GPU must match it exactly")
        assert np.abs(np64(M)[:, heads]).max() == 0.0
    else:
        check("segment M", np64(M)[:, heads], rM[:, heads], TOL_STATE)
    check("segment S~", np64(S)[:, heads], rS[:, heads], TOL_STATE)
    p.h0 = state.cpu().numpy()[None]
    t["h0"] = state[None].contiguous()
    o, f = run_fwd(kda, p, t)
    ro, rf = orc.forward(p, heads=heads)
    check("o", np64(o)[..., heads, :], ro[..., heads, :], TOL_BF16_OUT)
    check("final_state", np64(f)[:, heads], rf[:, heads], TOL_STATE)
    # the segment's summary applied to the rebuilt state gives its final state
    check("M X + S~", np64(torch.matmul(M[0], state) + S[0])[heads], np64(f)[0, heads], 1e-4)


def test_segment_small(gpu_lib):
    _segment_case(gpu_lib, ks.make("segment", T=300, H=2), heads=[0, 1])


# --------------------------------------------------------- full-size, sampled
def test_layer_full_all_heads(gpu_lib):
    """The benchmark workload at full size, every head against the oracle (its
    heads span slowly and fast decaying gates, so both diagonal-tile forms)."""
    fwd_case(gpu_lib, ks.make("layer"))


def test_varlen_full_sampled(gpu_lib):
    fwd_case(gpu_lib, ks.make("varlen"), heads=[0, 21])


def test_gqa_full_sampled(gpu_lib):
    fwd_case(gpu_lib, ks.make("gqa"), heads=[0, 5, 63])


def test_segment_full_sampled(gpu_lib):
    _segment_case(gpu_lib, ks.make("segment"), heads=[3])
