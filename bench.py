"""Benchmark: chunkwise KDA forward on one MI355X.

Default workload (the metric's): Kimi-Linear-shaped layer forward, B=1,
T=8192, H=32, dk=dv=128, bf16 q/k/v/gate/beta, in-kernel gate + L2Norm +
sigmoid, fp32 initial state.  ``--workload`` selects the other seeded
workloads (tiny, varlen, segment, gqa) with the same protocol.  Inputs are
synthetic, seeded and resident in HBM before timing starts.  One step = one
pass of the whole path over the workload: ``kda_chunk_fwd`` (chunk-local
kernel + state-scan/output kernel); for the segment workload the segment's
summary, the merge of the seven preceding summaries and the forward from the
rebuilt state.

Every step records HIP events on the stream the kernels run on, so step and
per-kernel times are reported as mean, median, min and p90.  Prints ONE JSON
line on stdout; progress goes to stderr.
"""
import argparse
import ctypes
import dataclasses
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "chunk-KDA fwd tokens/s + TFLOP/s (% bf16 MFMA peak), H=32 d=128 T=8192"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
BT = 64


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def flop_per_token_head(K, V):
    """Akk, Aqk and w (BT*K each), u and the intra-chunk output (BT*V each),
    w h, qg h and kg^T v_new (K*V each), two flops per multiply-add."""
    return 2 * BT * (3 * K + 2 * V) + 6 * K * V


def nbytes(a, es):
    return 0 if a is None else int(a.size) * es


def token_bytes(p, with_q=True, with_o=True):
    """Minimum HBM bytes of one pass over a problem's token tensors: q (optional),
    k, v, gate, beta read once, o (optional) written once."""
    es = 2 if p.dtype == "bf16" else 4
    b = nbytes(p.k, es) + nbytes(p.v, es) + nbytes(p.g, es) + nbytes(p.beta, es)
    if with_q:
        b += nbytes(p.q, es)
    if with_o:
        b += nbytes(p.v, es)
    b += nbytes(p.A_log, 4) + nbytes(p.dt_bias, 4)
    return b


def token_heads(p):
    return (p.B * p.T if p.layout == "bsnd" else p.T) * p.Hv


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime (recorded by the library on
    the stream its kernels run on, or by ``record`` here)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.all = []

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            out.append(h.value)
        self.all += out
        return out

    def record(self, ev, stream):
        assert self.hip.hipEventRecord(ev, stream) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self):
        for e in self.all:
            self.hip.hipEventDestroy(e)
        self.all = []


def stats_us(xs_ms):
    xs = sorted(x * 1e3 for x in xs_ms)
    p90 = xs[min(len(xs) - 1, int(round(0.9 * (len(xs) - 1))))]
    return {"mean": sum(xs) / len(xs), "median": statistics.median(xs), "min": xs[0], "p90": p90}


# ------------------------------------------------------------------ workloads
def setup(name, dev, hev, scan_segments=0):
    """Inputs on the device and a step function for one workload.

    Returns (step(marks) -> None, meta).  ``step`` records the events of the
    list ``marks`` (None: no events) at its stage boundaries; meta holds the
    problem, the algorithmic FLOP and bytes, each kernel's own algorithmic
    bytes and the names of the intervals between consecutive marks."""
    import numpy as np
    import torch

    import kda_synth as ks
    from chunkwise_kimi_delta_amd import kda
    from kda_synth.torch_io import flag_kwargs, to_torch

    p = ks.make("gqa" if name == "gqa_train" else name)
    t = to_torch(p, dev)
    kw = flag_kwargs(p)
    stream = torch.cuda.current_stream(dev).cuda_stream
    K, V, Hv = p.K, p.V, p.Hv
    N = p.num_seqs
    state = Hv * K * V * 4
    fpt = flop_per_token_head(K, V)
    th = token_heads(p)

    if name == "segment":
        prev = ks.preceding_summary_inputs(p)
        tp = to_torch(prev, dev)
        Mp, _ = kda.kda_segment_summary(tp["k"], tp["v"], tp["g"], tp["beta"], cu_seqlens=tp["cu"],
                                        cu_seqlens_host=tp["cu_host"], **flag_kwargs(prev))
        S_prev = torch.from_numpy(np.ascontiguousarray(p.extras["prev_S"])).to(dev)
        P = Mp.shape[0]
        rebuilt = torch.zeros((1, Hv, K, V), dtype=torch.float32, device=dev)
        o = torch.empty_like(t["v"])
        final = torch.empty((1, Hv, K, V), dtype=torch.float32, device=dev)
        M = torch.empty((1, Hv, K, K), dtype=torch.float32, device=dev)
        St = torch.empty((1, Hv, K, V), dtype=torch.float32, device=dev)
        ws = torch.empty(kda.workspace_bytes(t["q"], t["v"]), dtype=torch.uint8, device=dev)

        def step(m):
            kda.kda_segment_summary(t["k"], t["v"], t["g"], t["beta"], A_log=t["A_log"],
                                    dt_bias=t["dt_bias"], M=M, S_tilde=St, workspace=ws,
                                    stage_events=None if m is None else m[0:3], **kw)
            rebuilt.zero_()
            if m is not None:
                hev.record(m[3], stream)
            kda.kda_summary_merge(Mp, S_prev, rebuilt[0])
            kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=p.scale,
                              A_log=t["A_log"], dt_bias=t["dt_bias"], initial_state=rebuilt,
                              o=o, final_state=final, workspace=ws,
                              stage_events=None if m is None else m[4:7], **kw)

        flop = 2 * fpt * th + P * Hv * 2 * K * K * V
        b_sum = token_bytes(p, with_q=False, with_o=False) + Hv * K * (K + V) * 4
        b_merge = P * Hv * K * (K + V) * 4 + 2 * state
        b_fwd = token_bytes(p) + 2 * state
        meta = dict(p=p, flop=flop, bytes=b_sum + b_merge + b_fwd, nmarks=7,
                    intervals={"summary_chunk_local": (0, 1), "summary_scan": (1, 2),
                               "merge": (3, 4), "fwd_chunk_local": (4, 5), "fwd_scan": (5, 6)},
                    own_bytes={"summary_chunk_local": token_bytes(p, with_q=False, with_o=False),
                               "summary_scan": Hv * K * (K + V) * 4, "merge": b_merge,
                               "fwd_chunk_local": token_bytes(p, with_o=False),
                               "fwd_scan": nbytes(p.v, 2 if p.dtype == "bf16" else 4) + 2 * state},
                    config={"T": p.T, "H": Hv, "dk": K, "dv": V, "preceding_summaries": P})
        return step, meta

    if name == "gqa_train":
        # forward, then the backward given seeded do ~ N(0, 1) and dht ~ N(0, 0.01^2)
        rng = np.random.default_rng(2024)
        do = torch.from_numpy(ks.bf16_round(rng.standard_normal(p.v.shape).astype(np.float32))).to(
            dev, torch.bfloat16)
        dht = torch.from_numpy((rng.standard_normal((N, Hv, K, V)) * 0.01).astype(np.float32)).to(dev)
        o = torch.empty_like(t["v"])
        final = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev)
        ws = torch.empty(kda.workspace_bytes(t["q"], t["v"]), dtype=torch.uint8, device=dev)
        bws = torch.empty(kda_bwd_ws_bytes(kda, p, t), dtype=torch.uint8, device=dev)

        def step(m):
            kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=p.scale, A_log=t["A_log"],
                              dt_bias=t["dt_bias"], initial_state=t["h0"], o=o, final_state=final,
                              workspace=ws, stage_events=None if m is None else m[0:3], **kw)
            g = kda.kda_chunk_bwd(t["q"], t["k"], t["v"], t["g"], t["beta"], do, dht=dht, scale=p.scale,
                                  A_log=t["A_log"], dt_bias=t["dt_bias"], initial_state=t["h0"],
                                  workspace=bws, **kw)
            if m is not None:
                hev.record(m[3], stream)
            del g

        es = 2
        fwd_b = token_bytes(p) + 2 * N * state
        # backward: q, k, v, g, beta, do read; dq, dk, dv, dg, dbeta written in fp32; h0, dht read, dh0 written
        bwd_b = (token_bytes(p, with_o=False) + nbytes(p.v, es) + nbytes(p.q, 4) + nbytes(p.k, 4)
                 + nbytes(p.v, 4) + nbytes(p.g, 4) + nbytes(p.beta, 4) + 3 * N * state)
        meta = dict(p=p, flop=3 * fpt * th, bytes=fwd_b + bwd_b, nmarks=4,
                    intervals={"fwd_intra_kernel": (0, 1), "fwd_scan_kernel": (1, 2), "backward": (2, 3)},
                    own_bytes={"fwd_intra_kernel": token_bytes(p, with_o=False),
                               "fwd_scan_kernel": nbytes(p.v, es) + 2 * N * state, "backward": bwd_b},
                    config={"B": p.B, "T": p.T, "Hk": p.Hk, "H": Hv, "dk": K, "dv": V,
                            "step": "forward + backward (flop counted as 3x the forward's)"})
        return step, meta

    if name == "decode":
        o = torch.empty_like(t["v"])
        n_valid = int((p.state_indices >= 0).sum())

        def step(m):
            if m is not None:
                hev.record(m[0], stream)
            kda.kda_recurrent_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=p.scale,
                                  A_log=t["A_log"], dt_bias=t["dt_bias"], initial_state=t["h0"],
                                  cu_seqlens=t["cu"], cu_seqlens_host=t["cu_host"],
                                  state_indices=t["state_indices"], o=o, **kw)
            if m is not None:
                hev.record(m[1], stream)

        # per token and head: K*V for the decay, 2*K*V each for S^T k, the write and S^T q
        meta = dict(p=p, flop=th * 7 * K * V, bytes=token_bytes(p) + 2 * n_valid * state, nmarks=2,
                    intervals={"recurrent_kernel": (0, 1)},
                    own_bytes={"recurrent_kernel": token_bytes(p) + 2 * n_valid * state},
                    config={"seqs": N, "tokens_per_seq": p.T // N, "H": Hv, "dk": K, "dv": V,
                            "state_cache_rows": int(p.h0.shape[0]), "valid_indices": n_valid})
        return step, meta

    cache = p.state_indices is not None
    o = torch.empty_like(t["v"])
    if cache:
        final = t["h0"]
        n_states = 2 * int((p.state_indices >= 0).sum())
    else:
        final = torch.empty((N, Hv, K, V), dtype=torch.float32, device=dev)
        n_states = N * (2 if p.h0 is not None else 1)
    ws = torch.empty(kda.workspace_bytes(t["q"], t["v"], t["cu_host"], scan_segments=scan_segments),
                     dtype=torch.uint8, device=dev)

    def step(m):
        kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=p.scale, A_log=t["A_log"],
                          dt_bias=t["dt_bias"], initial_state=t["h0"], cu_seqlens=t["cu"],
                          cu_seqlens_host=t["cu_host"], state_indices=t["state_indices"], o=o,
                          final_state=final, workspace=ws, stage_events=m, scan_segments=scan_segments,
                          **kw)

    es = 2 if p.dtype == "bf16" else 4
    meta = dict(p=p, flop=fpt * th, bytes=token_bytes(p) + n_states * state, nmarks=3,
                intervals={"intra_kernel": (0, 1), "scan_kernel": (1, 2)},
                scan_segments=scan_segments,
                own_bytes={"intra_kernel": token_bytes(p, with_o=False),
                           "scan_kernel": nbytes(p.v, es) + n_states * state},
                config={"B": p.B, "T": p.T, "Hk": p.Hk, "H": Hv, "dk": K, "dv": V})
    if name == "varlen":
        meta["config"].update(seqs=N, tokens=p.T, state_cache_rows=int(p.h0.shape[0]))
    return step, meta


def kda_bwd_ws_bytes(kda, p, t):
    """Backward workspace bytes for a problem's shapes (through the C ABI)."""
    import ctypes
    lib = kda.load()
    from kda_synth.torch_io import flag_kwargs
    fl = flag_kwargs(p)
    flags = ((kda.KDA_GATE_IN_KERNEL if fl["gate_in_kernel"] else 0) | (kda.KDA_SAFE_GATE if fl["safe_gate"] else 0)
             | (kda.KDA_QK_L2NORM if fl["qk_l2norm"] else 0) | (kda.KDA_BETA_SIGMOID if fl["beta_sigmoid"] else 0))
    pr, _ = kda.make_problem(t["q"], t["v"], scale=p.scale, flags=flags, eps=p.eps, lower_bound=p.lower_bound,
                             cu_host=t["cu_host"])
    sz = ctypes.c_size_t()
    kda._check(lib.kda_chunk_bwd_workspace_size(ctypes.byref(pr), ctypes.byref(sz)))
    return sz.value


WORKLOAD_TEXT = {
    "tiny": "tiny KDA forward (fp32, precomputed gate, pre-normalised q/k)",
    "layer": "Kimi-Linear-shaped KDA layer forward",
    "varlen": "packed varlen prefill with a state cache (16 sequences, lengths U[512, 8192])",
    "segment": "one segment of a 1M-token sequence: summary + merge of 7 preceding summaries + forward",
    "gqa": "GQA long batch forward (16 q/k heads shared by 64 value heads, safe gate)",
    "decode": "decode step: one token for each of 64 sequences, state cache updated in place",
    "longseq": "long sequence over few heads (B=1, T=65536, H=4): segment-parallel scan",
    "gqa_train": "GQA long batch forward + backward (dq, dk, dv, dbeta, dg, dA_log, ddt_bias, dh0)",
}


# ------------------------------------------------------------------ baselines
def cpu_baseline(p, target_token_heads):
    """The fp64 oracle on a bounded sample of the workload: the first t tokens
    of every sequence over all value heads, t chosen so the sample holds about
    ``target_token_heads`` token-heads (repeated when the whole workload is
    smaller).  The rate is scaled to tokens/s of the whole workload
    (token-heads/s over the number of value heads)."""
    from threadpoolctl import threadpool_limits

    from oracle import kda_oracle as orc
    N = p.num_seqs
    lens = [b - a for (_, a, b) in p.seq_bounds()]
    t_max = min(max(lens), max(1, target_token_heads // (N * p.Hv)))
    per_run = sum(min(L, t_max) for L in lens) * p.Hv
    repeats = max(1, round(target_token_heads / per_run))
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for _ in range(repeats):
            orc.forward(p, t_max=t_max)
        dt = time.perf_counter() - t0
    return {"value": per_run * repeats / dt / p.Hv, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {t_max} tokens of each of {N} sequence(s) x all {p.Hv} value heads, "
                      f"{repeats} run(s) ({dt:.1f} s, numpy fp64 token recurrence, 1 thread)",
            "host_cpu": platform.processor() or platform.machine(),
            "host_cores_available": len(os.sched_getaffinity(0))}


def cpu_baseline_train(p, target_token_heads):
    """The fp64 oracle's forward and backward on the first t tokens of batch 0
    over all value heads (t sized to about ``target_token_heads``), scaled to
    tokens/s of the whole workload like ``cpu_baseline``."""
    import dataclasses

    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import kda_oracle as orc
    t = min(p.T, max(1, target_token_heads // (2 * p.Hv)))
    sub = dataclasses.replace(p, B=1, T=t, q=p.q[:1, :t], k=p.k[:1, :t], v=p.v[:1, :t], g=p.g[:1, :t],
                              beta=p.beta[:1, :t], h0=p.h0[:1])
    do = np.random.default_rng(0).standard_normal(sub.v.shape)
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        orc.forward(sub)
        orc.backward(sub, do, None)
        dt = time.perf_counter() - t0
    return {"value": t / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"forward + backward on the first {t} tokens of batch 0 x all {p.Hv} value heads "
                      f"({dt:.1f} s, numpy fp64, 1 thread)",
            "host_cpu": platform.processor() or platform.machine(),
            "host_cores_available": len(os.sched_getaffinity(0))}


# The sources of the forward step's kernels (the chunk-local kernel, the scan
# and the layouts they share): counters taken on them stay valid while these
# files are unchanged.
FWD_SOURCES = ("kda_common.h", "kda_launch.h", "kda_intra.hip", "kda_scan.hip")


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "chunkwise_kimi_delta_amd", "csrc")
    for f in FWD_SOURCES:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()


def _profile(name):
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    return d if d.get("source_sha256") == source_hash() else None


def traffic_for(kernels):
    """Calibrated HBM bytes per launch summed over ``kernels``, from committed
    PMC counters taken on the current sources (else None)."""
    d = _profile("pmc_traffic.json")
    if not d or any(k not in d for k in kernels):
        return None
    return sum(d[k]["bytes_per_launch"] for k in kernels)


def _per_dispatch_counters(path):
    """{kernel: {counter: [value per dispatch]}} from a rocprofv3 counter CSV
    (one row per dispatch and counter, already summed over the chip)."""
    import csv
    vals = {}
    for r in csv.DictReader(open(path)):
        d = vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], {})
        d[r["Dispatch_Id"]] = d.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return {k: {c: list(d.values()) for c, d in cs.items()} for k, cs in vals.items()}


SHORT = (("intra_kernel", "intra_kernel"), ("scan_kernel", "scan_kernel"))


def summarize_pmc(fetch_csv, write_csv, copy_bytes, out_json):
    """Per-launch HBM bytes of each KDA kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs, scaled by what the same counters read for the calibration copy of
    ``copy_bytes`` bytes (read once, written once: its largest dispatch)."""
    fetch, write = _per_dispatch_counters(fetch_csv), _per_dispatch_counters(write_csv)
    copy_name = max((k for k in fetch if "copy" in k.lower()), key=lambda k: max(fetch[k]["FETCH_SIZE"]))
    cf = copy_bytes / (max(fetch[copy_name]["FETCH_SIZE"]) * 1024.0)
    cw = copy_bytes / (max(write[copy_name]["WRITE_SIZE"]) * 1024.0)
    out = {"source_sha256": source_hash(),
           "calibration": {"kernel": copy_name, "bytes": copy_bytes, "fetch_factor": cf, "write_factor": cw}}
    lines = [f"calibration copy {copy_name}: {copy_bytes / 1e6:.1f} MB read + written; "
             f"FETCH_SIZE factor {cf:.4f}, WRITE_SIZE factor {cw:.4f} (bytes per counted byte)"]
    for short, key in SHORT:
        names = [k for k in fetch if key in k]
        if not names:
            continue
        k = names[0]
        fb = statistics.mean(fetch[k]["FETCH_SIZE"]) * 1024.0 * cf
        wb = statistics.mean(write[k]["WRITE_SIZE"]) * 1024.0 * cw
        out[short] = {"kernel": k, "fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                      "launches": len(fetch[k]["FETCH_SIZE"])}
        lines.append(f"{short}: fetch {fb / 1e6:.1f} MB + write {wb / 1e6:.1f} MB = "
                     f"{(fb + wb) / 1e6:.1f} MB per launch ({len(fetch[k]['FETCH_SIZE'])} launches)")
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
    return "\n".join(lines)


CU_NUM, SIMD_NUM, XCD_NUM, CLOCK_GHZ = 256, 1024, 8, 2.4


def summarize_mfma(csv_path, out_json):
    """Matrix-core and vector-ALU activity per kernel from one rocprofv3 --pmc
    run of SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_{BF16,F16,F32}
    (and _F8 where collected), SQ_INSTS_VALU, SQ_ACTIVE_INST_VALU,
    SQ_BUSY_CU_CYCLES and GRBM_GUI_ACTIVE.  GRBM_GUI_ACTIVE is summed over the
    XCDs: one XCD's count is the kernel's cycles.  MFMA util = busy cycles /
    (kernel cycles x SIMDs); VALU active = 4 x SQ_ACTIVE_INST_VALU (quad-cycles)
    / (kernel cycles x SIMDs); each MOPS counts 512 flop.  bf16 and fp16 products
    share one dense peak, so their sum is the 16-bit fraction of it."""
    data = _per_dispatch_counters(csv_path)
    out = {"source_sha256": source_hash()}
    lines = []
    for short, key in SHORT:
        names = [k for k in data if key in k]
        if not names:
            continue
        c = {n: statistics.mean(v) for n, v in data[names[0]].items()}
        cyc = c.get("GRBM_GUI_ACTIVE", 0.0) / XCD_NUM
        us = cyc / (CLOCK_GHZ * 1e3)
        util = c.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0) / (cyc * SIMD_NUM) if cyc else None
        flops = {d: c.get(f"SQ_INSTS_VALU_MFMA_MOPS_{d}", 0.0) * 512 for d in ("BF16", "F16", "F32", "F8")}
        valu = c.get("SQ_ACTIVE_INST_VALU", 0.0) * 4 / (cyc * SIMD_NUM) if cyc else None
        f16 = flops["BF16"] + flops["F16"]
        f16_frac = f16 / (us * 1e-6) / (PEAK_BF16_TFLOPS * 1e12) if us else None
        out[short] = {"kernel": names[0], "counters_mean_per_dispatch": c, "kernel_cycles": cyc,
                      "kernel_us_from_counter": us, "mfma_busy_frac": util, "mfma_flop": flops,
                      "mfma16_flop_frac_of_peak": f16_frac, "valu_insts": c.get("SQ_INSTS_VALU"),
                      "valu_active_frac": valu}
        lines.append(f"{short}: {us:.1f} us; MFMA busy {100 * util:.1f}% of SIMD cycles; MFMA flop bf16 "
                     f"{flops['BF16'] / 1e9:.2f} G + fp16 {flops['F16'] / 1e9:.2f} G ({100 * f16_frac:.1f}% "
                     f"of the 16-bit peak over the kernel), f32 {flops['F32'] / 1e9:.3f} G, "
                     f"f8 {flops['F8'] / 1e9:.3f} G; VALU insts "
                     f"{c.get('SQ_INSTS_VALU', 0) / 1e6:.1f} M, VALU active {100 * valu:.1f}% of SIMD cycles")
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
    return "\n".join(lines)


# ----------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="layer", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--scan-segments", type=int, default=0,
                    help="0: the library chooses the segment-parallel scan, 1: off, n > 1: forced")
    ap.add_argument("--cpu-token-heads", type=int, default=524288,
                    help="token-heads of the oracle's CPU-baseline sample (about 10 s at one thread)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="after timing, run a plain device copy of this many MB (PMC calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs and exit")
    ap.add_argument("--summarize-mfma", metavar="COUNTER_CSV",
                    help="summarise a rocprofv3 run of the matrix-core counters and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1],
                            args.calibration_copy_mb * 1024 * 1024,
                            os.path.join(ROOT, "profiles", "pmc_traffic.json")))
        return
    if args.summarize_mfma:
        print(summarize_mfma(args.summarize_mfma, os.path.join(ROOT, "profiles", "pmc_mfma.json")))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from chunkwise_kimi_delta_amd import kda

    kda.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    hev = HipEvents()
    log(f"generating inputs ({args.workload}) ...")
    step, meta = setup(args.workload, dev, hev, args.scan_segments)
    p = meta["p"]

    log(f"warmup {args.warmup} ...")
    for _ in range(args.warmup):
        step(None)
    torch.cuda.synchronize()

    nm = meta["nmarks"]
    evs = hev.create(nm * args.steps)
    marks = [evs[nm * i: nm * (i + 1)] for i in range(args.steps)]
    log(f"timing {args.steps} steps ...")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(marks[i])
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    steps_ms = [hev.elapsed_ms(m[0], m[-1]) for m in marks]
    kern = {k: [hev.elapsed_ms(m[a], m[b]) for m in marks] for k, (a, b) in meta["intervals"].items()}
    hev.destroy()

    if args.calibration_copy_mb:
        src = torch.empty(args.calibration_copy_mb * 1024 * 1024, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    st = stats_us(steps_ms)
    ms = wall_s * 1e3 / args.steps                  # whole-job time per step (host clock)
    tokens = p.B * p.T if p.layout == "bsnd" else p.T
    tok_s = tokens / (ms * 1e-3)
    tflops = meta["flop"] / (ms * 1e-3) / 1e12
    step_gbs = meta["bytes"] / (st["mean"] * 1e-6) / 1e9
    kernels = {}
    for k, xs in kern.items():
        ks_ = stats_us(xs)
        ob = meta["own_bytes"][k]
        kernels[k] = {**{f"us_{n}": v for n, v in ks_.items()}, "own_algorithmic_bytes": ob,
                      "own_gbs": ob / (ks_["mean"] * 1e-6) / 1e9,
                      "own_hbm_frac": ob / (ks_["mean"] * 1e-6) / 1e9 / PEAK_HBM_GBS}
    log(f"step {st['mean']:.1f} us (median {st['median']:.1f}, min {st['min']:.1f}, p90 {st['p90']:.1f}); "
        + ", ".join(f"{k} {v['us_mean']:.1f} us" for k, v in kernels.items()))

    traffic = traffic_for(["intra_kernel", "scan_kernel"]) if args.workload == "layer" else None
    mfma = _profile("pmc_mfma.json") if args.workload == "layer" else None
    res = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": p.dtype, "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "chunk": BT, **meta["config"],
                   "scan_segments": args.scan_segments,
                   "gate": "in-kernel -exp(A_log)*softplus(g+dt_bias)" if p.gate_in_kernel else "precomputed",
                   "safe_gate": p.safe_gate, "l2norm": p.l2norm, "beta_sigmoid": p.beta_sigmoid},
        "step_us": st, "tflops": tflops, "mfma_peak_frac": tflops / PEAK_BF16_TFLOPS,
        "algorithmic_flop": meta["flop"], "algorithmic_bytes": meta["bytes"],
        "hbm_roofline_frac": meta["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": "whole step (" + " + ".join(kernels) + ")",
                     "achieved": step_gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": step_gbs / PEAK_HBM_GBS, "traffic": traffic},
    }
    if mfma:
        res["mfma_counters"] = {k: {"mfma_busy_frac": v["mfma_busy_frac"],
                                    "mfma16_flop_frac_of_peak": v.get("mfma16_flop_frac_of_peak"),
                                    "valu_active_frac": v["valu_active_frac"]}
                                for k, v in mfma.items() if isinstance(v, dict) and "mfma_busy_frac" in v}
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on about {args.cpu_token_heads} token-heads ...")
        res["cpu_baseline"] = (cpu_baseline_train(p, args.cpu_token_heads) if args.workload == "gqa_train"
                               else cpu_baseline(p, args.cpu_token_heads))
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
