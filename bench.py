"""Benchmark: chunkwise KDA forward on one MI355X.

Workload: Kimi-Linear-shaped layer forward, B=1, T=8192, H=32, dk=dv=128,
bf16 q/k/v/gate/beta, in-kernel gate + L2Norm + sigmoid, fp32 initial state
(seeded synthetic inputs, resident in HBM before timing starts).  One step =
one kda_chunk_fwd call (chunk-local kernel + state-scan/output kernel).

Prints ONE JSON line on stdout.  Progress goes to stderr.
"""
import argparse
import ctypes
import hashlib
import json
import os
import platform
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


def algorithmic(B, T, H, K, V, Hk=None):
    """FLOP and minimum HBM bytes of one forward (per (token, v-head) figures)."""
    Hk = Hk or H
    th = B * T * H
    flop = th * (2 * BT * (3 * K + 2 * V) + 6 * K * V)
    # read q, k (per q/k head), v, g_raw, beta; write o; bf16
    tok_bytes = B * T * (Hk * 2 * K * 2 + H * (K * 2 + V * 2 + 2 + V * 2))
    state_bytes = 2 * B * H * K * V * 4     # h0 in, final state out (fp32)
    return flop, tok_bytes + state_bytes


class HipEvents:
    """Raw hipEvent_t handles from the HIP runtime (the library records them)."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            out.append(h.value)
        return out

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def cpu_baseline(p, sample_tokens, repeats):
    """The fp64 oracle on the first `sample_tokens` tokens of every head, run
    `repeats` times (the rate is over all runs)."""
    from threadpoolctl import threadpool_limits

    import dataclasses

    from oracle import kda_oracle as orc
    sample_tokens = min(sample_tokens, p.T)
    sl = slice(0, sample_tokens)
    sub = dataclasses.replace(p, T=sample_tokens, q=p.q[:, sl], k=p.k[:, sl], v=p.v[:, sl],
                              g=p.g[:, sl], beta=p.beta[:, sl])
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        for _ in range(repeats):
            orc.forward(sub)
        dt = time.perf_counter() - t0
    return {"value": repeats * sample_tokens * p.B / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {sample_tokens} tokens x all {p.Hv} heads of the workload, {repeats} runs "
                      f"({dt:.1f} s, numpy fp64 token recurrence, 1 thread)",
            "host_cpu": platform.processor() or platform.machine(),
            "host_cores_available": len(os.sched_getaffinity(0))}


def source_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "chunkwise_kimi_delta_amd", "csrc"))):
        with open(os.path.join(ROOT, "chunkwise_kimi_delta_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()


def traffic_for(kernel):
    """HBM bytes per launch from committed PMC counters, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    e = d.get(kernel)
    if not e or e.get("source_sha256") != source_hash():
        return None
    return e["bytes_per_launch"]


def summarize_pmc(fetch_csv, write_csv, copy_bytes, out_json):
    """Per-launch HBM bytes of each KDA kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE
    runs, scaled by what the same counters read for the calibration copy of
    `copy_bytes` bytes (read once, written once).  Writes `out_json` and
    returns a text summary."""
    import csv
    import statistics

    def per_kernel(path):
        vals = {}
        for r in csv.DictReader(open(path)):
            vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_csv), per_kernel(write_csv)
    copy_name = max((k for k in fetch if "copy" in k.lower()), key=lambda k: max(fetch[k]))
    cf = copy_bytes / (max(fetch[copy_name]) * 1024.0)
    cw = copy_bytes / (max(write[copy_name]) * 1024.0)
    out = {"calibration": {"kernel": copy_name, "bytes": copy_bytes, "fetch_factor": cf,
                           "write_factor": cw}}
    lines = [f"calibration copy {copy_name}: {copy_bytes / 1e6:.1f} MB read + written; "
             f"FETCH_SIZE factor {cf:.4f}, WRITE_SIZE factor {cw:.4f} (bytes per counted byte)"]
    for short, key in (("intra_kernel", "intra_kernel"), ("scan_kernel", "scan_kernel")):
        names = [k for k in fetch if key in k]
        if not names:
            continue
        k = names[0]
        fb = statistics.mean(fetch[k]) * 1024.0 * cf
        wb = statistics.mean(write[k]) * 1024.0 * cw
        out[short] = {"kernel": k, "fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                      "source_sha256": source_hash()}
        lines.append(f"{short}: fetch {fb / 1e6:.1f} MB + write {wb / 1e6:.1f} MB = "
                     f"{(fb + wb) / 1e6:.1f} MB per launch ({len(fetch[k])} launches)")
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--cpu-repeats", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibration-copy-mb", type=int, default=0,
                    help="after timing, run a plain device copy of this many MB (PMC calibration)")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="summarise rocprofv3 FETCH_SIZE / WRITE_SIZE runs and exit")
    args = ap.parse_args()
    if args.summarize_pmc:
        print(summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1],
                            args.calibration_copy_mb * 1024 * 1024,
                            os.path.join(ROOT, "profiles", "pmc_traffic.json")))
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import kda_synth as ks
    from chunkwise_kimi_delta_amd import kda
    from kda_synth.torch_io import flag_kwargs, to_torch

    kda.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log("generating inputs ...")
    p = ks.make("layer")
    t = to_torch(p, dev)
    B, T, H, K, V = p.B, p.T, p.Hv, p.K, p.V
    o = torch.empty_like(t["v"])
    final = torch.empty((B, H, K, V), dtype=torch.float32, device=dev)
    ws = torch.empty(kda.workspace_bytes(t["q"], t["v"]), dtype=torch.uint8, device=dev)
    kw = flag_kwargs(p)

    def step():
        kda.kda_chunk_fwd(t["q"], t["k"], t["v"], t["g"], t["beta"], scale=p.scale, A_log=t["A_log"],
                          dt_bias=t["dt_bias"], initial_state=t["h0"], o=o, final_state=final,
                          workspace=ws, **kw)

    log(f"warmup {args.warmup} ...")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    hev = HipEvents()
    evs = hev.create(3 * args.steps)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} steps ...")
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        kda.kda_set_stage_events(evs[3 * i], evs[3 * i + 1], evs[3 * i + 2])
        step()
    end.record()
    torch.cuda.synchronize()
    kda.kda_set_stage_events(None, None, None)
    total_ms = start.elapsed_time(end)
    intra = [hev.elapsed_ms(evs[3 * i], evs[3 * i + 1]) for i in range(args.steps)]
    scan = [hev.elapsed_ms(evs[3 * i + 1], evs[3 * i + 2]) for i in range(args.steps)]
    hev.destroy(evs)

    if args.calibration_copy_mb:
        src = torch.empty(args.calibration_copy_mb * 1024 * 1024, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms = total_ms / args.steps
    flop, nbytes = algorithmic(B, T, H, K, V)
    tok_s = B * T / (ms * 1e-3)
    tflops = flop / (ms * 1e-3) / 1e12
    hbm_gbs = nbytes / (ms * 1e-3) / 1e9
    t_intra, t_scan = sum(intra) / len(intra), sum(scan) / len(scan)
    dom_name, dom_ms = (("scan_kernel", t_scan) if t_scan >= t_intra else ("intra_kernel", t_intra))
    achieved = nbytes / (dom_ms * 1e-3) / 1e9
    traffic = traffic_for(dom_name)
    log(f"step {ms*1e3:.1f} us: intra {t_intra*1e3:.1f} us, scan {t_scan*1e3:.1f} us")

    res = {
        "metric": METRIC, "value": tok_s, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "Kimi-Linear-shaped KDA layer forward", "B": B, "T": T, "H": H,
                   "dk": K, "dv": V, "chunk": BT, "gate": "in-kernel -exp(A_log)*softplus(g+dt_bias)",
                   "l2norm": True, "beta_sigmoid": True, "initial_state": "fp32"},
        "tflops": tflops, "mfma_peak_frac": tflops / PEAK_BF16_TFLOPS,
        "hbm_algorithmic_gbs": hbm_gbs, "hbm_roofline_frac": hbm_gbs / PEAK_HBM_GBS,
        "kernels_us": {"intra_kernel": t_intra * 1e3, "scan_kernel": t_scan * 1e3},
        "roofline": {"bound": "hbm", "kernel": dom_name, "achieved": achieved, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_sample_tokens} tokens x {args.cpu_repeats} ...")
        res["cpu_baseline"] = cpu_baseline(p, args.cpu_sample_tokens, args.cpu_repeats)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
