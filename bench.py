#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

One step = one spec_verify call (row statistics, acceptance tests, first
rejection, final draw, emit) over one batch of synthetic logits already
resident in HBM.  The default workload is the largest named one:
B=256 sequences, K=8 draft tokens, V=152064 vocabulary, bf16 logits,
T=1, sampling (target ~ N(0,4) + log-Zipf bias, draft = target + N(0,2.5)).

Prints one JSON line: verified logits/s (B*(K+1)*V per second), the roofline
of the dominant kernel (k_rowstats: HBM-bound; algorithmic bytes = every target
row and every draft row of sampling sequences read once, V*s bytes per row,
divided by its average duration from HIP events recorded around it on the
launch stream), and the fp64 oracle's throughput on this host as a CPU
baseline.  Run `python bench.py --help` for options.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "verified logits/s (B·(K+1)·V per sec) + achieved HBM GB/s vs peak, 1 GPU"
HBM_PEAK_GBS = 8000.0
KERNEL_SRC = os.path.join(ROOT, "speculative_sampling_verification_06_amd", "csrc", "spec_verify.hip")
PROFILES = os.path.join(ROOT, "profiles")


def _source_sha() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()


def _traffic(workload_name: str):
    """HBM bytes per k_rowstats launch from the committed PMC summary, if it was
    taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"k_rowstats_{workload_name}_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    tot = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not tot or sha.group(1) != _source_sha():
        return None
    return float(tot.group(1))


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="cfg152k", choices=["cfg152k", "cfg128k", "cfg32k", "tiny"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the oracle timing (repeated whole-workload calls)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this size (for PMC byte scaling)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the verify step shards by sequence with no communication, so N GPUs run N "
              "independent copies of this single-GPU step.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from speculative_sampling_verification_06_amd import binding
    from speculative_sampling_verification_06_amd import inputs as I

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    binding.load_library()

    t_gen = time.perf_counter()
    w = I.CONFIGS[args.config]()
    gen_s = time.perf_counter() - t_gen
    print(f"[bench] workload {w.name}: generated in {gen_s:.1f}s", file=sys.stderr, flush=True)

    d = binding.to_device(w, dev)
    a = (d["target"], d["draft"], d["tokens"], d["uniforms"], d["temperature"], d["greedy"])
    call = binding.Bound(*a)                       # checks, outputs and workspace, once
    out = call.verify()
    stream = torch.cuda.current_stream(dev)

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: {n * 4} bytes read, {n * 4} bytes written", file=sys.stderr, flush=True)
        del src, dst

    for _ in range(args.warmup):
        call.stats()
        call.draw()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        evs[i][0].record(stream)
        call.stats()
        evs[i][1].record(stream)
        call.draw()
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    print(f"[bench] timed {K} steps", file=sys.stderr, flush=True)

    ms_per_step = (t1 - t0) * 1e3 / K
    stats_ms = np.array([evs[i][0].elapsed_time(evs[i][1]) for i in range(K)])
    draw_ms = np.array([evs[i][1].elapsed_time(evs[i][2]) for i in range(K)])
    step_ev_ms = stats_ms + draw_ms

    eager = I.eager_bytes(w)
    acc = out["accepted_len"].cpu().numpy()
    gpu = {k: v.cpu().numpy() for k, v in out.items()}
    needed = I.needed_bytes(w, acc)
    stats_avg_s = float(stats_ms.mean()) * 1e-3
    achieved_gbs = eager / stats_avg_s / 1e9

    result = {
        "metric": METRIC,
        "value": w.verified_logits / (ms_per_step * 1e-3),
        "unit": "logits/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "K": w.K, "V": w.V, "logits": I.DTYPE_NAMES[w.dtype],
                   "temperature": w.T, "greedy_sequences": int(w.greedy.sum()), "seed": w.seed,
                   "verified_logits_per_step": w.verified_logits},
        "roofline": {"bound": "hbm", "achieved": achieved_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved_gbs / HBM_PEAK_GBS, "traffic": _traffic(w.name),
                     "kernel": "k_rowstats", "algorithmic_bytes_per_launch": eager,
                     "avg_launch_ms": float(stats_ms.mean())},
        "timing_ms": {"step_events_median": float(np.median(step_ev_ms)),
                      "step_events_p10": float(np.percentile(step_ev_ms, 10)),
                      "step_events_p90": float(np.percentile(step_ev_ms, 90)),
                      "k_rowstats_median": float(np.median(stats_ms)),
                      "decide_search_median": float(np.median(draw_ms))},
        "method": {"accepted_len_hist": np.bincount(acc[acc >= 0], minlength=w.K + 1).tolist(),
                   "mean_accepted": float(acc[acc >= 0].mean()) if (acc >= 0).any() else None,
                   "needed_bytes": needed, "eager_bytes": eager,
                   "useful_bytes_fraction": needed / eager,
                   "page_context": "pages quote 2-3x end-to-end decode speed-up, no hardware stated"},
    }

    if not args.no_cpu_baseline:
        import oracle
        from oracle import parity
        oracle.build(force=False)
        ncpu = len(os.sched_getaffinity(0))
        med_s, used, calls = oracle.time_verify(w, reps=3, min_seconds=args.cpu_seconds, nthreads=ncpu)
        result["cpu_baseline"] = {"value": w.verified_logits / med_s, "unit": "logits/s", "cores": used,
                                  "kind": "oracle",
                                  "sample": f"whole workload ({w.B} sequences), {calls} calls, median "
                                            f"{med_s * 1e3:.1f} ms per call, fp64 C oracle, {used} threads"}
        try:
            rep = parity.compare(w, gpu, oracle.verify(w, nthreads=ncpu))
            result["parity"] = {"ok": True, "flagged": rep["flagged"],
                                "flagged_mismatch": len(rep["flagged_mismatch"]), "invalid": rep["invalid"]}
        except parity.ParityError as e:
            result["parity"] = {"ok": False, "error": str(e)[:500]}
    else:
        result["cpu_baseline"] = None

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
