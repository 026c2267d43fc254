#!/usr/bin/env python3
"""Throughput of the speculative-sampling verify step on one MI355X.

One step = one pass of the verify path (row statistics, acceptance tests,
first rejection, final draw, emit) over one batch of synthetic logits already
resident in HBM.  The default workload is the largest named one:
B=256 sequences, K=8 draft tokens, V=152064 vocabulary, bf16 logits, T=1,
sampling (target ~ N(0,4) + log-Zipf bias, draft = target + N(0,2.5)).
`--config lmhead` times the fused LM-head workload instead (hidden bf16
[32, 6, 4096] x W bf16 [4096, 128256] -> fp32 target logits, then the verify
step against bf16 draft logits; one step = spec_lmhead_verify).

Timing.  The step first runs untimed for --settle-ms (200 ms) of wall time,
so the timed steps see the GPU's steady clock rather than its ramp out of
idle, then W warm-up steps.  The headline (`ms_per_step`, `value`,
`roofline`) comes from K cache-flushed steps: before each, 1 GiB is read on
the launch stream (outside the timed region), so the 256 MB last-level cache
holds none of the inputs and every byte comes from HBM; HIP events on the
launch stream bracket each step.  `hot` repeats the measurement with the
inputs left in the caches by the previous step (K bare steps on the host
clock, and per-kernel events).

Prints one JSON line: verified logits/s (B*(K+1)*V per second), the roofline
of the dominant kernel (algorithmic bytes over its event-timed duration), the
fp64 oracle's throughput on this host as a CPU baseline, parity against the
oracle, and, for the default workload, the same figures for the other named
workloads under `workloads` (B=64 K=5 V=128256 bf16 half greedy, the fused
LM head, B=8 K=4 V=32000 fp32).  The dominant kernel depends on the schedule
the shape gets: under the per-sequence schedule the whole step is one launch
(k_seqg / k_seq), whose algorithmic bytes are the rows the method reaches
plus the draw's pass over row n; under the eager schedule k_rowstats, every
target row and every draft row of sampling sequences read once (V*s bytes
per row); under the lazy schedule the row-statistics launches over the rows
reached; for the LM head k_lmhead (the weight read once, the hidden states,
the fp32 logits written), with its MFMA rate beside it.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "speculative_sampling_verification_06_amd", "csrc")
PROFILES = os.path.join(ROOT, "profiles")


def _source_sha(name: str) -> str:
    return hashlib.sha256(open(os.path.join(CSRC, name), "rb").read()).hexdigest()


def _traffic(kernel: str, workload_name: str, source: str):
    """HBM bytes per launch of `kernel` from the committed PMC summary, if it
    was taken on the current kernel source; else None."""
    path = os.path.join(PROFILES, f"{kernel}_{workload_name}_traffic.txt")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    tot = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not sha or not tot or sha.group(1) != _source_sha(source):
        return None
    return float(tot.group(1))


def _settle(args, torch, *fns):
    """Run the step untimed for at least args.settle_ms of wall time before the
    warmup steps (synchronising every eight steps): a GPU coming out of idle
    ramps its clock over some tens of milliseconds, and the timed steps are
    meant to see the steady clock a serving loop runs at.  The timed region is
    unchanged: the warmup steps, then exactly K steps."""
    if args.settle_ms <= 0:
        return
    t_end = time.perf_counter() + args.settle_ms * 1e-3
    while True:
        for _ in range(8):
            for f in fns:
                f()
        torch.cuda.synchronize()
        if time.perf_counter() >= t_end:
            return


FLUSH_NOTE = ("1 GiB read on the launch stream before every step (outside the events): the 256 MB "
              "last-level cache then holds none of the inputs and no dirty lines")


class _Flush:
    """A 1 GiB read on the launch stream: afterwards the 256 MB last-level
    cache holds none of the step's inputs (a read, not a write: written lines
    would be written back during the timed part)."""

    def __init__(self, torch, stream, mib=1024):
        self.torch = torch
        self.junk = torch.ones(mib << 18, dtype=torch.float32, device=stream.device)
        self.sink = torch.empty((), dtype=torch.float32, device=stream.device)

    def __call__(self):
        self.torch.sum(self.junk, dim=0, out=self.sink)


def _cold_steps(torch, stream, K, parts):
    """K steps, each after a cache flush: HIP events around the whole step
    (ms array), then K more with events between the parts (list of ms arrays,
    one per part)."""
    import numpy as np
    flush = _Flush(torch, stream)
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        flush()
        ev[i][0].record(stream)
        for f in parts:
            f()
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    step = np.array([e[0].elapsed_time(e[1]) for e in ev])
    n = len(parts)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(K)]
    for i in range(K):
        flush()
        ev[i][0].record(stream)
        for k, f in enumerate(parts):
            f()
            ev[i][k + 1].record(stream)
    torch.cuda.synchronize()
    per = [np.array([e[k].elapsed_time(e[k + 1]) for e in ev]) for k in range(n)]
    return step, per


def _hot_steps(torch, stream, K, parts):
    """K bare steps between two synchronizations (host ms per step), then K
    more with events between the parts (an event record is a queue packet of
    its own, so those are not the steps the host clock times)."""
    import numpy as np
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        for f in parts:
            f()
    torch.cuda.synchronize()
    host = (time.perf_counter() - t0) * 1e3 / K
    n = len(parts)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(n + 1)] for _ in range(K)]
    for i in range(K):
        ev[i][0].record(stream)
        for k, f in enumerate(parts):
            f()
            ev[i][k + 1].record(stream)
    torch.cuda.synchronize()
    return host, [np.array([e[k].elapsed_time(e[k + 1]) for e in ev]) for k in range(n)]


def _measure(args, torch, stream, parts, steps):
    """Settle, warm up, then the hot and the cache-flushed timings of one step
    made of `parts` (callables launched in order on `stream`)."""
    _settle(args, torch, *parts)
    for _ in range(args.warmup):
        for f in parts:
            f()
    hot_host, hot_per = _hot_steps(torch, stream, steps, parts)
    cold_step, cold_per = _cold_steps(torch, stream, steps, parts)
    return {"hot_host_ms": hot_host, "hot_per": hot_per, "cold_step": cold_step, "cold_per": cold_per}


def _roofline(np, nbytes, per_ms, kernel, traffic, extra=None):
    """Roofline of the dominant kernel: algorithmic bytes over its mean duration."""
    ms = float(per_ms.mean())
    achieved = nbytes / (ms * 1e-3) / 1e9
    r = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
         "traffic": traffic, "kernel": kernel, "algorithmic_bytes_per_launch": nbytes, "avg_launch_ms": ms}
    if extra:
        r.update(extra)
    return r


def _base_result(w, K, warmup, ms_per_step, dtype_name):
    return {
        "metric": METRIC,
        "value": w.verified_logits / (ms_per_step * 1e-3),
        "unit": "logits/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_name,
        "data": "synthetic",
    }


def _method_stats(w, acc):
    import numpy as np
    ok = acc >= 0
    return {"accepted_len_hist": np.bincount(acc[ok], minlength=w.K + 1).tolist(),
            "mean_accepted": float(acc[ok].mean()) if ok.any() else None,
            "page_context": "pages quote 2-3x end-to-end decode speed-up, no hardware stated"}


SCHEDULES = {1: "eager (one launch streams every row)",
             2: "lazy (one launch per position, reached rows only)",
             3: "seq (one launch: each sequence's workgroups walk its positions, reached rows only, draws in place)"}


def _copy_calibration(args, torch, dev):
    """A device copy of known size for scaling the traffic counters (profiler runs)."""
    if args.copy_calibration_mib <= 0:
        return
    n = args.copy_calibration_mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] copy calibration: {n * 4} bytes read, {n * 4} bytes written", file=sys.stderr, flush=True)
    del src, dst


def hbm_ceiling(torch, np, binding, dev, mib=1024, reps=10):
    """What plain streaming kernels reach on this GPU (sv_hbm_probe): a 1 GiB
    read and a 1 GiB copy (read + write bytes), median over reps, HIP events
    on the launch stream."""
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    words = binding.hbm_probe(binding.PROBE_READ, src)
    out = {}
    for name, fn, nbytes in (("read", lambda: binding.hbm_probe(binding.PROBE_READ, src, words), n * 4),
                             ("copy", lambda: binding.hbm_probe(binding.PROBE_COPY, src, dst), 2 * n * 4)):
        fn()
        fn()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            e1.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = float(np.median(ts))
        out[f"{name}_GBps"] = nbytes / (ms * 1e-3) / 1e9
        out[f"{name}_ms"] = ms
    out["bytes_read"] = n * 4
    out["frac_of_peak"] = {"read": out["read_GBps"] / HBM_PEAK_GBS, "copy": out["copy_GBps"] / HBM_PEAK_GBS}
    out["kernels"] = "sv_hbm_probe read and copy over 1 GiB (16-byte non-temporal accesses), median of 10"
    del src, dst, words
    torch.cuda.synchronize()
    return out


def bench_verify(args, torch, np, binding, I, dev, w=None, steps=None):
    w = I.CONFIGS[args.config]() if w is None else w
    steps = args.steps if steps is None else steps
    print(f"[bench] workload {w.name}: generated", file=sys.stderr, flush=True)
    d = binding.to_device(w, dev)
    a = (d["target"], d["draft"], d["tokens"], d["uniforms"], d["temperature"], d["greedy"])
    call = binding.Bound(*a)                       # checks, outputs and workspace, once
    out = call.verify()
    stream = torch.cuda.current_stream(dev)
    _copy_calibration(args, torch, dev)
    t = _measure(args, torch, stream, (call.stats, call.draw), steps)
    print(f"[bench] {w.name}: timed {steps} hot and {steps} cache-flushed steps", file=sys.stderr, flush=True)

    eager = I.eager_bytes(w)
    acc = out["accepted_len"].cpu().numpy()
    gpu = {k: v.cpu().numpy() for k, v in out.items()}
    sched = binding.schedule(w.B, w.K, w.V, w.dtype)
    lazy = sched == binding.MODE_LAZY
    seq = sched == binding.MODE_SEQ
    # eager: every row once; lazy: the rows reached; seq: the whole step in one
    # launch, so the rows reached plus the draw's second pass over row n
    stats_bytes = I.needed_bytes(w, acc) if seq else (I.reached_bytes(w, acc) if lazy else eager)
    ms = float(t["cold_step"].mean())
    res = _base_result(w, steps, args.warmup, ms, "f32")
    res["config"] = {"workload": w.name, "B": w.B, "K": w.K, "V": w.V, "logits": I.DTYPE_NAMES[w.dtype],
                     "temperature": w.T, "greedy_sequences": int(w.greedy.sum()), "seed": w.seed,
                     "verified_logits_per_step": w.verified_logits,
                     "schedule": SCHEDULES[sched]}
    if seq:
        res["config"]["workgroups_per_sequence"] = binding.seq_groups(w.B, w.K, w.V, w.dtype)
        res["config"]["lookahead"] = binding.seq_lookahead(w.B, w.K, w.V, w.dtype)
    kname = {binding.MODE_EAGER: "k_rowstats", binding.MODE_LAZY: "k_rowstats_lazy",
             binding.MODE_SEQ: "k_seqg" if seq and binding.seq_groups(w.B, w.K, w.V, w.dtype) > 1 else "k_seq"}[sched]
    kdesc = {binding.MODE_EAGER: "k_rowstats",
             binding.MODE_LAZY: "k_rowstats_lazy (all K+1 launches of a step)",
             binding.MODE_SEQ: "k_seq/k_seqg (the whole step, draw included)"}[sched]
    res["roofline"] = _roofline(np, stats_bytes, t["cold_per"][0], kdesc, _traffic(kname, w.name, "spec_verify.hip"),
                                {"timing": FLUSH_NOTE})
    hot = _roofline(np, stats_bytes, t["hot_per"][0], kdesc, None)
    res["hot"] = {"ms_per_step": t["hot_host_ms"], "value": w.verified_logits / (t["hot_host_ms"] * 1e-3),
                  "achieved": hot["achieved"], "frac": hot["frac"], "avg_launch_ms": hot["avg_launch_ms"],
                  "timing": "K bare steps on the host clock; per-kernel events; inputs left in the caches by the previous step"}
    cs = t["cold_step"]
    res["timing_ms"] = {"step_median": float(np.median(cs)), "step_p10": float(np.percentile(cs, 10)),
                        "step_p90": float(np.percentile(cs, 90)),
                        "stats_median": float(np.median(t["cold_per"][0])),
                        "draw_median": float(np.median(t["cold_per"][1])),
                        "hot_stats_median": float(np.median(t["hot_per"][0])),
                        "hot_draw_median": float(np.median(t["hot_per"][1]))}
    res["method"] = _method_stats(w, acc)
    needed = I.needed_bytes(w, acc)
    # the compulsory-eager rate: the bytes an eager verify moves, over the step time
    res["method"].update(needed_bytes=needed, eager_bytes=eager, useful_bytes_fraction=needed / eager,
                         eager_equivalent_GBs=eager / (res["ms_per_step"] * 1e-3) / 1e9)
    return w, gpu, res, None


def bench_lmhead(args, torch, np, binding, I, dev, w=None, steps=None):
    w = I.cfg_lmhead() if w is None else w
    steps = args.steps if steps is None else steps
    print(f"[bench] workload {w.name}: generated", file=sys.stderr, flush=True)
    M, d, V = w.B * (w.K + 1), w.hidden.shape[-1], w.V
    hidden = binding.bf16_tensor(w.hidden, dev)
    wt = binding.lmhead_pack(binding.bf16_tensor(w.w_lm, dev))   # static weight, packed once
    dd = binding.to_device(w, dev)
    call = binding.BoundLMHeadVerify(hidden, wt, dd["draft"], dd["tokens"], dd["uniforms"], w.T, dd["greedy"])
    out = call()
    stream = torch.cuda.current_stream(dev)
    _copy_calibration(args, torch, dev)
    t = _measure(args, torch, stream, (call.gemm, call.rest), steps)
    print(f"[bench] {w.name}: timed {steps} hot and {steps} cache-flushed steps", file=sys.stderr, flush=True)

    acc = out["accepted_len"].cpu().numpy()
    gpu = {k: v.cpu().numpy() for k, v in out.items() if k != "target_logits"}
    gemm_bytes = V * d * 2 + M * d * 2 + M * V * 4
    flops = 2.0 * M * d * V
    ms = float(t["cold_step"].mean())
    res = _base_result(w, steps, args.warmup, ms, "bf16-mfma+f32")
    res["config"] = {"workload": w.name, "B": w.B, "K": w.K, "V": V, "d": d,
                     "logits": "f32 target / bf16 draft",
                     "temperature": w.T, "seed": w.seed, "verified_logits_per_step": w.verified_logits}

    def mfma(per):
        g = float(per.mean()) * 1e-3
        return {"mfma_tflops": flops / g / 1e12, "mfma_frac": flops / g / 1e12 / MFMA_BF16_PEAK_TFLOPS}
    res["roofline"] = _roofline(np, gemm_bytes, t["cold_per"][0], "k_lmhead",
                                _traffic("k_lmhead", w.name, "lmhead.hip"),
                                dict(mfma(t["cold_per"][0]), timing=FLUSH_NOTE))
    hot = _roofline(np, gemm_bytes, t["hot_per"][0], "k_lmhead", None, mfma(t["hot_per"][0]))
    res["hot"] = {"ms_per_step": t["hot_host_ms"], "value": w.verified_logits / (t["hot_host_ms"] * 1e-3),
                  "achieved": hot["achieved"], "frac": hot["frac"], "avg_launch_ms": hot["avg_launch_ms"],
                  "mfma_frac": hot["mfma_frac"],
                  "timing": "K bare steps on the host clock; per-kernel events; inputs left in the caches by the previous step"}
    res["timing_ms"] = {"step_median": float(np.median(t["cold_step"])),
                        "k_lmhead_median": float(np.median(t["cold_per"][0])),
                        "verify_median": float(np.median(t["cold_per"][1])),
                        "hot_k_lmhead_median": float(np.median(t["hot_per"][0])),
                        "hot_verify_median": float(np.median(t["hot_per"][1]))}
    res["method"] = _method_stats(w, acc)
    return w, gpu, res, "lmhead"


def _timed_one(torch, stream, K, fn):
    """A one-part step: host ms per step over K bare steps, then
    the event-timed ms of K more."""
    import numpy as np
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        fn()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    for i in range(K):
        evs[i][0].record(stream)
        fn()
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    return (t1 - t0) * 1e3 / K, np.array([evs[i][0].elapsed_time(evs[i][1]) for i in range(K)])


def bench_sample(args, torch, np, binding, I, dev):
    """Draft-side sampling step: one token per row of [256, 152064] bf16 logits."""
    w = I.synth_logits(1003, 256, 0, 152064, dtype=I.BF16, T=1.0, sigma=4.0, zipf=True, draft_scale=1.0,
                       draft_sigma=2.5, name="sample_B256_V152064_bf16")
    d = binding.to_device(w, dev)
    logits = d["target"][:, 0, :].contiguous()
    u = d["uniforms"][:, 0].contiguous()
    call = binding.BoundSample(logits, u, w.T)
    stream = torch.cuda.current_stream(dev)
    _settle(args, torch, call)
    for _ in range(args.warmup):
        call()
    ms, ev = _timed_one(torch, stream, args.steps, call)
    tok = call().cpu().numpy()
    # every row once (the bonus-row stream keeps its segment sums, so the draw
    # reads only the one segment it walks)
    bytes_ = w.B * w.V * 2 + w.B * 512 * 2
    res = _base_result(w, args.steps, args.warmup, ms, "f32")
    res["metric"] = "draft-step sampled logits/s (B·V per sec), 1 GPU"
    res["value"] = w.B * w.V / (ms * 1e-3)
    res["config"] = {"workload": w.name, "B": w.B, "V": w.V, "logits": "bf16", "temperature": w.T, "seed": w.seed,
                     "schedule": SCHEDULES[binding.schedule(w.B, 0, w.V, w.dtype)]}
    achieved = bytes_ / (float(ev.mean()) * 1e-3) / 1e9
    res["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": achieved / HBM_PEAK_GBS, "traffic": None, "kernel": "sv_sample (all launches)",
                       "algorithmic_bytes_per_launch": bytes_, "avg_launch_ms": float(ev.mean())}
    g = {"accepted_len": np.where(tok >= 0, 0, -1).astype(np.int32), "out_tokens": tok[:, None]}
    return w, g, res, "sample"


def bench_lookup(args, torch, np, binding, I, dev):
    """Prompt lookup: the proposer over B=256 histories of 2-4k tokens, then the
    verify step on its candidates (one-hot proposals) over [256, 9, 152064] bf16."""
    lw = I.lookup_152k()
    print(f"[bench] workload {lw.name}: generated", file=sys.stderr, flush=True)
    hist = torch.from_numpy(lw.history).to(dev)
    hl = torch.from_numpy(lw.hist_len).to(dev)
    tt = torch.from_numpy(lw.target.view(np.int16)).view(torch.bfloat16).to(dev)
    uni = torch.from_numpy(lw.uniforms).to(dev)
    call = binding.BoundLookup(hist, hl, lw.n_max, lw.n_min, tt, uni, lw.T)
    stream = torch.cuda.current_stream(dev)
    t = _measure(args, torch, stream, (call.propose, call.verify), args.steps)
    print(f"[bench] {lw.name}: timed {args.steps} hot and {args.steps} cache-flushed steps", file=sys.stderr,
          flush=True)
    klen = call.klen.cpu().numpy()
    out = call.outputs
    acc = out["accepted_len"].cpu().numpy()
    gpu = {k: v.cpu().numpy() for k, v in out.items()}
    gpu["_cand"], gpu["_klen"] = call.cand.cpu().numpy(), klen
    s = 2
    # per-sequence launch: target rows 0..n once (no draft rows: the proposal is
    # one-hot), then row n once more for the draw of every valid sampling sequence
    ok = acc >= 0
    ver_bytes = (int(np.sum(acc[ok] + 1)) + int(np.sum(ok & (lw.greedy == 0)))) * lw.V * s
    hist_bytes = int(lw.hist_len.sum()) * 4
    w = I.Workload(lw.name, lw.B, lw.K, lw.V, lw.dtype, lw.T, lw.target, np.zeros((lw.B, lw.K, 0), np.uint16),
                   gpu["_cand"], lw.uniforms, lw.greedy, seed=lw.seed)
    w.lookup = lw
    res = _base_result(w, args.steps, args.warmup, float(t["cold_step"].mean()), "f32")
    res["config"] = {"workload": lw.name, "B": lw.B, "K": lw.K, "V": lw.V, "logits": "bf16",
                     "history_tokens": int(lw.hist_len.sum()), "n_max": lw.n_max, "n_min": lw.n_min,
                     "temperature": lw.T, "seed": lw.seed,
                     "schedule": "automatic for one-hot proposals (per-sequence at this size)"}
    prop_ms = t["cold_per"][0]
    res["roofline"] = _roofline(np, ver_bytes, t["cold_per"][1],
                                "spec_verify_lookup (one launch: k_seqg with one-hot proposals)", None,
                                {"proposer_avg_ms": float(prop_ms.mean()), "proposer_history_bytes": hist_bytes,
                                 "proposer_gbs": hist_bytes / (float(prop_ms.mean()) * 1e-3) / 1e9,
                                 "timing": FLUSH_NOTE})
    hot = _roofline(np, ver_bytes, t["hot_per"][1], "spec_verify_lookup", None)
    res["hot"] = {"ms_per_step": t["hot_host_ms"], "value": w.verified_logits / (t["hot_host_ms"] * 1e-3),
                  "achieved": hot["achieved"], "frac": hot["frac"], "avg_launch_ms": hot["avg_launch_ms"]}
    res["timing_ms"] = {"propose_median": float(np.median(t["cold_per"][0])),
                        "verify_median": float(np.median(t["cold_per"][1])),
                        "step_median": float(np.median(t["cold_step"]))}
    res["method"] = _method_stats(w, acc)
    res["method"]["candidates_hist"] = np.bincount(np.maximum(klen, 0), minlength=lw.K + 1).tolist()
    return w, gpu, res, "lookup"


def bench_kvcommit(args, torch, np, binding, I, dev):
    """KV-cache commit: 64 planes (32 layers x keys/values) of 2048-byte rows
    (8 heads x 128 x bf16), B=256, K=8, staging block = previous final token +
    8 candidates, L=512; accepted lengths follow the 152k-vocab workload."""
    P, B, K, L, row = 64, 256, 8, 512, 2048
    rng = np.random.default_rng(7)
    hist = np.array([185, 57, 9, 5, 0, 0, 0, 0, 0], np.float64)
    acc = rng.choice(K + 1, size=B, p=hist / hist.sum()).astype(np.int32)
    cache = torch.empty(P, B, L, row, dtype=torch.uint8, device=dev)
    staged = torch.randint(0, 255, (P, B, K + 1, row), dtype=torch.uint8, device=dev)
    ln0 = torch.from_numpy(rng.integers(0, L - K - 2, size=B).astype(np.int32)).to(dev)
    ln = ln0.clone()
    acc_d = torch.from_numpy(acc).to(dev)
    call = binding.BoundKvCommit(cache, ln, staged, acc_d, 1)
    stream = torch.cuda.current_stream(dev)

    def step():
        ln.copy_(ln0)          # same starting lengths every step
        call()
    _settle(args, torch, step)
    for _ in range(args.warmup):
        step()
    ms, ev = _timed_one(torch, stream, args.steps, step)
    committed = int((acc + 1).sum()) * P * row
    bytes_ = 2 * committed                              # read staged rows, write cache rows

    class _W:
        name, B_, verified_logits = f"kvcommit_P{P}_B{B}_K{K}_row{row}", B, 0
    res = _base_result(_W, args.steps, args.warmup, ms, "u8")
    res["metric"] = "committed KV bytes/s, 1 GPU"
    res["value"] = committed / (ms * 1e-3)
    res["unit"] = "B/s"
    res["config"] = {"workload": _W.name, "planes": P, "B": B, "K": K, "L": L, "row_bytes": row,
                     "committed_bytes_per_step": committed}
    achieved = bytes_ / (float(ev.mean()) * 1e-3) / 1e9
    res["roofline"] = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                       "kernel": "k_kv_copy + k_kv_len (+ a length reset copy)",
                       "algorithmic_bytes_per_launch": bytes_, "avg_launch_ms": float(ev.mean())}
    return None, None, res, "kv"


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="untimed run of the step before the warmup steps, in ms of wall time (0: none)")
    ap.add_argument("--config", default="cfg152k",
                    choices=["cfg152k", "cfg128k", "cfg32k", "tiny", "lmhead", "sample", "kvcommit", "lookup",
                             "shard_batch", "shard_vocab"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="wall-clock budget of the oracle timing (repeated whole-workload calls)")
    ap.add_argument("--mode", choices=["auto", "eager", "lazy", "seq"], default="auto",
                    help="row-statistics schedule (the library chooses per call under auto)")
    ap.add_argument("--seq-groups", type=int, default=0,
                    help="cap on workgroups per sequence under --mode seq (0: as many as the device holds)")
    ap.add_argument("--seq-lookahead", type=int, default=-1, choices=[-1, 0, 1, 2],
                    help="lookahead of --mode seq (-1: by shape)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="default workload only: skip the other named workloads' figures (`workloads`)")
    ap.add_argument("--workload-steps", type=int, default=30,
                    help="timed steps (hot and cache-flushed each) of every other named workload")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before timing, run one plain device copy of this size (for PMC byte scaling)")
    ap.add_argument("--ceiling-only", action="store_true",
                    help="print only the HBM ceiling (plain streaming read and copy) as one JSON line")
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
    binding.set_mode({"auto": binding.MODE_AUTO, "eager": binding.MODE_EAGER, "lazy": binding.MODE_LAZY,
                      "seq": binding.MODE_SEQ}[args.mode])
    binding.set_seq_groups(args.seq_groups)
    binding.set_seq_lookahead(args.seq_lookahead)
    if args.ceiling_only:
        print(json.dumps({"hbm_ceiling": hbm_ceiling(torch, np, binding, dev)}), flush=True)
        return 0

    fn = {"lmhead": bench_lmhead, "sample": bench_sample, "kvcommit": bench_kvcommit,
          "lookup": bench_lookup}.get(args.config, bench_verify)
    w, gpu, result, kind = fn(args, torch, np, binding, I, dev)

    if kind == "kv":
        result["cpu_baseline"] = None
    elif kind == "lookup" and not args.no_cpu_baseline:
        import oracle
        from oracle import lookup, parity
        oracle.build(force=False)
        lw = w.lookup
        pick = np.arange(16)                       # bounded sample: the first 16 sequences
        t_start = time.perf_counter()
        ts = []
        while len(ts) < 2 or time.perf_counter() - t_start < args.cpu_seconds:
            t0 = time.perf_counter()
            co, ko = lookup.propose(lw.history[pick], lw.hist_len[pick], lw.n_max, lw.n_min, lw.K)
            orc = lookup.verify_lookup(I.logits_as_f64(lw.target[pick], lw.dtype), co, ko, lw.uniforms[pick],
                                       lw.T, lw.greedy[pick], len(pick), lw.K, lw.V)
            ts.append(time.perf_counter() - t0)
        med = float(np.median(ts))
        result["cpu_baseline"] = {"value": len(pick) * (lw.K + 1) * lw.V / med, "unit": "logits/s", "cores": 1,
                                  "kind": "oracle",
                                  "sample": f"first 16 of {lw.B} sequences (proposer + one-hot verify), "
                                            f"{len(ts)} calls, median {med * 1e3:.1f} ms, python proposer + fp64 C "
                                            f"verify, 1 thread; scaled to verified logits/s"}
        ok = np.array_equal(gpu["_klen"][pick], ko) and np.array_equal(gpu["_cand"][pick], co)
        try:
            sub = {k: v[pick] for k, v in gpu.items() if not k.startswith("_")}
            wsub = I.Workload(w.name, len(pick), w.K, w.V, w.dtype, w.T, None, None, co, None, lw.greedy[pick])
            rep = parity.compare(wsub, sub, orc)
            result["parity"] = {"ok": ok, "flagged": rep["flagged"], "sample": "first 16 sequences",
                                "flagged_mismatch": len(rep["flagged_mismatch"]), "invalid": rep["invalid"]}
        except parity.ParityError as e:
            result["parity"] = {"ok": False, "error": str(e)[:500]}
    elif kind == "lookup":
        result["cpu_baseline"] = None
    elif not args.no_cpu_baseline:
        import oracle
        from oracle import parity
        oracle.build(force=False)
        ncpu = len(os.sched_getaffinity(0))
        tgt = None
        gemm_s = 0.0
        if kind == "lmhead":
            t0 = time.perf_counter()
            tgt = oracle.lmhead_logits(w.hidden, w.w_lm)
            gemm_s = time.perf_counter() - t0
        t_start = time.perf_counter()
        ts = []
        orc = None
        while len(ts) < 3 or time.perf_counter() - t_start < args.cpu_seconds:
            t0 = time.perf_counter()
            orc = oracle.verify(w, nthreads=ncpu, target=tgt)
            ts.append(time.perf_counter() - t0)
        med = float(np.median(ts))
        sample = (f"whole workload ({w.B} sequences), {len(ts)} calls, median {med * 1e3:.1f} ms per call, "
                  f"fp64 C oracle, {orc['nthreads']} threads")
        if kind == "lmhead":
            sample += f"; plus one fp64 numpy LM-head product of {gemm_s:.2f} s per step"
        result["cpu_baseline"] = {"value": w.verified_logits / (med + gemm_s), "unit": "logits/s",
                                  "cores": orc["nthreads"], "kind": "oracle", "sample": sample}
        try:
            rep = parity.compare(w, gpu, orc)
            result["parity"] = {"ok": True, "flagged": rep["flagged"],
                                "flagged_mismatch": len(rep["flagged_mismatch"]), "invalid": rep["invalid"]}
        except parity.ParityError as e:
            result["parity"] = {"ok": False, "error": str(e)[:500]}
    else:
        result["cpu_baseline"] = None
    result["settle_ms"] = args.settle_ms

    if args.config == "cfg152k" and not args.no_workloads:
        result["workloads"] = {}
        for name, leg, make in (("cfg128k", bench_verify, I.cfg_128k), ("lmhead", bench_lmhead, I.cfg_lmhead),
                                ("cfg32k", bench_verify, I.cfg_32k)):
            wl, gl, rl, kl = leg(args, torch, np, binding, I, dev, w=make(), steps=args.workload_steps)
            result["workloads"][name] = _summary(rl, _parity(np, wl, gl, kl))
            print(f"[bench] {name}: {result['workloads'][name]}", file=sys.stderr, flush=True)
        # the NEXT rows (sampling step, KV commit, prompt lookup + its verify), fewer steps each
        import copy
        a2 = copy.copy(args)
        a2.steps, a2.settle_ms = args.workload_steps, 50.0
        result["next_rows"] = {}
        for name, leg in (("sample", bench_sample), ("kvcommit", bench_kvcommit), ("lookup", bench_lookup)):
            wl, gl, rl, kl = leg(a2, torch, np, binding, I, dev)
            rf = rl["roofline"]
            entry = {"workload": rl["config"]["workload"], "ms_per_step": rl["ms_per_step"], "value": rl["value"],
                     "unit": rl["unit"], "kernel": rf["kernel"], "algorithmic_bytes": rf["algorithmic_bytes_per_launch"],
                     "avg_launch_ms": rf["avg_launch_ms"], "achieved_GBs": rf["achieved"], "roofline_frac": rf["frac"]}
            if "hot" in rl:
                entry["hot_ms_per_step"] = rl["hot"]["ms_per_step"]
            if kl == "sample":
                entry["parity"] = _parity(np, wl, gl, kl)
            result["next_rows"][name] = entry
            print(f"[bench] {name}: {entry}", file=sys.stderr, flush=True)
        result["hbm_ceiling"] = hbm_ceiling(torch, np, binding, dev)
        print(f"[bench] hbm ceiling: {result['hbm_ceiling']}", file=sys.stderr, flush=True)
        # every kernel's rate against what a plain read (a copy, for the KV commit) reaches in this run
        rd, cp = result["hbm_ceiling"]["read_GBps"], result["hbm_ceiling"]["copy_GBps"]
        result["roofline"]["frac_of_read_ceiling"] = result["roofline"]["achieved"] / rd
        for v in result["workloads"].values():
            v["frac_of_read_ceiling"] = v["achieved_GBs"] / rd
        for k, v in result["next_rows"].items():
            v["frac_of_copy_ceiling" if k == "kvcommit" else "frac_of_read_ceiling"] = \
                v["achieved_GBs"] / (cp if k == "kvcommit" else rd)

    print(json.dumps(result), flush=True)
    return 0


def _parity(np, w, gpu, kind):
    """The oracle on the same inputs (no timing) and the parity report."""
    import oracle
    from oracle import parity
    oracle.build(force=False)
    tgt = oracle.lmhead_logits(w.hidden, w.w_lm) if kind == "lmhead" else None
    orc = oracle.verify(w, target=tgt)
    try:
        rep = parity.compare(w, gpu, orc)
        return {"ok": True, "flagged": rep["flagged"], "flagged_mismatch": len(rep["flagged_mismatch"]),
                "invalid": rep["invalid"]}
    except parity.ParityError as e:
        return {"ok": False, "error": str(e)[:300]}


def _summary(r, par):
    """The figures of one named workload for the `workloads` entry."""
    rf, hot = r["roofline"], r["hot"]
    out = {"workload": r["config"]["workload"], "ms_per_step": r["ms_per_step"], "value": r["value"],
           "unit": r["unit"], "dominant_kernel": rf["kernel"], "algorithmic_bytes": rf["algorithmic_bytes_per_launch"],
           "avg_launch_ms": rf["avg_launch_ms"], "achieved_GBs": rf["achieved"], "roofline_frac": rf["frac"],
           "hot_ms_per_step": hot["ms_per_step"], "hot_frac": hot["frac"], "timing_ms": r["timing_ms"],
           "parity": par, "accepted_len_hist": r["method"]["accepted_len_hist"]}
    if "schedule" in r["config"]:
        out["schedule"] = r["config"]["schedule"]
    if "mfma_frac" in rf:
        out["mfma_frac"] = rf["mfma_frac"]
    return out


if __name__ == "__main__":
    sys.exit(main())
