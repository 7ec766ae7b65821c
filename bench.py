#!/usr/bin/env python3
"""MoE decode benchmark on one MI355X.

Workload (default): Mixtral-8x7B-shaped decode -- 32 MoE layers, hidden 4096,
expert intermediate 14336, 8 experts per layer with 3.00-bit RVQ records
(66,322,432 bytes each, all 256 resident in HBM), softmax top-2 with
renormalisation, batch 1 token, seeded fp32 layer inputs.  One step = one
token through all 32 layers (route -> top-k -> RVQ SwiGLU experts ->
combine), issued by the library's decode driver.

Prints one JSON line: tok/s, expert-weight HBM GB/s against the 8 TB/s peak
(the decode step, timed with HIP events on the stream it runs on), and the
CPU oracle timed on this host's cores on a bounded sample of the same
workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM bytes per decode launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs
# (each scaled by the same counter on a 1 GiB device copy; the runs and the
# factors are in profiles/k_decode_persistent_mixtral_hbm_counters.txt),
# valid for the kernel source they were taken on: reported as null once that
# source has changed.
DECODE_TRAFFIC = {"kernel_source": "routed_expert_streaming_amd/csrc/kernels_decode.hip",
                  "sha256_prefix": "83d09abc5f859a2c", "bytes_per_launch": 4681542778}


def measured_traffic():
    import hashlib
    try:
        with open(os.path.join(ROOT, DECODE_TRAFFIC["kernel_source"]), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    return DECODE_TRAFFIC["bytes_per_launch"] if digest.startswith(DECODE_TRAFFIC["sha256_prefix"]) else None


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def git_commit() -> str:
    """HEAD read from the .git directory (no child process: under a profiler a
    child inherits the profiler's preloaded library)."""
    try:
        head = open(os.path.join(ROOT, ".git", "HEAD")).read().strip()
        if head.startswith("ref: "):
            ref = head[5:]
            path = os.path.join(ROOT, ".git", ref)
            if os.path.exists(path):
                return open(path).read().strip()[:7]
            for line in open(os.path.join(ROOT, ".git", "packed-refs")):
                if line.rstrip().endswith(" " + ref):
                    return line.split()[0][:7]
            return "unknown"
        return head[:7]
    except OSError:
        return "unknown"


def cpu_baseline(cfg, x_np, sample_tokens: int):
    """The fp64 oracle on `sample_tokens` tokens x all layers of the workload."""
    import numpy as np

    import oracle
    import synth
    threads = min(16, len(os.sched_getaffinity(0)))
    oracle.set_threads(threads)
    wl = synth.Workload(cfg)
    # inputs of the oracle: records of the experts its own router selects
    # (generation is not timed)
    jobs = []
    for t in range(sample_tokens):
        for L in range(cfg.layers):
            x64 = x_np[t, L][None].astype(np.float64)
            ridx, _, _ = oracle.route(wl.router(L), wl.bias(L), x64, cfg.k, cfg.score)
            jobs.append((L, x64, set(int(e) for e in ridx.reshape(-1))))
    empty = np.zeros(1, np.uint8)
    t_total = 0.0
    for L, x64, needed in jobs:
        recs = [wl.record(L, e) if e in needed else empty for e in range(cfg.E)]
        sh = wl.shared(L)
        t0 = time.perf_counter()
        oracle.layer(wl.router(L), wl.bias(L), cfg.k, cfg.score, recs, sh, cfg.H, cfg.I, x64)
        t_total += time.perf_counter() - t0
    return {"value": round(sample_tokens / t_total, 4), "unit": "tok/s", "cores": threads, "kind": "oracle",
            "sample": f"{sample_tokens} tokens x {cfg.layers} layers of the {cfg.name} decode (fp64, "
                      f"{threads} threads); {t_total:.1f} s"}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64, help="timed decode tokens")
    ap.add_argument("--warmup", type=int, default=2, help="untimed decode tokens")
    ap.add_argument("--config", default="mixtral", choices=["mixtral", "kimi_linear", "batched", "k3_slice"],
                    help="mixtral / kimi_linear: resident decode; batched: one 256-token grouped layer call "
                         "per step; k3_slice: streamed decode through the HBM slot cache (cold start)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB three times (reference for the HBM byte "
                         "counters FETCH_SIZE / WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): this build has no multi-GPU path; "
              "see the sharding design notes.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import synth
    import routed_expert_streaming_amd as moe
    from routed_expert_streaming_amd.device_workload import DeviceWorkload

    moe.lib()
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "repeats": 3}))
        return 0
    cfg = synth.get_config(args.config)
    if args.config == "batched":
        return bench_batched(args, cfg)
    if args.config == "k3_slice":
        return bench_streamed(args, cfg)
    n_tok = args.warmup + args.steps
    if n_tok > cfg.tokens:
        cfg = cfg.replace(tokens=n_tok)
    t0 = time.time()
    dw = DeviceWorkload(cfg)
    x = dw.inputs()
    log(f"workload {cfg.name}: {cfg.layers} layers x {cfg.E} experts uploaded in {time.time() - t0:.1f} s "
        f"(input redraws {dw.wl.redraws})")
    layers = dw.layers
    ws = torch.empty(moe.decode_workspace_bytes(layers), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def step(t):
        moe.decode_forward(layers, x[t:t + 1], ws=ws, out=out[t:t + 1], want_idx=False)

    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step(args.warmup + i)
        ends[i].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    step_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]

    tok_s = args.steps / elapsed
    bytes_tok = synth.expert_bytes_per_token(cfg)
    mean_step_s = float(np.mean(step_ms)) / 1e3
    achieved = bytes_tok / mean_step_s / 1e9
    record = {
        "metric": "MoE decode tok/s on 1 MI355X; expert-weight HBM GB/s as % of peak",
        "value": round(tok_s, 3),
        "unit": "tok/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32 accumulate, fp16 x RVQ-3bit weights",
        "data": "synthetic (seeded; random RVQ records and router weights)",
        "config": {"workload": f"{cfg.name} decode: {cfg.layers} layers, H {cfg.H}, I {cfg.I}, "
                               f"{cfg.E} experts, top-{cfg.k} {cfg.score}, batch 1",
                   "tokens": args.steps, "expert_bytes_per_token": bytes_tok},
        "expert_gbs": round(bytes_tok * tok_s / 1e9, 1),
        "expert_hbm_frac": round(bytes_tok * tok_s / 1e9 / HBM_PEAK_GBS, 4),
        "step_ms_min_max": [round(min(step_ms), 4), round(max(step_ms), 4)],
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if cfg.name == "mixtral" else None,
                     "kernel": "k_decode_persistent (route, top-k, RVQ gate/up, RVQ down, combine; all layers of "
                               "one token per launch)",
                     "algorithmic_bytes_per_launch": bytes_tok},
        "device": torch.cuda.get_device_name(0),
        "commit": git_commit(),
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample ...")
        record["cpu_baseline"] = cpu_baseline(cfg, x.cpu().numpy(), args.cpu_sample_tokens)
    print(json.dumps(record), flush=True)
    return 0


def bench_batched(args, cfg) -> int:
    """One step = one 256-token batched layer call on the grouped matrix-core path."""
    import numpy as np
    import torch

    import synth
    import routed_expert_streaming_amd as moe
    from routed_expert_streaming_amd.device_workload import DeviceWorkload
    t0 = time.time()
    dw = DeviceWorkload(cfg)
    x = dw.inputs().to(torch.bfloat16).contiguous()
    log(f"workload {cfg.name}: {cfg.E} experts uploaded in {time.time() - t0:.1f} s")
    layer = dw.layers[0]
    ws = torch.empty(moe.grouped_workspace_bytes(layer, cfg.tokens), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.tokens, cfg.H), dtype=torch.float32, device="cuda")
    for _ in range(args.warmup):
        moe.layer_forward_grouped(layer, x, ws=ws, out=out)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    t_start = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        moe.layer_forward_grouped(layer, x, ws=ws, out=out)
        ends[i].record(stream)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    step_ms = [a.elapsed_time(b) for a, b in zip(starts, ends)]
    # every expert is touched (P(unused) ~ 2e-5): bytes = all records + shared
    nbytes = cfg.E * synth.expert_bytes(cfg) + synth.shared_record_bytes(cfg.H, cfg.I)
    flops = 2.0 * cfg.tokens * (cfg.k + 1) * 3 * cfg.H * cfg.I + 2.0 * cfg.tokens * cfg.E * cfg.H
    mean_s = float(np.mean(step_ms)) / 1e3
    rec = {"metric": "batched MoE layer tokens/s on 1 MI355X (grouped bf16 MFMA)",
           "value": round(cfg.tokens * args.steps / elapsed, 1), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(elapsed * 1e3 / args.steps, 4),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16 MFMA, fp32 accumulate",
           "data": "synthetic", "config": {"workload": f"batched layer: T {cfg.tokens}, H {cfg.H}, I {cfg.I}, "
                                                        f"{cfg.E} experts, top-{cfg.k} + shared"},
           "roofline": {"bound": "hbm", "achieved": round(nbytes / mean_s / 1e9, 1), "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": round(nbytes / mean_s / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                        "kernel": "batched layer call", "algorithmic_bytes_per_launch": nbytes},
           "mfma": {"flops_per_call": flops, "achieved_tflops": round(flops / mean_s / 1e12, 2),
                    "peak_tflops": 2500.0, "utilisation": round(flops / mean_s / 1e12 / 2500.0, 4)},
           "commit": git_commit()}
    print(json.dumps(rec), flush=True)
    return 0


def bench_streamed(args, cfg) -> int:
    """K3-scale slice: 8 layers x 768 experts in pinned host memory, a 25%
    HBM slot cache (1536 slots) starting cold; one step = one token."""
    import numpy as np
    import torch

    import synth
    import routed_expert_streaming_amd as moe
    from routed_expert_streaming_amd.device_workload import DeviceWorkload, HostRecordPool
    n_tok = args.warmup + args.steps
    if n_tok > cfg.tokens:
        cfg = cfg.replace(tokens=n_tok)
    t0 = time.time()
    dw = DeviceWorkload(cfg, with_records=False)
    x = dw.inputs()
    hp = HostRecordPool(cfg, list(range(cfg.layers)))
    log(f"host pool {len(hp.chunks)} chunks, {cfg.layers * cfg.E} records ready in {time.time() - t0:.1f} s")
    cap = cfg.cache_capacity
    pool = torch.empty(cap * hp.stride, dtype=torch.uint8, device="cuda")
    cache = moe.ExpertCache(cap, hp.stride, pool)
    tables = [hp.table(L) for L in range(cfg.layers)]
    ws = torch.empty(moe.streamed_workspace_bytes(dw.layers[0]), dtype=torch.uint8, device="cuda")
    out = torch.empty((cfg.tokens, cfg.layers, cfg.H), dtype=torch.float32, device="cuda")
    copy_stream = torch.cuda.Stream()

    def token(t):
        for L in range(cfg.layers):
            moe.layer_forward_streamed(dw.layers[L], cache, L, None, x[t, L][None], copy_stream, ws=ws,
                                       out=out[t, L][None], host_table=tables[L])

    # the cold start is part of the workload: warm-up tokens are decoded (and
    # counted in the cache) but not timed
    for t in range(args.warmup):
        token(t)
    torch.cuda.synchronize()
    st0 = cache.stats()
    t_start = time.perf_counter()
    for i in range(args.steps):
        token(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    st = cache.stats()
    tr = cache.trace()
    hits = np.array([r[1] for r in tr])
    per_tok = cfg.layers * cfg.k
    half = (cfg.tokens // 2) * per_tok
    misses_timed = (st["lookups"] - st0["lookups"]) - (st["hits"] - st0["hits"])
    tok_s = args.steps / elapsed
    hbm_bytes = synth.expert_bytes_per_token(cfg)
    rec = {"metric": "streamed MoE decode tok/s on 1 MI355X (HBM LRU slot cache, misses over PCIe)",
           "value": round(tok_s, 3), "unit": "tok/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": round(elapsed * 1e3 / args.steps, 3), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "f32 accumulate, fp16 x RVQ-3bit weights", "data": "synthetic",
           "config": {"workload": f"k3_slice streamed decode: {cfg.layers} layers x {cfg.E} experts, H {cfg.H}, "
                                  f"I {cfg.I}, top-{cfg.k} sigmoid + shared, Zipf bias, cache {cap} slots",
                      "tokens": cfg.tokens},
           "hit_rate_all": round(float(hits.mean()), 4),
           "hit_rate_second_half": round(float(hits[half:].mean()), 4) if len(hits) > half else None,
           "misses_per_token_timed": round(misses_timed / args.steps, 2),
           "h2d_gbs": round(misses_timed * hp.stride / elapsed / 1e9, 2),
           "hbm_expert_gbs": round(hbm_bytes * tok_s / 1e9, 1),
           "cold_tier": {"records": cfg.layers * cfg.E, "pinned_records": hp.pinned_records,
                         "note": "the rest in pageable host memory (this host page-locks at most ~59 GiB)"},
           "commit": git_commit()}
    cache.close()
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    rc = main()
    # a successful run ends normally: leaving through SystemExit reorders the
    # runtime's teardown so that rocprofv3 loses its results
    if rc:
        sys.exit(rc)
