"""Throughput of the TQ3 codec on one MI355X.

A step is one pass of the TQ3 hot path over one layer of KV cache: quantize K
and V ([32768 tokens, 8 heads, 128] bf16 each, 2 x 524288 vectors) to 56-byte
records, then dequantize both back to bf16. `value` counts vectors taken
through the round trip per second (1,048,576 per step). Inputs are resident in
HBM before timing; the step rotates over several buffer sets whose total size
exceeds the 256 MB last-level cache, so every launch streams from HBM.

Prints one JSON line. Extra fields: per-kernel times and effective bandwidth,
the roofline of the dominant kernel (algorithmic bytes / average launch time,
HIP events on the launch stream), and the oracle's CPU throughput on a bounded
sample (the CPU baseline).
"""
import argparse
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TQ3 quantize+dequantize vectors/s and effective HBM GB/s (% of peak)"
PEAK_HBM_GBS = 8000.0
REC = 56


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--sets", type=int, default=4, help="rotating buffer sets")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    return p.parse_args()


def cpu_baseline(k_cpu, signs, seconds):
    """The oracle, as it stands, on a bounded sample of the workload: the first
    65536 K vectors, quantize + dequantize, repeated for about `seconds`."""
    import oracle
    sample = k_cpu.reshape(-1, 128)[:65536].to(torch.float32).numpy()
    s = signs.numpy()
    threads = min(os.cpu_count() or 1, 16)
    n_done, t0 = 0, time.perf_counter()
    while True:
        rec = oracle.tq3_quantize(sample, s, threads=threads)
        oracle.tq3_dequantize(rec, s, threads=threads)
        n_done += sample.shape[0]
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": n_done / el, "unit": "vectors/s", "cores": threads, "kind": "oracle",
            "sample": f"first 65536 K vectors (bf16 widened to fp32), quantize+dequantize, "
                      f"{n_done // 65536} passes in {el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); "
              "the codec is data-parallel per vector and needs no collective", file=sys.stderr)
        sys.exit(2)
    import datagen
    import randomized_hadamard_lloyd_amd as tq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    signs = datagen.tq3_signs()
    mask = tq.sign_mask(signs)
    k_cpu = datagen.kv_cache("K")
    v_cpu = datagen.kv_cache("V")
    n = k_cpu.numel() // 128                       # vectors per tensor

    sets = []
    for _ in range(args.sets):
        sets.append({
            "k": k_cpu.to(dev), "v": v_cpu.to(dev),
            "rk": torch.empty((n, REC), dtype=torch.uint8, device=dev),
            "rv": torch.empty((n, REC), dtype=torch.uint8, device=dev),
            "ok": torch.empty((n, 128), dtype=torch.bfloat16, device=dev),
            "ov": torch.empty((n, 128), dtype=torch.bfloat16, device=dev),
        })
    stream = torch.cuda.current_stream(dev)
    sp = tq._stream(sets[0]["k"])
    L = tq.lib

    def launch_q(x, r):
        st = L.tq3_quantize(tq._ptr(x), tq.TQ_BF16, n, 128, mask, tq._ptr(r), sp)
        assert st == 0, st

    def launch_dq(r, y):
        st = L.tq3_dequantize(tq._ptr(r), n, mask, tq._ptr(y), tq.TQ_BF16, 128, sp)
        assert st == 0, st

    def step(i, evs=None):
        b = sets[i % len(sets)]
        seq = [(launch_q, b["k"], b["rk"], "quantize"), (launch_q, b["v"], b["rv"], "quantize"),
               (launch_dq, b["rk"], b["ok"], "dequantize"), (launch_dq, b["rv"], b["ov"], "dequantize")]
        for fn, a, o, name in seq:
            if evs is not None:
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                fn(a, o)
                e1.record(stream)
                evs.append((name, e0, e1))
            else:
                fn(a, o)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: K steps, wall time by events around the whole region
    evs = []
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i, evs)
    t_end.record(stream)
    torch.cuda.synchronize()
    total_ms = t_start.elapsed_time(t_end)
    ms_step = total_ms / args.steps

    per = {}
    for name, e0, e1 in evs:
        per.setdefault(name, []).append(e0.elapsed_time(e1))
    bytes_per_vec = {"quantize": 128 * 2 + REC, "dequantize": REC + 128 * 2}
    kernels = {}
    for name, times in per.items():
        avg = sum(times) / len(times)
        gbs = bytes_per_vec[name] * n / (avg * 1e-3) / 1e9
        kernels[name] = {"avg_ms": avg, "launches": len(times), "bytes_per_vector": bytes_per_vec[name],
                         "vectors_per_launch": n, "GBps": gbs, "frac_peak_hbm": gbs / PEAK_HBM_GBS}
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"] * kernels[k]["launches"])
    vec_per_step = 2 * n
    value = vec_per_step / (ms_step * 1e-3)
    step_bytes = 2 * n * (bytes_per_vec["quantize"] + bytes_per_vec["dequantize"])
    eff_gbs = step_bytes / (ms_step * 1e-3) / 1e9

    # correctness spot check of the last set against the oracle (outside timing)
    import oracle
    b = sets[(args.steps - 1) % len(sets)]
    k32 = k_cpu.reshape(-1, 128)[:4096].to(torch.float32).numpy()
    ok = bool((b["rk"][:4096].cpu().numpy() == oracle.tq3_quantize(k32, signs.numpy())).all())

    result = {
        "metric": METRIC, "value": value, "unit": "vectors/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "TQ3 round trip of one KV-cache layer: K and V, 32768 tokens x "
                               "8 heads x 128, bf16 in, 56-byte records, bf16 out",
                   "vectors_per_step": vec_per_step, "buffer_sets": args.sets},
        "effective_GBps": eff_gbs, "pct_of_peak_hbm": 100.0 * eff_gbs / PEAK_HBM_GBS,
        "kernels": kernels,
        "roofline": {"bound": "hbm", "kernel": f"tq3_{dom}_kernel<bf16>",
                     "achieved": kernels[dom]["GBps"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": kernels[dom]["frac_peak_hbm"], "traffic": None},
        "parity_spot_check": ok,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(k_cpu, signs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
