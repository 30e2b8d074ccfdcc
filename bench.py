"""Throughput of the randomized-Hadamard + Lloyd-Max codecs on one MI355X.

Headline (`value`): the TQ3 hot path on one layer of KV cache. K and V
([32768 tokens, 8 heads, 128] bf16 each, 262144 vectors per tensor) sit in one
[2, 32768, 8, 128] buffer, the layout paged KV caches use; a step quantizes
the 524288 vectors to 56-byte records with one launch and dequantizes them
back to bf16 with another. `value` counts vectors taken through that round
trip per second. Inputs are resident in HBM before timing; steps rotate over
buffer sets whose total size exceeds the 256 MB last-level cache, so every
launch streams from HBM. The timed region is bracketed by device
synchronisation and measured with HIP events on the launch stream.

Before the warmup steps, a pre-roll runs steps for a fixed stretch of device
time (default 200 ms): the GPU idles at a low clock and needs some 20 ms of
load to reach its sustained one, whatever --warmup asks for.

Also reported, each timed with HIP events over repeated launches:
  * kernels: per-kernel average duration and effective bandwidth
    (algorithmic bytes read + written) of the headline step;
  * roofline: the dominant kernel of the step against MI355X's 8 TB/s HBM
    peak (algorithmic bytes per launch / average launch duration), with
    traffic from the committed rocprofv3 counter summary when it matches the
    kernel source;
  * valu: the same kernel's arithmetic and issued VALU lane-ops (from the
    committed SQ_INSTS_VALU summary) against the non-packed VALU issue peak;
  * codec_kernels: each codec workload's own kernel line (KV-layer bf16
    quantize and dequantize, 2^20 structured fp32 quantize and dequantize,
    2^24 decode records to bf16) against the HBM peak;
  * secondary: the same layer with K and V as separate tensors (four
    launches per step); 2^20 structured fp32 vectors; 2^24 records
    dequantized to bf16; the 12288 x 3072 OrbitQuant weight at 2/3/4 bits;
    a device-to-device copy;
  * cpu_baseline: the oracle on the host cores, on a bounded sample.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TQ3 quantize+dequantize vectors/s and effective HBM GB/s (% of peak)"
PEAK_HBM_GBS = 8000.0
# 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz: one non-packed 32-bit VALU operation
# per lane per cycle (the 157.3 TFLOP/s fp32 figure counts packed FMA as 4).
PEAK_VALU_LANE_OPS = 256 * 64 * 2.4e9
REC = 56
PROFILES = os.path.join(ROOT, "profiles")

# Arithmetic of the method per 128-vector, one op per fp32 multiply, add,
# divide, square root, max or compare ("tq3_core.py", tq3_quantize and
# tq3_dequantize). Quantize: 128 squares + 127 adds + sqrt + clamp (norm),
# 128 divisions (x / norm), 128 sign multiplies, 7 x 128 butterfly adds,
# 128 multiplies by 1/sqrt(128), 128 abs-max steps (scale), 128 divisions
# (y / scale), and per element 3 compares against the positive boundaries plus
# a sign test (the table is symmetric). Dequantize: 128 centroid x scale,
# 7 x 128 butterfly adds, 128 x 1/sqrt(128), 128 sign and 128 norm multiplies.
ALG_OPS_PER_VECTOR = {
    "quantize": 128 + 127 + 1 + 1 + 128 + 128 + 7 * 128 + 128 + 128 + 128 + 4 * 128,
    "dequantize": 128 + 7 * 128 + 128 + 128 + 128,
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    # The GPU idles at a low clock and takes some 20 ms of load to reach its
    # sustained one: 300 warmup steps (~25 ms) come before the timed region.
    p.add_argument("--steps", type=int, default=500)
    p.add_argument("--warmup", type=int, default=300)
    p.add_argument("--sets", type=int, default=4, help="rotating buffer sets")
    p.add_argument("--preroll-ms", type=float, default=200.0,
                   help="device time of untimed steps run before the warmup steps, so the "
                        "clock has ramped up whatever --warmup is")
    p.add_argument("--cpu-seconds", type=float, default=8.0,
                   help="seconds of oracle work per thread count (1 thread, all threads)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-secondary", action="store_true")
    p.add_argument("--only-secondary", action="store_true",
                   help="run only the secondary measurements and print them as one JSON line")
    p.add_argument("--profile", action="store_true",
                   help="short run for counter collection: one 256 MiB device copy "
                        "(calibration), 1 warmup + 3 steps, nothing else")
    p.add_argument("--profile-orbit", action="store_true",
                   help="short run for counter collection on the OrbitQuant weight codec: "
                        "one 256 MiB device copy (calibration), then for 2, 3 and 4 bits one "
                        "warmup + 3 launches each of quantize, rotated and full dequantize")
    args = p.parse_args()
    if args.profile:
        args.steps, args.warmup, args.preroll_ms = 3, 1, 0.0
        args.no_secondary = args.no_cpu_baseline = True
    return args


class Timer:
    """Average duration of repeated launches, HIP events on one stream."""

    def __init__(self, stream):
        self.stream = stream

    def run(self, fn, iters, warmup=5):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        # A spin kernel first, long enough for the host to enqueue every timed
        # launch behind it: the launches then run back to back and each event
        # pair brackets device time only, not the host's launch overhead.
        with torch.cuda.stream(self.stream):
            torch.cuda._sleep(int(iters * 100_000))
        evs = []
        for _ in range(iters):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(self.stream)
            fn()
            e1.record(self.stream)
            evs.append((e0, e1))
        torch.cuda.synchronize()
        ms = [a.elapsed_time(b) for a, b in evs]
        return sum(ms) / len(ms), min(ms)

    def run_batch(self, fn, iters, warmup=5):
        """Average duration of iters back-to-back calls between one event pair
        (queued behind the spin kernel like run's): for calls of several
        kernels, where an event pair around each call adds its own gaps."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        with torch.cuda.stream(self.stream):
            torch.cuda._sleep(int(iters * 100_000))
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        for _ in range(iters):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters


def rate(bytes_, ms):
    return bytes_ / (ms * 1e-3) / 1e9


# the sources the TQ3 kernels are compiled from (the dominant kernel's
# counters stay valid while these are unchanged)
TQ3_SOURCES = ("tq3.hip", "tq_common.h", "tq_kernels.h")
ALL_SOURCES = ("tq3.hip", "tq3_attn.hip", "orbit.hip", "orbit_linear.hip", "orbit_linear_lp.hip",
               "orbit_codes.h", "tq_common.h", "tq_kernels.h", "libtq.cpp")


def source_hash(files=TQ3_SOURCES):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "randomized_hadamard_lloyd_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel):
    """HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, each scaled by what the
    counter reads for a 256 MiB device copy) from the committed counter
    summary, if it was taken on the current kernel source; otherwise None."""
    path = os.path.join(PROFILES, "tq3_kv_layer_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != source_hash():
        return None
    k = t.get("kernels", {}).get(kernel)
    return None if k is None else k["hbm_bytes"]


def valu_per_vector():
    path = os.path.join(PROFILES, "tq3_valu_counts.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    return t if t.get("source_hash") == source_hash() else None


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(k_cpu, signs, seconds):
    """The oracle, as it stands, on a bounded sample of the workload: the first
    65536 K vectors, quantize + dequantize, repeated for about `seconds`, once
    on one thread and once on every thread this process may use (OpenMP over
    vectors). `value` is the all-threads rate."""
    import oracle
    sample = k_cpu.reshape(-1, 128)[:65536].to(torch.float32).numpy()
    s = signs.numpy()
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    env = os.environ.get("OMP_NUM_THREADS", "")
    threads_all = min(usable, int(env)) if env.isdigit() and int(env) > 0 else usable

    def leg(threads):
        n_done, t0 = 0, time.perf_counter()
        while True:
            rec = oracle.tq3_quantize(sample, s, threads=threads)
            oracle.tq3_dequantize(rec, s, threads=threads)
            n_done += sample.shape[0]
            el = time.perf_counter() - t0
            if el >= seconds:
                return n_done / el, n_done // sample.shape[0], el

    v1, p1, e1 = leg(1)
    va, pa, ea = leg(threads_all)
    return {"value": va, "unit": "vectors/s", "cores": threads_all, "kind": "oracle",
            "sample": f"first 65536 K vectors of the KV layer (bf16 widened to fp32), "
                      f"quantize + dequantize: {pa} passes in {ea:.1f} s on {threads_all} "
                      f"threads, {p1} passes in {e1:.1f} s on 1 thread",
            "single_thread_value": v1, "cpu_model": cpu_model(),
            "host_cpus": os.cpu_count(), "usable_cpus": usable,
            "omp_num_threads_env": env or None}


def secondary(tq, timer, dev, signs, mask):
    import datagen
    out = {}
    L = tq.lib
    sp = tq._stream(torch.empty(1, device=dev))

    # the KV layer with K and V as separate tensors: four launches per step
    kc, vc = datagen.kv_cache("K"), datagen.kv_cache("V")
    n = kc.numel() // 128
    bufs = [dict(k=kc.to(dev), v=vc.to(dev),
                 rk=torch.empty((n, REC), dtype=torch.uint8, device=dev),
                 rv=torch.empty((n, REC), dtype=torch.uint8, device=dev),
                 ok=torch.empty((n, 128), dtype=torch.bfloat16, device=dev),
                 ov=torch.empty((n, 128), dtype=torch.bfloat16, device=dev)) for _ in range(4)]
    calls = []
    for b in bufs:
        calls.append([(L.tq3_quantize, (tq._ptr(b["k"]), tq.TQ_BF16, n, 128, mask, tq._ptr(b["rk"]), sp)),
                      (L.tq3_quantize, (tq._ptr(b["v"]), tq.TQ_BF16, n, 128, mask, tq._ptr(b["rv"]), sp)),
                      (L.tq3_dequantize, (tq._ptr(b["rk"]), n, mask, tq._ptr(b["ok"]), tq.TQ_BF16, 128, sp)),
                      (L.tq3_dequantize, (tq._ptr(b["rv"]), n, mask, tq._ptr(b["ov"]), tq.TQ_BF16, 128, sp))])
    it = [0]

    def sep_step():
        for f, a in calls[it[0] % 4]:
            f(*a)
        it[0] += 1
    ms, _ = timer.run(sep_step, 40, warmup=8)
    out["tq3_kv_layer_separate_tensors"] = {
        "launches_per_step": 4, "vectors_per_step": 2 * n, "ms_per_step": ms,
        "vectors_per_s": 2 * n / (ms * 1e-3), "GBps": rate(2 * n * 2 * (256 + REC), ms)}
    del bufs, calls

    # the same layer (K and V in one buffer) on the page's three-array layout:
    # indices, norms and scales in separate tensors, one launch each way
    kv = torch.stack([kc, vc])
    n2 = kv.numel() // 128
    bufs = [dict(x=kv.to(dev), p=torch.empty((n2, 48), dtype=torch.uint8, device=dev),
                 nr=torch.empty(n2, dtype=torch.float32, device=dev),
                 sc=torch.empty(n2, dtype=torch.float32, device=dev),
                 o=torch.empty((n2, 128), dtype=torch.bfloat16, device=dev)) for _ in range(4)]
    calls = []
    for b in bufs:
        calls.append([(L.tq3_quantize_split, (tq._ptr(b["x"]), tq.TQ_BF16, n2, 128, mask,
                                              tq._ptr(b["p"]), tq._ptr(b["nr"]), tq._ptr(b["sc"]), sp)),
                      (L.tq3_dequantize_split, (tq._ptr(b["p"]), tq._ptr(b["nr"]), tq._ptr(b["sc"]),
                                                n2, mask, tq._ptr(b["o"]), tq.TQ_BF16, 128, sp))])
    it[0] = 0
    del kv
    ms, _ = timer.run(sep_step, 40, warmup=8)
    out["tq3_kv_layer_split_layout"] = {
        "launches_per_step": 2, "vectors_per_step": n2, "ms_per_step": ms,
        "vectors_per_s": n2 / (ms * 1e-3), "GBps": rate(n2 * 2 * (256 + REC), ms)}
    del bufs, calls

    # device copy ceiling at the size of one KV tensor's quantize traffic
    nbytes = 256 << 20
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    ms, _ = timer.run(lambda: b.copy_(a), 20)
    out["device_copy_256MiB"] = {"avg_ms": ms, "GBps": rate(2 * nbytes, ms)}
    del a, b

    # 2^20 structured fp32 vectors: quantize, and dequantize back to fp32
    x = datagen.structured_blocks().to(dev)
    n = x.shape[0]
    rec = torch.empty((n, REC), dtype=torch.uint8, device=dev)
    y = torch.empty((n, 128), dtype=torch.float32, device=dev)
    ms_q, _ = timer.run(lambda: L.tq3_quantize(tq._ptr(x), tq.TQ_F32, n, 128, mask,
                                               tq._ptr(rec), sp), 20)
    ms_d, _ = timer.run(lambda: L.tq3_dequantize(tq._ptr(rec), n, mask, tq._ptr(y),
                                                 tq.TQ_F32, 128, sp), 20)
    out["tq3_structured_1M_f32"] = {
        "vectors": n,
        "quantize": {"avg_ms": ms_q, "vectors_per_s": n / (ms_q * 1e-3),
                     "GBps": rate(n * (512 + REC), ms_q)},
        "dequantize": {"avg_ms": ms_d, "vectors_per_s": n / (ms_d * 1e-3),
                       "GBps": rate(n * (REC + 512), ms_d)}}
    del x, rec, y

    # 2^24 decode records to bf16
    rec = datagen.decode_records().to(dev)
    n = rec.shape[0]
    y = torch.empty((n, 128), dtype=torch.bfloat16, device=dev)
    ms_d, _ = timer.run(lambda: L.tq3_dequantize(tq._ptr(rec), n, mask, tq._ptr(y),
                                                 tq.TQ_BF16, 128, sp), 10)
    out["tq3_decode_16M_bf16"] = {"vectors": n, "avg_ms": ms_d,
                                  "vectors_per_s": n / (ms_d * 1e-3),
                                  "GBps": rate(n * (REC + 256), ms_d)}
    del rec, y

    # decode attention over the KV layer's records (32768 tokens x 8 KV heads):
    # one query token per head, 8 or 32 query heads (groups of 1 and 4)
    import ctypes
    kv_k = tq.tq3_quantize(datagen.kv_cache("K").to(dev), mask).reshape(-1, REC)
    kv_v = tq.tq3_quantize(datagen.kv_cache("V").to(dev), mask).reshape(-1, REC)
    n_tok, hkv = datagen.KV_TOKENS, datagen.KV_HEADS
    att = {}
    for group in (1, 4):
        hq = hkv * group
        qh = datagen.attention_queries(hq).to(dev)
        ws = torch.zeros(tq.tq3_attention_workspace_bytes(n_tok, hq, hkv), dtype=torch.uint8,
                         device=dev)
        o = torch.empty((hq, 128), dtype=torch.float32, device=dev)
        call = lambda: L.tq3_decode_attention(
            tq._ptr(qh), tq.TQ_F32, hq, tq._ptr(kv_k), tq._ptr(kv_v), n_tok, hkv, mask,
            ctypes.c_float(128 ** -0.5), tq._ptr(ws), ws.numel(), tq._ptr(o), tq.TQ_F32, sp)
        # one call is two kernels (partial results, then their merge): timed
        # back to back between one event pair, and with a pair around each call
        ms_a = timer.run_batch(call, 200, warmup=20)
        ms_p, _ = timer.run(call, 50, warmup=5)
        ent = {"query_heads": hq, "kv_heads": hkv, "tokens": n_tok, "avg_ms": ms_a,
               "avg_ms_event_pair_per_call": ms_p,
               "records_GBps": rate(2 * n_tok * hkv * REC, ms_a)}
        if group == 4:
            # the unfused path: dequantize K and V to fp32, then bmm / softmax / bmm
            kd = torch.empty((n_tok * hkv, 128), dtype=torch.float32, device=dev)
            vd = torch.empty_like(kd)

            def unfused():
                L.tq3_dequantize(tq._ptr(kv_k), n_tok * hkv, mask, tq._ptr(kd), tq.TQ_F32, 128, sp)
                L.tq3_dequantize(tq._ptr(kv_v), n_tok * hkv, mask, tq._ptr(vd), tq.TQ_F32, 128, sp)
                k3 = kd.view(n_tok, hkv, 128).permute(1, 0, 2).contiguous()
                v3 = vd.view(n_tok, hkv, 128).permute(1, 0, 2).contiguous()
                qg = qh.view(hkv, group, 128).transpose(1, 2).contiguous()
                p = torch.softmax(torch.bmm(k3, qg) * (128 ** -0.5), dim=1)
                return torch.bmm(p.transpose(1, 2).contiguous(), v3)
            ms_u, _ = timer.run(unfused, 10, warmup=3)
            ent["unfused_fp32_dequantize_bmm_softmax_bmm_ms"] = ms_u
            del kd, vd
        att[f"hq{hq}"] = ent
    out["tq3_decode_attention_kv_layer"] = att
    del kv_k, kv_v

    # OrbitQuant weight 12288 x 3072 at 2, 3, 4 bits
    d = 3072
    w = datagen.orbit_weight().to(dev)
    rows = w.shape[0]
    perm, sg = datagen.rpbh_params(d)
    perm_d = perm.to(torch.int32).to(dev)
    inv_d = torch.argsort(perm).to(torch.int32).to(dev)
    sg_d = sg.to(dev)
    norms = torch.empty(rows, dtype=torch.float32, device=dev)
    wout = torch.empty_like(w)
    orb = {}
    import ctypes
    for bits in (2, 3, 4):
        cb = tq.orbit_make_codebook(bits, d)
        cbh = (ctypes.c_float * len(cb))(*cb.tolist())
        cbp = ctypes.cast(cbh, ctypes.c_void_p)
        packed = torch.empty((rows, d * bits // 8), dtype=torch.uint8, device=dev)
        ms_q, _ = timer.run(lambda: L.orbit_quantize_weight(
            tq._ptr(w), rows, d, bits, tq._ptr(perm_d), tq._ptr(sg_d), cbp, tq.TQ_MSB_FIRST,
            tq._ptr(packed), tq._ptr(norms), sp), 10)
        ms_r, _ = timer.run(lambda: L.orbit_dequantize(
            tq._ptr(packed), tq._ptr(norms), rows, d, bits, tq._ptr(inv_d), tq._ptr(sg_d), cbp,
            tq.TQ_MSB_FIRST, 1, tq._ptr(wout), tq.TQ_F32, sp), 10)
        ms_f, _ = timer.run(lambda: L.orbit_dequantize(
            tq._ptr(packed), tq._ptr(norms), rows, d, bits, tq._ptr(inv_d), tq._ptr(sg_d), cbp,
            tq.TQ_MSB_FIRST, 0, tq._ptr(wout), tq.TQ_F32, sp), 10)
        row_bytes = 4 * d + d * bits // 8 + 4
        orb[f"{bits}bit"] = {
            "quantize": {"avg_ms": ms_q, "rows_per_s": rows / (ms_q * 1e-3),
                         "GBps": rate(rows * row_bytes, ms_q)},
            "dequantize_rotated": {"avg_ms": ms_r, "GBps": rate(rows * row_bytes, ms_r)},
            "dequantize_full": {"avg_ms": ms_f, "GBps": rate(rows * row_bytes, ms_f)}}
    out["orbit_12288x3072"] = orb

    # OrbitQuant runtime forward on the same weight at 3 bits: rotate the
    # activations, then the linear layer with the weight decoded on the fly
    # (fp32 MFMA); beside it torch's fp32 matmul on the pre-dequantized W'
    bits = 3
    cb = tq.orbit_make_codebook(bits, d)
    cbh = (ctypes.c_float * len(cb))(*cb.tolist())
    cbp = ctypes.cast(cbh, ctypes.c_void_p)
    packed = torch.empty((rows, d * bits // 8), dtype=torch.uint8, device=dev)
    L.orbit_quantize_weight(tq._ptr(w), rows, d, bits, tq._ptr(perm_d), tq._ptr(sg_d), cbp,
                            tq.TQ_MSB_FIRST, tq._ptr(packed), tq._ptr(norms), sp)
    L.orbit_dequantize(tq._ptr(packed), tq._ptr(norms), rows, d, bits, tq._ptr(inv_d),
                       tq._ptr(sg_d), cbp, tq.TQ_MSB_FIRST, 1, tq._ptr(wout), tq.TQ_F32, sp)
    wrt = wout.t().contiguous()
    fwd = {}
    for m in (16, 1024):
        xa = torch.randn(m, d, generator=torch.Generator().manual_seed(m)).to(dev)
        xr = torch.empty_like(xa)
        yo = torch.empty((m, rows), dtype=torch.float32, device=dev)
        ms_r, _ = timer.run(lambda: L.orbit_rotate(tq._ptr(xa), tq.TQ_F32, m, d, tq._ptr(perm_d),
                                                   tq._ptr(sg_d), tq._ptr(xr), sp), 20)
        ms_l, _ = timer.run(lambda: L.orbit_linear(tq._ptr(xr), tq.TQ_F32, m, d, tq._ptr(packed),
                                                   tq._ptr(norms), rows, bits, cbp,
                                                   tq.TQ_MSB_FIRST, None, tq._ptr(yo), sp), 20)
        ms_t, _ = timer.run(lambda: torch.matmul(xr, wrt), 20)
        flop = 2.0 * m * rows * d
        fwd[f"m{m}"] = {"rotate_ms": ms_r, "linear_ms": ms_l,
                        "linear_TFLOPs": flop / (ms_l * 1e-3) / 1e12,
                        "linear_frac_fp32_mfma_peak": flop / (ms_l * 1e-3) / 157.3e12,
                        "codes_GBps": rate(packed.numel() + 4 * m * d + 4 * m * rows, ms_l),
                        "torch_fp32_matmul_on_dequantized_ms": ms_t}
    out["orbit_forward_12288x3072_3bit"] = fwd
    del wrt
    # the same forward on bf16 activations (bf16 rotation, W' products and
    # matrix cores); beside it torch's bf16 matmul on the pre-dequantized
    # bf16 W' (the weight it reads is 5.3x the codes' size)
    wrt16 = tq.orbit_dequantize(packed, norms, d, bits, None, None, cb, rotated_only=True,
                                dtype=torch.float32).to(torch.bfloat16).t().contiguous()
    fwd16 = {}
    for m in (16, 128, 1024):
        xa = torch.randn(m, d, generator=torch.Generator().manual_seed(m)).to(dev).to(torch.bfloat16)
        xr = torch.empty_like(xa)
        yo = torch.empty((m, rows), dtype=torch.bfloat16, device=dev)
        ms_r, _ = timer.run(lambda: L.orbit_rotate(tq._ptr(xa), tq.TQ_BF16, m, d, tq._ptr(perm_d),
                                                   tq._ptr(sg_d), tq._ptr(xr), sp), 20)
        ms_l, _ = timer.run(lambda: L.orbit_linear(tq._ptr(xr), tq.TQ_BF16, m, d, tq._ptr(packed),
                                                   tq._ptr(norms), rows, bits, cbp,
                                                   tq.TQ_MSB_FIRST, None, tq._ptr(yo), sp), 20)
        ms_t, _ = timer.run(lambda: torch.matmul(xr, wrt16), 20)
        flop = 2.0 * m * rows * d
        entry = {"path": "row-major", "rotate_ms": ms_r, "linear_ms": ms_l}
        if m > 64:
            # orbit_forward's path above 64 rows: the rotation written in the
            # matrix-core operand layout, read straight into registers
            xt = torch.empty(tq.orbit_tiled_bytes(m, d) // 2, dtype=torch.bfloat16, device=dev)
            ms_rt, _ = timer.run(lambda: L.orbit_rotate_tiled(
                tq._ptr(xa), tq.TQ_BF16, m, d, tq._ptr(perm_d), tq._ptr(sg_d), tq._ptr(xt), sp), 20)
            ms_lt, _ = timer.run(lambda: L.orbit_linear_tiled(
                tq._ptr(xt), tq.TQ_BF16, m, d, tq._ptr(packed), tq._ptr(norms), rows, bits, cbp,
                tq.TQ_MSB_FIRST, None, tq._ptr(yo), sp), 20)
            entry = {"path": "tiled", "rotate_ms": ms_rt, "linear_ms": ms_lt,
                     "row_major_rotate_ms": ms_r, "row_major_linear_ms": ms_l}
            ms_l = ms_lt
        entry.update({"linear_TFLOPs": flop / (ms_l * 1e-3) / 1e12,
                      "linear_frac_bf16_mfma_peak": flop / (ms_l * 1e-3) / 2.5e15,
                      "codes_GBps": rate(packed.numel() + 2 * m * d + 2 * m * rows, ms_l),
                      "torch_bf16_matmul_on_dequantized_ms": ms_t,
                      "linear_vs_torch": ms_l / ms_t})
        fwd16[f"m{m}"] = entry
    out["orbit_forward_12288x3072_3bit_bf16"] = fwd16
    del wrt16
    return out


def stream_ceiling(dev, sp, kv_kernels):
    """What HBM gives the TQ3 kernels' own access patterns with no arithmetic:
    the probe kernels of libtqprobe.so (quantize pattern: 256-byte bf16 rows
    in, 56-byte records out; dequantize pattern: records in, rows out) over
    four rotating buffer sets of the KV layer's size, at the kernels' grid and
    at one block per 64 vectors, and the best probe's time as a fraction of
    each kernel's."""
    import ctypes
    path = os.path.join(ROOT, "randomized_hadamard_lloyd_amd", "libtqprobe.so")
    P = ctypes.CDLL(path)
    P.tqprobe_stream.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                 ctypes.c_int, ctypes.c_void_p]
    n = kv_kernels["quantize"]["vectors_per_launch"]
    rows = [torch.empty((n, 128), dtype=torch.bfloat16, device=dev) for _ in range(4)]
    recs = [torch.zeros((n, REC), dtype=torch.uint8, device=dev) for _ in range(4)]
    for r in rows:
        r.zero_()
    stream = torch.cuda.current_stream(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {}
    for kind, name, src, dst, kgrid in ((0, "quantize", rows, recs, 4 * 5 * cus),
                                        (1, "dequantize", recs, rows, 4 * cus)):
        best = None
        for label, grid in (("kernel_grid", kgrid), ("one_block_per_64_vectors", n // 64)):
            calls = [lambda i=i: P.tqprobe_stream(kind, src[i].data_ptr(), dst[i].data_ptr(), n, grid,
                                                  sp) for i in range(4)]
            for c in calls:
                assert c() == 0
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record(stream)
            for i in range(200):
                calls[i % 4]()
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / 200
            gbs = rate(312 * n, ms)
            res[f"{name}_pattern_{label}"] = {"grid": grid, "avg_ms": ms, "GBps": gbs,
                                              "frac_peak_hbm": gbs / PEAK_HBM_GBS}
            best = ms if best is None else min(best, ms)
        res[f"{name}_kernel_over_probe"] = best / kv_kernels[name]["avg_ms"]
    return res


def codec_kernels(tq, dev, mask, sp, iters, kv_kernels):
    """Each codec workload's kernel on its own, back-to-back launches over
    rotating buffers (every launch streams from HBM), one event pair around
    them: the KV layer's bf16 quantize and dequantize (from the headline run),
    the 2^20 structured fp32 vectors (quantize, dequantize to fp32) and the
    2^24 decode records to bf16."""
    import datagen
    L = tq.lib
    stream = torch.cuda.current_stream(dev)

    def avg_ms(calls, count):
        for i in range(5):
            calls[i % len(calls)]()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(count):
            calls[i % len(calls)]()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / count

    def line(kernel, ms, vectors, bpv):
        gbs = rate(bpv * vectors, ms)
        return {"kernel": kernel, "avg_ms": ms, "vectors": vectors, "bytes_per_vector": bpv,
                "vectors_per_s": vectors / (ms * 1e-3), "GBps": gbs,
                "frac_peak_hbm": gbs / PEAK_HBM_GBS}

    out = {}
    for name in ("quantize", "dequantize"):
        k = kv_kernels[name]
        out[f"{name}_kv_layer_bf16"] = line(k["kernel"], k["avg_ms"], k["vectors_per_launch"],
                                            k["bytes_per_vector"])
    out["stream_ceiling_kv_layer"] = stream_ceiling(dev, sp, kv_kernels)
    # 2^20 structured fp32 vectors, two buffer sets (1.1 GB in all)
    x = datagen.structured_blocks().to(dev)
    n = x.shape[0]
    xs = [x, x.clone()]
    recs = [torch.empty((n, REC), dtype=torch.uint8, device=dev) for _ in xs]
    ys = [torch.empty((n, 128), dtype=torch.float32, device=dev) for _ in xs]
    qc = [lambda i=i: L.tq3_quantize(tq._ptr(xs[i]), tq.TQ_F32, n, 128, mask, tq._ptr(recs[i]),
                                     sp) for i in range(2)]
    dc = [lambda i=i: L.tq3_dequantize(tq._ptr(recs[i]), n, mask, tq._ptr(ys[i]), tq.TQ_F32,
                                       128, sp) for i in range(2)]
    its = max(20, min(iters, 200))
    out["quantize_structured_2^20_f32"] = line("tq3_quantize_kernel<f32>", avg_ms(qc, its), n,
                                               512 + REC)
    out["dequantize_structured_2^20_f32"] = line("tq3_dequantize_kernel<f32>", avg_ms(dc, its),
                                                 n, REC + 512)
    del x, xs, recs, ys, qc, dc
    # 2^24 decode records to bf16 (896 MiB in, 4 GiB out per launch)
    rec = datagen.decode_records().to(dev)
    n = rec.shape[0]
    y = torch.empty((n, 128), dtype=torch.bfloat16, device=dev)
    dd = [lambda: L.tq3_dequantize(tq._ptr(rec), n, mask, tq._ptr(y), tq.TQ_BF16, 128, sp)]
    out["dequantize_decode_2^24_bf16"] = line("tq3_dequantize_kernel<bf16>",
                                              avg_ms(dd, max(10, min(iters, 40))), n, REC + 256)
    del rec, y, dd
    return out


def profile_orbit(tq, dev):
    """The 12288 x 3072 fp32 weight through the codec, a few launches per
    kernel, for counters taken under a profiler."""
    import ctypes
    import datagen
    a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    d = 3072
    w = datagen.orbit_weight().to(dev)
    rows = w.shape[0]
    perm, sg = datagen.rpbh_params(d)
    perm_d = perm.to(torch.int32).to(dev)
    inv_d = torch.argsort(perm).to(torch.int32).to(dev)
    sg_d = sg.to(dev)
    norms = torch.empty(rows, dtype=torch.float32, device=dev)
    wout = torch.empty_like(w)
    L, sp = tq.lib, tq._stream(w)
    for bits in (2, 3, 4):
        cb = tq.orbit_make_codebook(bits, d)
        cbh = (ctypes.c_float * len(cb))(*cb.tolist())
        cbp = ctypes.cast(cbh, ctypes.c_void_p)
        packed = torch.empty((rows, d * bits // 8), dtype=torch.uint8, device=dev)
        for _ in range(4):
            assert L.orbit_quantize_weight(tq._ptr(w), rows, d, bits, tq._ptr(perm_d),
                                           tq._ptr(sg_d), cbp, tq.TQ_MSB_FIRST, tq._ptr(packed),
                                           tq._ptr(norms), sp) == 0
        for rot in (1, 0):
            for _ in range(4):
                assert L.orbit_dequantize(tq._ptr(packed), tq._ptr(norms), rows, d, bits,
                                          tq._ptr(inv_d), tq._ptr(sg_d), cbp, tq.TQ_MSB_FIRST,
                                          rot, tq._ptr(wout), tq.TQ_F32, sp) == 0
    torch.cuda.synchronize()
    print(json.dumps({"profile_orbit": "done", "rows": rows, "d": d}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}): the codecs are "
              "data-parallel per vector or row, and one GPU's share is what it measures",
              file=sys.stderr)
        sys.exit(2)
    import datagen
    import randomized_hadamard_lloyd_amd as tq

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    signs = datagen.tq3_signs()
    mask = tq.sign_mask(signs)
    if args.profile_orbit:
        profile_orbit(tq, dev)
        return
    if args.only_secondary:
        stream = torch.cuda.current_stream(dev)
        print(json.dumps({"secondary": secondary(tq, Timer(stream), dev, signs, mask)}), flush=True)
        return
    k_cpu = datagen.kv_cache("K")
    v_cpu = datagen.kv_cache("V")
    # The layer's K and V live in one [2, tokens, heads, 128] buffer (the
    # layout paged KV caches use), so one launch covers both tensors.
    kv_cpu = torch.stack([k_cpu, v_cpu])
    n = kv_cpu.numel() // 128                      # vectors per step (K and V)

    sets = []
    for _ in range(args.sets):
        sets.append({
            "kv": kv_cpu.to(dev),
            "rec": torch.empty((n, REC), dtype=torch.uint8, device=dev),
            "out": torch.empty(kv_cpu.shape, dtype=torch.bfloat16, device=dev),
        })
    stream = torch.cuda.current_stream(dev)
    sp = tq._stream(sets[0]["kv"])
    L = tq.lib
    # launch arguments bound once per buffer set, so the timed loop does no
    # more host work than two library calls per step
    q_args = [(tq._ptr(b["kv"]), tq.TQ_BF16, n, 128, mask, tq._ptr(b["rec"]), sp) for b in sets]
    d_args = [(tq._ptr(b["rec"]), n, mask, tq._ptr(b["out"]), tq.TQ_BF16, 128, sp) for b in sets]
    fq, fd = L.tq3_quantize, L.tq3_dequantize
    assert fq(*q_args[0]) == 0 and fd(*d_args[0]) == 0

    def step(i):
        fq(*q_args[i % len(sets)])
        fd(*d_args[i % len(sets)])

    if args.profile:
        # reference kernel for scaling the HBM byte counters: copies 256 MiB
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    # Pre-roll: untimed steps for a fixed stretch of device time, so the clock
    # has ramped up before the warmup and timed steps (the GPU idles at a low
    # clock and needs about 20 ms of load to reach its sustained one).
    preroll_steps, preroll_ms = 0, 0.0
    if args.preroll_ms > 0:
        p0 = torch.cuda.Event(enable_timing=True)
        p1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        p0.record(stream)
        chunk = 50
        while preroll_ms < args.preroll_ms:
            for i in range(chunk):
                step(preroll_steps + i)
            preroll_steps += chunk
            p1.record(stream)
            p1.synchronize()
            preroll_ms = p0.elapsed_time(p1)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region: exactly `steps` steps
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # Per-kernel durations, two ways. In the step: the same steps again with an
    # event before, between and after the two launches (each event costs a
    # little). Alone: `steps` back-to-back launches of one kernel over the same
    # rotating buffer sets, bracketed by one pair of events -- the figure the
    # roofline uses. (Dequantize alone runs slower than in the step, where it
    # reads records the quantize launch has just left in the last-level cache
    # and its writes drain while the next quantize computes.)
    in_step = {"quantize": [], "dequantize": []}
    torch.cuda.synchronize()
    evs = []
    for i in range(args.steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(stream)
        fq(*q_args[i % len(sets)])
        e[1].record(stream)
        fd(*d_args[i % len(sets)])
        e[2].record(stream)
        evs.append(e)
    torch.cuda.synchronize()
    for e in evs:
        in_step["quantize"].append(e[0].elapsed_time(e[1]))
        in_step["dequantize"].append(e[1].elapsed_time(e[2]))
    per = {}
    for name, f, a in (("quantize", fq, q_args), ("dequantize", fd, d_args)):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            f(*a[i % len(sets)])
        e1.record(stream)
        torch.cuda.synchronize()
        per[name] = (e0.elapsed_time(e1) / args.steps, args.steps)
    bytes_per_vec = {"quantize": 128 * 2 + REC, "dequantize": REC + 128 * 2}
    kernels = {}
    for name, (avg, count) in per.items():
        gbs = rate(bytes_per_vec[name] * n, avg)
        st = sum(in_step[name]) / len(in_step[name])
        kernels[name] = {"kernel": f"tq3_{name}_kernel<bf16>", "avg_ms": avg,
                         "launches": count, "bytes_per_vector": bytes_per_vec[name],
                         "vectors_per_launch": n, "GBps": gbs, "frac_peak_hbm": gbs / PEAK_HBM_GBS,
                         "in_step_avg_ms": st, "in_step_GBps": rate(bytes_per_vec[name] * n, st)}
    dom = max(kernels, key=lambda k: kernels[k]["avg_ms"])
    vec_per_step = n
    value = vec_per_step / (ms_step * 1e-3)
    step_bytes = n * (bytes_per_vec["quantize"] + bytes_per_vec["dequantize"])
    eff_gbs = rate(step_bytes, ms_step)

    for name, k in kernels.items():
        k["alg_ops_per_vector"] = ALG_OPS_PER_VECTOR[name]
        k["alg_TOPs"] = ALG_OPS_PER_VECTOR[name] * n / (k["avg_ms"] * 1e-3) / 1e12
    # Roofline of the dominant kernel against HBM: the codec streams its input
    # once and writes its output once, so its algorithmic bytes (256 B of bf16
    # in + 56 B record out per vector) over its average launch duration,
    # measured alone, against the 8 TB/s peak.
    traffic = measured_traffic(kernels[dom]["kernel"])
    alg_bytes = bytes_per_vec[dom] * n
    ach = alg_bytes / (kernels[dom]["avg_ms"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "kernel": kernels[dom]["kernel"], "achieved": ach,
                "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                "traffic": traffic, "alg_bytes_per_launch": alg_bytes,
                "bytes_per_vector": bytes_per_vec[dom], "vectors_per_launch": n,
                "avg_launch_ms": kernels[dom]["avg_ms"]}
    # The same kernel's vector-ALU work: the method's arithmetic and (from the
    # committed SQ_INSTS_VALU summary, when it matches the source) the issued
    # lane-ops, both against the non-packed 32-bit VALU issue peak.
    peak_valu = PEAK_VALU_LANE_OPS / 1e12
    valu = {"kernel": kernels[dom]["kernel"], "alg_ops_per_vector": ALG_OPS_PER_VECTOR[dom],
            "alg_achieved": kernels[dom]["alg_TOPs"], "peak": peak_valu, "unit": "TOP/s",
            "alg_frac": kernels[dom]["alg_TOPs"] / peak_valu}
    vc = valu_per_vector()
    if vc is not None and kernels[dom]["kernel"] in vc.get("kernels", {}):
        ops = vc["kernels"][kernels[dom]["kernel"]]["valu_lane_ops_per_vector"]
        issued = ops * n / (kernels[dom]["avg_ms"] * 1e-3)
        valu.update({"issued_lane_ops_per_vector": ops, "issued_achieved": issued / 1e12,
                     "issued_frac": issued / PEAK_VALU_LANE_OPS})

    codec = None if args.profile else codec_kernels(tq, dev, mask, sp, args.steps, kernels)

    # correctness spot check of one set against the oracle (outside timing)
    import oracle
    b = sets[(args.steps - 1) % len(sets)]
    k32 = k_cpu.reshape(-1, 128)[:4096].to(torch.float32).numpy()
    v32 = v_cpu.reshape(-1, 128)[-4096:].to(torch.float32).numpy()
    ok = bool((b["rec"][:4096].cpu().numpy() == oracle.tq3_quantize(k32, signs.numpy())).all()
              and (b["rec"][-4096:].cpu().numpy() == oracle.tq3_quantize(v32, signs.numpy())).all())

    result = {
        "metric": METRIC, "value": value, "unit": "vectors/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "TQ3 round trip of one KV-cache layer: K and V, 32768 tokens x "
                               "8 heads x 128 (262144 vectors each) in one [2, 32768, 8, 128] "
                               "bf16 buffer; one quantize launch to 56-byte records and one "
                               "dequantize launch back to bf16 per step",
                   "vectors_per_step": vec_per_step, "buffer_sets": args.sets},
        "effective_GBps": eff_gbs, "pct_of_peak_hbm": 100.0 * eff_gbs / PEAK_HBM_GBS,
        "preroll": {"steps": preroll_steps, "device_ms": preroll_ms},
        "kernels": kernels,
        "roofline": roofline,
        "valu": valu,
        "codec_kernels": codec,
        "parity_spot_check": ok,
    }
    if not args.no_secondary:
        result["secondary"] = secondary(tq, Timer(stream), dev, signs, mask)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(k_cpu, signs, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
