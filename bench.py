"""Benchmark of the TurboQuant KV-cache hot path on one MI355X.

Headline workload (the default): the long-context decode layer -- 32 query /
8 KV heads, head dim 128, batch 1, 1,048,576 cached positions, bf16 K/V; keys
3-bit codes + 128-row QJL sketch, values 3-bit codes -- over 4 distinct layer
caches (3.96 GB, far above the 256 MB Infinity Cache), so that every decode
reads HBM.

A timed step is one decode pass over the layer caches (one
tq_decode_attention launch per layer).  `value` is the decode attention
throughput in GB/s of algorithmic bytes: the packed K and V records of every
attended position plus the query and output, divided by the step time.  The
quantize-append half of the metric is measured in its own timed region (the
whole-context prefill of every layer after the first), reported as
positions/s and against the fp32 roof of its sketch contraction.

`configs` repeats the measurement for the other seeded workloads that fit
the same contract: the Llama-3.1-8B-shaped 32K layer (32 layer caches), the
Command-R+-shaped 128K layer with q8 keys (64 caches) and the batched serving
workload (16 x 8K, 32 caches, 64 serving steps that each append one position
per sequence and decode over it in one launch).

Also printed: the roofline of the headline decode kernel (algorithmic bytes
per launch over its mean launch duration, from HIP events on the launch
stream around the timed region), the HBM traffic per launch measured with
rocprofv3 counters (from profiles/, when taken on the current kernel
sources), the median, minimum and maximum step time, the practical HBM read
ceiling (a plain streaming read of 2 GiB on the same GPU) with the decode
throughput as a fraction of it, and the oracle's CPU throughput on a bounded
sample of the headline workload (single-threaded).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 (matrix and vector)
FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix
HEADLINE = "long_b1_ctx1m"
CONFIG_SET = ("llama8b_b1_ctx32k", "cmdr104b_b1_ctx128k", "serving_b16_ctx8k")
# what the matrix-core decode computes in: packed codes enter the matrix
# cores as fp4 (e2m1) operands against exact digits in fp6 (e2m3, the query)
# or fp8 (e4m3, p * radius) with one E8M0 scale per 32 k-slots; every sum
# accumulates in fp32
DECODE_DTYPE = ("fp4 code operands x fp6 (query) and fp8 (p*radius) digit operands, fp32 accumulate (query: "
                "4 base-16 digits per 32-slot E8M0 block, about 15 significant bits; p*radius: 3 base-32 digits, "
                "about 14 bits; q8 keys: int8 x 3 base-128 int8 query digits, int32 accumulate)")
# name fragment of the dominant decode kernel (POLAR / POLAR_QJL keys)
DECODE_KERNEL = "decode_reg_kernel"
TRAFFIC_GLOB = os.path.join(ROOT, "profiles", "decode_reg_*_traffic.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "compressed_decode_attention_quantize_amd", "csrc", f)
                  for f in ("tq_decode_reg.hip", "tq_mfma_ops.h", "tq_quant_unit.h", "tq_device.h",
                            "tq_internal.h")]


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(workload, layers):
    """HBM bytes per decode launch measured with rocprofv3 counters (FETCH_SIZE
    + WRITE_SIZE, scaled by what they read for a copy of known size), if the
    committed measurement was taken on this workload and the kernel sources
    have not changed since; else None."""
    import glob
    for path in sorted(glob.glob(TRAFFIC_GLOB)):
        with open(path) as fh:
            kv = dict(l.strip().split("=", 1) for l in fh if "=" in l and not l.startswith("#"))
        if kv.get("workload") == workload and kv.get("source_hash") == kernel_source_hash():
            return int(float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"]))
    return None


def summarize_counters(fetch_csv, write_csv, copy_mib):
    """Per-dispatch FETCH_SIZE / WRITE_SIZE (KiB) of the decode kernel and of
    the calibration copy, from two rocprofv3 --pmc runs; prints key=value
    lines (bytes per decode launch after dividing by the copy's read/write
    factor)."""
    import csv

    def dispatches(path, counter):
        rows = []
        with open(path) as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") == counter:
                    rows.append((int(row["Dispatch_Id"]), row.get("Kernel_Name", ""), float(row["Counter_Value"])))
        return sorted(rows)

    out = {}
    for tag, path, counter in (("fetch", fetch_csv, "FETCH_SIZE"), ("write", write_csv, "WRITE_SIZE")):
        rows = dispatches(path, counter)
        dec = sorted(v for _, n, v in rows if DECODE_KERNEL in n)
        # the calibration copy: the run's last three dispatches (bench.py issues
        # the three copies after everything else), all of one kernel
        want = copy_mib * 1024.0
        tail = rows[-3:]
        if not dec or len(tail) < 3 or len({n for _, n, _ in tail}) != 1 or DECODE_KERNEL in tail[0][1]:
            raise SystemExit(f"{path}: no {DECODE_KERNEL} dispatches or no trailing calibration copies with {counter}")
        med = dec[len(dec) // 2]
        copy = sorted(v for _, _, v in tail)[1]
        factor = copy / want
        out[f"{tag}_kib_per_launch_raw"] = med
        out[f"{tag}_copy_kib"] = copy
        out[f"{tag}_copy_factor"] = round(factor, 4)
        out[f"{tag}_bytes_per_launch"] = round(med * 1024.0 / factor)
        out[f"{tag}_dispatches"] = len(dec)
    return out


def algorithmic_decode_bytes(w, cfg, tq, lens):
    kb, vb = tq.cache_bytes(cfg)
    slots = cfg.batch * cfg.n_kv_heads * ((cfg.max_ctx + 127) // 128) * 128
    krec, vrec = kb // slots, vb // slots
    recs = sum(lens) * cfg.n_kv_heads
    qo = 2 * cfg.batch * cfg.n_q_heads * cfg.head_dim * 4
    return recs * (krec + vrec) + qo, krec, vrec


def cpu_baseline(w, seed, n_pos):
    """Oracle, single-threaded, on a bounded sample of workload w: quantise the
    first n_pos positions of one layer (all KV heads; positions/s) and decode
    every query head over them (GB/s of the sample's algorithmic bytes)."""
    import numpy as np

    sys.path.insert(0, os.path.join(ROOT, "oracle"))
    import oracle
    from compressed_decode_attention_quantize_amd import synth

    ws = synth.with_ctx(w, n_pos)
    k, v = synth.make_kv(ws, n_pos, seed=seed)
    q = synth.make_q(ws, seed=seed + 1000).numpy()
    kn = k.to("cpu").float().numpy()
    vn = v.to("cpu").float().numpy()
    codec = {synth.RAW_F32: 0, synth.POLAR: 1, synth.POLAR_QJL: 2, synth.Q8_BLOCK32: 3}
    s = oracle.make_spec(d=w.d, n_q=w.n_q, n_kv=w.n_kv, batch=w.batch, max_ctx=n_pos, k_codec=codec[w.k_codec],
                         k_bits=w.k_bits, m=w.m, v_codec=codec[w.v_codec], v_bits=w.v_bits)
    P = oracle.Params(s, 42, 0)
    reps = 3   # about 10 s of single-threaded work at 32768 positions of the 32/8-head shape
    t_app = t_dec = 0.0
    lens = np.full(w.batch, n_pos, np.int32)
    # the oracle is single-threaded C; the calling thread is pinned to one
    # host core while it runs
    allowed = os.sched_getaffinity(0)
    core = min(allowed)
    os.sched_setaffinity(0, {core})
    try:
        for _ in range(reps):
            R = oracle.Records(s)
            t0 = time.perf_counter()
            for b in range(w.batch):
                oracle.quantize_into(s, P, R, kn[b], vn[b], b, 0)
            t_app += time.perf_counter() - t0
            t0 = time.perf_counter()
            oracle.decode(s, P, R, lens, q)
            t_dec += time.perf_counter() - t0
    finally:
        os.sched_setaffinity(0, allowed)
    t_app /= reps
    t_dec /= reps
    sz = oracle.spec_sizes(s)
    rec = sz["k_record"] + sz["v_record"]
    dec_bytes = w.batch * n_pos * w.n_kv * rec + 2 * w.batch * w.n_q * w.d * 4
    return {
        "value": dec_bytes / t_dec / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
        "sample": (f"the first {n_pos} positions of one layer of {w.name} (same shapes and input recipe), "
                   f"{reps} times: oracle quantize of {w.batch * n_pos} positions x {w.n_kv} KV heads "
                   f"({t_app:.1f} s each) then fp64 decode of all {w.n_q} query heads over them "
                   f"({t_dec:.1f} s each), single-threaded C on the host"),
        "append_tokens_per_s": w.batch * n_pos / t_app,
        "seconds": reps * (t_app + t_dec),
        "pinned_core": core,
        "host_cpus_allowed": len(allowed),
        "nproc": os.cpu_count(),
        "cpu_model": host_cpu_model(),
    }


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def serve_steps(args, w, layers, q, dev, tq, synth, seed, bytes_per_launch):
    """Serving steps over the layer stack: step s appends one position per
    sequence at length ctx + s to every layer and decodes q over ctx + s + 1
    positions.  Lengths are prepared per step beforehand, so the timed region
    holds only the library's launches."""
    import torch
    n_steps = args.steps
    total = args.warmup + n_steps
    g = torch.Generator(device=dev)
    g.manual_seed(seed + 3000)
    dt = torch.float32 if w.dtype == "f32" else torch.bfloat16
    kn = torch.randn((total, w.batch, 1, w.n_kv, w.d), generator=g, device=dev).to(dt)
    vn = torch.randn((total, w.batch, 1, w.n_kv, w.d), generator=g, device=dev).to(dt)
    lens = [torch.full((w.batch,), w.ctx + s, dtype=torch.int32, device=dev) for s in range(total + 1)]
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream()

    def step(s):
        for L in layers:
            if args.serve == "fused":
                tq.append_decode(L.cfg, L.params, L.k_cache, L.v_cache, lens[s], w.ctx + s, kn[s], vn[s], q, out,
                                 L.workspace)
            else:
                tq.quantize_append(L.cfg, L.params, L.k_cache, L.v_cache, lens[s], w.ctx + s, kn[s], vn[s])
                tq.decode_attention(L.cfg, L.params, L.k_cache, L.v_cache, lens[s + 1], w.ctx + s + 1, q, out,
                                    L.workspace)

    if args.settle_ms > 0:   # plain decodes (they leave the caches as they are)
        settle(layers, q, args.settle_ms / 1e3)
    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for s in range(args.warmup, total):
        step(s)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n_steps
    return {"serve": {"mode": args.serve, "steps": n_steps, "ms_per_step_all_layers": round(ms, 4),
                      "us_per_layer_step": round(ms * 1e3 / len(layers), 3),
                      "tokens_per_s": round(w.batch / (ms / 1e3), 1),
                      "decode_bytes_per_layer_step": bytes_per_launch}}


def read_ceiling(tq, dev, nbytes=2 << 30, reps=10):
    """The practical HBM read ceiling: a plain streaming read (tq_stream_read,
    16-byte non-temporal loads) over 2 GiB, well past the 256 MB last-level
    cache, timed with HIP events over `reps` back-to-back launches."""
    import torch
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    for _ in range(2):
        tq.stream_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        tq.stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = reps * nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9
    del buf
    return {"gbs": round(gbs, 1), "bytes": nbytes, "reps": reps, "kernel": "stream_read_kernel",
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def append_flop_per_position(w):
    """Arithmetic of quantising one (position, KV head): the raw FWHT of the
    key and of the value (d log2 d additions each) and, for QJL keys, the
    m x d sketch contraction (2 m d)."""
    import math
    fwht = w.d * int(math.log2(w.d))
    sketch = 2 * w.m * w.d if w.k_codec == "polar_qjl" else 0
    key = fwht if w.k_codec in ("polar", "polar_qjl", "polar_tree") else 0
    val = fwht if w.v_codec in ("polar", "polar_tree") else 0
    return sketch + key + val


def append_roofline(w, positions_per_s, krec, vrec):
    """Binding roof of the append: the m x d sketch contraction at fp32
    accuracy when it makes the append compute-bound, else HBM (inputs read,
    records written).  The contraction runs on the fp16 matrix instruction as
    three products of split operands (hi hi + lo hi + hi lo, fp32
    accumulate): `achieved` and `frac` count its fp32-equivalent flops
    against the fp32 roof (what an fp32 kernel could reach at most), and
    `fp16_matrix` the fp16 products actually issued against the fp16 roof."""
    flop = append_flop_per_position(w) * w.n_kv
    in_bytes = 2 * w.d * (4 if w.dtype == "f32" else 2)
    nbytes = (in_bytes + krec + vrec) * w.n_kv
    t_flop = flop / (FP32_PEAK_TFLOPS * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    if t_flop >= t_hbm:
        ach = positions_per_s * flop / 1e12
        sketch = 2 * w.m * w.d * w.n_kv if w.k_codec == "polar_qjl" else 0   # the contraction's share of `flop`
        f16 = 3 * positions_per_s * sketch / 1e12
        return {"bound": "fp32-equivalent", "achieved": round(ach, 2), "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / FP32_PEAK_TFLOPS, 4), "flop_per_position": flop,
                "arith": "sketch S r as three fp16 matrix products of split operands, fp32 accumulate",
                "fp16_matrix": {"achieved": round(f16, 2), "peak": FP16_PEAK_TFLOPS,
                                "frac": round(f16 / FP16_PEAK_TFLOPS, 4)},
                "kernel": "quant_kernel"}
    ach = positions_per_s * nbytes / 1e9
    return {"bound": "hbm", "achieved": round(ach, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "bytes_per_position": nbytes, "kernel": "quant_kernel"}


def build_layers(w, n_layers, args, dev, tq, room=0):
    """The workload's layer caches (or the mixed-codec / recursive polar stack
    the flags ask for)."""
    policy = None
    if args.policy:
        from compressed_decode_attention_quantize_amd import presets
        kt, vt, prot = (args.policy.split("/") + ["0"])[:3]
        policy = presets.layer_policy(n_layers, kt, vt, int(prot))
        layers = [tq.KVLayer(presets.config(tq.config_for(w, seed=42, layer=l, sparse_v=args.sparse_v),
                                            policy[l], l), dev, zero=False)
                  for l in range(n_layers)]
    elif args.tree_bits:
        tkb, tvb = (int(x) for x in args.tree_bits.split("/"))
        layers = [tq.KVLayer(tq.make_config(w.d, w.n_q, w.n_kv, w.batch, w.ctx, tq.POLAR_TREE, tkb, 0,
                                            tq.POLAR_TREE, tvb, 0, 42, l, args.sparse_v), dev, zero=False)
                  for l in range(n_layers)]
    else:
        layers = [tq.KVLayer(tq.config_for(w, seed=42, layer=l, sparse_v=args.sparse_v, max_ctx=w.ctx + room),
                             dev, zero=False)
                  for l in range(n_layers)]
    return layers, policy


def time_prefill(layers, k, v, stream):
    """Whole-context append of every layer: one untimed (layer 0), the rest
    timed back to back.  Returns seconds per layer."""
    import torch
    layers[0].append(k, v)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for L in layers[1:]:
        L.append(k, v)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / 1e3 / max(1, len(layers) - 1)


SETTLE_S = 0.15


def settle(layers, q, seconds):
    """Untimed decode passes over the layer stack for `seconds` of wall time.
    The GPU enters a run at its top clock and within a few ms of sustained
    decode drops under its power limit, then recovers over the next ~20 ms
    (1M context: ~175 us per launch for the first dozen launches, up to
    ~240 us, then ~186-195 us): the timed steps measure the sustained state,
    whatever the warm-up count."""
    import torch
    out = torch.empty_like(q)
    t0 = time.perf_counter()
    n = 0
    while True:
        for L in layers:
            L.decode(q, out=out)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
            if time.perf_counter() - t0 >= seconds:
                return n


def time_decode(layers, q, steps, warmup, stream, settle_s=SETTLE_S):
    """Decode passes over the layer stack: a settling phase (see settle), then
    `warmup` untimed, then `steps` timed with HIP events on the launch stream.
    Returns (mean ms per step, sorted per-step ms, wall seconds)."""
    import torch
    outs = [torch.empty_like(q) for _ in layers]

    def step():
        for i, L in enumerate(layers):
            L.decode(q, out=outs[i])

    if settle_s > 0:
        settle(layers, q, settle_s)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    marks[0].record(stream)
    for k_ in range(steps):
        step()
        marks[k_ + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = marks[0].elapsed_time(marks[-1]) / steps
    per_step = sorted(marks[k_].elapsed_time(marks[k_ + 1]) for k_ in range(steps))
    return step_ms, per_step, wall


def measure_config(name, args, dev, tq, synth):
    """One workload of the configs table: prefill and decode timings (the
    serving workload: fused serving steps) with their roofline fractions."""
    import torch
    w = synth.WORKLOADS[name]
    wi = synth.ORDER.index(name)
    seed = 1000 + wi
    stream = torch.cuda.current_stream()
    n_layers = w.layers
    steps = w.steps if w.steps else args.steps
    room = (args.warmup + steps) if w.steps else 0
    layers, _ = build_layers(w, n_layers, argparse.Namespace(policy="", tree_bits="", sparse_v=0), dev, tq, room)
    k, v = synth.make_kv(w, w.ctx, seed=seed, device=dev)
    q = synth.make_q(w, seed=seed + 1000, device=dev)
    app_s = time_prefill(layers, k, v, stream)
    del k, v
    cfg0 = layers[0].cfg
    nbytes, krec, vrec = algorithmic_decode_bytes(w, cfg0, tq, [w.ctx] * w.batch)
    pos_s = w.batch * w.ctx / app_s
    res = {"workload": name, "batch": w.batch, "context": w.ctx, "n_q_heads": w.n_q, "n_kv_heads": w.n_kv,
           "k_codec": f"{w.k_codec} b{w.k_bits} m{w.m}", "v_codec": f"{w.v_codec} b{w.v_bits}",
           "layers": n_layers, "record_bytes": {"k": krec, "v": vrec},
           "append_tokens_per_s": round(pos_s, 1), "append_ms_per_layer": round(app_s * 1e3, 4),
           "append_roofline": append_roofline(w, pos_s, krec, vrec)}
    if w.steps:
        sargs = argparse.Namespace(steps=steps, warmup=args.warmup, serve="fused", settle_ms=args.settle_ms)
        sv = serve_steps(sargs, w, layers, q, dev, tq, synth, seed, nbytes)["serve"]
        us = sv["us_per_layer_step"]
        # the decode of a step attends ctx + warmup + s + 1 positions, s = 0 .. steps - 1
        mean_len = w.ctx + args.warmup + (steps + 1) / 2.0
        step_bytes = algorithmic_decode_bytes(w, cfg0, tq, [mean_len] * w.batch)[0]
        gbs = step_bytes / (us * 1e-6) / 1e9
        res.update({"mode": "serving steps (tq_append_decode: append one position per sequence and decode, "
                            "one launch per layer)", "steps": steps,
                    "us_per_launch": us, "decode_bytes_per_launch": int(step_bytes),
                    "gbs": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "tokens_per_s": sv["tokens_per_s"], "ms_per_step_all_layers": sv["ms_per_step_all_layers"]})
    else:
        step_ms, per_step, _ = time_decode(layers, q, args.steps, args.warmup, stream, args.settle_ms / 1e3)
        us = step_ms * 1e3 / n_layers
        gbs = nbytes / (us * 1e-6) / 1e9
        res.update({"mode": "decode (tq_decode_attention, one launch per layer)", "steps": args.steps,
                    "us_per_launch": round(us, 3), "decode_bytes_per_launch": nbytes,
                    "gbs": round(gbs, 2), "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "ms_per_step_median": round(per_step[len(per_step) // 2], 4)})
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50,
                    help="untimed steps first (the clocks and caches settle within a few tens of ms)")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_S * 1e3,
                    help="untimed decode work before the warm-up steps, in ms of wall time (the GPU's clocks "
                         "swing under its power limit for the first ~20 ms of sustained decode)")
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--layers", type=int, default=0, help="layer caches to cycle (0 = workload default)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-configs", action="store_true", help="headline workload only")
    ap.add_argument("--cpu-sample", type=int, default=32768, metavar="N",
                    help="positions of the oracle's bounded CPU sample")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="after the run, copy MIB MiB device to device three times (counter calibration)")
    ap.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="print the traffic summary of two rocprofv3 --pmc runs and exit (no GPU)")
    ap.add_argument("--calibration-mib", type=int, default=256)
    ap.add_argument("--policy", default="", metavar="K/V/PROTECT",
                    help="per-layer cache types, e.g. turbo3/turbo2/2: keys turbo3, values turbo2, the first "
                         "and last 2 layers in q8_0 (a mixed-codec stack instead of the workload's codecs)")
    ap.add_argument("--sparse-v", type=int, default=0, metavar="T",
                    help="decode skips the value work of blocks whose weights are all below 2^(1-T) of the "
                         "running maximum (0 = dense)")
    ap.add_argument("--focus-every", type=int, default=0, metavar="E",
                    help="peaked attention: one planted key per E positions that the query heads score "
                         "about 16 nats above the rest (0 = the workload's plain keys)")
    ap.add_argument("--tree-bits", default="", metavar="KB/VB",
                    help="store keys and values with the recursive polar codec at KB and VB bits instead of the "
                         "workload's codecs (e.g. 3/2)")
    ap.add_argument("--serve", choices=["fused", "separate"], default="",
                    help="time serving steps instead of bare decodes: each step appends one position per sequence "
                         "to every layer and decodes over it, in one launch (fused) or two (separate)")
    args = ap.parse_args()
    if args.summarize_counters:
        res = summarize_counters(args.summarize_counters[0], args.summarize_counters[1], args.calibration_mib)
        res["source_hash"] = kernel_source_hash()
        res["workload"] = args.workload
        for k_, v_ in res.items():
            print(f"{k_}={v_}")
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from compressed_decode_attention_quantize_amd import synth, tq

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    wi = synth.ORDER.index(args.workload)
    w = synth.WORKLOADS[args.workload]
    n_layers = args.layers or w.layers
    data_seed = 1000 + wi
    variant = bool(args.policy or args.tree_bits or args.sparse_v or args.focus_every or args.serve)

    # ------------------------------------------------ inputs and layer caches
    k, v = synth.make_kv(w, w.ctx, seed=data_seed, device=dev)
    q = synth.make_q(w, seed=data_seed + 1000, device=dev)
    if args.focus_every:
        k, _ = synth.plant_focus_keys(w, k, q, seed=data_seed + 2000, every=args.focus_every)
    room = (args.warmup + args.steps) if args.serve else 0   # serving steps append past the prefill
    layers, policy = build_layers(w, n_layers, args, dev, tq, room)
    torch.cuda.synchronize()

    # ------------------------------------------ append: prefill of every layer
    stream = torch.cuda.current_stream()
    append_s = time_prefill(layers, k, v, stream)
    append_tok_s = w.batch * w.ctx / append_s
    del k, v

    # --------------------------------------------------------------- decode
    lens = [w.ctx] * w.batch
    cfg0 = layers[0].cfg
    bytes_per_launch, krec, vrec = algorithmic_decode_bytes(w, cfg0, tq, lens)
    if policy is not None:   # mean over the stack's layers
        per_layer = [algorithmic_decode_bytes(w, L.cfg, tq, lens)[0] for L in layers]
        bytes_per_launch = sum(per_layer) // n_layers
    step_ms, per_step, wall = time_decode(layers, q, args.steps, args.warmup, stream, args.settle_ms / 1e3)
    ceiling = read_ceiling(tq, dev)

    # average duration of one decode launch: the timed region (HIP events on
    # the launch stream) holds only back-to-back decode launches
    launch_ms = step_ms / n_layers

    value = n_layers * bytes_per_launch / (step_ms / 1e3) / 1e9
    achieved = bytes_per_launch / (launch_ms / 1e3) / 1e9
    result = {
        "metric": "decode attention HBM GB/s on packed KV (% of peak); quantize-append tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(step_ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DECODE_DTYPE,
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "context": w.ctx, "n_q_heads": w.n_q,
                   "n_kv_heads": w.n_kv, "head_dim": w.d, "k_codec": f"{w.k_codec} b{w.k_bits} m{w.m}",
                   "v_codec": f"{w.v_codec} b{w.v_bits}", "k_dtype": w.dtype, "layers": n_layers,
                   "record_bytes": {"k": krec, "v": vrec}},
        "hbm_frac": round(value / HBM_PEAK_GBS, 4),
        "append_tokens_per_s": round(append_tok_s, 1),
        "append_ms_per_layer": round(append_s * 1e3, 4),
        "append_roofline": append_roofline(w, append_tok_s, krec, vrec),
        "decode_us_per_layer": round(step_ms * 1e3 / n_layers, 3),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 4),
        "ms_per_step_min": round(per_step[0], 4),
        "ms_per_step_max": round(per_step[-1], 4),
        "hbm_read_ceiling": ceiling,
        "frac_of_read_ceiling": round(value / ceiling["gbs"], 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": committed_traffic(w.name, n_layers),
                     "kernel": DECODE_KERNEL, "bytes_per_launch": bytes_per_launch,
                     "launch_us": round(launch_ms * 1e3, 3)},
        "wall_s_timed": round(wall, 4),
        "device": torch.cuda.get_device_name(0),
    }
    if policy is not None:
        packed = sum(sum(tq.cache_bytes(L.cfg)) for L in layers)
        fp16 = n_layers * w.batch * ((w.ctx + 127) // 128) * 128 * w.n_kv * 2 * w.d * 2
        result["metric"] = "decode attention HBM GB/s over a mixed-codec layer stack"
        result["config"]["policy"] = {"spec": args.policy, "layers": [f"{c.k_type}/{c.v_type}" for c in policy]}
        result["config"]["k_codec"] = result["config"]["v_codec"] = "per layer"
        result["config"].pop("record_bytes")
        result["cache_bytes_total"] = packed
        result["compression_vs_fp16"] = round(fp16 / packed, 3)
        result["roofline"]["traffic"] = None
        for key in ("append_tokens_per_s", "append_ms_per_layer", "append_roofline"):
            result.pop(key)
    if args.tree_bits:
        result["metric"] = "decode attention HBM GB/s on packed KV, recursive polar codec; quantize-append tokens/s"
        result["config"]["k_codec"] = f"polar_tree b{args.tree_bits.split('/')[0]}"
        result["config"]["v_codec"] = f"polar_tree b{args.tree_bits.split('/')[1]}"
        result["roofline"]["traffic"] = None
        result["roofline"]["kernel"] = "decode_kernel"
        result["dtype"] = "fp32"
        result.pop("append_roofline")
    if args.sparse_v or args.focus_every:
        result["config"]["sparse_v"] = args.sparse_v
        result["config"]["focus_every"] = args.focus_every
        result["data"] = "synthetic, planted focus keys" if args.focus_every else "synthetic"
    if args.serve:
        result.update(serve_steps(args, w, layers, q, dev, tq, synth, data_seed, bytes_per_launch))
    del layers
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    if not variant and not args.no_configs and args.workload == HEADLINE:
        result["configs"] = {name: measure_config(name, args, dev, tq, synth) for name in CONFIG_SET}
    if not args.no_cpu_baseline and not variant:
        result["cpu_baseline"] = cpu_baseline(w, data_seed, min(args.cpu_sample, w.ctx))
    if args.copy_calibration:
        src = torch.empty(args.copy_calibration << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
