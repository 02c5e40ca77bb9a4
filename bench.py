"""Benchmark: quantized-KV decode attention on one MI355X.

A step is one decode step of a whole LLaMA-7B-shaped model at 32K context: for each of
the model's layers, kvq_quantize_append of the new token's key and value, then
kvq_qk_matvec and kvq_pv_matvec over that layer's compressed cache.  Every layer has its
own cache (different seeded inputs), so a step reads ~3.7 GB of compressed KV and no
layer's cache is still resident in the 256 MB last-level cache when it is read again.

Prints ONE JSON line.  value = algorithmic HBM bytes per step / step time (GB/s).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llama7b_32k")
    p.add_argument("--outlier-frac", type=float, default=None,
                   help="override the workload's outlier fraction f (k = ceil(f * 128) per vector)")
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-fp16-baseline", dest="fp16_baseline", action="store_false",
                   help="skip timing the uncompressed fp16 kernels at the same shape")
    p.add_argument("--no-codebook-fit", dest="codebook_fit", action="store_false",
                   help="skip timing the codebook fit on the layer's key calibration set")
    p.add_argument("--no-fused", dest="fused", action="store_false",
                   help="skip timing the single-pass kernel (profiling runs of the two-call path)")
    p.add_argument("--cpu-heads", type=int, default=32, help="kv-head streams per layer the oracle times in the CPU leg")
    p.add_argument("--cpu-layers", type=int, default=4, help="layers the oracle times in the CPU leg")
    p.add_argument("--kernel-steps", type=int, default=5,
                   help="rounds of back-to-back launches (one per layer) timed per entry point for the roofline")
    p.add_argument("--traffic-probe", action="store_true",
                   help="after the run, launch a 256 MiB int32 bitwise_not (known bytes) to calibrate HBM counters")
    p.add_argument("--summarize-counters", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="write profiles/traffic.json from rocprofv3 FETCH_SIZE / WRITE_SIZE runs of this script "
                        "with --traffic-probe, then exit")
    p.add_argument("--no-graph", dest="graph", action="store_false",
                   help="launch every kernel eagerly instead of replaying one HIP graph per step")
    return p.parse_args()


def algorithmic_bytes(wl, L):
    """Bytes one layer's kernels must move at cache length L (per step)."""
    k = wl.n_outliers
    tok_heads = wl.batch * wl.n_kv_heads * L
    q_tok = wl.batch * wl.n_q_heads * L
    qk = tok_heads * (wl.head_dim * wl.k_bits // 8 + 3 * k) + q_tok * 4  # K records + outliers, logits write
    pv = tok_heads * (wl.head_dim * wl.v_bits // 8 + 3 * k + 2) + q_tok * 4  # V tiles + outliers + scale, logits read
    # append: read 2 fp16 vectors, write one key record, read-modify-write one value tile,
    # outliers and scale, per (sequence, kv head)
    nvec = wl.batch * wl.n_kv_heads * wl.n_new
    app = nvec * (2 * wl.head_dim * 2 + wl.head_dim * wl.k_bits // 8 + 2 * 1024 * wl.v_bits + 6 * k + 2)
    return qk, pv, app


def source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_decode_kvq_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload, kernel, src_hash):
    """HBM bytes per launch measured with rocprofv3 counters on this workload, if the
    committed measurement was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(workload, {}).get(kernel)
    if not e or e.get("source_hash") != src_hash:
        return None
    return e.get("hbm_bytes_per_launch")


PROBE_BYTES = 256 << 20  # the calibration kernel reads and writes this many bytes


def counter_means(d, counter):
    """Mean value of `counter` per dispatch, by kernel, from rocprofv3 counter CSVs under d."""
    import csv
    import glob
    import re
    acc = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") != counter:
                continue
            m = re.search(r"::(qk_lut_kernel|qk_kernel|pv_partial_kernel|pv_combine_kernel|append_kernel)\b|(bitwise_not)",
                          row.get("Kernel_Name", ""))
            if m:
                acc.setdefault(m.group(1) or m.group(2), []).append(float(row["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_counters(fetch_dir, write_dir, workload):
    """HBM bytes per launch = FETCH_SIZE and WRITE_SIZE (KiB per dispatch) each scaled by the
    factor that maps the same counter of the calibration kernel onto its known bytes."""
    fetch, write = counter_means(fetch_dir, "FETCH_SIZE"), counter_means(write_dir, "WRITE_SIZE")
    f_scale = PROBE_BYTES / (fetch["bitwise_not"] * 1024.0)
    w_scale = PROBE_BYTES / (write["bitwise_not"] * 1024.0)
    out = {"calibration": {"kernel": "bitwise_not over 256 MiB int32", "fetch_kib": fetch["bitwise_not"],
                           "write_kib": write["bitwise_not"], "fetch_scale": f_scale, "write_scale": w_scale}}
    groups = {"qk_lut_kernel": (["qk_lut_kernel"], ["qk_lut.hip", "kvq_device.h"]),
              "qk_kernel": (["qk_kernel"], ["qk.hip", "kvq_device.h"]),
              "pv_partial_kernel+pv_combine_kernel": (["pv_partial_kernel", "pv_combine_kernel"],
                                                      ["pv.hip", "kvq_device.h"])}
    for name, (kerns, src) in groups.items():
        if not all(k in fetch and k in write for k in kerns):
            continue
        fk, wk = sum(fetch[k] for k in kerns), sum(write[k] for k in kerns)
        out[name] = {"source_hash": source_hash(src), "fetch_kib": fk, "write_kib": wk,
                     "hbm_bytes_per_launch": round(fk * 1024.0 * f_scale + wk * 1024.0 * w_scale)}
    path = os.path.join(ROOT, "profiles", "traffic.json")
    allw = {}
    if os.path.exists(path):
        with open(path) as f:
            allw = json.load(f)
        if "calibration" in allw:  # single-workload layout of older files
            allw = {}
    allw[workload] = out
    with open(path, "w") as f:
        json.dump(allw, f, indent=1)
    print(json.dumps(out, indent=1))


def cpu_model():
    """The host CPU's model name (Linux), or the platform string."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


def cpu_baseline(wl, seed, n_streams, n_layers):
    """Time the oracle (as it stands) on a bounded sample of the same step: the decode-step
    append and full-length decode attention for n_streams (sequence, kv head) streams of
    each of n_layers layers, on one thread; report the rate scaled to algorithmic bytes
    per second."""
    import torch
    from threadpoolctl import threadpool_limits

    L = wl.seq_len
    sm = 1.0 / math.sqrt(wl.head_dim)
    elapsed = 0.0
    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        for li in range(n_layers):
            for i in range(n_streams):
                elapsed += cpu_stream(wl, seed + li, i, L, sm)
    return {"value": round(stream_bytes(wl) * n_streams * n_layers / elapsed / 1e9, 6), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n_streams} of {wl.batch * wl.n_kv_heads} kv-head streams x {n_layers} layers, L={L + 1}: "
                      f"append of the new token + float64 decode attention, {elapsed:.1f} s, 1 thread, "
                      f"{cpu_model()}"}


def cpu_baseline_parallel(wl, seed, n_streams, n_layers, workers):
    """The same sample spread over `workers` single-threaded processes (spawned, so they
    share nothing with this process's GPU state).  Each worker times its streams as the
    serial leg does; the slowest worker's timed total is the parallel run's time."""
    import multiprocessing as mp

    L = wl.seq_len
    sm = 1.0 / math.sqrt(wl.head_dim)
    tasks = [(wl, seed + li, i, L, sm) for li in range(n_layers) for i in range(n_streams)]
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers, initializer=_cpu_worker_init, initargs=(wl, seed, sm)) as pool:
        timed = pool.starmap(_cpu_worker_task, [(w, tasks[w::workers]) for w in range(workers)])
    slowest = max(timed)
    return {"value": round(stream_bytes(wl) * len(tasks) / slowest / 1e9, 6), "unit": "GB/s", "cores": workers,
            "kind": "oracle",
            "sample": f"the serial leg's sample over {workers} single-threaded processes: slowest worker "
                      f"{slowest:.2f} s of timed oracle work (total {sum(timed):.1f} s), {cpu_model()}"}


def _cpu_worker_init(wl, seed, sm):
    from threadpoolctl import threadpool_limits
    import torch
    threadpool_limits(limits=1)
    torch.set_num_threads(1)
    cpu_stream(wl, seed, 0, 64, sm)  # untimed warm-up of the oracle's code paths


def _cpu_worker_task(w, tasks):
    return sum(cpu_stream(*t) for t in tasks)


def stream_bytes(wl):
    """Algorithmic bytes of one (sequence, kv head) stream's share of a decode step."""
    qk, pv, app = algorithmic_bytes(wl, wl.seq_len + 1)
    return (qk + pv + app) / (wl.batch * wl.n_kv_heads)


def cpu_stream(wl, seed, i, L, sm):
    """Oracle seconds for stream i (sequence i // Hkv, kv head i % Hkv) of one layer: the
    new token's quantization and the decode attention of every query head of its group
    over all L + 1 tokens (the prefix quantization is not timed)."""
    import numpy as np

    import oracle
    import synth

    b, h = divmod(i, wl.n_kv_heads)
    ks = synth.key_scale(seed, wl)
    cbk, cbv = synth.codebook(seed, wl.k_bits, "k"), synth.codebook(seed, wl.v_bits, "v")
    q = synth.queries(seed, wl)
    kx = synth.keys(seed, wl, b, h, L + 1).numpy()
    vx = synth.values(seed, wl, b, h, L + 1).numpy()
    cache = oracle.quantize_stream(kx[:L], vx[:L], ks[h], cbk, cbv, wl.n_outliers)  # prefix: not timed
    t0 = time.perf_counter()
    new = oracle.quantize_stream(kx[L:], vx[L:], ks[h], cbk, cbv, wl.n_outliers)
    full = oracle.StreamCache(*(np.concatenate([a, b]) for a, b in zip(
        (cache.k_codes, cache.k_idx, cache.k_val, cache.v_codes, cache.v_idx, cache.v_val, cache.v_scale),
        (new.k_codes, new.k_idx, new.k_val, new.v_codes, new.v_idx, new.v_val, new.v_scale))))
    oracle.pack_key_records(new.k_codes, wl.k_bits)
    for hq in range(h * wl.group, (h + 1) * wl.group):
        oracle.decode_head(q[b, hq].float().numpy().astype(np.float64), full, ks[h], cbk, cbv, wl.rope_base, sm)
    return time.perf_counter() - t0


def stream_ceiling(nbytes=1 << 30, reps=10):
    """HBM read bandwidth of the library's plain streaming-read kernel over a 1 GiB buffer
    (four times the last-level cache), the practical ceiling beside the 8 TB/s peak."""
    import torch

    import long_context_decode_kvq_amd as kvq
    buf = torch.zeros(nbytes // 4, dtype=torch.int32, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    kvq.stream_read(buf, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        kvq.stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del buf
    return {"kernel": "kvq_stream_read", "bytes": nbytes, "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "pct_of_peak": round(100 * nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 1)}


def key_scale_leg(wl, cfg, seed):
    """Per-channel key scale over a whole prompt of the workload (the keys a prefill
    appends), each vector's outliers left out, and the per-channel outlier threshold at a
    1 % share over the same keys; returns each one's time and bytes read per second."""
    import torch

    import long_context_decode_kvq_amd as kvq
    import synth
    n = wl.seq_len
    keys = torch.empty(wl.batch, n, wl.n_kv_heads, wl.head_dim, dtype=torch.float16, device="cuda")
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            keys[b, :, h] = synth.keys(seed, wl, b, h, n, "cuda")
    out = torch.empty(wl.n_kv_heads, wl.head_dim, dtype=torch.float32, device="cuda")
    kvq.key_scale(cfg, keys, True, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        kvq.key_scale(cfg, keys, True, out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 5
    nbytes = keys.numel() * 2
    # the per-channel outlier rule's threshold over the same prompt (two passes over the keys)
    ws = torch.empty((kvq.key_threshold_workspace_bytes(cfg, n) + 3) // 4, dtype=torch.int32, device="cuda")
    kvq.key_threshold(cfg, keys, 0.01, out, ws)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(5):
        kvq.key_threshold(cfg, keys, 0.01, out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms_t = e0.elapsed_time(e1) / 5
    del keys, ws
    return ({"tokens": wl.batch * n, "exclude_outliers": True, "ms": round(ms, 4),
             "gbs": round(nbytes / (ms * 1e-3) / 1e9, 1)},
            {"tokens": wl.batch * n, "outlier_frac": 0.01, "ms": round(ms_t, 4),
             "gbs_per_pass": round(2 * nbytes / (ms_t * 1e-3) / 1e9, 1)})


def codebook_fit_leg(wl, seed, iters=20, n_calib=4096):
    """Codebook fit (k-means) on the key calibration set of one layer: every kv head's
    n_calib calibration tokens divided by the per-channel key scale, fitted for wl.k_bits."""
    import torch

    import long_context_decode_kvq_amd as kvq
    import synth
    ks = torch.from_numpy(synth.key_scale(seed, wl)).cuda()
    u = torch.cat([(synth.keys(seed, wl, 0, h, n_calib, "cuda").float() / ks[h]).reshape(-1)
                   for h in range(wl.n_kv_heads)]).contiguous()
    out = torch.empty(1 << wl.k_bits, dtype=torch.float16, device="cuda")
    ws = torch.empty(int(kvq.load_library().kvq_fit_workspace_bytes()), dtype=torch.uint8, device="cuda")
    kvq.fit_codebook(u, wl.k_bits, iters, out, ws)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        kvq.fit_codebook(u, wl.k_bits, iters, out, ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    per_iter = ms / iters
    return {"inputs": u.numel(), "bits": wl.k_bits, "iterations": iters, "ms": round(ms, 4),
            "ms_per_iteration": round(per_iter, 5), "gbs_per_pass": round(4 * u.numel() / (per_iter * 1e-3) / 1e9, 1),
            "codebook": [float(x) for x in out.float().cpu()]}


def fp16_baseline(wl, cfg, L, kernel_steps, kt, n_layers=4):
    """The uncompressed fp16 kernels on the same shape: seeded fp16 caches of n_layers layers
    (each larger than the 256 MB last-level cache), per-launch times measured like the
    compressed kernels', and the compressed path's speed-up over them."""
    import torch

    import long_context_decode_kvq_amd as kvq
    import synth
    gen = torch.Generator(device="cuda").manual_seed(12345)
    caches = []
    for li in range(n_layers):
        c = kvq.Fp16Cache(cfg)
        c.k.copy_(torch.randn(c.k.shape, generator=gen, device="cuda").half())
        c.v.copy_(torch.randn(c.v.shape, generator=gen, device="cuda").half())
        c.set_lengths([L] * cfg.batch)
        caches.append((c, synth.queries(li, wl, "cuda"), kvq.DecodeBuffers(c)))
    torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)
    rounds = {"qk": [], "pv": []}
    for _ in range(kernel_steps + 1):
        e0, e1, e2 = ev(), ev(), ev()
        e0.record()
        for c, q, b in caches:
            kvq.fp16_qk_matvec(c, q, b.logits, max_len=L)
        e1.record()
        for c, q, b in caches:
            kvq.fp16_pv_matvec(c, b.logits, b.out, b.workspace, max_len=L)
        e2.record()
        rounds["qk"].append((e0, e1))
        rounds["pv"].append((e1, e2))
    torch.cuda.synchronize()
    ms = {k: sum(a.elapsed_time(b) for a, b in v[1:]) / (kernel_steps * n_layers) for k, v in rounds.items()}
    per_head_tok = cfg.batch * cfg.n_kv_heads * L
    byt = {"qk": per_head_tok * 256 + 4 * cfg.batch * cfg.n_q_heads * L,
           "pv": per_head_tok * 256 + 4 * cfg.batch * cfg.n_q_heads * L}
    del caches
    torch.cuda.empty_cache()
    return {"kernel_ms": {k: round(v, 5) for k, v in ms.items()},
            "kernel_gbs": {k: round(byt[k] / (ms[k] * 1e-3) / 1e9, 1) for k in ms},
            "speedup_of_quantized": {"qk": round(ms["qk"] / kt["qk"], 3), "pv": round(ms["pv"] / kt["pv"], 3),
                                     "qk+pv": round((ms["qk"] + ms["pv"]) / (kt["qk"] + kt["pv"]), 3)},
            "layers_timed": n_layers, "data": "seeded N(0,1) fp16 keys (as stored after RoPE) and values"}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "kvq runs on one GPU; --gpus must be 1 "
                          "(sharding across GPUs is designed, not built)"}))
        sys.exit(2)
    import torch

    import long_context_decode_kvq_amd as kvq
    import synth

    wl = synth.WORKLOADS[args.workload]
    if args.outlier_frac is not None:
        wl = wl.with_(outlier_frac=args.outlier_frac)
    dev = "cuda"
    kvq.load_library()
    L0 = wl.seq_len
    total_new = (args.warmup + args.steps + args.kernel_steps) * wl.n_new
    max_seq = ((L0 + total_new + 63) // 64) * 64
    cfg = kvq.CacheConfig(wl.batch, wl.n_q_heads, wl.n_kv_heads, max_seq, wl.k_bits, wl.v_bits, wl.n_outliers,
                          wl.head_dim, wl.rope_base)

    # ---- build one cache per layer (prefill through kvq_quantize_append) --------------
    layers = []
    for li in range(args.layers):
        s = args.seed * 1000 + li
        ks = torch.from_numpy(synth.key_scale(s, wl))
        cache = kvq.KVCache(cfg, ks, torch.from_numpy(synth.codebook(s, wl.k_bits, "k")),
                            torch.from_numpy(synth.codebook(s, wl.v_bits, "v")), dev)
        n_all = L0 + total_new
        kraw = torch.empty(wl.batch, n_all, wl.n_kv_heads, wl.head_dim, dtype=torch.float16, device=dev)
        vraw = torch.empty_like(kraw)
        for b in range(wl.batch):
            for h in range(wl.n_kv_heads):
                kraw[b, :, h] = synth.keys(s, wl, b, h, n_all, dev)
                vraw[b, :, h] = synth.values(s, wl, b, h, n_all, dev)
        kvq.quantize_append(cache, kraw[:, :L0].contiguous(), vraw[:, :L0].contiguous())
        new_k = [kraw[:, L0 + i * wl.n_new: L0 + (i + 1) * wl.n_new].contiguous() for i in range(total_new // wl.n_new)]
        new_v = [vraw[:, L0 + i * wl.n_new: L0 + (i + 1) * wl.n_new].contiguous() for i in range(total_new // wl.n_new)]
        del kraw, vraw
        layers.append(dict(cache=cache, q=synth.queries(s, wl, dev), bufs=kvq.DecodeBuffers(cache),
                           new_k=new_k, new_v=new_v))
        torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)
    n_graph_steps = args.warmup + args.steps

    def eager_step(i):
        for lay in layers:
            c = lay["cache"]
            kvq.quantize_append(c, lay["new_k"][i], lay["new_v"][i])
            L = max(c.lengths)
            kvq.qk_matvec(c, lay["q"], lay["bufs"].logits, max_len=L)
            kvq.pv_matvec(c, lay["bufs"].logits, lay["bufs"].out, lay["bufs"].workspace, max_len=L)

    # One HIP graph per decode step: every layer's device-positioned append of that
    # step's new token, then q.K^T and softmax.V over the whole capacity bound (kernels
    # read the live length from the device).
    graphs = []
    if args.graph:
        for i in range(n_graph_steps):
            g = torch.cuda.CUDAGraph()
            saved = [list(l["cache"].lengths) for l in layers]
            with torch.cuda.graph(g):
                for lay in layers:
                    c = lay["cache"]
                    kvq.quantize_append(c, lay["new_k"][i], lay["new_v"][i], device_positions=True)
                    kvq.qk_matvec(c, lay["q"], lay["bufs"].logits, max_len=max_seq)
                    kvq.pv_matvec(c, lay["bufs"].logits, lay["bufs"].out, lay["bufs"].workspace, max_len=max_seq)
            for l, sv in zip(layers, saved):
                l["cache"].lengths = sv
            graphs.append(g)
        torch.cuda.synchronize()

    def run_step(i):
        if args.graph:
            graphs[i].replay()
            for l in layers:
                l["cache"].lengths = [x + wl.n_new for x in l["cache"].lengths]
        else:
            eager_step(i)

    for i in range(args.warmup):
        run_step(i)
    torch.cuda.synchronize()
    start_len = max(layers[0]["cache"].lengths)
    t_start, t_end = ev(), ev()
    w0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        run_step(args.warmup + i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps
    assert [int(x) for x in layers[0]["cache"].seq_len.cpu()] == layers[0]["cache"].lengths

    # Per-launch kernel durations: HIP events (on the launch stream) around the layers'
    # back-to-back launches of one entry point, so launch overhead overlaps execution.
    L_now = max(layers[0]["cache"].lengths)
    kern_events = {"qk": [], "pv": []}
    for _ in range(args.kernel_steps):
        e0, e1, e2 = ev(), ev(), ev()
        e0.record()
        for lay in layers:
            kvq.qk_matvec(lay["cache"], lay["q"], lay["bufs"].logits, max_len=L_now)
        e1.record()
        for lay in layers:
            kvq.pv_matvec(lay["cache"], lay["bufs"].logits, lay["bufs"].out, lay["bufs"].workspace, max_len=L_now)
        e2.record()
        kern_events["qk"].append((e0, e1))
        kern_events["pv"].append((e1, e2))
    torch.cuda.synchronize()
    # the single-pass kernel (one query head per kv head, 2/3-bit keys) on the same layers
    fused_events = []
    if args.fused and wl.group == 1 and wl.k_bits <= 3:
        for _ in range(args.kernel_steps):
            e0, e1 = ev(), ev()
            e0.record()
            for lay in layers:
                kvq.fused_decode_attention(lay["cache"], lay["q"], lay["bufs"].out, lay["bufs"].workspace, max_len=L_now)
            e1.record()
            fused_events.append((e0, e1))
        torch.cuda.synchronize()

    # the decode step's append alone: every layer's device-positioned append of one token
    # per sequence, back to back (the capacity holds these tokens too)
    # per decode step (recorded once as a HIP graph when graphs are on, so the host's launch
    # rate does not set the time of these short kernels)
    def appends():
        for j in range(args.kernel_steps):
            for lay in layers:
                kvq.quantize_append(lay["cache"], lay["new_k"][n_graph_steps + j], lay["new_v"][n_graph_steps + j],
                                    device_positions=True)
    e0, e1 = ev(), ev()
    if args.graph:
        g_app = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_app):
            appends()
        torch.cuda.synchronize()
        e0.record()
        g_app.replay()
        e1.record()
    else:
        e0.record()
        appends()
        e1.record()
    torch.cuda.synchronize()
    app_events = [(e0, e1)]
    for lay in layers:
        lay["cache"].lengths = [x + wl.n_new * args.kernel_steps for x in lay["cache"].lengths]
    ceiling = stream_ceiling()

    # bytes: lengths grow by n_new per step; use the mean length over the timed steps
    L_mean = start_len + wl.n_new * (args.steps + 1) / 2.0
    qk_b, pv_b, app_b = algorithmic_bytes(wl, L_mean)
    step_bytes = args.layers * (qk_b + pv_b + app_b)
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    # the same without the logits (written by q.K^T, read by softmax.V: 8 bytes per query
    # head and token), the KV-only figure a single-pass kernel would be judged by
    kv_only_gbs = (step_bytes - args.layers * 8 * wl.batch * wl.n_q_heads * L_mean) / (ms_step * 1e-3) / 1e9
    kv_tok_s = args.layers * wl.batch * L_mean / (ms_step * 1e-3)

    n_lay = len(layers)
    kt = {k: sum(a.elapsed_time(b) for a, b in v) / (len(v) * n_lay) for k, v in kern_events.items()}  # ms/launch
    qk_bk, pv_bk, _ = algorithmic_bytes(wl, L_now)
    dom = max(kt, key=kt.get)
    dom_bytes = {"qk": qk_bk, "pv": pv_bk}[dom]
    achieved = dom_bytes / (kt[dom] * 1e-3) / 1e9
    qk_name, qk_src = (("qk_lut_kernel", "qk_lut.hip") if wl.group == 1 and wl.k_bits <= 3 else ("qk_kernel", "qk.hip"))
    dom_name = {"qk": qk_name, "pv": "pv_partial_kernel+pv_combine_kernel"}[dom]
    src = {"qk": [qk_src, "kvq_device.h"], "pv": ["pv.hip", "kvq_device.h"]}[dom]
    # counted traffic is stored per workload as defined (another outlier count moves other bytes)
    traffic = traffic_from_profile(args.workload, dom_name, source_hash(src)) if args.outlier_frac is None else None

    line = {
        "metric": "quantized-KV decode attention: achieved HBM GB/s (% of peak) + KV-tokens/s",
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded N(0,1) keys with 4 x10 channels, N(0,1) values; fp16 queries)",
        "config": {"workload": args.workload, "layers": args.layers, "batch": wl.batch,
                   "q_heads": wl.n_q_heads, "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim,
                   "seq_len": wl.seq_len, "k_bits": wl.k_bits, "v_bits": wl.v_bits,
                   "outliers_per_vector": wl.n_outliers, "new_tokens_per_step": wl.n_new},
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "kv_only_gbs": round(kv_only_gbs, 1),
        "kv_tokens_per_s": round(kv_tok_s, 1),
        "kernel_ms": {k: round(v, 5) for k, v in kt.items()},
        "kernel_gbs": {"qk": round(qk_bk / (kt["qk"] * 1e-3) / 1e9, 1),
                       "pv": round(pv_bk / (kt["pv"] * 1e-3) / 1e9, 1)},
        "append_us_per_layer": round(1000 * app_events[0][0].elapsed_time(app_events[0][1]) / (args.kernel_steps * n_lay), 2),
        "hbm_read_ceiling": ceiling,
        "graph": bool(args.graph),
        "wall_s_timed": round(wall, 3),
        "roofline": {"kernel": dom_name, "launches_timed": args.kernel_steps * n_lay,
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    if fused_events:
        fms = sum(a.elapsed_time(b) for a, b in fused_events) / (len(fused_events) * n_lay)
        line["fused_single_pass"] = {"ms_per_layer": round(fms, 5), "two_call_ms_per_layer": round(kt["qk"] + kt["pv"], 5),
                                     "gbs": round((qk_bk + pv_bk - 8 * wl.batch * wl.n_q_heads * L_now) / (fms * 1e-3) / 1e9, 1)}
    if args.codebook_fit:
        line["key_scale_calibration"], line["key_threshold_calibration"] = key_scale_leg(wl, cfg, args.seed * 1000 + 7)
        line["codebook_fit"] = codebook_fit_leg(wl, args.seed * 1000)
    if args.fp16_baseline:
        line["fp16_baseline"] = fp16_baseline(wl, cfg, L_now, args.kernel_steps, kt)
    if args.traffic_probe:
        src_p = torch.ones(PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
        dst_p = torch.empty_like(src_p)
        torch.bitwise_not(src_p, out=dst_p)
        torch.cuda.synchronize()
        del src_p, dst_p
    if not args.no_cpu_baseline:
        n_streams = min(args.cpu_heads, wl.batch * wl.n_kv_heads)
        line["cpu_baseline"] = cpu_baseline(wl, args.seed * 1000, n_streams, args.cpu_layers)
        # at most 16 worker processes (a host's share per GPU), whatever the host reports
        workers = max(1, min(16, len(os.sched_getaffinity(0))))
        if workers > 1:
            line["cpu_baseline_parallel"] = cpu_baseline_parallel(wl, args.seed * 1000, n_streams, args.cpu_layers,
                                                                  workers)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
