"""Benchmark: quantized-KV decode attention on one MI355X.

Default step: one decode step of a whole LLaMA-7B-shaped model (32 layers, 32 heads of
128) at 1,048,576 tokens of context with 2-bit keys and values and 1 % outliers per
vector: for each layer, kvq_quantize_append of the new token's key and value (position
read on the device), then kvq_qk_matvec and kvq_pv_matvec over that layer's compressed
cache, captured as one HIP graph per step.  All 32 layers stay resident (83.8 GB), so a
step reads 92 GB and no layer is still in the 256 MB last-level cache when read again.

The same JSON line carries the other decode workloads (the 128K-token 4-bit layer at 0,
0.5 and 1 % outliers, the batch-16 Llama-3-8B-shaped GQA layer at 64K tokens and the
32K-token 3-bit layer), measured the same way on a few resident layers each.

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
METRIC = "quantized-KV decode attention: achieved HBM GB/s (% of peak) + KV-tokens/s"
DTYPE = "f32 (softmax.V dense terms: f16 x f16 products summed in f32)"
# decode workloads reported beside the headline: name -> (outlier fractions, layers); each
# step is a whole 32-layer model's decode step, as in the headline (LLaMA-7B and
# Llama-3-8B both have 32 layers), so one graph launch per step is spread over 32 layers
EXTRA = {"llama7b_128k_4bit": ((0.0, 0.005, 0.01), 32), "llama3_8b_gqa_b16_64k": ((None,), 32),
         "llama7b_32k": ((None,), 32)}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--workload", default="llama7b_1m_2bit")
    p.add_argument("--outlier-frac", type=float, default=None,
                   help="override the workload's outlier fraction f (k = ceil(f * 128) per vector)")
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--seed", type=int, default=0)
    p.add_argument("--no-cpu-baseline", action="store_true",
                   help="skip the oracle leg (its parity check of a sampled stream and its timing)")
    p.add_argument("--no-extra", dest="extra", action="store_false",
                   help="skip the other decode workloads")
    p.add_argument("--no-fp16-baseline", dest="fp16_baseline", action="store_false",
                   help="skip timing the uncompressed fp16 kernels at the same shape")
    p.add_argument("--no-codebook-fit", dest="codebook_fit", action="store_false",
                   help="skip timing the calibration steps (key scale, key threshold, codebook fit)")
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
    # append, per new (sequence, kv head): read the fp16 key and value vectors, write the
    # key record, the value codes (set in place), both vectors' outliers and the value scale
    nvec = wl.batch * wl.n_kv_heads * wl.n_new
    app = nvec * (2 * wl.head_dim * 2 + wl.head_dim * (wl.k_bits + wl.v_bits) // 8 + 6 * k + 2)
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
KERNEL_SOURCES = {"qk_lut_kernel": ["qk_lut.hip", "kvq_device.h"], "qk_kernel": ["qk.hip", "kvq_device.h"],
                  "qk_mfma_kernel": ["qk_mfma.hip", "kvq_device.h"],
                  "pv_partial_kernel+pv_combine_kernel": ["pv.hip", "kvq_device.h"]}


def counter_means(d, counter):
    """Mean value of `counter` per dispatch, by kernel, from rocprofv3 counter output under
    d (CSV files or rocpd databases)."""
    import csv
    import glob
    import re
    import sqlite3
    pat = re.compile(r"::(qk_lut_kernel|qk_mfma_kernel|qk_kernel|pv_partial_kernel|pv_combine_kernel|append_kernel)\b"
                     r"|(bitwise_not)")
    acc = {}

    def add(name, value):
        m = pat.search(name or "")
        if m:
            acc.setdefault(m.group(1) or m.group(2), []).append(float(value))

    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for row in csv.DictReader(open(f)):
            if row.get("Counter_Name") == counter:
                add(row.get("Kernel_Name"), row["Counter_Value"])
    for f in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
        con = sqlite3.connect(f)
        for name, value in con.execute("select kernel_name, value from counters_collection where counter_name = ?",
                                       (counter,)):
            add(name, value)
    return {k: sum(v) / len(v) for k, v in acc.items()}


def summarize_counters(fetch_dir, write_dir, workload):
    """HBM bytes per launch = FETCH_SIZE and WRITE_SIZE (KiB per dispatch) each scaled by the
    factor that maps the same counter of the calibration kernel onto its known bytes."""
    fetch, write = counter_means(fetch_dir, "FETCH_SIZE"), counter_means(write_dir, "WRITE_SIZE")
    f_scale = PROBE_BYTES / (fetch["bitwise_not"] * 1024.0)
    w_scale = PROBE_BYTES / (write["bitwise_not"] * 1024.0)
    out = {"calibration": {"kernel": "bitwise_not over 256 MiB int32", "fetch_kib": fetch["bitwise_not"],
                           "write_kib": write["bitwise_not"], "fetch_scale": f_scale, "write_scale": w_scale}}
    for name, src in KERNEL_SOURCES.items():
        kerns = name.split("+")
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


def stream_bytes(wl, L):
    """Algorithmic bytes of one (sequence, kv head) stream's share of a decode step."""
    qk, pv, app = algorithmic_bytes(wl, L)
    return (qk + pv + app) / (wl.batch * wl.n_kv_heads)


def cpu_baseline_and_gate(wl, lay, seed, b, h, L0):
    """The oracle leg, run before the timed region on one sampled (sequence, kv head)
    stream of the first layer, whose prompt of L0 tokens the GPU has appended:
      - parity gate: the oracle quantizes the same seeded prompt; the GPU cache must hold
        the same packed codes, outlier indices/values and value scales bit for bit, and
        kvq_qk_matvec / kvq_pv_matvec over it must match the oracle's logits and outputs
        for every query head of the stream's group within the 1e-3 relative criterion
        (exits non-zero otherwise);
      - cpu_baseline: the oracle's decode-step work for that stream (quantizing one new
        token, then float64 decode attention of every query head of the group over the
        L0 + 1 tokens) timed on one thread, as algorithmic bytes per second (the prompt's
        quantization is set-up, not timed)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import long_context_decode_kvq_amd as kvq
    import oracle
    import synth

    c = lay["cache"]
    cfg = c.cfg
    sm = 1.0 / math.sqrt(wl.head_dim)
    ks = lay["k_scale"]
    cbk, cbv = lay["cbk"], lay["cbv"]
    t_gate = time.perf_counter()
    # GPU side: the layer's logits and outputs at the prompt length
    kvq.qk_matvec(c, lay["q"], lay["bufs"].logits, max_len=L0)
    kvq.pv_matvec(c, lay["bufs"].logits, lay["bufs"].out, lay["bufs"].workspace, max_len=L0)
    torch.cuda.synchronize()
    hq0, hq1 = h * wl.group, (h + 1) * wl.group
    g_logits = lay["bufs"].logits[b, hq0:hq1, :L0].cpu().numpy()
    g_out = lay["bufs"].out[b, hq0:hq1].cpu().numpy()
    g_rec = c.k_records()[b, h, :L0].cpu().numpy()
    g_tiles = c.v_tiles()[b, h, : (L0 + 63) // 64].cpu().numpy()
    # the stream as the GPU drew it (the device generator, same length), then on the host:
    # the prompt and the decode step's first token
    k16 = synth.keys(seed, wl, b, h, lay["n_all"], "cuda")[:L0 + 1].cpu().numpy()
    v16 = synth.values(seed, wl, b, h, lay["n_all"], "cuda")[:L0 + 1].cpu().numpy()
    st = oracle.quantize_stream(k16[:L0], v16[:L0], ks[h], cbk, cbv, wl.n_outliers)
    codes_ok = np.array_equal(g_rec, oracle.pack_key_records(st.k_codes, wl.k_bits))
    codes_ok &= np.array_equal(g_tiles, oracle.pack_value_tiles(st.v_codes, wl.v_bits, g_tiles.shape[0] * 64))
    k = wl.n_outliers
    if k:
        for kind, idx, val in (("k", st.k_idx, st.k_val), ("v", st.v_idx, st.v_val)):
            gi, gv = c.outliers(kind)
            codes_ok &= np.array_equal(gi[b, h, :L0].cpu().numpy(), idx)
            codes_ok &= np.array_equal(gv[b, h, :L0].cpu().numpy().view(np.uint16), val)
    scales = c.v_scale.view(cfg.batch, cfg.n_kv_heads, cfg.max_seq)[b, h, :L0].cpu().numpy().view(np.uint16)
    codes_ok &= np.array_equal(scales, st.v_scale)
    worst_l = worst_o = rel_l = rel_o = 0.0

    def max_rel(got, ref):
        # largest |got - ref| / |ref| over the elements with |ref| above 1e-2 of ref's rms
        r = np.abs(ref)
        m = r > 1e-2 * np.sqrt(np.mean(ref * ref))
        return float((np.abs(got - ref)[m] / r[m]).max()) if m.any() else 0.0

    q = lay["q"]
    for j, hq in enumerate(range(hq0, hq1)):
        qh = q[b, hq].float().cpu().numpy().astype(np.float64)
        ref_l, ref_o = oracle.decode_head(qh, st, ks[h], cbk, cbv, wl.rope_base, sm)
        tl = oracle.logit_tolerance_scale(qh, st, ks[h], cbk, wl.rope_base, sm)
        to = oracle.output_tolerance_scale(ref_l, st, cbv)
        worst_l = max(worst_l, float((np.abs(g_logits[j] - ref_l) / np.maximum(tl, 1e-300)).max()))
        worst_o = max(worst_o, float((np.abs(g_out[j] - ref_o) / np.maximum(to, 1e-300)).max()))
        rel_l, rel_o = max(rel_l, max_rel(g_logits[j], ref_l)), max(rel_o, max_rel(g_out[j], ref_o))
    gate = {"layer": 0, "stream": [b, h], "tokens": L0, "codes_bit_exact": bool(codes_ok),
            "worst_logit_err_over_scale": worst_l, "worst_output_err_over_scale": worst_o, "criterion": 1e-3,
            # reported only: the plain relative error where the reference is not near zero
            "max_rel_err_logits": rel_l, "max_rel_err_outputs": rel_o, "rel_err_where": "|ref| > 1e-2 rms(ref)",
            "passed": bool(codes_ok and worst_l <= 1e-3 and worst_o <= 1e-3),
            "seconds": round(time.perf_counter() - t_gate, 1)}
    if not gate["passed"]:
        print(json.dumps({"error": "parity gate failed before timing", "parity_gate": gate}), flush=True)
        sys.exit(3)
    # the oracle's decode step for this stream, one thread, repeated until about 10 s of work
    with threadpool_limits(limits=1):
        torch.set_num_threads(1)
        t0 = time.perf_counter()
        reps = 0
        while reps == 0 or (time.perf_counter() - t0 < 10.0 and reps < 16):
            new = oracle.quantize_stream(k16[L0:], v16[L0:], ks[h], cbk, cbv, wl.n_outliers)
            full = oracle.StreamCache(*(np.concatenate([x, y]) for x, y in zip(
                (st.k_codes, st.k_idx, st.k_val, st.v_codes, st.v_idx, st.v_val, st.v_scale),
                (new.k_codes, new.k_idx, new.k_val, new.v_codes, new.v_idx, new.v_val, new.v_scale))))
            oracle.pack_key_records(new.k_codes, wl.k_bits)
            for hq in range(hq0, hq1):
                oracle.decode_head(q[b, hq].float().cpu().numpy().astype(np.float64), full, ks[h], cbk, cbv,
                                   wl.rope_base, sm)
            reps += 1
        elapsed = time.perf_counter() - t0
    torch.set_num_threads(max(1, os.cpu_count() or 1))
    cpu = {"value": round(reps * stream_bytes(wl, L0 + 1) / elapsed / 1e9, 6), "unit": "GB/s", "cores": 1,
           "kind": "oracle",
           "sample": f"1 of {wl.batch * wl.n_kv_heads} (sequence, kv head) streams of one layer, stream {b},{h}, "
                     f"L={L0 + 1}: quantization of the new token + float64 decode attention of its "
                     f"{wl.group} query head(s), {reps} times, {elapsed:.1f} s on 1 thread, {cpu_model()}"}
    return gate, cpu


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


def key_scale_leg(wl, cfg, seed, max_tokens=1 << 20):
    """Per-channel key scale over a prompt of the workload (the keys a prefill appends),
    each vector's outliers left out, and the per-channel outlier threshold at a 1 % share
    over the same keys; returns each one's time and bytes read per second."""
    import torch

    import long_context_decode_kvq_amd as kvq
    import synth
    n = min(wl.seq_len, max_tokens)
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


def fp16_baseline(wl, cfg, L, kernel_steps, kt, n_layers):
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


def build_layers(wl, n_layers, seed, n_extra, dev="cuda"):
    """One compressed cache per layer, filled through kvq_quantize_append with the seeded
    prompt (wl.seq_len tokens per sequence), plus the n_extra decode-step tokens each
    layer appends later (kept on the device)."""
    import numpy as np  # noqa: F401
    import torch

    import long_context_decode_kvq_amd as kvq
    import synth
    L0 = wl.seq_len
    max_seq = ((L0 + n_extra * wl.n_new + 63) // 64) * 64
    cfg = kvq.CacheConfig(wl.batch, wl.n_q_heads, wl.n_kv_heads, max_seq, wl.k_bits, wl.v_bits, wl.n_outliers,
                          wl.head_dim, wl.rope_base)
    layers = []
    for li in range(n_layers):
        s = seed * 1000 + li
        ks = synth.key_scale(s, wl)
        cbk, cbv = synth.codebook(s, wl.k_bits, "k"), synth.codebook(s, wl.v_bits, "v")
        cache = kvq.KVCache(cfg, torch.from_numpy(ks), torch.from_numpy(cbk), torch.from_numpy(cbv), dev)
        n_all = L0 + n_extra * wl.n_new
        kraw = torch.empty(wl.batch, n_all, wl.n_kv_heads, wl.head_dim, dtype=torch.float16, device=dev)
        vraw = torch.empty_like(kraw)
        for b in range(wl.batch):
            for h in range(wl.n_kv_heads):
                kraw[b, :, h] = synth.keys(s, wl, b, h, n_all, dev)
                vraw[b, :, h] = synth.values(s, wl, b, h, n_all, dev)
        kvq.quantize_append(cache, kraw[:, :L0].contiguous(), vraw[:, :L0].contiguous())
        # copies (a slice of one token is a contiguous view that would keep the prompt alive)
        new_k = [kraw[:, L0 + i * wl.n_new: L0 + (i + 1) * wl.n_new].clone() for i in range(n_extra)]
        new_v = [vraw[:, L0 + i * wl.n_new: L0 + (i + 1) * wl.n_new].clone() for i in range(n_extra)]
        del kraw, vraw
        layers.append(dict(cache=cache, q=synth.queries(s, wl, dev), bufs=kvq.DecodeBuffers(cache),
                           new_k=new_k, new_v=new_v, seed=s, k_scale=ks, cbk=cbk, cbv=cbv, n_all=n_all))
        torch.cuda.synchronize()
    return layers, cfg, max_seq


def run_workload(wl, layers, max_seq, steps, warmup, kernel_steps, graph):
    """Time `steps` decode steps (after `warmup`), one HIP graph per step: every layer's
    device-positioned append of the step's token, then q.K^T and softmax.V over the whole
    capacity bound (kernels read the live length from the device).  Then per-launch times
    of each entry point over back-to-back launches on the layers, and of the appends."""
    import torch

    import long_context_decode_kvq_amd as kvq
    ev = lambda: torch.cuda.Event(enable_timing=True)
    n_graph_steps = warmup + steps

    def eager_step(i):
        for lay in layers:
            c = lay["cache"]
            kvq.quantize_append(c, lay["new_k"][i], lay["new_v"][i])
            L = max(c.lengths)
            kvq.qk_matvec(c, lay["q"], lay["bufs"].logits, max_len=L)
            kvq.pv_matvec(c, lay["bufs"].logits, lay["bufs"].out, lay["bufs"].workspace, max_len=L)

    graphs = []
    if graph:
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
        if graph:
            graphs[i].replay()
            for l in layers:
                l["cache"].lengths = [x + wl.n_new for x in l["cache"].lengths]
        else:
            eager_step(i)

    for i in range(warmup):
        run_step(i)
    torch.cuda.synchronize()
    start_len = max(layers[0]["cache"].lengths)
    t_start, t_end = ev(), ev()
    w0 = time.perf_counter()
    t_start.record()
    for i in range(steps):
        run_step(warmup + i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = t_start.elapsed_time(t_end) / steps
    assert [int(x) for x in layers[0]["cache"].seq_len.cpu()] == layers[0]["cache"].lengths
    del graphs

    # Per-launch kernel durations: HIP events (on the launch stream) around the layers'
    # back-to-back launches of one entry point, so launch overhead overlaps execution.
    L_now = max(layers[0]["cache"].lengths)
    kern_events = {"qk": [], "pv": []}
    for _ in range(kernel_steps):
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
    n_lay = len(layers)
    kt = {k: sum(a.elapsed_time(b) for a, b in v) / (len(v) * n_lay) for k, v in kern_events.items()}  # ms/launch

    # the decode step's append alone: every layer's device-positioned append of one token
    # per sequence (recorded once as a HIP graph when graphs are on, so the host's launch
    # rate does not set the time of these short kernels)
    def appends():
        for j in range(kernel_steps):
            for lay in layers:
                kvq.quantize_append(lay["cache"], lay["new_k"][n_graph_steps + j], lay["new_v"][n_graph_steps + j],
                                    device_positions=True)
    e0, e1 = ev(), ev()
    if graph:
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
    for lay in layers:
        lay["cache"].lengths = [x + wl.n_new * kernel_steps for x in lay["cache"].lengths]
    app_us = 1000 * e0.elapsed_time(e1) / (kernel_steps * n_lay)
    return dict(ms_step=ms_step, wall=wall, start_len=start_len, L_now=L_now, kt=kt, app_us=app_us)


def summarize(wl, n_layers, r, steps):
    """GB/s, KV-tokens/s and per-kernel rates of a run_workload result."""
    L_mean = r["start_len"] + wl.n_new * (steps + 1) / 2.0
    qk_b, pv_b, app_b = algorithmic_bytes(wl, L_mean)
    step_bytes = n_layers * (qk_b + pv_b + app_b)
    gbs = step_bytes / (r["ms_step"] * 1e-3) / 1e9
    # the same without the logits (written by q.K^T, read by softmax.V: 8 bytes per query
    # head and token)
    kv_only = (step_bytes - n_layers * 8 * wl.batch * wl.n_q_heads * L_mean) / (r["ms_step"] * 1e-3) / 1e9
    qk_bk, pv_bk, _ = algorithmic_bytes(wl, r["L_now"])
    kt = r["kt"]
    return {"ms_per_step": round(r["ms_step"], 4), "gbs": round(gbs, 2), "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "kv_only_gbs": round(kv_only, 1),
            "kv_tokens_per_s": round(n_layers * wl.batch * L_mean / (r["ms_step"] * 1e-3), 1),
            "kernel_ms": {k: round(v, 5) for k, v in kt.items()},
            "kernel_gbs": {"qk": round(qk_bk / (kt["qk"] * 1e-3) / 1e9, 1), "pv": round(pv_bk / (kt["pv"] * 1e-3) / 1e9, 1),
                           "qk+pv": round((qk_bk + pv_bk) / ((kt["qk"] + kt["pv"]) * 1e-3) / 1e9, 1)},
            "append_us_per_layer": round(r["app_us"], 2)}


def workload_config(wl, n_layers):
    return {"workload": wl.name, "layers": n_layers, "batch": wl.batch, "q_heads": wl.n_q_heads,
            "kv_heads": wl.n_kv_heads, "head_dim": wl.head_dim, "seq_len": wl.seq_len, "k_bits": wl.k_bits,
            "v_bits": wl.v_bits, "outliers_per_vector": wl.n_outliers, "new_tokens_per_step": wl.n_new}


def main():
    args = parse()
    if args.summarize_counters:
        summarize_counters(*args.summarize_counters, args.workload)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU; --gpus must be 1 "
                          "(sharding across GPUs is described in the design notes, not built)"}))
        sys.exit(2)
    import torch

    import long_context_decode_kvq_amd as kvq
    import synth

    wl = synth.WORKLOADS[args.workload]
    if args.outlier_frac is not None:
        wl = wl.with_(outlier_frac=args.outlier_frac)
    kvq.load_library()
    n_extra = args.warmup + args.steps + args.kernel_steps
    t_build = time.perf_counter()
    layers, cfg, max_seq = build_layers(wl, args.layers, args.seed, n_extra)
    build_s = time.perf_counter() - t_build
    free_b, total_b = torch.cuda.mem_get_info()
    footprint = {"layers": args.layers, "cache_bytes": args.layers * kvq.cache_sizes(cfg).total,
                 "device_total_bytes": total_b, "device_free_bytes_after_build": free_b,
                 "build_s": round(build_s, 1)}

    gate = cpu = None
    if not args.no_cpu_baseline:
        b_s, h_s = 0, min(9, wl.n_kv_heads - 1)
        gate, cpu = cpu_baseline_and_gate(wl, layers[0], layers[0]["seed"], b_s, h_s, wl.seq_len)

    r = run_workload(wl, layers, max_seq, args.steps, args.warmup, args.kernel_steps, args.graph)
    s = summarize(wl, args.layers, r, args.steps)
    kt = r["kt"]
    qk_bk, pv_bk, _ = algorithmic_bytes(wl, r["L_now"])
    dom = max(kt, key=kt.get)
    dom_bytes = {"qk": qk_bk, "pv": pv_bk}[dom]
    achieved = dom_bytes / (kt[dom] * 1e-3) / 1e9
    qk_name = ("qk_lut_kernel" if wl.group == 1 else "qk_kernel" if wl.k_bits == 4 else "qk_mfma_kernel")
    dom_name = {"qk": qk_name, "pv": "pv_partial_kernel+pv_combine_kernel"}[dom]
    # counted traffic is stored per workload as defined (another outlier count moves other bytes)
    traffic = (traffic_from_profile(args.workload, dom_name, source_hash(KERNEL_SOURCES[dom_name]))
               if args.outlier_frac is None else None)
    ceiling = stream_ceiling()

    line = {
        "metric": METRIC,
        "value": s["gbs"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": s["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DTYPE,
        "data": "synthetic (seeded N(0,1) keys with 4 x10 channels per kv head, N(0,1) values; fp16 queries)",
        "config": workload_config(wl, args.layers),
        "pct_of_hbm_peak": s["pct_of_hbm_peak"],
        "kv_only_gbs": s["kv_only_gbs"],
        "kv_tokens_per_s": s["kv_tokens_per_s"],
        "kernel_ms": s["kernel_ms"],
        "kernel_gbs": s["kernel_gbs"],
        "append_us_per_layer": s["append_us_per_layer"],
        "footprint": footprint,
        "hbm_read_ceiling": ceiling,
        "graph": bool(args.graph),
        "wall_s_timed": round(r["wall"], 3),
        "roofline": {"kernel": dom_name, "launches_timed": args.kernel_steps * args.layers,
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic},
    }
    if gate is not None:
        line["parity_gate"] = gate
    if cpu is not None:
        line["cpu_baseline"] = cpu
    if args.codebook_fit:
        line["key_scale_calibration"], line["key_threshold_calibration"] = key_scale_leg(wl, cfg, args.seed * 1000 + 7)
        line["codebook_fit"] = codebook_fit_leg(wl, args.seed * 1000)
    if args.fp16_baseline:
        n_fp16 = 2 if wl.seq_len * wl.batch * wl.n_kv_heads * 512 > (8 << 30) else 4
        line["fp16_baseline"] = fp16_baseline(wl, cfg, r["L_now"], args.kernel_steps, kt, n_fp16)
    del layers
    torch.cuda.empty_cache()
    if args.extra:
        extra = {}
        for name, (fracs, n_lay) in EXTRA.items():
            if name == args.workload:
                continue
            for f in fracs:
                w = synth.WORKLOADS[name] if f is None else synth.WORKLOADS[name].with_(outlier_frac=f)
                e_steps, e_warm, e_ks = 10, 2, 5
                ls, _, ms = build_layers(w, n_lay, args.seed + 1, e_steps + e_warm + e_ks)
                rr = run_workload(w, ls, ms, e_steps, e_warm, e_ks, args.graph)
                entry = {"config": workload_config(w, n_lay), **summarize(w, n_lay, rr, e_steps)}
                extra[name if f is None else f"{name}@k={w.n_outliers}"] = entry
                del ls
                torch.cuda.empty_cache()
        line["workloads"] = extra
    if args.traffic_probe:
        src_p = torch.ones(PROBE_BYTES // 4, dtype=torch.int32, device="cuda")
        dst_p = torch.empty_like(src_p)
        torch.bitwise_not(src_p, out=dst_p)
        torch.cuda.synchronize()
        del src_p, dst_p
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
