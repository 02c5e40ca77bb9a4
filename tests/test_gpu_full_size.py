"""Parity at the full layer sizes, in the launch configuration the benchmark times.

The whole layer is built by a bulk kvq_quantize_append of the prompt and one
device-positioned decode-step append (one token per sequence), then q.K^T and softmax.V
run with the grid bounded by the full capacity, as `bench.py` does.  The oracle then
checks sampled (sequence, kv head) streams completely: packed key records, value tiles,
outlier indices/values and value scales bit for bit over every token, and for every
query head of the stream's group every logit (|dl| <= 1e-3 sm sum_c |q_c y_c|) and the
output (|do| <= 1e-3 sum_t p_t |v~_t|).  Sizes: the LLaMA-7B-shaped layer at 32K tokens
(3-bit), 128K (4-bit, Laplace outlier channels) and 1M (2-bit), and the Llama-3-8B-shaped
GQA layer (batch 16, 32 query heads on 8 kv heads, 64K tokens each), the 32K layer
again under the per-channel key outlier rule, and the 1M and 128K shapes cut to 27K
tokens, where the one-head q.K^T blocks end part-way through their rounds between
barriers; the oracle needs about a minute of host time for the 1M stream.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kvq_testlib import assert_logits_close, assert_out_close, gpu_buffers

pytestmark = pytest.mark.gpu

D = 128

# workload -> (sequence, kv head) streams checked against the oracle
SAMPLED = {
    "llama7b_32k": [(0, 0), (0, 17), (0, 31)],
    "llama7b_128k_4bit": [(0, 5)],
    "llama7b_1m_2bit": [(0, 9)],
    "llama3_8b_gqa_b16_64k": [(0, 0), (9, 5), (15, 7)],
    # the per-channel key outlier rule, each channel's scale the 0.99 quantile of |key|
    "llama7b_32k@per_channel": [(0, 3), (0, 30)],
    # 53 super-tiles of 512 tokens per head over 8 blocks per head: blocks of 7 steps and
    # one of 4, so the one-head q.K^T leaves its 4-step (2-bit) and 2-step (4-bit) rounds
    # between block barriers part-way, with 2 and 4 record sets
    "llama7b_1m_2bit@27k": [(0, 4), (0, 27)],
    "llama7b_128k_4bit@27k": [(0, 2), (0, 19)],
}
# shape overrides of the variants above
VARIANTS = {"llama7b_1m_2bit@27k": dict(seq_len=27036), "llama7b_128k_4bit@27k": dict(seq_len=27036)}


@pytest.mark.parametrize("name", sorted(SAMPLED))
def test_full_layer_sampled_heads(name):
    import long_context_decode_kvq_amd as kvq
    per_channel = name.endswith("@per_channel")
    wl = synth.WORKLOADS[name.split("@")[0]].with_(**VARIANTS.get(name, {}))
    seed = 0
    L0 = wl.seq_len
    n = L0 + 1  # the prompt plus one decode-step token
    S = ((n + 63) // 64) * 64
    cfg = kvq.CacheConfig(wl.batch, wl.n_q_heads, wl.n_kv_heads, S, wl.k_bits, wl.v_bits, wl.n_outliers, D,
                          wl.rope_base, int(per_channel))
    ks = synth.key_scale(seed, wl, quantile=0.99 if per_channel else None)
    cbk, cbv = synth.codebook(seed, wl.k_bits, "k"), synth.codebook(seed, wl.v_bits, "v")
    cache = kvq.KVCache(cfg, torch.from_numpy(ks), torch.from_numpy(cbk), torch.from_numpy(cbv), "cuda")
    kraw = torch.empty(wl.batch, n, wl.n_kv_heads, D, dtype=torch.float16, device="cuda")
    vraw = torch.empty_like(kraw)
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            kraw[b, :, h] = synth.keys(seed, wl, b, h, n, "cuda")
            vraw[b, :, h] = synth.values(seed, wl, b, h, n, "cuda")
    kvq.quantize_append(cache, kraw[:, :L0].contiguous(), vraw[:, :L0].contiguous())
    kvq.quantize_append(cache, kraw[:, L0:].contiguous(), vraw[:, L0:].contiguous(), device_positions=True)
    q = synth.queries(seed, wl, "cuda").contiguous()
    bufs = kvq.DecodeBuffers(cache)
    bufs.logits.fill_(float("nan"))
    kvq.qk_matvec(cache, q, bufs.logits, max_len=S)
    kvq.pv_matvec(cache, bufs.logits, bufs.out, bufs.workspace, max_len=S)
    fused = None
    if wl.group == 1 and wl.k_bits <= 3:  # the single-pass kernel on the same cache
        fused = torch.full_like(bufs.out, float("nan"))
        ws = torch.empty(kvq.workspace_bytes(cfg, S) // 4, dtype=torch.float32, device="cuda")
        kvq.fused_decode_attention(cache, q, fused, ws, max_len=S)
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == [n] * wl.batch
    sm = 1.0 / math.sqrt(D)
    for b, h in SAMPLED[name]:
        k16 = kraw[b, :, h].cpu().numpy()
        v16 = vraw[b, :, h].cpu().numpy()
        c = oracle.quantize_stream(k16, v16, ks[h], cbk, cbv, wl.n_outliers, per_channel_keys=per_channel)
        got = gpu_buffers(cache, b, h)
        what = f"{name} b={b} h={h}"
        assert np.array_equal(got["k_rec"][:n], oracle.pack_key_records(c.k_codes, wl.k_bits)), f"{what} k_rec"
        assert np.array_equal(got["v_tiles"], oracle.pack_value_tiles(c.v_codes, wl.v_bits, S)), f"{what} v_tiles"
        for key in ("k_idx", "k_val", "v_idx", "v_val", "v_scale"):
            assert np.array_equal(got[key][:n], getattr(c, key)), f"{what} {key}"
        del got
        for hq in range(h * wl.group, (h + 1) * wl.group):
            qh = q[b, hq].float().cpu().numpy().astype(np.float64)
            ref_l, ref_o = oracle.decode_head(qh, c, ks[h], cbk, cbv, wl.rope_base, sm)
            scale_l = oracle.logit_tolerance_scale(qh, c, ks[h], cbk, wl.rope_base, sm)
            wl_err = assert_logits_close(bufs.logits[b, hq, :n].cpu().numpy(), ref_l, scale_l, what=f"{what} hq={hq}")
            assert torch.isnan(bufs.logits[b, hq, n:]).all(), "logits written past seq_len"
            scale_o = oracle.output_tolerance_scale(ref_l, c, cbv)
            wo_err = assert_out_close(bufs.out[b, hq].cpu().numpy(), ref_o, scale_o, what=f"{what} hq={hq}")
            msg = f"{what} hq={hq}: worst logit rel err {wl_err:.2e}, worst output rel err {wo_err:.2e}"
            if fused is not None:
                wf_err = assert_out_close(fused[b, hq].cpu().numpy(), ref_o, scale_o, what=f"{what} hq={hq} single-pass")
                msg += f", single-pass {wf_err:.2e}"
            print(msg)


# single (sequence, kv head) streams: the value pass splits each one into more than 64
# parts (the combine's register-resident merge holds 64, the rest take its second loop)
LONG_STREAMS = {"llama7b_128k_4bit": 131072, "llama7b_1m_2bit": 1048576}


@pytest.mark.parametrize("name", sorted(LONG_STREAMS))
def test_long_single_stream_with_positional_values(name):
    """One long stream whose values are non-negative and code the position (channel 0
    rises as t / L, channel 1 falls as 1 - t / L, the rest |N(0,1)|), quantized with a
    non-negative value codebook: the outputs have no cancellation, so the tolerance
    1e-3 sum_t p_t |v~_t| is a plain relative bound,
    and a split part dropped, counted twice or merged with the wrong weight moves the
    position channels by more than it allows."""
    import long_context_decode_kvq_amd as kvq
    L = LONG_STREAMS[name]
    wl = synth.WORKLOADS[name].with_(batch=1, n_q_heads=1, n_kv_heads=1, seq_len=L)
    seed = 4
    S = ((L + 63) // 64) * 64
    cfg = kvq.CacheConfig(1, 1, 1, S, wl.k_bits, wl.v_bits, wl.n_outliers, D, wl.rope_base)
    ks = synth.key_scale(seed, wl)
    cbk = synth.codebook(seed, wl.k_bits, "k")
    # a value codebook of non-negative levels j / (2^b - 1): non-negative values then decode
    # to non-negative values (the zero code decodes to 0)
    cbv = np.float16(np.arange(1 << wl.v_bits) / ((1 << wl.v_bits) - 1)).astype(np.float32)
    cache = kvq.KVCache(cfg, torch.from_numpy(ks), torch.from_numpy(cbk), torch.from_numpy(cbv), "cuda")
    k16 = synth.keys(seed, wl, 0, 0, L, "cuda")
    v16 = synth.values(seed, wl, 0, 0, L, "cuda").abs()
    ramp = torch.arange(L, device="cuda", dtype=torch.float32) / L
    v16[:, 0] = ramp.half()
    v16[:, 1] = (1.0 - ramp).half()
    kvq.quantize_append(cache, k16[None, :, None].contiguous(), v16[None, :, None].contiguous())
    q = synth.queries(seed, wl, "cuda").contiguous()
    bufs = kvq.DecodeBuffers(cache)
    kvq.qk_matvec(cache, q, bufs.logits, max_len=S)
    kvq.pv_matvec(cache, bufs.logits, bufs.out, bufs.workspace, max_len=S)
    torch.cuda.synchronize()
    # with one stream the value pass splits it into min(block slots, ceil(tiles / 16)) parts,
    # at least 256 block slots on this device: more than 64 parts for both lengths
    assert -(-L // (64 * 16)) > 64
    c = oracle.quantize_stream(k16.cpu().numpy(), v16.cpu().numpy(), ks[0], cbk, cbv, wl.n_outliers)
    qh = q[0, 0].float().cpu().numpy().astype(np.float64)
    sm = 1.0 / math.sqrt(D)
    ref_l, ref_o = oracle.decode_head(qh, c, ks[0], cbk, cbv, wl.rope_base, sm)
    scale_l = oracle.logit_tolerance_scale(qh, c, ks[0], cbk, wl.rope_base, sm)
    assert_logits_close(bufs.logits[0, 0, :L].cpu().numpy(), ref_l, scale_l, what=name)
    got = bufs.out[0, 0].cpu().numpy().astype(np.float64)
    assert np.all(ref_o >= 0)
    scale_o = oracle.output_tolerance_scale(ref_l, c, cbv)
    assert np.allclose(scale_o, ref_o, rtol=1e-12, atol=0)  # no cancellation: the two bounds coincide
    err = np.abs(got - ref_o)
    assert np.all(err <= 1e-3 * ref_o), f"{name}: worst relative output error {(err / ref_o).max():.3g}"
    print(f"{name}: worst relative output error {(err / ref_o).max():.2e}, "
          f"position channels {got[0]:.6f} / {got[1]:.6f}")


def test_32_layer_1m_cache_is_resident():
    """The full 32-layer cache of the 1M-token 2-bit LLaMA-7B-shaped model (k = 2) fits
    on the device: every layer's buffers allocated at once, sized by kvq_cache_sizes."""
    import long_context_decode_kvq_amd as kvq
    wl = synth.WORKLOADS["llama7b_1m_2bit"]
    S = wl.capacity
    cfg = kvq.CacheConfig(wl.batch, wl.n_q_heads, wl.n_kv_heads, S, wl.k_bits, wl.v_bits, wl.n_outliers, D,
                          wl.rope_base)
    per_layer = kvq.cache_sizes(cfg).total
    torch.cuda.empty_cache()
    free0, total = torch.cuda.mem_get_info()
    ks = torch.ones(wl.n_kv_heads, D)
    cbk, cbv = torch.from_numpy(synth.codebook(0, 2, "k")), torch.from_numpy(synth.codebook(0, 2, "v"))
    layers = [kvq.KVCache(cfg, ks, cbk, cbv, "cuda") for _ in range(32)]
    torch.cuda.synchronize()
    held = sum(sum(t.numel() * t.element_size() for t in (c.k_codes, c.v_codes, c.k_out_idx, c.k_out_val,
                                                            c.v_out_idx, c.v_out_val, c.v_scale, c.k_scale,
                                                            c.k_codebook, c.v_codebook, c.seq_len))
               for c in layers)
    free1, _ = torch.cuda.mem_get_info()
    print(f"32 layers x {per_layer / 1e9:.3f} GB = {held / 1e9:.2f} GB held; device {total / 1e9:.1f} GB, "
          f"free {free0 / 1e9:.1f} GB before, {free1 / 1e9:.1f} GB after")
    assert held == 32 * per_layer
    assert 83e9 < held < 85e9
    assert free0 - free1 >= held
    del layers
    torch.cuda.empty_cache()
