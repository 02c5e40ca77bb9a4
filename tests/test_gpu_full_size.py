"""Parity at the full layer sizes, in the launch configuration the benchmark times.

The whole layer is built by a bulk kvq_quantize_append of the prompt and one
device-positioned decode-step append (one token per sequence), then q.K^T and softmax.V
run with the grid bounded by the full capacity, as `bench.py` does.  The oracle then
checks sampled (sequence, kv head) streams completely: packed key records, value tiles,
outlier indices/values and value scales bit for bit over every token, and for every
query head of the stream's group every logit (|dl| <= 1e-3 sm sum_c |q_c y_c|) and the
output (|do| <= 1e-3 sum_t p_t |v~_t|).  Sizes: the LLaMA-7B-shaped layer at 32K tokens
(3-bit), 128K (4-bit, Laplace outlier channels) and 1M (2-bit), and the Llama-3-8B-shaped
GQA layer (batch 16, 32 query heads on 8 kv heads, 64K tokens each), and the 32K layer
again under the per-channel key outlier rule; the oracle needs about a minute of host
time for the 1M stream.
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
}


@pytest.mark.parametrize("name", sorted(SAMPLED))
def test_full_layer_sampled_heads(name):
    import long_context_decode_kvq_amd as kvq
    per_channel = name.endswith("@per_channel")
    wl = synth.WORKLOADS[name.split("@")[0]]
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
