"""Parity of the uncompressed fp16 baseline kernels (through the C ABI) with the oracle's
exact attention over the same fp16 tensors.

The cache holds keys after the rotary embedding: the oracle rotates the fp16 keys in
float64 (pair (i, i + 64) by t * base^(-2i/D)) and the rounded fp16 result is the
cache's content, so both sides read identical fp16 keys and values.  Tolerances as for the
compressed path: |dl| <= 1e-3 * sm * sum_c |q_c k_c| per logit, |do| <= 1e-3 * sum_t
p_t |v_t,c| per output.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kvq_testlib import assert_logits_close, assert_out_close

pytestmark = pytest.mark.gpu

D = 128
W = synth.WORKLOADS


def _wl(base, **kw):
    return W[base].with_(**kw)


def _build(wl, lens, seed, max_seq=None):
    """fp16 cache filled from the seeded workload; host copies of the rotated keys."""
    import long_context_decode_kvq_amd as kvq
    S = max_seq or ((max(lens) + 63) // 64) * 64
    cfg = kvq.CacheConfig(wl.batch, wl.n_q_heads, wl.n_kv_heads, S, wl.k_bits, wl.v_bits, wl.n_outliers)
    cache = kvq.Fp16Cache(cfg)
    k_rot, v_host = {}, {}
    for b in range(wl.batch):
        n = int(lens[b])
        for h in range(wl.n_kv_heads):
            k16 = synth.keys(seed, wl, b, h, max(n, 1)).numpy()[:n]
            v16 = synth.values(seed, wl, b, h, max(n, 1)).numpy()[:n]
            kr16 = oracle.rope(k16.astype(np.float64), np.arange(n), wl.rope_base).astype(np.float16)
            k_rot[b, h], v_host[b, h] = kr16, v16
            cache.k[b, h, :n] = torch.from_numpy(kr16).cuda()
            cache.v[b, h, :n] = torch.from_numpy(v16).cuda()
    cache.set_lengths(lens)
    return cache, k_rot, v_host


CASES = {
    "mha1_ragged_fp32q": (_wl("single_head_4k", seq_len=4100), [4100], torch.float32),
    "mha4_fp16q": (_wl("llama7b_32k", n_q_heads=4, n_kv_heads=4, seq_len=2100), [2100], torch.float16),
    "gqa4_ragged_batch": (_wl("llama3_8b_gqa_b16_64k", batch=3, n_q_heads=8, n_kv_heads=2, seq_len=1300),
                          [1300, 517, 1], torch.float16),
    "gqa8": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=8, n_kv_heads=1, seq_len=700), [700, 64], torch.float16),
    "length_one": (_wl("single_head_4k", seq_len=1), [1], torch.float32),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_fp16_baseline_matches_exact_attention(name):
    import long_context_decode_kvq_amd as kvq
    wl, lens, qdt = CASES[name]
    cache, k_rot, v_host = _build(wl, lens, seed=11)
    q = synth.queries(11, wl).to(qdt)
    bufs = kvq.DecodeBuffers(cache)
    bufs.logits.fill_(float("nan"))
    kvq.fp16_decode_attention(cache, q.cuda().contiguous(), bufs)
    torch.cuda.synchronize()
    logits, out = bufs.logits.cpu().numpy(), bufs.out.cpu().numpy()
    sm = 1.0 / math.sqrt(D)
    qn = q.double().numpy()
    for b in range(wl.batch):
        n = int(lens[b])
        for hq in range(wl.n_q_heads):
            h = hq // wl.group
            kr = k_rot[b, h].astype(np.float64)
            ref_l = oracle.qk_logits(qn[b, hq], kr, sm)
            assert_logits_close(logits[b, hq, :n], ref_l, sm * (np.abs(kr) @ np.abs(qn[b, hq])),
                                what=f"{name} b={b} hq={hq}")
            assert np.all(np.isnan(logits[b, hq, n:])), "logits written past seq_len"
            ref_o = oracle.attend(ref_l, v_host[b, h])
            scale_o = oracle.softmax(ref_l) @ np.abs(v_host[b, h].astype(np.float64))
            assert_out_close(out[b, hq], ref_o, scale_o, what=f"{name} b={b} hq={hq}")


def test_fp16_baseline_full_layer_sampled_heads():
    """The 32K-token LLaMA-7B layer shape in the launch configuration the benchmark times,
    checked on three heads against the oracle (all 32 heads run)."""
    import long_context_decode_kvq_amd as kvq
    wl = W["llama7b_32k"]
    L = wl.seq_len
    cfg = kvq.CacheConfig(1, 32, 32, L, wl.k_bits, wl.v_bits, wl.n_outliers)
    cache = kvq.Fp16Cache(cfg)
    gen = torch.Generator(device="cuda").manual_seed(5)
    cache.k.copy_(torch.randn(cache.k.shape, generator=gen, device="cuda").half())
    cache.v.copy_(torch.randn(cache.v.shape, generator=gen, device="cuda").half())
    cache.set_lengths([L])
    q = synth.queries(0, wl).cuda().contiguous()
    bufs = kvq.DecodeBuffers(cache)
    kvq.fp16_decode_attention(cache, q, bufs)
    torch.cuda.synchronize()
    sm = 1.0 / math.sqrt(D)
    for h in (0, 13, 31):
        kr = cache.k[0, h].double().cpu().numpy()
        vv = cache.v[0, h].double().cpu().numpy()
        qn = q[0, h].double().cpu().numpy()
        ref_l = oracle.qk_logits(qn, kr, sm)
        assert_logits_close(bufs.logits[0, h].cpu().numpy(), ref_l, sm * (np.abs(kr) @ np.abs(qn)), what=f"h={h}")
        assert_out_close(bufs.out[0, h].cpu().numpy(), oracle.attend(ref_l, vv), oracle.softmax(ref_l) @ np.abs(vv),
                         what=f"h={h}")
