"""Parity of the HIP path (through the C ABI) with the CPU oracle.

Packed codes, outlier indices/values and value scales must match bit for bit.  Logits
must satisfy |l_gpu - l_ref| <= 1e-3 * sm_scale * sum_c |q_c y_{t,c}| (y the rotated
dequantized key) and outputs |o_gpu - o_ref| <= 1e-3 * sum_t p_t |v~_{t,c}|, for every
element.  Sizes span several tiles and blocks, with ragged tails.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import synth
from kvq_testlib import Case, assert_logits_close, assert_out_close, gpu_buffers

pytestmark = pytest.mark.gpu

D = 128
W = synth.WORKLOADS


def _wl(base, **kw):
    return W[base].with_(**kw)


# name -> (workload, lens, append chunks)
CASES = {
    "single_head_ragged": (_wl("single_head_4k", seq_len=4100), [4100], None),
    "mha32_3bit": (_wl("llama7b_32k", seq_len=1500), [1500], None),
    "mha4_4bit_k2_laplace": (_wl("llama7b_128k_4bit", n_q_heads=4, n_kv_heads=4, seq_len=1100), [1100], None),
    "mha4_4bit_k1": (_wl("llama7b_128k_4bit", n_q_heads=4, n_kv_heads=4, seq_len=1100, outlier_frac=0.005),
                     [1100], None),
    "mha4_4bit_k0": (_wl("llama7b_128k_4bit", n_q_heads=4, n_kv_heads=4, seq_len=1100, outlier_frac=0.0),
                     [1100], None),
    "mha4_2bit": (_wl("llama7b_1m_2bit", n_q_heads=4, n_kv_heads=4, seq_len=2100), [2100], None),
    "mha2_2bit_k1": (_wl("llama7b_1m_2bit", n_q_heads=2, n_kv_heads=2, seq_len=1500, outlier_frac=0.005), [1500], None),
    "gqa_ragged_batch": (_wl("llama3_8b_gqa_b16_64k", batch=3, n_q_heads=8, n_kv_heads=2, seq_len=1300),
                         [1300, 517, 1], None),
    "gqa_g8": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=8, n_kv_heads=1, seq_len=700), [700, 64], None),
    "all_outliers": (_wl("single_head_4k", n_q_heads=2, n_kv_heads=2, seq_len=300, outlier_frac=1.0),
                     [300], None),
    "mixed_bits": (_wl("llama7b_32k", n_q_heads=4, n_kv_heads=4, seq_len=333, k_bits=2, v_bits=4), [333], None),
    "incremental_appends": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=4, n_kv_heads=2, seq_len=400),
                            [400, 257], [1, 62, 1, 64, 65, 3, 200, 1, 100]),
    "length_one": (_wl("single_head_4k", seq_len=1), [1], None),
    # k = ceil(f D) = 5 and 3: the first two outliers of a token travel with its record, the
    # rest go through the kernels' general loop
    "mha2_3bit_k5": (_wl("llama7b_32k", n_q_heads=2, n_kv_heads=2, seq_len=1300, outlier_frac=0.035), [1300], None),
    "mha2_2bit_k3": (_wl("llama7b_1m_2bit", n_q_heads=2, n_kv_heads=2, seq_len=1100, outlier_frac=0.02), [1100], None),
    "gqa4_k5_ragged": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=4, n_kv_heads=1, seq_len=900, outlier_frac=0.035),
                       [900, 333], None),
    # 4-bit keys and values with k = 5: the 4-bit key kernel's loop over the outliers past
    # the second, with one head and with grouped heads
    "mha2_4bit_k5": (_wl("llama7b_128k_4bit", n_q_heads=2, n_kv_heads=2, seq_len=1100, outlier_frac=0.035),
                     [1100], None),
    # one head with 4-bit keys (separable table rows) and fp32 queries, ragged batch
    "mha2_4bit_q32_batch": (_wl("llama7b_128k_4bit", batch=3, n_q_heads=2, n_kv_heads=2, seq_len=1300, q_dtype="fp32"),
                            [1300, 517, 1], None),
    "gqa2_4bit_k5": (_wl("llama7b_128k_4bit", batch=2, n_q_heads=4, n_kv_heads=2, seq_len=700, outlier_frac=0.035),
                     [700, 131], None),
    # grouped heads with 2-bit keys (the per-pair table path of the general kernel)
    "gqa2_2bit": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=4, n_kv_heads=2, seq_len=800, k_bits=2),
                  [800, 391], None),
    "gqa8_2bit": (_wl("llama3_8b_gqa_b16_64k", batch=1, n_q_heads=8, n_kv_heads=1, seq_len=1000, k_bits=2, v_bits=2),
                  [1000], None),
    # every (bits, group) instantiation the C ABI accepts: 4-bit keys with grouped heads,
    # 2-bit keys at g = 4, 2- and 4-bit values with grouped heads
    "gqa2_4bit": (_wl("llama7b_128k_4bit", batch=2, n_q_heads=4, n_kv_heads=2, seq_len=700), [700, 333], None),
    "gqa4_4bitk_2bitv": (_wl("llama7b_128k_4bit", batch=1, n_q_heads=8, n_kv_heads=2, seq_len=900, v_bits=2),
                         [900], None),
    "gqa8_4bit": (_wl("llama7b_128k_4bit", batch=1, n_q_heads=8, n_kv_heads=1, seq_len=1000), [1000], None),
    "gqa4_2bitk_4bitv": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=8, n_kv_heads=2, seq_len=800, k_bits=2,
                              v_bits=4), [800, 65], None),
    "gqa2_3bitk_2bitv": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=4, n_kv_heads=2, seq_len=600, v_bits=2),
                         [600, 129], None),
    # fp32 queries with grouped heads (the matrix-core kernel's two-part fp16 split)
    "gqa4_3bit_q32": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=8, n_kv_heads=2, seq_len=700, q_dtype="fp32"),
                      [700, 190], None),
    "gqa8_2bit_q32": (_wl("llama3_8b_gqa_b16_64k", batch=1, n_q_heads=8, n_kv_heads=1, seq_len=600, k_bits=2,
                          q_dtype="fp32"), [600], None),
    "gqa2_2bit_q32": (_wl("llama3_8b_gqa_b16_64k", batch=1, n_q_heads=4, n_kv_heads=2, seq_len=555, k_bits=2,
                          q_dtype="fp32"), [555], None),
    # grouped heads on the matrix cores without outliers, with one, and with a sequence of
    # one token beside a ragged one
    "gqa4_3bit_k0": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=8, n_kv_heads=2, seq_len=640, outlier_frac=0.0),
                     [640, 100], None),
    "gqa8_2bit_k1": (_wl("llama3_8b_gqa_b16_64k", batch=1, n_q_heads=8, n_kv_heads=1, seq_len=777, k_bits=2, v_bits=2,
                         outlier_frac=0.005), [777], None),
    "gqa2_len1": (_wl("llama3_8b_gqa_b16_64k", batch=3, n_q_heads=4, n_kv_heads=2, seq_len=65), [1, 65, 2], None),
    # one query head per kv head with the remaining (key, value) bit widths of the
    # single-pass kernel
    "mha2_k2v3": (_wl("llama7b_32k", n_q_heads=2, n_kv_heads=2, seq_len=900, k_bits=2, v_bits=3), [900], None),
    "mha2_k3v2": (_wl("llama7b_32k", n_q_heads=2, n_kv_heads=2, seq_len=900, k_bits=3, v_bits=2), [900], None),
    "mha2_k3v4": (_wl("llama7b_32k", n_q_heads=2, n_kv_heads=2, seq_len=900, k_bits=3, v_bits=4), [900], None),
    # the per-channel key outlier rule (key_outliers = 1): the frozen key scale is a
    # per-channel quantile of |key| over the calibration draw and doubles as the threshold
    "pc_mha4_3bit_k2": (_wl("llama7b_32k", n_q_heads=4, n_kv_heads=4, seq_len=1100), [1100], None),
    "pc_mha2_3bit_k5": (_wl("llama7b_32k", n_q_heads=2, n_kv_heads=2, seq_len=1300, outlier_frac=0.035),
                        [1300], None),
    "pc_mha4_4bit_laplace": (_wl("llama7b_128k_4bit", n_q_heads=4, n_kv_heads=4, seq_len=1100), [1100], None),
    "pc_mha2_2bit_capped": (_wl("llama7b_1m_2bit", n_q_heads=2, n_kv_heads=2, seq_len=900), [900], None),
    "pc_gqa_incremental": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=8, n_kv_heads=2, seq_len=700),
                           [700, 333], [1, 62, 1, 64, 65, 3, 200, 1, 400]),
    "pc_k0": (_wl("llama7b_32k", n_q_heads=2, n_kv_heads=2, seq_len=500, outlier_frac=0.0), [500], None),
}

# per-channel cases -> the quantile of |key| taken as each channel's scale; 0.99 leaves about
# 1.3 candidates per 128-entry vector (often more than k = 2), 0.5 about 64 (k always binds)
PER_CHANNEL = {"pc_mha4_3bit_k2": 0.99, "pc_mha2_3bit_k5": 0.965, "pc_mha4_4bit_laplace": 0.99,
               "pc_mha2_2bit_capped": 0.5, "pc_gqa_incremental": 0.99, "pc_k0": 0.99}


def make_case(name, wl, lens, device="cuda", seed=3):
    if name in PER_CHANNEL:
        ks = synth.key_scale(seed, wl, quantile=PER_CHANNEL[name])
        return Case(wl, seed=seed, lens=lens, device=device, k_scale=ks, key_outliers=1)
    return Case(wl, seed=seed, lens=lens, device=device)


@pytest.fixture(scope="module", params=sorted(CASES))
def built(request):
    wl, lens, chunks = CASES[request.param]
    case = make_case(request.param, wl, lens)
    cache = case.build_gpu(chunks)
    torch.cuda.synchronize()
    return request.param, case, cache


def test_append_bit_exact(built):
    name, case, cache = built
    assert cache.seq_len.cpu().tolist() == [int(x) for x in case.lens]
    for b in range(case.wl.batch):
        for h in range(case.wl.n_kv_heads):
            exp = case.expected_buffers(b, h)
            got = gpu_buffers(cache, b, h)
            n = int(case.lens[b])
            for key in ("k_rec", "k_idx", "k_val", "v_idx", "v_val", "v_scale"):
                assert np.array_equal(got[key][:n], exp[key][:n]), f"{name} b={b} h={h} {key}"
            assert np.array_equal(got["v_tiles"], exp["v_tiles"]), f"{name} b={b} h={h} v_tiles"


def _run_decode(case, cache):
    import long_context_decode_kvq_amd as kvq
    bufs = kvq.DecodeBuffers(cache)
    bufs.logits.fill_(float("nan"))
    kvq.decode_attention(cache, case.q, bufs)
    torch.cuda.synchronize()
    return bufs.logits.cpu().numpy(), bufs.out.cpu().numpy()


def test_qk_and_pv_parity(built):
    name, case, cache = built
    logits, out = _run_decode(case, cache)
    sm = 1.0 / math.sqrt(D)
    worst_l = worst_o = 0.0
    for b in range(case.wl.batch):
        n = int(case.lens[b])
        for hq in range(case.wl.n_q_heads):
            h = hq // case.wl.group
            c = case.oracle_stream(b, h)
            ref_l, ref_o = case.oracle_decode(b, hq)
            scale_l = oracle.logit_tolerance_scale(case.q_head(b, hq), c, case.ks[h], case.cbk,
                                                   case.wl.rope_base, sm)
            worst_l = max(worst_l, assert_logits_close(logits[b, hq, :n], ref_l, scale_l,
                                                       what=f"{name} b={b} hq={hq}"))
            assert np.all(np.isnan(logits[b, hq, n:])), "logits written past seq_len"
            scale_o = oracle.output_tolerance_scale(ref_l, c, case.cbv)
            worst_o = max(worst_o, assert_out_close(out[b, hq], ref_o, scale_o, what=f"{name} b={b} hq={hq}"))
    print(f"{name}: worst logit rel err {worst_l:.2e}, worst output rel err {worst_o:.2e}")


@pytest.mark.parametrize("q_log2", [-40, 40])
@pytest.mark.parametrize("k_bits", [2, 3])
def test_grouped_fp32_query_magnitudes(q_log2, k_bits):
    """fp32 queries far outside fp16's range (|q| near 2^42 or 2^-38) with grouped heads:
    the per-head power-of-two prescale before the two-part fp16 split keeps every logit
    within the tolerance (outputs are not compared: at 2^40 the softmax is a one-hot of
    logits whose tolerance exceeds their gaps)."""
    wl = _wl("llama3_8b_gqa_b16_64k", batch=1, n_q_heads=8, n_kv_heads=2, seq_len=300, k_bits=k_bits, q_dtype="fp32")
    case = make_case("q_magnitude", wl, [300])
    case.q = case.q * (2.0 ** q_log2)
    cache = case.build_gpu()
    logits, _ = _run_decode(case, cache)
    sm = 1.0 / math.sqrt(D)
    for hq in range(wl.n_q_heads):
        h = hq // wl.group
        c = case.oracle_stream(0, h)
        ref_l, _ = case.oracle_decode(0, hq)
        scale_l = oracle.logit_tolerance_scale(case.q_head(0, hq), c, case.ks[h], case.cbk, wl.rope_base, sm)
        assert_logits_close(logits[0, hq, :300], ref_l, scale_l, what=f"q 2^{q_log2} k_bits={k_bits} hq={hq}")


def test_fused_decode_matches_oracle(built):
    """The single-pass kernel (no logits written) against the oracle, within the output
    criterion, for every case it serves (one query head per kv head, 2/3-bit keys); other
    shapes are refused before launch."""
    import long_context_decode_kvq_amd as kvq
    name, case, cache = built
    out = torch.full((case.wl.batch, case.wl.n_q_heads, D), float("nan"), device="cuda")
    ws = torch.empty(kvq.workspace_bytes(cache.cfg, cache.cfg.max_seq) // 4, dtype=torch.float32, device="cuda")
    if case.wl.group != 1 or case.wl.k_bits > 3:
        with pytest.raises(kvq.KvqError):
            kvq.fused_decode_attention(cache, case.q, out, ws)
        return
    kvq.fused_decode_attention(cache, case.q, out, ws)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    worst = 0.0
    for b in range(case.wl.batch):
        for hq in range(case.wl.n_q_heads):
            h = hq // case.wl.group
            ref_l, ref_o = case.oracle_decode(b, hq)
            scale_o = oracle.output_tolerance_scale(ref_l, case.oracle_stream(b, h), case.cbv)
            worst = max(worst, assert_out_close(got[b, hq], ref_o, scale_o, what=f"fused {name} b={b} hq={hq}"))
    print(f"fused {name}: worst output rel err {worst:.2e}")


def test_decode_is_deterministic(built):
    """Two runs of the two-pass decode, and of the single-pass kernel where it applies, give
    bitwise identical logits and outputs: every sum the kernels form runs in a fixed order,
    and the outlier corrections, which meet in LDS through atomics, are summed as integers
    (fixed point), whose sum does not depend on the order the atomics land in."""
    import long_context_decode_kvq_amd as kvq
    name, case, cache = built
    l1, o1 = _run_decode(case, cache)
    l2, o2 = _run_decode(case, cache)
    assert np.array_equal(l1, l2, equal_nan=True)
    assert np.array_equal(o1, o2, equal_nan=True)
    if case.wl.group == 1 and case.wl.k_bits <= 3:
        ws = torch.empty(kvq.workspace_bytes(cache.cfg, cache.cfg.max_seq) // 4, dtype=torch.float32, device="cuda")
        runs = []
        for _ in range(2):
            out = torch.full((case.wl.batch, case.wl.n_q_heads, D), float("nan"), device="cuda")
            kvq.fused_decode_attention(cache, case.q, out, ws)
            torch.cuda.synchronize()
            runs.append(out.cpu().numpy())
        assert np.array_equal(runs[0], runs[1], equal_nan=True)


@pytest.mark.parametrize("key_outliers", [0, 1])
def test_device_position_appends_match_oracle(key_outliers):
    """Appends that read their positions from the device seq_len (no host lengths) give
    the same cache as host-positioned appends, advance seq_len, and drop tokens of a
    sequence without room while leaving its length unchanged (both key outlier rules)."""
    import long_context_decode_kvq_amd as kvq
    from kvq_testlib import stack_new
    wl = _wl("llama3_8b_gqa_b16_64k", batch=3, n_q_heads=4, n_kv_heads=2, seq_len=200)
    lens = np.array([190, 127, 62])
    ks = synth.key_scale(5, wl, quantile=0.99) if key_outliers else None
    case = Case(wl, seed=5, lens=lens, device="cuda", max_seq=192, k_scale=ks, key_outliers=key_outliers)
    cache = case.build_gpu(upto=np.minimum(lens, 60))  # host positions for the first 60 tokens
    pos = np.minimum(lens, 60)
    while (pos < lens).any():
        n = 3
        hi = np.minimum(pos + n, lens)
        k_new, v_new = stack_new(wl, case.streams, pos, hi, n, "cuda")
        kvq.quantize_append(cache, k_new, v_new, n_new=(hi - pos).tolist(), device_positions=True)
        pos = hi
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == lens.tolist()
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            exp = case.expected_buffers(b, h)
            got = gpu_buffers(cache, b, h)
            n = int(lens[b])
            for key in ("k_rec", "k_idx", "k_val", "v_idx", "v_val", "v_scale"):
                assert np.array_equal(got[key][:n], exp[key][:n]), f"b={b} h={h} {key}"
            assert np.array_equal(got["v_tiles"], exp["v_tiles"]), f"b={b} h={h} v_tiles"
    # sequence 0 holds 190 of 192: a 3-token append does not fit and is dropped
    before = cache.k_codes.clone()
    k_new = torch.ones(3, 3, 2, D, dtype=torch.float16, device="cuda")
    kvq.quantize_append(cache, k_new, k_new.clone(), n_new=[3, 0, 0], device_positions=True)
    torch.cuda.synchronize()
    assert cache.seq_len.cpu().tolist() == lens.tolist()
    assert torch.equal(before, cache.k_codes)


@pytest.mark.parametrize("key_outliers", [0, 1])
def test_graph_replay_of_decode_step_matches_eager(key_outliers):
    """A decode step (device-positioned append, q.K^T, softmax.V) recorded once in a HIP
    graph and replayed several times, with eager work in between, gives every step the
    same result as running the same step eagerly on an identical cache (both key outlier
    rules)."""
    import long_context_decode_kvq_amd as kvq
    from kvq_testlib import stack_new
    wl = _wl("llama7b_32k", n_q_heads=4, n_kv_heads=4, seq_len=600)
    lens = np.array([600])
    steps = 4
    ks = synth.key_scale(7, wl, quantile=0.99) if key_outliers else None
    case = Case(wl, seed=7, lens=lens + steps, device="cuda", k_scale=ks, key_outliers=key_outliers)
    pre = [int(lens[0])]
    c_eager = Case.__new__(Case)
    c_eager.__dict__.update(case.__dict__)
    c_eager.lens = lens
    cache_g = c_eager.build_gpu()
    cache_e = c_eager.build_gpu()
    news = [stack_new(wl, case.streams, lens + i, lens + i + 1, 1, "cuda") for i in range(steps)]
    k_in = torch.empty_like(news[0][0])
    v_in = torch.empty_like(news[0][1])
    bufs_g = kvq.DecodeBuffers(cache_g)
    bufs_e = kvq.DecodeBuffers(cache_e)
    ml = cache_g.cfg.max_seq
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        kvq.quantize_append(cache_g, k_in, v_in, device_positions=True)
        kvq.decode_attention(cache_g, case.q, bufs_g, max_len=ml)
    # capture only records; the cache is untouched until replay
    cache_g.lengths = list(pre)
    torch.cuda.synchronize()
    assert cache_g.seq_len.cpu().tolist() == pre
    for i in range(steps):
        k_in.copy_(news[i][0])
        v_in.copy_(news[i][1])
        g.replay()
        kvq.quantize_append(cache_e, news[i][0], news[i][1])
        kvq.decode_attention(cache_e, case.q, bufs_e)
        torch.cuda.synchronize()
        assert cache_g.seq_len.cpu().tolist() == [pre[0] + i + 1]
        L = pre[0] + i + 1
        assert torch.equal(bufs_g.logits[..., :L], bufs_e.logits[..., :L])
        o_g, o_e = bufs_g.out.cpu().numpy(), bufs_e.out.cpu().numpy()
        assert np.allclose(o_g, o_e, rtol=1e-5, atol=1e-6)
    assert torch.equal(cache_g.k_codes, cache_e.k_codes) and torch.equal(cache_g.v_codes, cache_e.v_codes)
    for kind in ("k", "v"):
        for a, b in zip(cache_g.outliers(kind), cache_e.outliers(kind)):
            assert torch.equal(a, b)


# name -> (workload, lens): several split parts per stream for every group size, plus an
# empty sequence.
MERGE_CASES = {
    "g1": (_wl("llama7b_32k", batch=2, n_q_heads=2, n_kv_heads=2, seq_len=3000), [3000, 0]),
    "g2": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=4, n_kv_heads=2, seq_len=2600), [2600, 0]),
    "g4": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=4, n_kv_heads=1, seq_len=9000), [9000, 0]),
    "g8": (_wl("llama3_8b_gqa_b16_64k", batch=2, n_q_heads=8, n_kv_heads=1, seq_len=5000), [5000, 0]),
}


@pytest.mark.parametrize("name", sorted(MERGE_CASES))
def test_pv_split_merge_across_calls_on_one_workspace(name):
    """softmax.V splits each stream over several blocks and merges their partials.  Two
    logit sets from the oracle (A and -A) alternate on one workspace, with two grid sizes
    (max_len = max_seq and = the longest length), so a partial left by the previous call
    would show: every output must match the oracle's attention over the same float32
    logits, and the empty sequence must give zeros."""
    import long_context_decode_kvq_amd as kvq
    wl, lens = MERGE_CASES[name]
    case = Case(wl, seed=7, lens=lens, device="cuda")
    cache = case.build_gpu()
    n = int(lens[0])
    S = cache.cfg.max_seq
    la = np.zeros((wl.batch, wl.n_q_heads, S), np.float32)
    for hq in range(wl.n_q_heads):
        la[0, hq, :n] = case.oracle_decode(0, hq)[0].astype(np.float32)
    expected = {}
    for sign in (1.0, -1.0):
        lg = (sign * la).astype(np.float32)
        for hq in range(wl.n_q_heads):
            c = case.oracle_stream(0, hq // wl.group)
            vd = oracle.dequant_values(c.v_codes, c.v_idx, c.v_val, c.v_scale, case.cbv)
            l64 = lg[0, hq, :n].astype(np.float64)
            expected[sign, hq] = (oracle.attend(l64, vd), oracle.output_tolerance_scale(l64, c, case.cbv))
    bufs = kvq.DecodeBuffers(cache)
    dev = {s: torch.from_numpy(s * la).cuda() for s in (1.0, -1.0)}
    for it in range(6):
        for sign in (1.0, -1.0):
            bufs.logits.copy_(dev[sign])
            bufs.out.fill_(float("nan"))
            kvq.pv_matvec(cache, bufs.logits, bufs.out, bufs.workspace, max_len=S if it % 2 == 0 else n)
            torch.cuda.synchronize()
            got = bufs.out.cpu().numpy()
            for hq in range(wl.n_q_heads):
                ref, scale = expected[sign, hq]
                assert_out_close(got[0, hq], ref, scale, what=f"{name} it={it} sign={sign} hq={hq}")
            assert np.all(got[1] == 0.0), f"{name}: empty sequence output not zero"


def _logit_patterns(n: int, rng) -> dict:
    """Logit sequences that move a running softmax max in different ways: slow and steep
    ramps (the max rises on every tile; with slope 0.2 weights relative to a max set one
    tile earlier reach e^12.8), a fall, single spikes just under and far over 16 above the
    rest, steps of +-40 between tiles, and tiles alternating between 0 and 15.9 (weights
    near e^15.9 on every other tile of each wave when the max is not raised)."""
    t = np.arange(n, dtype=np.float64)
    noise = rng.normal(size=n)
    return {
        "ramp_0.2": 0.2 * t,
        "ramp_1": 1.0 * t,
        "fall": -0.5 * t,
        "spike_15.9": noise + 15.9 * (t == n // 2),
        "spike_30": noise + 30.0 * (t == n // 3),
        "steps": 40.0 * ((t // 64) % 3 - 1) + noise,
        "sawtooth_15.9": 15.9 * ((t // 64) % 2),
    }


@pytest.mark.parametrize("name", ["g1", "g4", "g8"])
def test_pv_running_max_under_logit_ramps_and_spikes(name):
    """softmax.V keeps a running max per wave; with one query head it is raised only when a
    logit exceeds it by more than 16, so weights reach e^16, and grouped heads share one
    fixed-point outlier scale.  Logit patterns fed directly (a different one per head of a
    group, so within a tile the heads' weights differ by many orders of magnitude) must
    give the oracle's attention over the same float32 logits."""
    import long_context_decode_kvq_amd as kvq
    wl, lens = MERGE_CASES[name]
    case = Case(wl, seed=11, lens=lens, device="cuda")
    cache = case.build_gpu()
    n = int(lens[0])
    S = cache.cfg.max_seq
    pats = _logit_patterns(n, np.random.default_rng(5))
    names = sorted(pats)
    bufs = kvq.DecodeBuffers(cache)
    vds = {}
    for rot in range(len(names)):
        la = np.zeros((wl.batch, wl.n_q_heads, S), np.float32)
        for hq in range(wl.n_q_heads):
            la[0, hq, :n] = pats[names[(rot + hq) % len(names)]].astype(np.float32)
        bufs.logits.copy_(torch.from_numpy(la).cuda())
        bufs.out.fill_(float("nan"))
        kvq.pv_matvec(cache, bufs.logits, bufs.out, bufs.workspace)
        torch.cuda.synchronize()
        got = bufs.out.cpu().numpy()
        for hq in range(wl.n_q_heads):
            h = hq // wl.group
            c = case.oracle_stream(0, h)
            if h not in vds:
                vds[h] = oracle.dequant_values(c.v_codes, c.v_idx, c.v_val, c.v_scale, case.cbv)
            l64 = la[0, hq, :n].astype(np.float64)
            ref = oracle.attend(l64, vds[h])
            scale = oracle.output_tolerance_scale(l64, c, case.cbv)
            assert_out_close(got[0, hq], ref, scale,
                             what=f"{name} pattern={names[(rot + hq) % len(names)]} hq={hq}")
        assert np.all(got[1] == 0.0), f"{name}: empty sequence output not zero"
