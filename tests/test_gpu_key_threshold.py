"""kvq_key_threshold against the oracle, bit for bit: the per-channel (m+1)-th largest |x_c|
over the calibration keys, m = floor(f N).  Cases: several heads and batches, shares from
0 (the channel maximum) to 1 (threshold 0), a single vector, no vectors, heavy ties with
infinities and a NaN, many histogram blocks with a ragged last one, and the benchmark's
32K-token, 32-head prompt.  Then the GPU thresholds drive a per-channel-rule cache whose
buffers match the oracle's."""
import numpy as np
import pytest
import torch

import oracle
import synth
from kvq_testlib import gpu_buffers

pytestmark = pytest.mark.gpu

D = 128


def _keys(wl, batch, n_kv, n, seed):
    k = torch.empty(batch, n, n_kv, D, dtype=torch.float16, device="cuda")
    for b in range(batch):
        for h in range(n_kv):
            k[b, :, h] = synth.keys(seed, wl, b, h, n, "cuda")
    return k


def _cfg(batch, n_kv, key_outliers=0, k=2):
    import long_context_decode_kvq_amd as kvq
    return kvq.CacheConfig(batch, n_kv, n_kv, 64, 3, 3, k, D, 10000.0, key_outliers)


def _oracle(keys_cpu, f):
    B, n, H, _ = keys_cpu.shape
    return np.stack([oracle.key_threshold_from_keys(keys_cpu[:, :, h].reshape(B * n, D), f) for h in range(H)])


def _check(keys, f, what):
    import long_context_decode_kvq_amd as kvq
    B, n, H, _ = keys.shape
    got = torch.full((H, D), float("nan"), device="cuda")
    kvq.key_threshold(_cfg(B, H), keys, f, out=got)
    torch.cuda.synchronize()
    exp = _oracle(keys.cpu().numpy(), f)
    g = got.cpu().numpy()
    assert np.array_equal(g.view(np.uint32), exp.view(np.uint32)), (
        f"{what}: {int((g.view(np.uint32) != exp.view(np.uint32)).sum())} channels differ")
    return g


# (workload, batch, kv heads, tokens, shares)
CASES = [
    ("llama7b_32k", 1, 4, 4096, (0.0, 0.01, 0.2, 0.5, 0.999, 1.0)),
    ("llama3_8b_gqa_b16_64k", 3, 2, 517, (0.01, 0.05)),
    ("llama7b_128k_4bit", 2, 1, 40000, (0.01,)),   # 256 histogram blocks, the last one ragged
    ("single_head_4k", 1, 1, 1, (0.0, 0.01, 1.0)),
    ("llama7b_32k", 2, 3, 7, (0.1, 0.3)),
]


@pytest.mark.parametrize("name,batch,n_kv,n,shares", CASES)
def test_key_threshold_matches_oracle(name, batch, n_kv, n, shares):
    wl = synth.WORKLOADS[name]
    keys = _keys(wl, batch, n_kv, n, seed=4)
    for f in shares:
        _check(keys, f, f"{name} B={batch} H={n_kv} n={n} f={f}")


def test_key_threshold_of_no_vectors_is_zero():
    import long_context_decode_kvq_amd as kvq
    keys = torch.empty(2, 0, 3, D, dtype=torch.float16, device="cuda")
    got = torch.full((3, D), float("nan"), device="cuda")
    kvq.key_threshold(_cfg(2, 3), keys, 0.01, out=got)
    torch.cuda.synchronize()
    assert torch.equal(got.cpu(), torch.zeros(3, D))


def test_key_threshold_with_ties_infinities_and_nan():
    """Entries drawn from a few values (many ties across the low-bit pass), both signs,
    signed zeros, +-inf in some channels and one NaN (ranked above +inf)."""
    rng = np.random.default_rng(12)
    vals = np.float16([0.0, -0.0, 1e-7, 0.25, -0.25, 1.0, -1.0, 1.0009765625, 3.0, -3.0, 65504.0])
    x = rng.choice(vals, size=(2, 900, 2, D)).astype(np.float16)
    x[0, 5, 0, 7] = np.float16(np.inf)
    x[1, 9, 1, 7] = np.float16(-np.inf)
    x[0, 3, 1, 100] = np.float16(np.nan)
    keys = torch.from_numpy(x).cuda().contiguous()
    for f in (0.0, 0.001, 0.01, 0.4):
        _check(keys, f, f"ties f={f}")


def test_key_threshold_full_prompt():
    """The benchmark's prompt: 32K tokens of the LLaMA-7B-shaped layer's 32 kv heads."""
    wl = synth.WORKLOADS["llama7b_32k"]
    keys = _keys(wl, 1, wl.n_kv_heads, wl.seq_len, seed=0)
    g = _check(keys, 0.01, "32K prompt f=0.01")
    # about 1 % of every channel's entries lie above its threshold, never more
    above = (keys.float().abs() > torch.from_numpy(g).cuda()[None, None]).sum(dim=(0, 1)).cpu().numpy()
    assert above.max() <= int(0.01 * wl.seq_len)


def test_gpu_thresholds_drive_a_per_channel_cache():
    """Calibrate on a prompt, then append it under the per-channel rule with the GPU
    thresholds: the cache equals the oracle's built from the oracle's thresholds."""
    import long_context_decode_kvq_amd as kvq
    wl = synth.WORKLOADS["llama7b_32k"]
    B, H, n = 2, 2, 700
    keys = _keys(wl, B, H, n, seed=6)
    vals = torch.stack([torch.stack([synth.values(6, wl, b, h, n, "cuda") for h in range(H)], dim=1)
                        for b in range(B)]).contiguous()
    cfg = kvq.CacheConfig(B, H, H, 704, 3, 3, 2, D, 10000.0, 1)
    ks_gpu = kvq.key_threshold(cfg, keys, 0.01)
    cbk, cbv = synth.codebook(6, 3, "k"), synth.codebook(6, 3, "v")
    cache = kvq.KVCache(cfg, ks_gpu.cpu(), torch.from_numpy(cbk), torch.from_numpy(cbv), "cuda")
    kvq.quantize_append(cache, keys, vals)
    torch.cuda.synchronize()
    ks_ref = _oracle(keys.cpu().numpy(), 0.01)
    assert np.array_equal(ks_gpu.cpu().numpy().view(np.uint32), ks_ref.view(np.uint32))
    for b in range(B):
        for h in range(H):
            c = oracle.quantize_stream(keys[b, :, h].cpu().numpy(), vals[b, :, h].cpu().numpy(), ks_ref[h], cbk, cbv, 2,
                                       per_channel_keys=True)
            got = gpu_buffers(cache, b, h)
            assert np.array_equal(got["k_rec"][:n], oracle.pack_key_records(c.k_codes, 3)), (b, h)
            for key in ("k_idx", "k_val", "v_idx", "v_val", "v_scale"):
                assert np.array_equal(got[key][:n], getattr(c, key)), (b, h, key)
            assert (c.k_idx == oracle.NO_OUTLIER).any() and (c.k_idx != oracle.NO_OUTLIER).any()
