"""Per-channel key scale on the GPU (kvq_key_scale) against the oracle: bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl_name,batch,heads,n,frac", [
    ("llama7b_32k", 1, 4, 4096, 0.01), ("llama7b_128k_4bit", 2, 3, 1000, 0.005),
    ("llama3_8b_gqa_b16_64k", 3, 2, 517, 0.01), ("llama7b_32k", 1, 2, 1, 0.01), ("llama7b_32k", 2, 1, 0, 0.01),
    ("single_head_4k", 1, 1, 300, 1.0),
    ("llama7b_32k", 1, 32, 32768, 0.01)])  # the 32K-token, 32-head prompt the benchmark times
def test_key_scale_matches_oracle(wl_name, batch, heads, n, frac):
    import long_context_decode_kvq_amd as kvq
    wl = synth.WORKLOADS[wl_name].with_(batch=batch, n_kv_heads=heads, n_q_heads=heads, outlier_frac=frac)
    k = wl.n_outliers
    cfg = kvq.CacheConfig(batch, heads, heads, 64, wl.k_bits, wl.v_bits, k)
    keys = torch.zeros(batch, n, heads, 128, dtype=torch.float16)
    for b in range(batch):
        for h in range(heads):
            if n:
                keys[b, :, h] = synth.keys(9, wl, b, h, n)
    for excl in (False, True):
        got = kvq.key_scale(cfg, keys.cuda().contiguous(), exclude_outliers=excl).cpu().numpy()
        for h in range(heads):
            vecs = keys[:, :, h].reshape(-1, 128).numpy()
            ref = oracle.key_scale_from_keys(vecs, k if excl else 0)
            assert np.array_equal(got[h], ref), (wl_name, excl, h)
