"""Codebook fitting on the GPU (kvq_fit_codebook) against the oracle's k-means.

The fit's decisions are integer and float32 comparisons and its means exact fixed-point
sums, so the fp16 codebooks must agree bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import synth

pytestmark = pytest.mark.gpu


def _inputs(kind, n, seed):
    rng = np.random.default_rng(seed)
    if kind == "gauss":
        return (rng.standard_normal(n) * 0.35).astype(np.float32)
    if kind == "laplace":
        return (rng.laplace(0.0, 0.2, n)).astype(np.float32)
    if kind == "wide":  # a fifth of the inputs outside [-1, 1]: clamped
        return (rng.standard_normal(n) * 0.8).astype(np.float32)
    if kind == "constant":  # every input in one bin: the other entries stay where they start
        return np.full(n, 0.3, dtype=np.float32)
    if kind == "uniform":
        return ((np.arange(n) + 0.5) / n * 2.0 - 1.0).astype(np.float32)
    raise ValueError(kind)


CASES = [("gauss", 2, 10, 100003), ("gauss", 3, 12, 262147), ("laplace", 4, 15, 65537), ("wide", 3, 8, 50000),
         ("constant", 2, 3, 1000), ("uniform", 4, 6, 40001), ("gauss", 3, 0, 1000), ("gauss", 4, 5, 0),
         ("gauss", 3, 1, 1)]


@pytest.mark.parametrize("kind,bits,iters,n", CASES)
def test_fit_matches_oracle_bit_for_bit(kind, bits, iters, n):
    import long_context_decode_kvq_amd as kvq
    u = _inputs(kind, n, seed=bits * 1000 + iters)
    got = kvq.fit_codebook(torch.from_numpy(u).cuda(), bits, iters).cpu().numpy()
    ref = oracle.fit_codebook(u, bits, iters)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), (kind, bits, iters, n, got, ref)
    assert np.all(np.diff(got.astype(np.float64)) > 0) and got.min() >= -1 and got.max() <= 1


def test_fit_on_normalised_keys_and_values_of_the_32k_layer():
    """Calibration activations of the 32K LLaMA-7B workload's generator: keys divided by
    their per-channel scale and values by their per-vector scale (4 heads x 4096 tokens)."""
    import long_context_decode_kvq_amd as kvq
    wl = synth.WORKLOADS["llama7b_32k"]
    ks = synth.key_scale(0, wl)
    keys, vals = [], []
    for h in range(4):
        k16 = synth.keys(0, wl, 0, h, 4096).numpy().astype(np.float32)
        v16 = synth.values(0, wl, 0, h, 4096).numpy().astype(np.float32)
        keys.append((k16 / ks[h][None, :]).reshape(-1))
        vals.append((v16 / np.abs(v16).max(axis=1, keepdims=True)).reshape(-1))
    for u, bits in ((np.concatenate(keys).astype(np.float32), 3), (np.concatenate(vals).astype(np.float32), 3)):
        got = kvq.fit_codebook(torch.from_numpy(u).cuda(), bits, 12).cpu().numpy()
        ref = oracle.fit_codebook(u, bits, 12)
        assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
        # the fitted codebook quantizes its own calibration data better than the uniform grid
        assert oracle.quantization_mse(u, got.astype(np.float32)) < oracle.quantization_mse(u, synth.uniform_codebook(bits))


def test_fit_at_bench_scale():
    """16.8M inputs (the size of a 32-head, 4096-token key calibration set): bit-exact."""
    import long_context_decode_kvq_amd as kvq
    u = (np.random.default_rng(11).standard_normal(1 << 24) * 0.3).astype(np.float32)
    got = kvq.fit_codebook(torch.from_numpy(u).cuda(), 3, 4).cpu().numpy()
    ref = oracle.fit_codebook(u, 3, 4)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16))
