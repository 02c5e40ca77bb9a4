"""Per-layer codebook fitting: unweighted 1-D k-means (Lloyd iterations) on normalised
calibration activations.

TEST INFRASTRUCTURE ONLY (as the rest of this package): imported by tests, the smoke
check and the benchmark's CPU leg, never by the product path.

Source: [P1] "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
Quantization" (study.space summary), abstract paragraph, technique (iii): a non-uniform
datatype per layer, derived offline from calibration data; [P2] the KVQuant paper note,
"Four components" paragraph, item (3): one codebook per layer.  The pages weight the fit
by each activation's sensitivity, which needs a trained model's gradients; this fit is
the unweighted version (plain k-means on the activations), a stated reading.

Readings (the pages give no algorithm for the fit):
  * inputs are activations already divided by their scale (keys by the per-channel
    scale, values by the per-vector scale), clamped to [-1, 1] in float32;
  * initial centroids: the midpoints -1 + (2j + 1)/K of K equal bins, K = 2^bits;
  * one iteration: each input goes to its nearest centroid by the quantizer's own rule
    (smallest j minimising the float32 |u - c_j|), then each centroid with at least one
    input moves to their mean; an empty cluster keeps its centroid;
  * the mean is formed exactly: every input is rounded to the grid 2^-30 (error below
    5e-10), the per-cluster sums are integers, and c_j = float32(sum / (count 2^30))
    with one float64 division, so the result does not depend on summation order;
  * the result is rounded to fp16 and made strictly ascending: each value is raised to
    at least the next fp16 above its predecessor, then, if the last exceeds 1, lowered
    from the top to at most the next fp16 below its successor.
"""
from __future__ import annotations

import numpy as np

from .kvquant import nearest_code

FRAC_BITS = 30


def fit_init(bits: int) -> np.ndarray:
    """Midpoints of 2^bits equal bins of [-1, 1], float32."""
    k = 1 << bits
    return np.array([-1.0 + (2.0 * j + 1.0) / k for j in range(k)], dtype=np.float32)


def clamp_inputs(u) -> np.ndarray:
    return np.clip(np.asarray(u, dtype=np.float32), np.float32(-1.0), np.float32(1.0))


def fixed_point(u32: np.ndarray) -> np.ndarray:
    """u rounded to the grid 2^-30, as integers (round half to even)."""
    return np.rint(u32.astype(np.float64) * float(1 << FRAC_BITS)).astype(np.int64)


def fit_step(u32: np.ndarray, c32: np.ndarray):
    """One Lloyd iteration on clamped float32 inputs.  Returns (new centroids float32,
    per-cluster integer sums, counts, codes)."""
    codes = nearest_code(u32, c32)
    q = fixed_point(u32)
    k = len(c32)
    sums = np.zeros(k, dtype=np.int64)
    counts = np.zeros(k, dtype=np.int64)
    for j in range(k):
        m = codes == j
        counts[j] = int(m.sum())
        sums[j] = int(q[m].sum())
    new = c32.copy()
    for j in range(k):
        if counts[j] > 0:
            new[j] = np.float32(np.float64(sums[j]) / (np.float64(counts[j]) * float(1 << FRAC_BITS)))
    return new, sums, counts, codes


def finalize(c32: np.ndarray) -> np.ndarray:
    """fp16 rounding, then strictly ascending within [-1, 1] (see the module readings)."""
    h = np.asarray(c32, dtype=np.float32).astype(np.float16)
    inf16, one = np.float16(np.inf), np.float16(1.0)
    for j in range(1, len(h)):
        floor_j = np.nextafter(h[j - 1], inf16)
        if h[j] < floor_j:
            h[j] = floor_j
    if h[-1] > one:
        h[-1] = one
        for j in range(len(h) - 2, -1, -1):
            ceil_j = np.nextafter(h[j + 1], -inf16)
            if h[j] > ceil_j:
                h[j] = ceil_j
    return h


def fit_codebook(u, bits: int, iters: int) -> np.ndarray:
    """Codebook of 2^bits fp16 values fitted to the inputs by ``iters`` Lloyd iterations."""
    u32 = clamp_inputs(u).reshape(-1)
    c = fit_init(bits)
    for _ in range(iters):
        c = fit_step(u32, c)[0]
    return finalize(c)


def quantization_mse(u, c) -> float:
    """Mean squared error of the inputs against their nearest entries (float64)."""
    u32 = clamp_inputs(u).reshape(-1)
    cb = np.asarray(c, dtype=np.float32)
    codes = nearest_code(u32, cb)
    return float(np.mean((u32.astype(np.float64) - cb[codes].astype(np.float64)) ** 2))
