"""Seeded synthetic inputs for quantized-KV decode attention.

This module produces *inputs only*: raw fp16 key/value streams, queries, codebooks
and the frozen per-channel key scale.  It holds none of the quantizer's arithmetic
(no outlier selection, no normalisation, no code search, no packing), so that the
CPU oracle and the HIP path can both consume it without sharing method code.

Shapes and distributions follow the KVQuant pages' workloads: LLaMA-7B-shaped
layers (32 heads x head_dim 128), a Llama-3-8B-shaped GQA layer (32 query heads on
8 KV heads), keys ~N(0,1) per channel with a few channels scaled x10 (heavy-tailed
Laplace in the 4-bit sweep), values ~N(0,1), codebooks of 2^b sorted entries in
[-1, 1].  The pages measure perplexity on Wikitext-2 / C4 with trained weights; these
seeded tensors stand in for those activations (same shapes, no dataset).

Large streams are drawn with ``torch`` generators on the requested device, one
independent generator per (tensor, batch row, kv head), so any slice can be
regenerated alone.  The CPU and GPU generators are different engines: a GPU test
draws on the GPU and copies the same tensors to the host for the oracle.
"""
from __future__ import annotations

import hashlib
import math
from dataclasses import dataclass, replace

import numpy as np
import torch

HEAD_DIM = 128
TILE = 64  # tokens per cache tile (capacity granularity)


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    seq_len: int          # tokens already in the cache before the decode step
    k_bits: int
    v_bits: int
    outlier_frac: float   # fraction of entries per (token, kv-head) vector kept in fp16
    q_dtype: str          # "fp32" or "fp16"
    key_tail: str = "normal"   # distribution of the x10 key channels: "normal" | "laplace"
    n_scaled_channels: int = 4
    channel_gain: float = 10.0
    rope_base: float = 10000.0
    n_new: int = 1        # tokens appended per decode step (per sequence)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def n_outliers(self) -> int:
        """Outliers per vector: ceil(f * D) (0 at f = 0)."""
        return int(math.ceil(round(self.outlier_frac * self.head_dim, 9)))

    @property
    def capacity(self) -> int:
        """Cache capacity: room for the prefix and one decode step, rounded to a tile."""
        need = self.seq_len + self.n_new
        return ((need + TILE - 1) // TILE) * TILE

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The decode-path workloads: a single head at 4K, LLaMA-7B-shaped layers at 32K (3-bit),
# 128K (4-bit, outlier sweep) and 1M (2-bit) tokens, and a Llama-3-8B-shaped GQA layer
# at batch 16 x 64K.
WORKLOADS = {
    "single_head_4k": Workload("single_head_4k", 1, 1, 1, HEAD_DIM, 4096, 3, 3, 0.01, "fp32"),
    "llama7b_32k": Workload("llama7b_32k", 1, 32, 32, HEAD_DIM, 32768, 3, 3, 0.01, "fp16"),
    "llama7b_128k_4bit": Workload("llama7b_128k_4bit", 1, 32, 32, HEAD_DIM, 131072, 4, 4, 0.01,
                                  "fp16", key_tail="laplace"),
    "llama7b_1m_2bit": Workload("llama7b_1m_2bit", 1, 32, 32, HEAD_DIM, 1048576, 2, 2, 0.01, "fp16"),
    "llama3_8b_gqa_b16_64k": Workload("llama3_8b_gqa_b16_64k", 16, 32, 8, HEAD_DIM, 65536, 3, 3,
                                      0.01, "fp16"),
}
# The 4-bit workload is swept over these outlier fractions.
OUTLIER_SWEEP = (0.0, 0.005, 0.01)


def _seed(*parts) -> int:
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _np_rng(*parts) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(_seed(*parts)))


def _torch_gen(device, *parts) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*parts))
    return g


def codebook(seed: int, bits: int, which: str) -> np.ndarray:
    """2^bits distinct values drawn U(-1, 1), rounded to fp16-representable values,
    sorted ascending; returned as float32.  ``which`` separates the key and value
    codebooks ("k" / "v")."""
    rng = _np_rng("codebook", seed, bits, which)
    n = 1 << bits
    vals: set = set()
    while len(vals) < n:
        v = float(np.float16(rng.uniform(-1.0, 1.0)))
        if -1.0 <= v <= 1.0:
            vals.add(v)
    return np.array(sorted(vals), dtype=np.float32)


def uniform_codebook(bits: int) -> np.ndarray:
    """Evenly spaced levels -1 + 2j/(2^b - 1) (float32), the symmetric uniform grid."""
    n = 1 << bits
    return np.array([-1.0 + 2.0 * j / (n - 1) for j in range(n)], dtype=np.float32)


def scaled_channels(seed: int, wl: Workload, kvh: int) -> np.ndarray:
    """The key channels of kv head ``kvh`` whose activations are scaled by the gain."""
    rng = _np_rng("scaled_channels", seed, wl.head_dim, kvh)
    return np.sort(rng.choice(wl.head_dim, size=wl.n_scaled_channels, replace=False))


def _key_draw(gen, n, wl: Workload, chans: np.ndarray, device) -> torch.Tensor:
    x = torch.randn(n, wl.head_dim, generator=gen, device=device, dtype=torch.float32)
    if len(chans):
        ci = torch.as_tensor(chans, device=device, dtype=torch.long)
        if wl.key_tail == "laplace":
            u = torch.rand(n, len(chans), generator=gen, device=device, dtype=torch.float64) - 0.5
            u = u.clamp(-0.5 + 1e-12, 0.5 - 1e-12)
            lap = (-torch.sign(u) * torch.log1p(-2.0 * u.abs())).to(torch.float32)
            x[:, ci] = lap * wl.channel_gain
        else:
            x[:, ci] = x[:, ci] * wl.channel_gain
    return x.to(torch.float16)


def keys(seed: int, wl: Workload, b: int, kvh: int, n: int, device="cpu") -> torch.Tensor:
    """Pre-RoPE key stream of sequence ``b``, kv head ``kvh``: fp16 [n, head_dim]."""
    gen = _torch_gen(device, "keys", seed, wl.name, wl.key_tail, b, kvh)
    return _key_draw(gen, n, wl, scaled_channels(seed, wl, kvh), device)


def values(seed: int, wl: Workload, b: int, kvh: int, n: int, device="cpu") -> torch.Tensor:
    """Value stream of sequence ``b``, kv head ``kvh``: fp16 [n, head_dim], N(0,1)."""
    gen = _torch_gen(device, "values", seed, wl.name, b, kvh)
    return torch.randn(n, wl.head_dim, generator=gen, device=device).to(torch.float16)


def queries(seed: int, wl: Workload, device="cpu") -> torch.Tensor:
    """Decode-step queries [batch, n_q_heads, head_dim], N(0,1), already rotated at
    their own position; float32 or float16 per the workload."""
    rng = _np_rng("queries", seed, wl.name)
    q = rng.standard_normal((wl.batch, wl.n_q_heads, wl.head_dim)).astype(np.float32)
    t = torch.from_numpy(q)
    if wl.q_dtype == "fp16":
        t = t.to(torch.float16)
    return t.to(device)


def key_scale(seed: int, wl: Workload, n_calib: int = 4096, quantile: float | None = None) -> np.ndarray:
    """Frozen per-channel key scale [n_kv_heads, head_dim] float32 from a separately
    seeded calibration draw of ``n_calib`` tokens: the largest raw |key| per channel
    (``quantile`` None; tokens seen later may exceed it and then land on an end code),
    or the ``quantile`` of |key| per channel (linear interpolation in float64, rounded
    to float32), a threshold that about a 1 - quantile share of entries exceed."""
    out = np.zeros((wl.n_kv_heads, wl.head_dim), dtype=np.float32)
    for h in range(wl.n_kv_heads):
        gen = _torch_gen("cpu", "calib", seed, wl.name, wl.key_tail, h)
        x = _key_draw(gen, n_calib, wl, scaled_channels(seed, wl, h), "cpu")
        a = x.float().abs()
        if quantile is None:
            out[h] = a.amax(dim=0).numpy()
        else:
            out[h] = np.quantile(a.numpy().astype(np.float64), quantile, axis=0).astype(np.float32)
    return out


def seq_lens(wl: Workload, ragged: bool = False, seed: int = 0) -> np.ndarray:
    """Per-sequence cache lengths before the decode step.  ``ragged`` draws unequal
    lengths in [seq_len/2, seq_len] for batch > 1 (the first sequence keeps seq_len)."""
    if not ragged or wl.batch == 1:
        return np.full(wl.batch, wl.seq_len, dtype=np.int32)
    rng = _np_rng("seq_lens", seed, wl.name)
    lens = rng.integers(wl.seq_len // 2, wl.seq_len + 1, size=wl.batch).astype(np.int32)
    lens[0] = wl.seq_len
    return lens
