"""Shared helpers for the parity tests: build the same seeded case on the HIP path and in
the oracle, and compare them.  Inputs come only from ``synth``; expected values only
from ``oracle``."""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import synth

D = 128


def make_streams(wl: synth.Workload, seed: int, lens, device):
    """Raw fp16 K/V per (sequence, kv head), each of length lens[b]: dict (b, h) -> (k, v)."""
    out = {}
    for b in range(wl.batch):
        for h in range(wl.n_kv_heads):
            out[(b, h)] = (synth.keys(seed, wl, b, h, int(lens[b]), device),
                           synth.values(seed, wl, b, h, int(lens[b]), device))
    return out


def stack_new(wl: synth.Workload, streams, lo, hi, n_max, device):
    """fp16 [B][n_max][Hkv][D] holding tokens lo[b]..hi[b]-1 of each stream (zero pad)."""
    k = torch.zeros(wl.batch, n_max, wl.n_kv_heads, D, dtype=torch.float16, device=device)
    v = torch.zeros_like(k)
    for (b, h), (ks, vs) in streams.items():
        n = int(hi[b]) - int(lo[b])
        if n > 0:
            k[b, :n, h] = ks[int(lo[b]):int(hi[b])]
            v[b, :n, h] = vs[int(lo[b]):int(hi[b])]
    return k.contiguous(), v.contiguous()


class Case:
    """One seeded workload instance: the oracle's view and (optionally) the GPU cache."""

    def __init__(self, wl: synth.Workload, seed: int = 0, lens=None, device="cpu", max_seq=None,
                 k_codebook=None, v_codebook=None, k_scale=None, key_outliers=0):
        self.wl, self.seed, self.device = wl, seed, device
        self.key_outliers = key_outliers  # 0: per-vector top-k; 1: per-channel thresholds
        self.lens = np.asarray(synth.seq_lens(wl) if lens is None else lens, dtype=np.int64)
        need = int(self.lens.max())
        self.max_seq = max_seq or max(64, ((need + 63) // 64) * 64)
        self.k = wl.n_outliers
        self.cbk = synth.codebook(seed, wl.k_bits, "k") if k_codebook is None else k_codebook
        self.cbv = synth.codebook(seed, wl.v_bits, "v") if v_codebook is None else v_codebook
        self.ks = synth.key_scale(seed, wl) if k_scale is None else k_scale
        self.q = synth.queries(seed, wl, device)
        self.streams = make_streams(wl, seed, self.lens, device)
        self._oracle = {}

    # ---------------------------------------------------------------- oracle side --
    def oracle_stream(self, b, h) -> oracle.StreamCache:
        if (b, h) not in self._oracle:
            ks, vs = self.streams[(b, h)]
            self._oracle[(b, h)] = oracle.quantize_stream(ks.cpu().numpy(), vs.cpu().numpy(), self.ks[h],
                                                          self.cbk, self.cbv, self.k,
                                                          per_channel_keys=self.key_outliers == 1)
        return self._oracle[(b, h)]

    def q_head(self, b, hq) -> np.ndarray:
        return self.q[b, hq].float().cpu().numpy().astype(np.float64)

    def oracle_decode(self, b, hq):
        h = hq // self.wl.group
        c = self.oracle_stream(b, h)
        sm = 1.0 / math.sqrt(D)
        return oracle.decode_head(self.q_head(b, hq), c, self.ks[h], self.cbk, self.cbv, self.wl.rope_base, sm)

    # ------------------------------------------------------------------- GPU side --
    def build_gpu(self, chunks=None, upto=None):
        """Fill a KVCache through kvq_quantize_append.  ``chunks``: list of per-call token
        counts (same for every sequence, clipped to its length); default one bulk call.
        ``upto``: per-sequence lengths to stop at (default: the case's lengths)."""
        import long_context_decode_kvq_amd as kvq
        wl = self.wl
        cfg = kvq.CacheConfig(wl.batch, wl.n_q_heads, wl.n_kv_heads, self.max_seq, wl.k_bits, wl.v_bits,
                              self.k, D, wl.rope_base, self.key_outliers)
        cache = kvq.KVCache(cfg, torch.from_numpy(self.ks), torch.from_numpy(self.cbk),
                            torch.from_numpy(self.cbv), device=self.device)
        target = self.lens if upto is None else np.asarray(upto, dtype=np.int64)
        total = int(target.max())
        chunks = chunks or [total]
        pos = np.zeros(wl.batch, dtype=np.int64)
        for n in chunks:
            hi = np.minimum(pos + n, target)
            cnt = hi - pos
            if cnt.max() <= 0:
                continue
            k_new, v_new = stack_new(wl, self.streams, pos, hi, int(cnt.max()), self.device)
            kvq.quantize_append(cache, k_new, v_new, n_new=cnt.tolist())
            pos = hi
        assert np.array_equal(pos, target)
        return cache

    # ------------------------------------------------------------ expected buffers --
    def expected_buffers(self, b, h):
        """The oracle's packed buffers for stream (b, h), padded to max_seq with zeros."""
        c = self.oracle_stream(b, h)
        n, S, k = c.length, self.max_seq, self.k
        rec = np.zeros((S, D * self.wl.k_bits // 8), np.uint8)
        rec[:n] = oracle.pack_key_records(c.k_codes, self.wl.k_bits)
        tiles = oracle.pack_value_tiles(c.v_codes, self.wl.v_bits, S)
        pad = lambda a, dt: np.concatenate([a, np.zeros((S - n,) + a.shape[1:], dt)]) if S > n else a
        return dict(k_rec=rec, v_tiles=tiles, k_idx=pad(c.k_idx, np.uint8), k_val=pad(c.k_val, np.uint16),
                    v_idx=pad(c.v_idx, np.uint8), v_val=pad(c.v_val, np.uint16),
                    v_scale=pad(c.v_scale, np.uint16))


def gpu_buffers(cache, b, h):
    """Download stream (b, h) of a KVCache in the documented layouts."""
    ki, kv = cache.outliers("k")
    vi, vv = cache.outliers("v")
    S = cache.cfg.max_seq
    return dict(k_rec=cache.k_records()[b, h].cpu().numpy(),
                v_tiles=cache.v_tiles()[b, h].cpu().numpy(),
                k_idx=ki[b, h].cpu().numpy(), k_val=kv[b, h].cpu().numpy().view(np.uint16),
                v_idx=vi[b, h].cpu().numpy(), v_val=vv[b, h].cpu().numpy().view(np.uint16),
                v_scale=cache.v_scale.view(cache.cfg.batch, cache.cfg.n_kv_heads, S)[b, h].cpu().numpy().view(np.uint16))


def assert_logits_close(got, ref, scale, rel=1e-3, what=""):
    """|got - ref| <= rel * scale elementwise (scale = sm * sum_c |q_c y_c|)."""
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = err > rel * scale
    assert not bad.any(), (f"{what}: {bad.sum()} logits out of tolerance; worst ratio "
                           f"{(err / np.maximum(rel * scale, 1e-300)).max():.3g}")
    return float((err / np.maximum(scale, 1e-300)).max())


def assert_out_close(got, ref, scale, rel=1e-3, what=""):
    err = np.abs(np.asarray(got, np.float64) - ref)
    bad = err > rel * scale
    assert not bad.any(), (f"{what}: {bad.sum()} outputs out of tolerance; worst ratio "
                           f"{(err / np.maximum(rel * scale, 1e-300)).max():.3g}")
    return float((err / np.maximum(scale, 1e-300)).max())
