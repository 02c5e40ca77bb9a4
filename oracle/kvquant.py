"""Plain, slow CPU oracle for KVQuant-style quantized-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The product path never calls it and shares
no code with it; the only thing both sides consume is the seeded input generator.

Sources (the KVQuant pages):
  [P1] "KVQuant: Towards 10 Million Context Length LLM Inference with KV Cache
       Quantization" (study.space summary), abstract paragraph: techniques (i) per-channel
       key quantization, (ii) pre-RoPE key quantization, (iii) non-uniform per-layer
       datatypes, (iv) per-vector dense-and-sparse quantization that isolates outliers
       separately for each vector; decode is memory- and bandwidth-bound.
  [P2] "KVQuant" paper note (phantomic12 inference-research), "Four components"
       paragraph: keys quantized per channel and before the rotary embedding (the
       position-dependent rotation would otherwise mix values between quantization
       levels); a codebook per layer; outliers isolated per vector, not globally.

The pages give the components in prose only; every step below that they leave open is
a stated reading (see the notes on each function).  Precision: the quantization
decision (normalise, nearest code) is taken in float32 exactly as the device kernel
takes it, so codes can be compared bit for bit; decode, RoPE, logits, softmax and the
value product are float64.
"""
from __future__ import annotations

import math

import numpy as np

# ----------------------------------------------------------------------------------
# Quantization of one (token, kv head) vector
# ----------------------------------------------------------------------------------


def _as_f16(x) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return x.view(np.float16)
    return x.astype(np.float16)


def select_outliers(x16, k: int) -> np.ndarray:
    """Per-vector outlier channels [P1 (iv); P2 item (4)].

    For each row (one vector of D fp16 entries) return the ``k`` channels of largest
    raw magnitude |x_c|, ties broken toward the lower channel, listed in ascending
    channel order.  Shape [N, k], int64.  Reading: magnitude is the raw |x| (not |x|
    divided by a scale); "1 %" per vector means k = ceil(0.01 * D)."""
    x = _as_f16(x16)
    n, d = x.shape
    if k == 0:
        return np.zeros((n, 0), dtype=np.int64)
    mag = np.abs(x.astype(np.float64))
    # Stable sort on descending magnitude keeps ascending channel order among ties.
    order = np.argsort(-mag, axis=1, kind="stable")
    return np.sort(order[:, :k], axis=1)


# Channel index of an unused outlier slot (key vectors under the per-channel rule).
NO_OUTLIER = 255


def select_outliers_by_threshold(x16, k_scale32, k: int):
    """Key outliers under the per-channel reading of [P1 (iv)]: keys are quantized per
    channel [P1 (i); P2 item (1)], so a key entry counts as an outlier by its own
    channel's standard, the frozen per-channel scale s_c, which then also bounds every
    dense entry it leaves.

    Entry c of a vector is a candidate iff |x_c| > s_c (float32 comparison).  A vector
    keeps at most ``k`` candidates: those with the largest float32 ratio |x_c| / s_c
    (+inf where s_c = 0), ties toward the lower channel; candidates beyond k stay dense.
    Returns (idx int64 [N, k]: the kept channels in ascending order, then NO_OUTLIER in
    the unused slots; count int64 [N])."""
    x = _as_f16(x16)
    n, d = x.shape
    idx = np.full((n, k), NO_OUTLIER, dtype=np.int64)
    count = np.zeros(n, dtype=np.int64)
    if k == 0:
        return idx, count
    mag = np.abs(x.astype(np.float32))
    s = np.asarray(k_scale32, dtype=np.float32)
    for r in range(n):
        cand = [c for c in range(d) if mag[r, c] > s[c]]
        ratio = {c: (np.float32(mag[r, c] / s[c]) if s[c] > 0 else np.float32(np.inf)) for c in cand}
        kept = sorted(sorted(cand, key=lambda c: (-float(ratio[c]), c))[:k])
        idx[r, :len(kept)] = kept
        count[r] = len(kept)
    return idx, count


def nearest_code(u32: np.ndarray, codebook32: np.ndarray) -> np.ndarray:
    """Non-uniform code assignment [P1 (iii); P2 item (3)].

    code = the smallest j minimising |u - cb_j|, with both the difference and its
    magnitude rounded to float32, scanned in ascending j with a strict '<'."""
    u = np.asarray(u32, dtype=np.float32)
    cb = np.asarray(codebook32, dtype=np.float32)
    best = np.zeros(u.shape, dtype=np.uint8)
    best_d = np.abs((u - cb[0]).astype(np.float32)).astype(np.float32)
    for j in range(1, len(cb)):
        dj = np.abs((u - cb[j]).astype(np.float32)).astype(np.float32)
        better = dj < best_d
        best = np.where(better, np.uint8(j), best)
        best_d = np.where(better, dj, best_d)
    return best


def _dense_part(x16, idx) -> np.ndarray:
    """x with its outlier entries set to zero, as float32 (the dense half of the
    dense-and-sparse split x = dense + sparse); NO_OUTLIER slots are skipped."""
    d = _as_f16(x16).astype(np.float32).copy()
    idx = np.asarray(idx, np.int64)
    r, j = np.nonzero(idx != NO_OUTLIER)
    d[r, idx[r, j]] = 0.0
    return d


def _normalise(d32: np.ndarray, s32: np.ndarray) -> np.ndarray:
    """u = d / s in float32 (IEEE division); u = 0 where s == 0."""
    s = np.broadcast_to(s32, d32.shape).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    u = (d32 / safe).astype(np.float32)
    return np.where(s > 0, u, np.float32(0.0)).astype(np.float32)


def quantize_keys(x16, k_scale32, codebook32, k: int, per_channel: bool = False):
    """Quantize key vectors of one kv head, pre-RoPE, with a per-channel scale.

    [P1 (i), (ii), (iii), (iv); P2 items (1)-(4)]
      x16         fp16 [N, D] pre-RoPE keys
      k_scale32   float32 [D]: this kv head's frozen per-channel scale
      codebook32  float32 [2^b], ascending, the layer's key codebook
      per_channel False: each vector's k largest |x_c| are its outliers
                  (select_outliers); True: the per-channel rule
                  (select_outliers_by_threshold), unused slots NO_OUTLIER with value 0
    Returns (codes uint8 [N, D], out_idx uint8 [N, k], out_val uint16 [N, k]).
    The dense part (outliers zeroed) is divided channel-wise by the scale and mapped
    to the nearest code; outliers keep their fp16 bits unchanged."""
    x = _as_f16(x16)
    if per_channel:
        idx = select_outliers_by_threshold(x, k_scale32, k)[0]
    else:
        idx = select_outliers(x, k)
    d = _dense_part(x, idx)
    u = _normalise(d, np.asarray(k_scale32, dtype=np.float32)[None, :])
    codes = nearest_code(u, codebook32)
    rows = np.arange(x.shape[0])[:, None]
    used = idx != NO_OUTLIER
    val = x.view(np.uint16)[rows, np.where(used, idx, 0)] if k else np.zeros((x.shape[0], 0), np.uint16)
    val = np.where(used, val, np.uint16(0))
    return codes, idx.astype(np.uint8), np.ascontiguousarray(val, dtype=np.uint16)


def quantize_values(x16, codebook32, k: int):
    """Quantize value vectors with one scale per (token, kv head) vector.

    The pages fix per-channel quantization for keys only; values take the other axis,
    one scale per vector: s = max over dense channels of |x_c| (an fp16 value, so it is
    stored exactly as fp16).  [P1 (i), (iii), (iv)]
    Returns (codes uint8 [N, D], out_idx uint8 [N, k], out_val uint16 [N, k],
    scale uint16 [N] (fp16 bits))."""
    x = _as_f16(x16)
    idx = select_outliers(x, k)
    d = _dense_part(x, idx)
    s = np.abs(d).max(axis=1).astype(np.float32)
    u = _normalise(d, s[:, None])
    codes = nearest_code(u, codebook32)
    rows = np.arange(x.shape[0])[:, None]
    val = x.view(np.uint16)[rows, idx] if k else np.zeros((x.shape[0], 0), np.uint16)
    return (codes, idx.astype(np.uint8), np.ascontiguousarray(val, dtype=np.uint16),
            s.astype(np.float16).view(np.uint16))


def zero_code(codebook32) -> int:
    """The code every dense-zero entry (in particular every outlier slot) receives:
    the smallest j minimising |0 - cb_j|."""
    return int(nearest_code(np.zeros(1, np.float32), codebook32)[0])


# ----------------------------------------------------------------------------------
# Bit packing (storage layout of the compressed cache)
# ----------------------------------------------------------------------------------

TILE = 64


def key_field_channels(d: int) -> np.ndarray:
    """Channel stored in each b-bit field of a key record: fields alternate between the
    two halves of a rotary pair, field 2i -> channel i, field 2i+1 -> channel i + D/2."""
    half = d // 2
    f = np.arange(d)
    return f // 2 + half * (f % 2)


def _pack_bits(fields: np.ndarray, bits: int) -> np.ndarray:
    """Little-endian bitstream: bit i of field f is stream bit f*bits + i; stream bit p
    lives in byte p // 8 at bit position p % 8.  fields: [..., F] -> bytes [..., F*bits/8]."""
    f = np.asarray(fields, dtype=np.uint8)
    planes = (f[..., None] >> np.arange(bits, dtype=np.uint8)) & 1
    stream = planes.reshape(*f.shape[:-1], f.shape[-1] * bits)
    return np.packbits(stream, axis=-1, bitorder="little")


def _unpack_bits(data: np.ndarray, bits: int, n_fields: int) -> np.ndarray:
    stream = np.unpackbits(np.asarray(data, np.uint8), axis=-1, bitorder="little")
    stream = stream[..., : n_fields * bits].reshape(*stream.shape[:-1], n_fields, bits)
    weights = (1 << np.arange(bits)).astype(np.uint16)
    return (stream.astype(np.uint16) * weights).sum(axis=-1).astype(np.uint8)


def pack_key_records(codes: np.ndarray, bits: int) -> np.ndarray:
    """Key cache record per token: D*bits/8 bytes, fields in rotary-pair order
    (see key_field_channels).  codes [N, D] -> uint8 [N, D*bits/8]."""
    d = codes.shape[-1]
    return _pack_bits(np.asarray(codes)[..., key_field_channels(d)], bits)


def unpack_key_records(records: np.ndarray, bits: int, d: int) -> np.ndarray:
    fields = _unpack_bits(records, bits, d)
    codes = np.empty_like(fields)
    codes[..., key_field_channels(d)] = fields
    return codes


def pack_value_tiles(codes: np.ndarray, bits: int, capacity: int) -> np.ndarray:
    """Value cache of one (sequence, kv head) stream, channel-major inside 64-token tiles.

    Tile T holds tokens 64T..64T+63.  Inside a tile, channel c owns 8*bits bytes: the
    little-endian bitstream of its 64 codes in token order.  Channels follow in order.
    Tokens at or beyond N (not yet written) have all-zero codes.
    codes [N, D] -> uint8 [capacity/64, D*8*bits]."""
    n, d = codes.shape
    assert capacity % TILE == 0 and n <= capacity
    full = np.zeros((capacity, d), dtype=np.uint8)
    full[:n] = codes
    tiles = full.reshape(capacity // TILE, TILE, d).transpose(0, 2, 1)  # [T, D, 64]
    return _pack_bits(tiles, bits).reshape(capacity // TILE, d * 8 * bits)


def unpack_value_tiles(tiles: np.ndarray, bits: int, d: int, n: int) -> np.ndarray:
    t = np.asarray(tiles, np.uint8).reshape(tiles.shape[0], d, 8 * bits)
    codes = _unpack_bits(t, bits, TILE)  # [T, D, 64]
    return codes.transpose(0, 2, 1).reshape(-1, d)[:n]


# ----------------------------------------------------------------------------------
# Decode (dequantization) of the dense-and-sparse representation
# ----------------------------------------------------------------------------------


def _scatter_outliers(x: np.ndarray, idx, val) -> np.ndarray:
    """Outlier channels take their stored fp16 value; NO_OUTLIER slots change nothing."""
    idx = np.asarray(idx, np.int64)
    v = np.asarray(val, np.uint16).view(np.float16).astype(np.float64)
    r, j = np.nonzero(idx != NO_OUTLIER)
    x[r, idx[r, j]] = v[r, j]
    return x


def dequant_keys(codes, out_idx, out_val, k_scale32, codebook32) -> np.ndarray:
    """x~_c = cb[code_c] * s_c for dense channels; outlier channels take their stored
    fp16 value exactly.  float64 [N, D] (pre-RoPE)."""
    cb = np.asarray(codebook32, np.float64)
    x = cb[np.asarray(codes, np.int64)] * np.asarray(k_scale32, np.float64)[None, :]
    return _scatter_outliers(x, out_idx, out_val)


def dequant_values(codes, out_idx, out_val, scale16, codebook32) -> np.ndarray:
    """x~_c = cb[code_c] * s_t for dense channels (s_t the vector's fp16 scale); outlier
    channels take their stored fp16 value exactly.  float64 [N, D]."""
    cb = np.asarray(codebook32, np.float64)
    s = np.asarray(scale16, np.uint16).view(np.float16).astype(np.float64)
    x = cb[np.asarray(codes, np.int64)] * s[:, None]
    return _scatter_outliers(x, out_idx, out_val)


# ----------------------------------------------------------------------------------
# Rotary embedding applied after dequantization, then attention
# ----------------------------------------------------------------------------------


def rope_frequencies(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/D), i < D/2, float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / d)


def rope(x: np.ndarray, positions, base: float) -> np.ndarray:
    """Rotate-half rotary embedding in float64 [P2 item (2): applied to keys after
    dequantization, at each cached token's own position].  Pair (i, i + D/2) is rotated
    by the angle position * theta_i."""
    x = np.asarray(x, np.float64)
    d = x.shape[-1]
    half = d // 2
    phi = np.asarray(positions, np.float64)[:, None] * rope_frequencies(d, base)[None, :]
    c, s = np.cos(phi), np.sin(phi)
    a, b = x[:, :half], x[:, half:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=1)


def qk_logits(q: np.ndarray, k_rot: np.ndarray, sm_scale: float) -> np.ndarray:
    """l_t = sm_scale * q . k_rot_t.  q [D], k_rot [N, D] -> float64 [N]."""
    return sm_scale * (np.asarray(k_rot, np.float64) @ np.asarray(q, np.float64))


def softmax(logits: np.ndarray) -> np.ndarray:
    l = np.asarray(logits, np.float64)
    e = np.exp(l - l.max())
    return e / e.sum()


def attend(logits: np.ndarray, v_deq: np.ndarray) -> np.ndarray:
    """softmax(l) . V over the given tokens; float64 [D]."""
    return softmax(logits) @ np.asarray(v_deq, np.float64)


# ----------------------------------------------------------------------------------
# One (sequence, kv head) stream end to end
# ----------------------------------------------------------------------------------


class StreamCache:
    """The compressed cache of one (sequence, kv head): what the oracle quantized."""

    def __init__(self, k_codes, k_idx, k_val, v_codes, v_idx, v_val, v_scale):
        self.k_codes, self.k_idx, self.k_val = k_codes, k_idx, k_val
        self.v_codes, self.v_idx, self.v_val, self.v_scale = v_codes, v_idx, v_val, v_scale

    @property
    def length(self) -> int:
        return self.k_codes.shape[0]


def quantize_stream(k16, v16, k_scale32, k_codebook32, v_codebook32, k: int,
                    per_channel_keys: bool = False) -> StreamCache:
    """Keys and values of one stream; per_channel_keys selects the keys' outlier rule."""
    kc, ki, kv = quantize_keys(k16, k_scale32, k_codebook32, k, per_channel_keys)
    vc, vi, vv, vs = quantize_values(v16, v_codebook32, k)
    return StreamCache(kc, ki, kv, vc, vi, vv, vs)


def decode_head(q, cache: StreamCache, k_scale32, k_codebook32, v_codebook32,
                rope_base: float, sm_scale: float, length: int | None = None):
    """Decode attention of one query head against one kv stream of ``length`` tokens.
    Returns (logits float64 [length], out float64 [D])."""
    n = cache.length if length is None else length
    kd = dequant_keys(cache.k_codes[:n], cache.k_idx[:n], cache.k_val[:n], k_scale32, k_codebook32)
    kr = rope(kd, np.arange(n), rope_base)
    logits = qk_logits(q, kr, sm_scale)
    vd = dequant_values(cache.v_codes[:n], cache.v_idx[:n], cache.v_val[:n], cache.v_scale[:n],
                        v_codebook32)
    return logits, attend(logits, vd)


def logit_tolerance_scale(q, cache: StreamCache, k_scale32, k_codebook32, rope_base: float,
                          sm_scale: float, length: int | None = None) -> np.ndarray:
    """sm_scale * sum_c |q_c * y_{t,c}| per token (y the rotated dequantized key): the
    magnitude a relative logit error is measured against."""
    n = cache.length if length is None else length
    kd = dequant_keys(cache.k_codes[:n], cache.k_idx[:n], cache.k_val[:n], k_scale32, k_codebook32)
    kr = rope(kd, np.arange(n), rope_base)
    return sm_scale * (np.abs(kr) @ np.abs(np.asarray(q, np.float64)))


def output_tolerance_scale(logits, cache: StreamCache, v_codebook32, length: int | None = None):
    """sum_t p_t |v~_{t,c}| per channel: the magnitude a relative output error is
    measured against."""
    n = cache.length if length is None else length
    vd = dequant_values(cache.v_codes[:n], cache.v_idx[:n], cache.v_val[:n], cache.v_scale[:n],
                        v_codebook32)
    return softmax(logits[:n]) @ np.abs(vd)


# ----------------------------------------------------------------------------------
# Key scale calibration
# ----------------------------------------------------------------------------------


def exceed_budget(outlier_frac: float, n: int) -> int:
    """How many of a channel's n calibration entries may lie above its threshold:
    floor(outlier_frac * n), the product formed in float64 (an IEEE double product,
    then floor)."""
    return int(math.floor(float(outlier_frac) * float(n)))


def key_threshold_from_keys(k16, outlier_frac: float) -> np.ndarray:
    """Per-channel key threshold for the per-channel outlier rule (R19 reading of
    [P1 (i), (iv); P2 items (1), (4)]): the pages give no calibration for it, so the
    threshold is the plainest one that keeps a chosen share of each channel's entries
    out of range.  With N calibration vectors and m = exceed_budget(outlier_frac, N),
    s_c is the smallest |x_c| of the calibration set that at most m entries of channel c
    exceed, i.e. its (m+1)-th largest magnitude; 0 when m >= N (so also for N = 0).

    Magnitudes are ordered as fp16 bit patterns with the sign cleared (numeric order for
    finite numbers; a NaN ranks above +inf), and s_c is that fp16 magnitude as float32
    (exact).  k16: [N, D] fp16 vectors of one kv head.  Returns float32 [D]."""
    x = _as_f16(k16)
    n, d = x.shape
    m = exceed_budget(outlier_frac, n)
    out = np.zeros(d, dtype=np.float32)
    if m >= n:
        return out
    mag = (x.view(np.uint16) & np.uint16(0x7FFF)).astype(np.int64)
    for c in range(d):
        ordered = np.sort(mag[:, c])[::-1]           # largest first
        out[c] = np.uint16(ordered[m]).view(np.float16).astype(np.float32)
    return out


def key_scale_from_keys(k16, k: int = 0) -> np.ndarray:
    """Per-channel key scale from calibration keys [P1 (i): keys are quantized per channel;
    P2 item (1)]: s_c = max over the given vectors of |x_c| (float32, exact for fp16
    inputs).  With k > 0 each vector's k outliers (``select_outliers``) are left out first,
    so the scale covers the dense part the quantizer sees (the reading in which outliers
    are held aside before the range is set).  k16: [N, D] fp16 vectors of one kv head."""
    x = _as_f16(k16)
    mag = np.abs(x.astype(np.float32))
    if k > 0:
        idx = select_outliers(x, k)
        mag = mag.copy()
        np.put_along_axis(mag, idx, 0.0, axis=1)
    return mag.max(axis=0) if len(mag) else np.zeros(x.shape[1], dtype=np.float32)
