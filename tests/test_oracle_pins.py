"""Pins of the CPU oracle against things other than itself: exact rational brute force,
closed forms, textbook/library special cases, invariants and hand-derived bytes.

No GPU.  Each pin is chosen so a plausible mistake in the oracle (a dropped term, a
flipped sign, a transposed operand, a wrong tie rule or scale axis) fails it; the
mutation tests at the end plant such mistakes in the oracle and check that a pin fires.
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
D = 128


def _fp16_codebook(rng, bits):
    vals = set()
    while len(vals) < (1 << bits):
        vals.add(float(np.float16(rng.uniform(-1, 1))))
    return np.array(sorted(vals), np.float32)


# ---------------------------------------------------------------- nearest code ----

@pytest.mark.parametrize("bits", [2, 3, 4])
def test_nearest_code_matches_exact_rational_argmin(bits):
    """Exact Fraction argmin (ties -> lowest j) agrees with the fp32 scan except where
    the two best exact distances are within fp32 rounding of each other."""
    rng = np.random.default_rng(100 + bits)
    cb = _fp16_codebook(rng, bits)
    u = rng.uniform(-1.3, 1.3, size=400).astype(np.float32)
    # adversarial: exact midpoints between neighbours, and points one ulp either side
    mids = ((cb[:-1].astype(np.float64) + cb[1:]) / 2).astype(np.float32)
    u = np.concatenate([u, mids, np.nextafter(mids, np.float32(2)), np.nextafter(mids, np.float32(-2)),
                        cb, np.float32([0.0, -0.0, 1.0, -1.0])]).astype(np.float32)
    got = oracle.nearest_code(u, cb)
    for ui, gi in zip(u, got):
        fu = Fraction(float(ui))
        dist = [abs(fu - Fraction(float(c))) for c in cb]
        best = min(range(len(cb)), key=lambda j: (dist[j], j))
        if gi != best:
            # an exact tie must go to the lower index; otherwise only an fp32 near-tie
            # may differ from exact arithmetic
            assert dist[gi] != dist[best]
            assert abs(dist[gi] - dist[best]) <= Fraction(2) ** -23 * max(dist[best], Fraction(1, 2 ** 30))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_uniform_codebook_no_outliers_is_textbook_symmetric_uniform(bits):
    """Uniform codebook, k = 0: value quantization is the textbook symmetric absmax
    quantizer code = round((x/max|x| + 1)(2^b - 1)/2)."""
    rng = np.random.default_rng(7 + bits)
    cb = synth.uniform_codebook(bits)
    x = rng.standard_normal((64, D)).astype(np.float16)
    codes, idx, val, s16 = oracle.quantize_values(x, cb, 0)
    assert idx.shape == (64, 0) and val.shape == (64, 0)
    s = np.abs(x.astype(np.float64)).max(axis=1)
    assert np.array_equal(s16.view(np.float16).astype(np.float64), s)
    levels = (1 << bits) - 1
    t = (x.astype(np.float64) / s[:, None] + 1.0) * levels / 2.0
    expect = np.floor(t + 0.5)
    near_tie = np.abs(t - np.floor(t) - 0.5) < 1e-5
    assert np.array_equal(codes[~near_tie], expect[~near_tie].astype(np.uint8))
    # and the reconstruction error is at most half a step
    deq = oracle.dequant_values(codes, idx, val, s16, cb)
    # (the fp32-rounded grid levels may overshoot half a step by an fp32 ulp)
    assert np.all(np.abs(deq - x.astype(np.float64)) <= s[:, None] / levels * (1 + 1e-6))


# ------------------------------------------------------------------- outliers ----

def test_outlier_selection_matches_full_sort_with_ties():
    rng = np.random.default_rng(3)
    # few distinct magnitudes -> many ties
    x = rng.choice(np.float16([-3, -2, -1, 0, 1, 2, 3, 2.5, -2.5]), size=(50, D)).astype(np.float16)
    for k in (0, 1, 2, 5, D):
        got = oracle.select_outliers(x, k)
        for r in range(x.shape[0]):
            order = sorted(range(D), key=lambda c: (-abs(float(x[r, c])), c))
            assert list(got[r]) == sorted(order[:k])


def test_outliers_chosen_by_raw_magnitude_not_scaled():
    x = np.zeros((1, D), np.float16)
    x[0, 5] = 8.0     # larger raw magnitude, but a large channel scale
    x[0, 9] = 3.0     # smaller raw magnitude, small channel scale
    ks = np.ones(D, np.float32)
    ks[5] = 100.0
    codes, idx, val = oracle.quantize_keys(x, ks, synth.uniform_codebook(3), 1)
    assert list(idx[0]) == [5]
    assert val[0, 0] == np.float16(8.0).view(np.uint16)


def test_key_scale_axis_is_the_channel():
    """Scaling one channel's scale by 2 while doubling that channel's data leaves its
    codes unchanged and touches no other channel (per-channel key scale)."""
    rng = np.random.default_rng(11)
    cb = _fp16_codebook(rng, 3)
    x = rng.standard_normal((40, D)).astype(np.float16)
    ks = np.full(D, 4.0, np.float32)
    c1, _, _ = oracle.quantize_keys(x, ks, cb, 0)
    x2 = x.copy()
    x2[:, 17] = (x2[:, 17].astype(np.float32) * 2).astype(np.float16)
    ks2 = ks.copy()
    ks2[17] = 8.0
    c2, _, _ = oracle.quantize_keys(x2, ks2, cb, 0)
    assert np.array_equal(c1, c2)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_uniform_codebook_keys_are_the_textbook_per_channel_quantizer(bits):
    """Uniform codebook, k = 0, a different non-unit scale on every channel: key
    quantization is the textbook per-channel symmetric quantizer
    code_c = round((x_c / s_c + 1)(2^b - 1)/2) (clamped to the grid), it decodes to
    s_c (-1 + 2 code_c / (2^b - 1)), and each dense entry is within half a step,
    s_c / (2^b - 1), of x_c.  A decode that drops, swaps or transposes the per-channel
    scale misses all three."""
    rng = np.random.default_rng(70 + bits)
    s = (0.5 + np.arange(D) * 0.0625).astype(np.float32)   # 0.5 .. 8.4375, all distinct
    x = (rng.uniform(-1, 1, size=(96, D)) * s[None, :]).astype(np.float16)
    cb = synth.uniform_codebook(bits)
    codes, idx, val = oracle.quantize_keys(x, s, cb, 0)
    assert idx.shape == (96, 0) and val.shape == (96, 0)
    levels = (1 << bits) - 1
    t = (x.astype(np.float64) / s.astype(np.float64)[None, :] + 1.0) * levels / 2.0
    expect = np.clip(np.floor(t + 0.5), 0, levels)
    near_tie = np.abs(t - np.floor(t) - 0.5) < 1e-5
    assert np.array_equal(codes[~near_tie], expect[~near_tie].astype(np.uint8))
    deq = oracle.dequant_keys(codes, idx, val, s, cb)
    textbook = s.astype(np.float64)[None, :] * (-1.0 + 2.0 * codes.astype(np.float64) / levels)
    assert np.allclose(deq, textbook, rtol=1e-6, atol=0)
    err = np.abs(deq - x.astype(np.float64))
    assert np.all(err <= s.astype(np.float64)[None, :] / levels * (1 + 1e-6))


def _hand_example():
    """A two-token stream whose logits, outputs and tolerance scales are derived by hand.

    Key and value codebook cb = (-1, -1/2, 1/2, 1) (2-bit), k = 0.  Key scales s_0 = 2,
    s_64 = 4, every other channel 1.  Both key vectors hold x_0 = 1, x_64 = -4 and zeros
    elsewhere: u_0 = 1/2 -> code 2 (1/2), u_64 = -1 -> code 0 (-1), so the dequantized
    key has k~_0 = 1/2 * 2 = 1 and k~_64 = -1 * 4 = -4 (a zero entry, u = 0, ties between
    -1/2 and 1/2 and takes -1/2; the query is zero on those channels).  The query is
    q_0 = 1, q_64 = 2, zero elsewhere.  Rotary pair (0, 64) turns by t radians (theta_0 = 1),
    so y_0 = cos t + 4 sin t, y_64 = sin t - 4 cos t and
        l_t = sm (q_0 y_0 + q_64 y_64) = sm (6 sin t - 7 cos t),
        tolerance scale_t = sm (|y_0| + 2 |y_64|).
    Values: token 0 holds v_0 = 2, v_1 = -1 (max |v| = 2: codes 3 and 1, decoded 2 and
    -1), token 1 holds v_0 = -4, v_1 = 4 (scale 4: codes 0 and 3); every other channel is
    zero and decodes to the zero code -1/2 times the token's scale: -1 and -2."""
    cb = np.float32([-1.0, -0.5, 0.5, 1.0])
    s = np.ones(D, np.float32)
    s[0], s[64] = 2.0, 4.0
    k16 = np.zeros((2, D), np.float16)
    k16[:, 0], k16[:, 64] = 1.0, -4.0
    v16 = np.zeros((2, D), np.float16)
    v16[0, :2] = [2.0, -1.0]
    v16[1, :2] = [-4.0, 4.0]
    q = np.zeros(D)
    q[0], q[64] = 1.0, 2.0
    sm = 1.0 / math.sqrt(D)
    logits = np.array([sm * (6 * math.sin(t) - 7 * math.cos(t)) for t in (0, 1)])
    tol_l = np.array([sm * (abs(math.cos(t) + 4 * math.sin(t)) + 2 * abs(math.sin(t) - 4 * math.cos(t)))
                      for t in (0, 1)])
    p1 = 1.0 / (1.0 + math.exp(logits[0] - logits[1]))
    p = np.array([1.0 - p1, p1])
    v_dec = np.full((2, D), 0.0)
    v_dec[0], v_dec[1] = -1.0, -2.0
    v_dec[0, :2] = [2.0, -1.0]
    v_dec[1, :2] = [-4.0, 4.0]
    out = p @ v_dec
    tol_o = p @ np.abs(v_dec)
    return dict(cb=cb, s=s, k16=k16, v16=v16, q=q, sm=sm, logits=logits, tol_l=tol_l, out=out, tol_o=tol_o)


def test_per_channel_key_decode_hand_example():
    """decode_head on the dense path with channel-dependent key scales, against the
    hand-derived logits and output of _hand_example."""
    e = _hand_example()
    c = oracle.quantize_stream(e["k16"], e["v16"], e["s"], e["cb"], e["cb"], 0)
    assert list(c.k_codes[0, [0, 64, 1]]) == [2, 0, 1]
    logits, out = oracle.decode_head(e["q"], c, e["s"], e["cb"], e["cb"], 10000.0, e["sm"])
    assert np.allclose(logits, e["logits"], rtol=0, atol=1e-12)
    assert np.allclose(out, e["out"], rtol=0, atol=1e-12)


def test_tolerance_scales_hand_example():
    """The logit tolerance scale is sm * sum_c |q_c y_c| and the output one
    sum_t p_t |v~_t,c|, on the hand-derived example (a dropped sm_scale, a signed sum or
    unnormalised weights fail it)."""
    e = _hand_example()
    c = oracle.quantize_stream(e["k16"], e["v16"], e["s"], e["cb"], e["cb"], 0)
    tl = oracle.logit_tolerance_scale(e["q"], c, e["s"], e["cb"], 10000.0, e["sm"])
    assert np.allclose(tl, e["tol_l"], rtol=0, atol=1e-12)
    to = oracle.output_tolerance_scale(e["logits"], c, e["cb"])
    assert np.allclose(to, e["tol_o"], rtol=0, atol=1e-12)


def test_value_scale_is_per_vector_max_of_dense_part():
    rng = np.random.default_rng(12)
    cb = _fp16_codebook(rng, 3)
    x = rng.standard_normal((30, D)).astype(np.float16)
    codes, idx, val, s16 = oracle.quantize_values(x, cb, 2)
    xf = x.astype(np.float64)
    for r in range(30):
        dense = np.delete(xf[r], idx[r].astype(int))
        assert s16[r] == np.float16(np.abs(dense).max()).view(np.uint16)
        # the largest dense entry normalises to +-1 -> the end code nearest it
        c = int(np.delete(np.arange(D), idx[r].astype(int))[np.argmax(np.abs(dense))])
        end = len(cb) - 1 if xf[r, c] > 0 else 0
        assert codes[r, c] == end


def test_all_zero_dense_part_decodes_to_zero():
    cb = synth.codebook(0, 3, "v")
    x = np.zeros((3, D), np.float16)
    x[:, 4] = 5.0
    codes, idx, val, s16 = oracle.quantize_values(x, cb, 1)
    assert np.all(s16.view(np.float16) == 0)
    assert np.all(codes == oracle.zero_code(cb))
    deq = oracle.dequant_values(codes, idx, val, s16, cb)
    expect = np.zeros((3, D))
    expect[:, 4] = 5.0
    assert np.array_equal(deq, expect)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_dequant_error_bound(bits):
    """For dense channels with |u| <= 1: |x~ - x| <= s * max(half the largest codebook
    gap, distance from the ends to +-1)."""
    rng = np.random.default_rng(20 + bits)
    cb = _fp16_codebook(rng, bits)
    x = rng.standard_normal((200, D)).astype(np.float16)
    codes, idx, val, s16 = oracle.quantize_values(x, cb, 2)
    deq = oracle.dequant_values(codes, idx, val, s16, cb)
    cbd = cb.astype(np.float64)
    bound = max(np.max(np.diff(cbd)) / 2, 1 - cbd[-1], cbd[0] + 1)
    s = s16.view(np.float16).astype(np.float64)
    err = np.abs(deq - x.astype(np.float64))
    assert np.all(err <= s[:, None] * bound * (1 + 1e-6) + 1e-12)
    rows = np.arange(200)[:, None]
    assert np.all(err[rows, idx.astype(int)] == 0)  # outliers exact


# ---------------------------------------------------------------------- packing ----

def test_golden_pack_examples():
    with open(os.path.join(GOLDEN, "pack_examples.json")) as f:
        g = json.load(f)
    for ex in g["key_records"]:
        codes = np.zeros((1, D), np.uint8)
        for c, v in ex["codes"].items():
            codes[0, int(c)] = v
        rec = oracle.pack_key_records(codes, ex["bits"])
        assert rec.shape == (1, D * ex["bits"] // 8)
        for byte, v in ex["expect_bytes"].items():
            assert rec[0, int(byte)] == v, ex["derivation"]
        assert int(rec.astype(np.int64).sum()) == sum(ex["expect_bytes"].values())
    for ex in g["value_tiles"]:
        n = ex["token"] + 1
        codes = np.zeros((n, D), np.uint8)
        codes[ex["token"], ex["channel"]] = ex["code"]
        cap = ((n + 63) // 64) * 64
        tiles = oracle.pack_value_tiles(codes, ex["bits"], cap)
        tile = tiles[ex.get("tile", 0)]
        for byte, v in ex["expect_bytes"].items():
            assert tile[int(byte)] == v, ex["derivation"]
        assert int(tile.astype(np.int64).sum()) == sum(ex["expect_bytes"].values())


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_roundtrip(bits):
    rng = np.random.default_rng(bits)
    codes = rng.integers(0, 1 << bits, size=(130, D)).astype(np.uint8)
    rec = oracle.pack_key_records(codes, bits)
    assert rec.shape == (130, D * bits // 8)
    assert np.array_equal(oracle.unpack_key_records(rec, bits, D), codes)
    tiles = oracle.pack_value_tiles(codes, bits, 192)
    assert tiles.shape == (3, D * 8 * bits)
    assert np.array_equal(oracle.unpack_value_tiles(tiles, bits, D, 130), codes)
    # unwritten tail of the last tile is zero
    assert np.all(oracle.unpack_value_tiles(tiles, bits, D, 192)[130:] == 0)


# ------------------------------------------------------------------------- RoPE ----

def _rope_complex(x, pos, base):
    """Independent formulation: pair (i, i+D/2) as the complex number x_i + j x_{i+D/2},
    multiplied by exp(j * pos * theta_i) with theta_i = exp(-(2i/D) ln base)."""
    half = x.shape[1] // 2
    theta = np.exp(-(2.0 * np.arange(half) / x.shape[1]) * math.log(base))
    z = (x[:, :half] + 1j * x[:, half:]) * np.exp(1j * np.outer(pos, theta))
    return np.concatenate([z.real, z.imag], axis=1)


def test_rope_matches_complex_rotation_and_invariants():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((40, D))
    pos = np.concatenate([np.arange(20), rng.integers(0, 2_000_000, size=20)])
    y = oracle.rope(x, pos, 10000.0)
    assert np.allclose(y, _rope_complex(x, pos, 10000.0), rtol=0, atol=1e-9)
    # norm of every rotary pair preserved
    h = D // 2
    assert np.allclose(np.hypot(y[:, :h], y[:, h:]), np.hypot(x[:, :h], x[:, h:]), atol=1e-12)
    # R(0) = I
    assert np.array_equal(oracle.rope(x, np.zeros(40, int), 10000.0), x)
    # R(a) R(b) = R(a + b)
    a, b = 1234, 98765
    lhs = oracle.rope(oracle.rope(x, np.full(40, a), 1e4), np.full(40, b), 1e4)
    assert np.allclose(lhs, oracle.rope(x, np.full(40, a + b), 1e4), atol=1e-9)
    # relative position: R(p)q . R(t)k = q . R(t-p)k
    q = rng.standard_normal((1, D))
    p, t = 777, 5000
    l1 = (oracle.rope(q, [p], 1e4) * oracle.rope(x[:1], [t], 1e4)).sum()
    l2 = (q * oracle.rope(x[:1], [t - p], 1e4)).sum()
    assert abs(l1 - l2) < 1e-9


def test_rope_frequencies_closed_form():
    th = oracle.rope_frequencies(D, 10000.0)
    assert th[0] == 1.0
    assert np.allclose(th, 10000.0 ** (-np.arange(64) / 64.0), rtol=1e-15)
    assert np.all(np.diff(th) < 0)


# ------------------------------------------------------------------- attention ----

def _exact_attention(q, k16, v16, base, sm):
    """Textbook attention on the unquantized fp16 K/V: complex-rotated keys and
    torch's scaled_dot_product_attention in float64."""
    kr = _rope_complex(k16.astype(np.float64), np.arange(k16.shape[0]), base)
    qt = torch.tensor(q, dtype=torch.float64).view(1, 1, 1, -1)
    kt = torch.tensor(kr).view(1, 1, -1, k16.shape[1])
    vt = torch.tensor(v16.astype(np.float64)).view(1, 1, -1, k16.shape[1])
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, scale=sm)
    logits = sm * (kr @ q)
    return logits, out.view(-1).numpy()


def test_all_outliers_is_exact_attention():
    """k = D: every entry is kept in fp16, so decode attention over the compressed cache
    is exact attention over the fp16 keys and values."""
    wl = synth.WORKLOADS["single_head_4k"]
    n = 300
    k16 = synth.keys(1, wl, 0, 0, n).numpy()
    v16 = synth.values(1, wl, 0, 0, n).numpy()
    ks = synth.key_scale(1, wl)[0]
    cbk, cbv = synth.codebook(1, 3, "k"), synth.codebook(1, 3, "v")
    cache = oracle.quantize_stream(k16, v16, ks, cbk, cbv, D)
    q = synth.queries(1, wl)[0, 0].numpy().astype(np.float64)
    sm = 1 / math.sqrt(D)
    logits, out = oracle.decode_head(q, cache, ks, cbk, cbv, 1e4, sm)
    el, eo = _exact_attention(q, k16, v16, 1e4, sm)
    assert np.allclose(logits, el, rtol=0, atol=1e-10)
    assert np.allclose(out, eo, rtol=0, atol=1e-12)


def test_softmax_shift_invariance_and_special_cases():
    rng = np.random.default_rng(9)
    l = rng.standard_normal(50) * 5
    v = rng.standard_normal((50, D))
    assert np.allclose(oracle.attend(l, v), oracle.attend(l + 123.0, v), atol=1e-13)
    assert np.allclose(oracle.attend(np.zeros(50), v), v.mean(axis=0), atol=1e-13)
    assert np.allclose(oracle.attend(l[:1], v[:1]), v[0], atol=0)


def test_split_softmax_combine_equals_single_pass():
    """The log-sum-exp merge of per-chunk (max, sum, weighted sum) partials equals the
    single-pass softmax product, for any chunking (the split-K identity)."""
    rng = np.random.default_rng(10)
    l = rng.standard_normal(1000) * 4
    v = rng.standard_normal((1000, D))
    ref = oracle.attend(l, v)
    for chunk in (1, 7, 64, 333, 1000):
        ms, ss, os_ = [], [], []
        for s in range(0, 1000, chunk):
            lc = l[s:s + chunk]
            m = lc.max()
            p = np.exp(lc - m)
            ms.append(m); ss.append(p.sum()); os_.append(p @ v[s:s + chunk])
        M = max(ms)
        w = np.exp(np.array(ms) - M)
        out = (w[:, None] * np.array(os_)).sum(0) / (w * np.array(ss)).sum()
        assert np.allclose(out, ref, atol=1e-13)


# ------------------------------------------------------------- planted mistakes ----

def test_pins_catch_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle (CPU only) and check a pin fires."""
    # 1. RoPE with a flipped sine
    good_rope = oracle.kvquant.rope

    def bad_rope(x, positions, base):
        y = good_rope(x, positions, base)
        h = y.shape[1] // 2
        xx = np.asarray(x, np.float64)
        phi = np.asarray(positions, np.float64)[:, None] * oracle.rope_frequencies(x.shape[1], base)
        return np.concatenate([xx[:, :h] * np.cos(phi) + xx[:, h:] * np.sin(phi), y[:, h:]], axis=1)

    monkeypatch.setattr(oracle.kvquant, "rope", bad_rope)
    with pytest.raises(AssertionError):
        test_all_outliers_is_exact_attention()
    monkeypatch.setattr(oracle.kvquant, "rope", good_rope)

    # 2. outliers dropped from the decode (sparse term lost)
    good_scatter = oracle.kvquant._scatter_outliers
    monkeypatch.setattr(oracle.kvquant, "_scatter_outliers", lambda x, i, v: x)
    with pytest.raises(AssertionError):
        test_all_outliers_is_exact_attention()
    monkeypatch.setattr(oracle.kvquant, "_scatter_outliers", good_scatter)

    # 3. key fields stored in channel order instead of rotary-pair order
    good_fields = oracle.kvquant.key_field_channels
    monkeypatch.setattr(oracle.kvquant, "key_field_channels", lambda d: np.arange(d))
    with pytest.raises(AssertionError):
        test_golden_pack_examples()
    monkeypatch.setattr(oracle.kvquant, "key_field_channels", good_fields)

    # 4. nearest-code ties resolved toward the higher index
    good_nc = oracle.kvquant.nearest_code

    def bad_nc(u, cb):
        cbr = np.asarray(cb)[::-1]
        return (len(cbr) - 1 - good_nc(u, cbr)).astype(np.uint8)

    monkeypatch.setattr(oracle, "nearest_code", bad_nc)
    with pytest.raises(AssertionError):
        test_nearest_code_matches_exact_rational_argmin(3)
    monkeypatch.setattr(oracle, "nearest_code", good_nc)

    # 5. the key threshold's exceed budget off by one, or taken from a float32 fraction
    good_budget = oracle.kvquant.exceed_budget
    monkeypatch.setattr(oracle.kvquant, "exceed_budget", lambda f, n: good_budget(f, n) + 1)
    with pytest.raises(AssertionError):
        test_key_threshold_is_characterised_by_counting()
    monkeypatch.setattr(oracle.kvquant, "exceed_budget", lambda f, n: int(math.floor(float(np.float32(f)) * n)))
    monkeypatch.setattr(oracle, "exceed_budget", oracle.kvquant.exceed_budget)
    with pytest.raises(AssertionError):
        test_key_threshold_special_cases()
    monkeypatch.setattr(oracle.kvquant, "exceed_budget", good_budget)
    monkeypatch.setattr(oracle, "exceed_budget", good_budget)

    # 6. the per-channel key scale dropped from, or reversed across channels in, the decode
    good_dk = oracle.kvquant.dequant_keys
    for bad_scale in (lambda s: np.ones_like(np.asarray(s, np.float32)), lambda s: np.asarray(s)[::-1]):
        def bad_dk(codes, out_idx, out_val, k_scale32, codebook32, f=bad_scale):
            return good_dk(codes, out_idx, out_val, f(k_scale32), codebook32)
        monkeypatch.setattr(oracle.kvquant, "dequant_keys", bad_dk)
        monkeypatch.setattr(oracle, "dequant_keys", bad_dk)
        with pytest.raises(AssertionError):
            test_per_channel_key_decode_hand_example()
        with pytest.raises(AssertionError):
            test_uniform_codebook_keys_are_the_textbook_per_channel_quantizer(3)
    monkeypatch.setattr(oracle.kvquant, "dequant_keys", good_dk)
    monkeypatch.setattr(oracle, "dequant_keys", good_dk)

    # 7. the logit tolerance without sm_scale; the output tolerance as a signed sum
    good_tl, good_to = oracle.kvquant.logit_tolerance_scale, oracle.kvquant.output_tolerance_scale
    monkeypatch.setattr(oracle, "logit_tolerance_scale",
                        lambda q, c, ks, cb, base, sm, length=None: good_tl(q, c, ks, cb, base, 1.0, length))
    with pytest.raises(AssertionError):
        test_tolerance_scales_hand_example()
    monkeypatch.setattr(oracle, "logit_tolerance_scale", good_tl)

    def signed_to(logits, c, cb, length=None):
        n = c.length if length is None else length
        vd = oracle.dequant_values(c.v_codes[:n], c.v_idx[:n], c.v_val[:n], c.v_scale[:n], cb)
        return np.abs(oracle.softmax(logits[:n]) @ vd)
    monkeypatch.setattr(oracle, "output_tolerance_scale", signed_to)
    with pytest.raises(AssertionError):
        test_tolerance_scales_hand_example()
    monkeypatch.setattr(oracle, "output_tolerance_scale", good_to)


# ---- codebook fitting (unweighted k-means, oracle/codebook_fit.py) -----------------------

def test_fit_uniform_inputs_keep_the_uniform_quantizer():
    """For inputs spread evenly over [-1, 1] the optimal K-level quantizer (Lloyd-Max) has
    its levels at the midpoints of K equal bins: iterating must not move them."""
    from fractions import Fraction
    n = 1 << 14
    u = np.array([(i + 0.5) / n * 2.0 - 1.0 for i in range(n)], dtype=np.float32)
    for bits in (2, 3, 4):
        k = 1 << bits
        c = oracle.fit_init(bits)
        for _ in range(5):
            c = oracle.fit_step(u, c)[0]
        expect = [float(Fraction(-1) + Fraction(2 * j + 1, k)) for j in range(k)]
        assert np.allclose(c.astype(np.float64), expect, atol=1e-6), (bits, c)


def test_fit_moves_each_centroid_to_its_cluster_mean():
    """Tight clusters, one inside each initial bin: one iteration puts every centroid on
    its cluster's exact mean (rational arithmetic), to the float32 rounding."""
    from fractions import Fraction
    rng = np.random.default_rng(7)
    for bits in (2, 3, 4):
        k = 1 << bits
        width = 2.0 / k
        centers = -1.0 + width * (np.arange(k) + 0.5 + rng.uniform(-0.3, 0.3, k))
        pts = [np.float32(c + rng.uniform(-0.02, 0.02, rng.integers(5, 40)) * width).astype(np.float32) for c in centers]
        u = np.concatenate(pts)
        c1 = oracle.fit_step(u, oracle.fit_init(bits))[0]
        for j, p in enumerate(pts):
            mean = float(sum(Fraction(float(x)) for x in p) / len(p))
            assert abs(float(c1[j]) - mean) <= 2e-7 * max(1.0, abs(mean)), (bits, j)


def test_fit_distortion_never_increases():
    """Lloyd's invariant: neither the assignment nor the mean update can raise the mean
    squared error."""
    rng = np.random.default_rng(3)
    u = oracle.clamp_inputs(rng.standard_normal(20000) * 0.4)
    for bits in (2, 3, 4):
        c = oracle.fit_init(bits)
        prev = oracle.quantization_mse(u, c)
        for _ in range(8):
            c = oracle.fit_step(u, c)[0]
            cur = oracle.quantization_mse(u, c)
            assert cur <= prev + 1e-12, (bits, cur, prev)
            prev = cur


def test_fit_empty_cluster_keeps_its_centroid_and_result_is_a_valid_codebook():
    u = np.full(100, 0.3, dtype=np.float32)  # every input in one bin
    c1, sums, counts, _ = oracle.fit_step(u, oracle.fit_init(2))
    assert counts.tolist() == [0, 0, 100, 0]
    assert c1[0] == oracle.fit_init(2)[0] and c1[3] == oracle.fit_init(2)[3]
    assert abs(float(c1[2]) - 0.3) < 1e-7
    for cand in ([0.5, 0.5, 0.5, 1.0], [0.999, 1.0, 1.0, 1.0], [-1.0, -1.0, 0.2, 0.2]):
        h = oracle.finalize(np.array(cand, dtype=np.float32))
        assert np.all(np.diff(h.astype(np.float64)) > 0) and h.min() >= -1 and h.max() <= 1, (cand, h)
        # values already in place are kept
        assert h[0] == np.float16(cand[0]) or cand[0] > 0.99


def test_key_scale_is_the_channel_max_of_the_dense_part():
    """Brute force on small inputs: for every channel, the largest |x| among the entries
    that are not one of their vector's k largest (ties to the lower channel)."""
    rng = np.random.default_rng(5)
    for k in (0, 1, 2, 5):
        x = rng.standard_normal((40, 16)).astype(np.float16)
        x[3, :] = np.float16(2.0)  # a vector of ties: its outliers are its lowest channels
        got = oracle.key_scale_from_keys(x, k)
        exp = np.zeros(16)
        for t in range(40):
            row = [(abs(float(x[t, c])), c) for c in range(16)]
            out = {c for _, c in sorted(row, key=lambda e: (-e[0], e[1]))[:k]}
            for c in range(16):
                if c not in out:
                    exp[c] = max(exp[c], abs(float(x[t, c])))
        assert np.array_equal(got.astype(np.float64), exp), k
    assert np.array_equal(oracle.key_scale_from_keys(x, 16), np.zeros(16, np.float32))


# ---- per-channel key outliers (candidates |x_c| > s_c, at most k, largest |x_c|/s_c) ----

def test_per_channel_rule_properties_on_many_vectors():
    """Checked against what the rule must satisfy, not a restatement of it: every kept
    channel exceeds its scale; the count is min(#candidates, k); no dropped candidate beats
    a kept one in (ratio, -channel) order; kept channels ascend, unused slots hold the
    sentinel; the dense part then lies in [-s_c, s_c] outside the dropped candidates."""
    rng = np.random.default_rng(11)
    x = rng.choice(np.float16([-6, -3, -2, -1, -0.5, 0, 0.5, 1, 2, 3, 6]), size=(200, D)).astype(np.float16)
    s = rng.choice(np.float32([0.0, 0.5, 1.0, 2.0, 3.0, 4.0]), size=D).astype(np.float32)
    for k in (0, 1, 2, 4, D):
        idx, count = oracle.select_outliers_by_threshold(x, s, k)
        for r in range(x.shape[0]):
            mag = [abs(float(x[r, c])) for c in range(D)]
            cand = [c for c in range(D) if mag[c] > s[c]]
            kept = [int(c) for c in idx[r] if c != oracle.NO_OUTLIER]
            assert count[r] == len(kept) == min(len(cand), k)
            assert kept == sorted(kept) and all(c in cand for c in kept)
            assert all(c == oracle.NO_OUTLIER for c in idx[r][len(kept):])
            ratio = lambda c: Fraction(mag[c]) / Fraction(float(s[c])) if s[c] > 0 else math.inf
            for c in cand:
                if c in kept:
                    continue
                for kc in kept:  # a dropped candidate never outranks a kept one
                    assert (ratio(kc), -kc) > (ratio(c), -c)


def test_per_channel_rule_reduces_to_top_k_for_a_uniform_power_of_two_threshold():
    """With the same power-of-two scale below every |x_c| in every channel, |x_c|/s orders
    exactly like |x_c|: the rule is the per-vector top-k rule."""
    rng = np.random.default_rng(5)
    x = (rng.choice(np.float16([1, 2, 3, 4, 5, 6, 7, 8]), size=(100, D)) *
         rng.choice(np.float16([-1, 1]), size=(100, D))).astype(np.float16)
    s = np.full(D, 0.5, np.float32)
    for k in (1, 2, 5):
        idx, count = oracle.select_outliers_by_threshold(x, s, k)
        assert np.all(count == k)
        assert np.array_equal(idx, oracle.select_outliers(x, k))


def test_per_channel_keys_decode_and_sentinel_slots():
    """Unused slots (sentinel channel, value 0) change nothing when decoding; kept outliers
    decode exactly; dense entries are within the quantizer's error bound of x; a candidate
    dropped by the cap lands on an end code."""
    cb = synth.uniform_codebook(3)
    x = np.zeros((2, D), np.float16)
    s = np.ones(D, np.float32)
    x[0, 3], x[0, 70], x[0, 9] = 5.0, -7.0, 0.75   # two candidates, k = 4 -> two sentinels
    x[1, [1, 2, 3]] = [9.0, 4.0, 2.0]               # three candidates, k = 2 -> channel 3 stays dense
    codes, idx, val = oracle.quantize_keys(x, s, cb, 4, per_channel=True)
    assert list(idx[0]) == [3, 70, oracle.NO_OUTLIER, oracle.NO_OUTLIER] and list(val[0][2:]) == [0, 0]
    deq = oracle.dequant_keys(codes, idx, val, s, cb)
    assert deq[0, 3] == 5.0 and deq[0, 70] == -7.0
    assert abs(deq[0, 9] - 0.75) <= (2.0 / 7) / 2 + 1e-12
    codes2, idx2, val2 = oracle.quantize_keys(x, s, cb, 2, per_channel=True)
    assert list(idx2[1]) == [1, 2]
    assert codes2[1, 3] == len(cb) - 1  # u = 2 clamps to the top entry
    # the same codes with the sentinel slots removed decode identically
    assert np.array_equal(oracle.dequant_keys(codes, idx[:, :2], val[:, :2], s, cb)[0], deq[0])


def test_per_channel_keys_with_all_entries_outliers_is_exact_attention():
    """k = D and tiny scales: every nonzero entry is an outlier, so the keys decode exactly
    and attention equals exact attention over the fp16 keys."""
    rng = np.random.default_rng(2)
    n = 40
    k16 = rng.standard_normal((n, D)).astype(np.float16)
    v16 = rng.standard_normal((n, D)).astype(np.float16)
    s = np.full(D, 1e-30, np.float32)
    c = oracle.quantize_stream(k16, v16, s, synth.uniform_codebook(2), synth.uniform_codebook(2), D,
                               per_channel_keys=True)
    kd = oracle.dequant_keys(c.k_codes, c.k_idx, c.k_val, s, synth.uniform_codebook(2))
    assert np.array_equal(kd, k16.astype(np.float64))


# ---- per-channel key threshold (calibration for the per-channel outlier rule) ----------

def test_key_threshold_golden_example():
    """Hand-derived thresholds of a 5-vector, 4-channel example (tests/golden)."""
    with open(os.path.join(os.path.dirname(__file__), "golden", "key_threshold_example.json")) as f:
        g = json.load(f)
    x = np.array(g["keys"], dtype=np.float16)
    for case in g["cases"]:
        assert oracle.exceed_budget(case["outlier_frac"], x.shape[0]) == case["m"], case
        got = oracle.key_threshold_from_keys(x, case["outlier_frac"])
        assert got.dtype == np.float32 and got.tolist() == case["threshold"], case


def test_key_threshold_is_characterised_by_counting():
    """Not a re-sort: s_c is a magnitude present in channel c, at most m entries lie above
    it and at least m + 1 at or above it (so no smaller threshold keeps within m); s_c = 0
    when m >= N.  Data with heavy ties, signed zeros and both signs."""
    rng = np.random.default_rng(8)
    vals = np.float16([0, -0.0, 0.25, -0.25, 1, -1, 1.5, 3, -3, 3, 7, 65504, -65504])
    for n in (1, 2, 7, 64, 300):
        x = rng.choice(vals, size=(n, 24)).astype(np.float16)
        for f in (0.0, 0.001, 0.01, 0.1, 0.33, 0.5, 0.999, 1.0):
            m = oracle.exceed_budget(f, n)
            s = oracle.key_threshold_from_keys(x, f)
            for c in range(24):
                mag = [abs(float(v)) for v in x[:, c]]
                if m >= n:
                    assert s[c] == 0.0
                    continue
                above = sum(1 for a in mag if a > s[c])
                at_or_above = sum(1 for a in mag if a >= s[c])
                assert float(s[c]) in mag and above <= m < at_or_above, (n, f, c)


def test_key_threshold_special_cases():
    """f = 0 gives the channel maximum (the max-scale calibration without outliers); the
    exceed budget is formed in float64 (0.01 of 300 is 3, where a float32 0.01 would
    give 2); an empty calibration set gives zeros; the threshold does not depend on the
    order of the vectors, and each channel only on its own entries."""
    rng = np.random.default_rng(3)
    x = rng.standard_normal((500, D)).astype(np.float16)
    assert np.array_equal(oracle.key_threshold_from_keys(x, 0.0), oracle.key_scale_from_keys(x, 0))
    assert oracle.exceed_budget(0.01, 300) == 3 and oracle.exceed_budget(0.5, 7) == 3
    assert oracle.exceed_budget(1.0, 12345) == 12345
    assert np.array_equal(oracle.key_threshold_from_keys(np.zeros((0, D), np.float16), 0.01), np.zeros(D, np.float32))
    s = oracle.key_threshold_from_keys(x, 0.01)
    perm_t, perm_c = rng.permutation(500), rng.permutation(D)
    assert np.array_equal(oracle.key_threshold_from_keys(x[perm_t], 0.01), s)
    assert np.array_equal(oracle.key_threshold_from_keys(x[:, perm_c], 0.01), s[perm_c])
    # about 1 % of each channel's entries lie above its threshold
    above = (np.abs(x.astype(np.float32)) > s).sum(axis=0)
    assert np.all(above <= 5)
