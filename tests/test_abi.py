"""The C ABI without a GPU: the library loads, exports every entry point the header
declares, sizes buffers as the documented layout says, and rejects bad arguments with
the documented status codes before touching the device."""
import ctypes
import os
import re

import pytest

import long_context_decode_kvq_amd as kvq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kvq.LIB_PATH), reason="libkvq.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = kvq.load_library()
    names = declared_functions()
    assert set(names) == set(kvq.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert lib.kvq_abi_version() == kvq.ABI_VERSION


def cfg(**kw):
    base = dict(batch=2, n_q_heads=8, n_kv_heads=2, max_seq=256, k_bits=3, v_bits=4, n_outliers=2)
    base.update(kw)
    return kvq.CacheConfig(**base)


def test_cache_sizes_match_layout():
    c = cfg()
    s = kvq.cache_sizes(c)
    slots = 2 * 2 * 256
    assert s.k_codes == slots * 128 * 3 // 8
    assert s.v_codes == slots * 128 * 4 // 8
    assert s.k_out_idx == slots * 2 and s.k_out_val == slots * 4
    assert s.v_scale == slots * 2
    assert s.k_scale == 2 * 128 * 4 and s.k_codebook == 8 * 2 and s.v_codebook == 16 * 2
    assert s.total == sum(getattr(s, f) for f, _ in kvq.Sizes._fields_ if f != "total")


def test_million_token_layer_footprint_fits():
    """32 layers of a LLaMA-7B-shaped 2-bit cache with 1 % outliers at 1M tokens."""
    c = cfg(batch=1, n_q_heads=32, n_kv_heads=32, max_seq=1 << 20, k_bits=2, v_bits=2, n_outliers=2)
    per_layer = kvq.cache_sizes(c).total
    fp16 = 2 * 32 * (1 << 20) * 128 * 2
    assert 32 * per_layer < 288e9
    assert fp16 / per_layer > 6.0


def test_workspace_bytes():
    c = cfg()
    assert kvq.workspace_bytes(c, 1) == 2 * 8 * 1 * 130 * 4
    assert kvq.workspace_bytes(c, 1025) == 2 * 8 * 2 * 130 * 4
    assert kvq.workspace_bytes(c, 0) == 0


@pytest.mark.parametrize("field,value,status", [
    ("head_dim", 64, -2), ("k_bits", 5, -2), ("v_bits", 1, -2), ("n_q_heads", 6, -2),
    ("max_seq", 100, -1), ("n_outliers", 129, -1), ("n_outliers", -1, -1), ("batch", 0, -1),
    ("rope_base", 0.5, -1), ("key_outliers", 2, -1), ("key_outliers", -1, -1)])
def test_bad_shapes_rejected(field, value, status):
    c = cfg(**{field: value})
    out = kvq.Sizes()
    st = kvq.load_library().kvq_cache_sizes(ctypes.byref(c.shape()), ctypes.byref(out))
    assert st == status


def test_entry_points_reject_before_launch():
    lib = kvq.load_library()
    c = cfg()
    shape = c.shape()
    desc = kvq.CacheDesc()  # all NULL
    lens = (ctypes.c_int32 * 2)(0, 0)
    assert lib.kvq_quantize_append(ctypes.byref(shape), ctypes.byref(desc), None, None, 1, None, lens, None) == -1
    assert lib.kvq_qk_matvec(ctypes.byref(shape), None, None, 0, 1.0, None, 10, None) == -1
    # a descriptor with fake (never dereferenced) pointers: capacity and workspace checks
    fake = kvq.CacheDesc(*([ctypes.c_void_p(4096)] * len(kvq.CacheDesc._fields_)))
    big = (ctypes.c_int32 * 2)(250, 0)
    assert lib.kvq_quantize_append(ctypes.byref(shape), ctypes.byref(fake), 4096, 4096, 10, None, big, None) == -3
    assert lib.kvq_pv_matvec(ctypes.byref(shape), ctypes.byref(fake), 4096, 4096, 4096, 16, 10, None) == -4
    assert lib.kvq_qk_matvec(ctypes.byref(shape), ctypes.byref(fake), 4096, 2, 1.0, 4096, 10, None) == -1
    assert lib.kvq_qk_matvec(ctypes.byref(shape), ctypes.byref(fake), 4096, 0, 1.0, 4096, 257, None) == -1
    for s in (0, -1, -2, -3, -4, -5, 7):
        assert lib.kvq_status_string(s)


def test_fp16_baseline_entry_points_reject_before_launch():
    lib = kvq.load_library()
    c = cfg()
    shape = c.shape()
    p = 4096  # fake device pointers, never dereferenced: every case fails its host checks
    assert lib.kvq_fp16_qk_matvec(ctypes.byref(shape), None, p, p, 0, 1.0, p, 10, None) == -1
    assert lib.kvq_fp16_qk_matvec(ctypes.byref(shape), p, p, p, 2, 1.0, p, 10, None) == -1
    assert lib.kvq_fp16_qk_matvec(ctypes.byref(shape), p, p, p, 0, 1.0, p, c.max_seq + 1, None) == -1
    assert lib.kvq_fp16_pv_matvec(ctypes.byref(shape), p, p, p, p, p, 16, 10, None) == -4
    assert lib.kvq_fp16_pv_matvec(ctypes.byref(shape), p, None, p, p, p, 1 << 20, 10, None) == -1
    bad = cfg(head_dim=64).shape()
    assert lib.kvq_fp16_qk_matvec(ctypes.byref(bad), p, p, p, 0, 1.0, p, 10, None) == -2
    # bit widths and outliers do not concern the fp16 cache
    odd = cfg(k_bits=5, n_outliers=-1).shape()
    assert lib.kvq_fp16_pv_matvec(ctypes.byref(odd), p, p, p, p, p, 16, 10, None) == -4


def test_fused_entry_point_rejects_before_launch():
    lib = kvq.load_library()
    p = 4096  # fake device pointers, never dereferenced
    fake = kvq.CacheDesc(*([ctypes.c_void_p(p)] * len(kvq.CacheDesc._fields_)))
    mha = cfg(n_q_heads=2, n_kv_heads=2, k_bits=3).shape()
    assert lib.kvq_decode_attention(ctypes.byref(mha), None, p, 0, 1.0, p, p, 1 << 20, 10, None) == -1
    assert lib.kvq_decode_attention(ctypes.byref(mha), ctypes.byref(fake), p, 0, 1.0, p, p, 16, 10, None) == -4
    assert lib.kvq_decode_attention(ctypes.byref(mha), ctypes.byref(fake), p, 2, 1.0, p, p, 1 << 20, 10, None) == -1
    # grouped heads and 4-bit keys are served by the two-call path
    gqa = cfg(k_bits=3).shape()
    assert lib.kvq_decode_attention(ctypes.byref(gqa), ctypes.byref(fake), p, 0, 1.0, p, p, 1 << 20, 10, None) == -2
    k4 = cfg(n_q_heads=2, n_kv_heads=2, k_bits=4).shape()
    assert lib.kvq_decode_attention(ctypes.byref(k4), ctypes.byref(fake), p, 0, 1.0, p, p, 1 << 20, 10, None) == -2


def test_fit_codebook_entry_point_rejects_before_launch():
    lib = kvq.load_library()
    p, ws = 4096, int(lib.kvq_fit_workspace_bytes())
    assert ws >= 320
    assert lib.kvq_fit_codebook(p, 10, 5, 3, p, p, ws, None) == -2        # bits
    assert lib.kvq_fit_codebook(None, 10, 3, 3, p, p, ws, None) == -1     # inputs missing
    assert lib.kvq_fit_codebook(p, -1, 3, 3, p, p, ws, None) == -1        # negative count
    assert lib.kvq_fit_codebook(p, 10, 3, -1, p, p, ws, None) == -1       # negative iterations
    assert lib.kvq_fit_codebook(p, 1 << 33, 3, 1, p, p, ws, None) == -1   # integer sums could overflow
    assert lib.kvq_fit_codebook(p, 10, 3, 3, None, p, ws, None) == -1     # no output
    assert lib.kvq_fit_codebook(p, 10, 3, 3, p, p, ws - 1, None) == -4    # workspace


def test_key_scale_entry_point_rejects_before_launch():
    lib = kvq.load_library()
    shape = cfg().shape()
    p = 4096
    assert lib.kvq_key_scale(ctypes.byref(shape), None, 10, 0, p, None) == -1
    assert lib.kvq_key_scale(ctypes.byref(shape), p, -1, 0, p, None) == -1
    assert lib.kvq_key_scale(ctypes.byref(shape), p, 10, 2, p, None) == -1
    assert lib.kvq_key_scale(ctypes.byref(shape), p, 10, 0, None, None) == -1
    assert lib.kvq_key_scale(ctypes.byref(cfg(head_dim=64).shape()), p, 10, 0, p, None) == -2


def test_key_threshold_entry_point_rejects_before_launch():
    lib = kvq.load_library()
    c = cfg()
    shape = c.shape()
    p = 4096
    ws = lib.kvq_key_threshold_workspace_bytes(ctypes.byref(shape), 10)
    assert ws > 0 and lib.kvq_key_threshold_workspace_bytes(ctypes.byref(shape), 0) == 0
    assert lib.kvq_key_threshold_workspace_bytes(ctypes.byref(shape), -1) == 0
    assert lib.kvq_key_threshold_workspace_bytes(ctypes.byref(shape), 2 ** 30) == 0  # 2 * 2^30 vectors
    # 256 blocks' high-bit histograms (at least 64 vectors each), the summed ones, the selections
    assert ws == 4 * (2 * 1 * 256 * 128 + 2 * 256 * 128) + 8 * 2 * 128
    big = lib.kvq_key_threshold_workspace_bytes(ctypes.byref(shape), 1 << 20)
    assert big == 4 * (2 * 128 * 256 * 128 + 2 * 256 * 128) + 8 * 2 * 128
    T = lib.kvq_key_threshold
    assert T(ctypes.byref(shape), None, 10, 0.01, p, p, ws, None) == -1          # no keys
    assert T(ctypes.byref(shape), p, -1, 0.01, p, p, ws, None) == -1             # negative length
    assert T(ctypes.byref(shape), p, 10, -0.1, p, p, ws, None) == -1             # fraction below 0
    assert T(ctypes.byref(shape), p, 10, 1.5, p, p, ws, None) == -1              # fraction above 1
    assert T(ctypes.byref(shape), p, 10, float("nan"), p, p, ws, None) == -1     # NaN fraction
    assert T(ctypes.byref(shape), p, 10, 0.01, None, p, ws, None) == -1          # no output
    assert T(ctypes.byref(shape), p, 2 ** 30, 0.01, p, p, ws, None) == -1        # 2^31 vectors
    assert T(ctypes.byref(shape), p, 10, 0.01, p, None, ws, None) == -4          # no workspace
    assert T(ctypes.byref(shape), p, 10, 0.01, p, p, ws - 1, None) == -4         # short workspace
    assert T(ctypes.byref(cfg(head_dim=64).shape()), p, 10, 0.01, p, p, ws, None) == -2


def test_stream_read_rejects_before_launch():
    lib = kvq.load_library()
    assert lib.kvq_stream_read(4096, 100, 4096, None) == -1      # size not a multiple of 16
    assert lib.kvq_stream_read(4104, 160, 4096, None) == -1      # misaligned buffer
    assert lib.kvq_stream_read(None, 160, 4096, None) == -1      # no buffer
    assert lib.kvq_stream_read(4096, 160, None, None) == -1      # no sink


def test_noalloc_value_pass_rejects_before_launch():
    """kvq_pv_matvec_noalloc checks its arguments like kvq_pv_matvec and refuses sizes whose
    split partials exceed its fixed device array, before touching the device."""
    lib = kvq.load_library()
    p = 4096  # fake device pointers, never dereferenced
    fake = kvq.CacheDesc(*([ctypes.c_void_p(p)] * len(kvq.CacheDesc._fields_)))
    f = lib.kvq_pv_matvec_noalloc
    shape = cfg().shape()
    assert f(ctypes.byref(shape), None, p, p, 10, None) == -1                    # no cache
    assert f(ctypes.byref(shape), ctypes.byref(fake), None, p, 10, None) == -1   # no logits
    assert f(ctypes.byref(shape), ctypes.byref(fake), p, None, 10, None) == -1   # no output
    assert f(ctypes.byref(shape), ctypes.byref(fake), p, p, 0, None) == -1       # empty bound
    assert f(ctypes.byref(shape), ctypes.byref(fake), p, p, 257, None) == -1     # beyond capacity
    assert f(ctypes.byref(cfg(head_dim=64).shape()), ctypes.byref(fake), p, p, 10, None) == -2
    # 32 query heads of one sequence: partials of ceil(L / 1024) parts of 130 floats each
    limit = kvq.NOALLOC_SCRATCH_BYTES
    fits = 1024 * (limit // (32 * 130 * 4))             # the longest bound that fits
    big = cfg(batch=1, n_q_heads=32, n_kv_heads=32, max_seq=fits + 1024).shape()
    assert kvq.workspace_bytes(cfg(batch=1, n_q_heads=32, n_kv_heads=32, max_seq=fits + 1024), fits) <= limit
    assert f(ctypes.byref(big), ctypes.byref(fake), p, p, fits + 1, None) == -4
