"""Quantized-KV decode attention on MI355X (gfx950): Python binding of libkvq.so.

Argument marshalling only: every step of the path (quantize-append, the q.K^T matvec
with RoPE after dequantization, the split softmax.V matvec and its combine) runs in the
HIP kernels behind the C ABI declared in ``include/kvq.h``.  PyTorch supplies device
memory and the current stream.  There is no fallback: if libkvq.so is missing or fails to
load, every entry point raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvq.so")

KVQ_OK = 0
STATUS_NAMES = {0: "KVQ_OK", -1: "KVQ_ERR_INVALID", -2: "KVQ_ERR_UNSUPPORTED",
                -3: "KVQ_ERR_CAPACITY", -4: "KVQ_ERR_WORKSPACE", -5: "KVQ_ERR_HIP"}
EXPORTED = ("kvq_cache_sizes", "kvq_workspace_bytes", "kvq_quantize_append", "kvq_qk_matvec",
            "kvq_pv_matvec", "kvq_pv_matvec_noalloc", "kvq_decode_attention", "kvq_key_scale", "kvq_key_threshold_workspace_bytes",
            "kvq_key_threshold", "kvq_fit_workspace_bytes", "kvq_fit_codebook", "kvq_stream_read",
            "kvq_fp16_qk_matvec", "kvq_fp16_pv_matvec", "kvq_status_string",
            "kvq_abi_version")
ABI_VERSION = 4


class KvqError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({msg})")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("max_seq", ctypes.c_int32), ("k_bits", ctypes.c_int32), ("v_bits", ctypes.c_int32),
                ("n_outliers", ctypes.c_int32), ("rope_base", ctypes.c_float), ("key_outliers", ctypes.c_int32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "k_codes", "v_codes", "k_out_idx", "k_out_val", "v_out_idx", "v_out_val", "v_scale",
        "k_scale", "k_codebook", "v_codebook", "seq_len")]


class Sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in (
        "k_codes", "v_codes", "k_out_idx", "k_out_val", "v_out_idx", "v_out_val", "v_scale",
        "k_scale", "k_codebook", "v_codebook", "seq_len", "total")]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """dlopen libkvq.so and declare its signatures (raises if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() or "
                           "python long_context_decode_kvq_amd/build.py")
    lib = ctypes.CDLL(path)
    P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.kvq_cache_sizes.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(Sizes)]
    lib.kvq_cache_sizes.restype = ctypes.c_int
    lib.kvq_workspace_bytes.argtypes = [ctypes.POINTER(Shape), I32]
    lib.kvq_workspace_bytes.restype = SZ
    lib.kvq_quantize_append.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(CacheDesc), P, P, I32,
                                        P, P, P]
    lib.kvq_quantize_append.restype = ctypes.c_int
    lib.kvq_qk_matvec.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(CacheDesc), P, I32,
                                  ctypes.c_float, P, I32, P]
    lib.kvq_qk_matvec.restype = ctypes.c_int
    lib.kvq_pv_matvec.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(CacheDesc), P, P, P, SZ,
                                  I32, P]
    lib.kvq_pv_matvec.restype = ctypes.c_int
    lib.kvq_pv_matvec_noalloc.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(CacheDesc), P, P, I32, P]
    lib.kvq_pv_matvec_noalloc.restype = ctypes.c_int
    lib.kvq_decode_attention.argtypes = [ctypes.POINTER(Shape), ctypes.POINTER(CacheDesc), P, I32, ctypes.c_float,
                                         P, P, SZ, I32, P]
    lib.kvq_decode_attention.restype = ctypes.c_int
    lib.kvq_key_scale.argtypes = [ctypes.POINTER(Shape), P, I32, I32, P, P]
    lib.kvq_key_scale.restype = ctypes.c_int
    lib.kvq_key_threshold_workspace_bytes.argtypes = [ctypes.POINTER(Shape), I32]
    lib.kvq_key_threshold_workspace_bytes.restype = SZ
    lib.kvq_key_threshold.argtypes = [ctypes.POINTER(Shape), P, I32, ctypes.c_double, P, P, SZ, P]
    lib.kvq_key_threshold.restype = ctypes.c_int
    lib.kvq_fit_workspace_bytes.argtypes = []
    lib.kvq_fit_workspace_bytes.restype = SZ
    lib.kvq_fit_codebook.argtypes = [P, ctypes.c_int64, I32, I32, P, P, SZ, P]
    lib.kvq_fit_codebook.restype = ctypes.c_int
    lib.kvq_fp16_qk_matvec.argtypes = [ctypes.POINTER(Shape), P, P, P, I32, ctypes.c_float, P, I32, P]
    lib.kvq_fp16_qk_matvec.restype = ctypes.c_int
    lib.kvq_fp16_pv_matvec.argtypes = [ctypes.POINTER(Shape), P, P, P, P, P, SZ, I32, P]
    lib.kvq_fp16_pv_matvec.restype = ctypes.c_int
    lib.kvq_stream_read.argtypes = [P, SZ, P, P]
    lib.kvq_stream_read.restype = ctypes.c_int
    lib.kvq_status_string.argtypes = [ctypes.c_int]
    lib.kvq_status_string.restype = ctypes.c_char_p
    lib.kvq_abi_version.argtypes = []
    lib.kvq_abi_version.restype = ctypes.c_int
    if lib.kvq_abi_version() != ABI_VERSION:
        raise RuntimeError(f"libkvq.so ABI {lib.kvq_abi_version()} != binding ABI {ABI_VERSION}")
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != KVQ_OK:
        msg = load_library().kvq_status_string(status).decode()
        raise KvqError(fn, status, msg)


def _stream(stream=None) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


@dataclass
class CacheConfig:
    batch: int
    n_q_heads: int
    n_kv_heads: int
    max_seq: int
    k_bits: int
    v_bits: int
    n_outliers: int
    head_dim: int = 128
    rope_base: float = 10000.0
    key_outliers: int = 0  # 0: per vector (k largest |x|); 1: per channel (|x_c| > k_scale[c], at most k)

    def shape(self) -> Shape:
        return Shape(self.batch, self.n_q_heads, self.n_kv_heads, self.head_dim, self.max_seq,
                     self.k_bits, self.v_bits, self.n_outliers, self.rope_base, self.key_outliers)


def cache_sizes(cfg: CacheConfig) -> Sizes:
    """Byte size of every cache buffer (host-side, from the C library)."""
    out = Sizes()
    _check("kvq_cache_sizes", load_library().kvq_cache_sizes(ctypes.byref(cfg.shape()), ctypes.byref(out)))
    return out


def workspace_bytes(cfg: CacheConfig, max_len: int) -> int:
    return int(load_library().kvq_workspace_bytes(ctypes.byref(cfg.shape()), int(max_len)))


def _fp16_codebook(cb: torch.Tensor, device) -> torch.Tensor:
    """The codebook as fp16 bits (int16 storage); its values must be fp16 numbers."""
    c = cb.detach().to("cpu")
    h = c.to(torch.float16)
    if not torch.equal(h.to(c.dtype), c):
        raise ValueError("codebook entries must be exactly representable in fp16")
    return h.view(torch.int16).to(device).contiguous()


class KVCache:
    """Device buffers of one layer's compressed KV cache, laid out as ``include/kvq.h``
    documents; all zero-filled at creation."""

    def __init__(self, cfg: CacheConfig, k_scale: torch.Tensor, k_codebook: torch.Tensor,
                 v_codebook: torch.Tensor, device="cuda"):
        self.cfg = cfg
        sz = cache_sizes(cfg)
        u8 = dict(dtype=torch.uint8, device=device)
        i16 = dict(dtype=torch.int16, device=device)
        self.k_codes = torch.zeros(sz.k_codes, **u8)
        self.v_codes = torch.zeros(sz.v_codes, **u8)
        k = max(cfg.n_outliers, 0)
        n_slots = cfg.batch * cfg.n_kv_heads * cfg.max_seq
        self.k_out_idx = torch.zeros(n_slots * k, **u8)
        self.k_out_val = torch.zeros(n_slots * k, **i16)
        self.v_out_idx = torch.zeros(n_slots * k, **u8)
        self.v_out_val = torch.zeros(n_slots * k, **i16)
        self.v_scale = torch.zeros(n_slots, **i16)
        self.k_scale = k_scale.to(device=device, dtype=torch.float32).contiguous()
        self.k_codebook = _fp16_codebook(k_codebook, device)
        self.v_codebook = _fp16_codebook(v_codebook, device)
        assert self.k_scale.numel() == cfg.n_kv_heads * cfg.head_dim
        assert self.k_codebook.numel() == 1 << cfg.k_bits and self.v_codebook.numel() == 1 << cfg.v_bits
        self.seq_len = torch.zeros(cfg.batch, dtype=torch.int32, device=device)
        self.lengths = [0] * cfg.batch  # host mirror of seq_len
        self._desc = CacheDesc(*(_ptr(t) for t in (
            self.k_codes, self.v_codes, self.k_out_idx if k else None, self.k_out_val if k else None,
            self.v_out_idx if k else None, self.v_out_val if k else None, self.v_scale,
            self.k_scale, self.k_codebook, self.v_codebook, self.seq_len)))
        self._shape = cfg.shape()

    @property
    def nbytes(self) -> int:
        return cache_sizes(self.cfg).total

    # views in the documented layouts ------------------------------------------------
    def k_records(self):
        c = self.cfg
        return self.k_codes.view(c.batch, c.n_kv_heads, c.max_seq, c.head_dim * c.k_bits // 8)

    def v_tiles(self):
        c = self.cfg
        return self.v_codes.view(c.batch, c.n_kv_heads, c.max_seq // 64, c.head_dim * 8 * c.v_bits)

    def outliers(self, which: str):
        c = self.cfg
        idx = self.k_out_idx if which == "k" else self.v_out_idx
        val = self.k_out_val if which == "k" else self.v_out_val
        shp = (c.batch, c.n_kv_heads, c.max_seq, c.n_outliers)
        return idx.view(shp), val.view(shp)


def quantize_append(cache: KVCache, k_new: torch.Tensor, v_new: torch.Tensor, n_new=None, stream=None,
                    device_positions: bool = False):
    """kvq_quantize_append: k_new, v_new fp16 [B][n_max][Hkv][D] (keys pre-RoPE).

    device_positions=True passes no host lengths: the kernel reads each sequence's
    position from the device seq_len (graph-capturable).  The host mirror
    ``cache.lengths`` is advanced for sequences that had room."""
    cfg = cache.cfg
    assert k_new.dtype == torch.float16 and v_new.dtype == torch.float16
    assert k_new.shape == v_new.shape and k_new.dim() == 4
    assert k_new.shape[0] == cfg.batch and k_new.shape[2] == cfg.n_kv_heads and k_new.shape[3] == cfg.head_dim
    assert k_new.is_contiguous() and v_new.is_contiguous()
    n_max = k_new.shape[1]
    counts = [n_max] * cfg.batch if n_new is None else [int(x) for x in n_new]
    starts = None if device_positions else (ctypes.c_int32 * cfg.batch)(*cache.lengths)
    cnt = (ctypes.c_int32 * cfg.batch)(*counts)
    st = load_library().kvq_quantize_append(ctypes.byref(cache._shape), ctypes.byref(cache._desc),
                                            k_new.data_ptr(), v_new.data_ptr(), n_max, cnt, starts,
                                            _stream(stream))
    _check("kvq_quantize_append", st)
    cache.lengths = [a + b if a + b <= cfg.max_seq else a for a, b in zip(cache.lengths, counts)]


def qk_matvec(cache: KVCache, q: torch.Tensor, logits: torch.Tensor, sm_scale: float | None = None,
              max_len: int | None = None, stream=None):
    """kvq_qk_matvec: q [B][Hq][D] fp32/fp16 -> logits fp32 [B][Hq][max_seq]."""
    cfg = cache.cfg
    assert q.shape == (cfg.batch, cfg.n_q_heads, cfg.head_dim) and q.is_contiguous()
    assert q.dtype in (torch.float32, torch.float16)
    assert logits.dtype == torch.float32 and logits.is_contiguous()
    assert logits.numel() == cfg.batch * cfg.n_q_heads * cfg.max_seq
    sm = 1.0 / math.sqrt(cfg.head_dim) if sm_scale is None else float(sm_scale)
    ml = max(max(cache.lengths), 1) if max_len is None else int(max_len)
    st = load_library().kvq_qk_matvec(ctypes.byref(cache._shape), ctypes.byref(cache._desc), q.data_ptr(),
                                      1 if q.dtype == torch.float16 else 0, sm, logits.data_ptr(), ml,
                                      _stream(stream))
    _check("kvq_qk_matvec", st)


def pv_matvec(cache: KVCache, logits: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
              max_len: int | None = None, stream=None):
    """kvq_pv_matvec: logits fp32 [B][Hq][max_seq] -> out fp32 [B][Hq][D]."""
    cfg = cache.cfg
    assert out.dtype == torch.float32 and out.numel() == cfg.batch * cfg.n_q_heads * cfg.head_dim
    assert logits.dtype == torch.float32 and out.is_contiguous() and workspace.is_contiguous()
    ml = max(max(cache.lengths), 1) if max_len is None else int(max_len)
    st = load_library().kvq_pv_matvec(ctypes.byref(cache._shape), ctypes.byref(cache._desc),
                                      logits.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                      workspace.numel() * workspace.element_size(), ml, _stream(stream))
    _check("kvq_pv_matvec", st)


NOALLOC_SCRATCH_BYTES = 32 << 20  # KVQ_NOALLOC_SCRATCH_BYTES


def pv_matvec_noalloc(cache: KVCache, logits: torch.Tensor, out: torch.Tensor, max_len: int | None = None,
                      stream=None):
    """kvq_pv_matvec_noalloc: kvq_pv_matvec with the split partials in the library's own
    device array (no workspace; calls overlapping on one device race)."""
    cfg = cache.cfg
    assert out.dtype == torch.float32 and out.numel() == cfg.batch * cfg.n_q_heads * cfg.head_dim
    assert logits.dtype == torch.float32 and out.is_contiguous()
    ml = max(max(cache.lengths), 1) if max_len is None else int(max_len)
    st = load_library().kvq_pv_matvec_noalloc(ctypes.byref(cache._shape), ctypes.byref(cache._desc),
                                              logits.data_ptr(), out.data_ptr(), ml, _stream(stream))
    _check("kvq_pv_matvec_noalloc", st)


def fused_decode_attention(cache: KVCache, q: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                           sm_scale: float | None = None, max_len: int | None = None, stream=None) -> torch.Tensor:
    """kvq_decode_attention: q [B][Hq][D] fp32/fp16 -> out fp32 [B][Hq][D] in one pass
    (one query head per kv head, 2/3-bit keys)."""
    cfg = cache.cfg
    assert q.shape == (cfg.batch, cfg.n_q_heads, cfg.head_dim) and q.is_contiguous()
    assert q.dtype in (torch.float32, torch.float16)
    assert out.dtype == torch.float32 and out.numel() == cfg.batch * cfg.n_q_heads * cfg.head_dim
    assert out.is_contiguous() and workspace.is_contiguous()
    sm = 1.0 / math.sqrt(cfg.head_dim) if sm_scale is None else float(sm_scale)
    ml = max(max(cache.lengths), 1) if max_len is None else int(max_len)
    st = load_library().kvq_decode_attention(ctypes.byref(cache._shape), ctypes.byref(cache._desc), q.data_ptr(),
                                             1 if q.dtype == torch.float16 else 0, sm, out.data_ptr(),
                                             workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                             ml, _stream(stream))
    _check("kvq_decode_attention", st)
    return out


class DecodeBuffers:
    """Logits, output and split workspace for decode steps over ``cache``."""

    def __init__(self, cache: KVCache, device="cuda"):
        cfg = cache.cfg
        self.logits = torch.empty(cfg.batch, cfg.n_q_heads, cfg.max_seq, dtype=torch.float32, device=device)
        self.out = torch.empty(cfg.batch, cfg.n_q_heads, cfg.head_dim, dtype=torch.float32, device=device)
        self.workspace = torch.empty(workspace_bytes(cfg, cfg.max_seq) // 4, dtype=torch.float32, device=device)


def decode_attention(cache: KVCache, q: torch.Tensor, bufs: DecodeBuffers, sm_scale=None, max_len=None,
                     stream=None) -> torch.Tensor:
    """q.K^T then softmax.V over the compressed cache; returns bufs.out [B][Hq][D]."""
    qk_matvec(cache, q, bufs.logits, sm_scale, max_len, stream)
    pv_matvec(cache, bufs.logits, bufs.out, bufs.workspace, max_len, stream)
    return bufs.out


class Fp16Cache:
    """A plain fp16 KV cache (the baseline the compressed kernels are compared with):
    k, v fp16 [B][Hkv][max_seq][D], keys stored after the rotary embedding, and the device
    lengths seq_len int32 [B]."""

    def __init__(self, cfg: CacheConfig, device="cuda"):
        self.cfg = cfg
        shape = (cfg.batch, cfg.n_kv_heads, cfg.max_seq, cfg.head_dim)
        self.k = torch.zeros(shape, dtype=torch.float16, device=device)
        self.v = torch.zeros(shape, dtype=torch.float16, device=device)
        self.seq_len = torch.zeros(cfg.batch, dtype=torch.int32, device=device)
        self.lengths = [0] * cfg.batch
        self._shape = cfg.shape()

    def set_lengths(self, lengths):
        self.lengths = [int(x) for x in lengths]
        self.seq_len.copy_(torch.tensor(self.lengths, dtype=torch.int32))

    @property
    def nbytes(self) -> int:
        return self.k.numel() * 2 + self.v.numel() * 2


def fp16_qk_matvec(cache: Fp16Cache, q: torch.Tensor, logits: torch.Tensor, sm_scale: float | None = None,
                   max_len: int | None = None, stream=None):
    """kvq_fp16_qk_matvec: q [B][Hq][D] fp32/fp16 -> logits fp32 [B][Hq][max_seq]."""
    cfg = cache.cfg
    assert q.shape == (cfg.batch, cfg.n_q_heads, cfg.head_dim) and q.is_contiguous()
    assert q.dtype in (torch.float32, torch.float16)
    assert logits.dtype == torch.float32 and logits.is_contiguous()
    assert logits.numel() == cfg.batch * cfg.n_q_heads * cfg.max_seq
    sm = 1.0 / math.sqrt(cfg.head_dim) if sm_scale is None else float(sm_scale)
    ml = max(max(cache.lengths), 1) if max_len is None else int(max_len)
    st = load_library().kvq_fp16_qk_matvec(ctypes.byref(cache._shape), cache.k.data_ptr(), cache.seq_len.data_ptr(),
                                           q.data_ptr(), 1 if q.dtype == torch.float16 else 0, sm,
                                           logits.data_ptr(), ml, _stream(stream))
    _check("kvq_fp16_qk_matvec", st)


def fp16_pv_matvec(cache: Fp16Cache, logits: torch.Tensor, out: torch.Tensor, workspace: torch.Tensor,
                   max_len: int | None = None, stream=None):
    """kvq_fp16_pv_matvec: logits fp32 [B][Hq][max_seq] -> out fp32 [B][Hq][D]."""
    cfg = cache.cfg
    assert out.dtype == torch.float32 and out.numel() == cfg.batch * cfg.n_q_heads * cfg.head_dim
    assert logits.dtype == torch.float32 and out.is_contiguous() and workspace.is_contiguous()
    ml = max(max(cache.lengths), 1) if max_len is None else int(max_len)
    st = load_library().kvq_fp16_pv_matvec(ctypes.byref(cache._shape), cache.v.data_ptr(), cache.seq_len.data_ptr(),
                                           logits.data_ptr(), out.data_ptr(), workspace.data_ptr(),
                                           workspace.numel() * workspace.element_size(), ml, _stream(stream))
    _check("kvq_fp16_pv_matvec", st)


def fp16_decode_attention(cache: Fp16Cache, q: torch.Tensor, bufs: DecodeBuffers, sm_scale=None, max_len=None,
                          stream=None) -> torch.Tensor:
    """q.K^T then softmax.V over the fp16 cache; returns bufs.out [B][Hq][D]."""
    fp16_qk_matvec(cache, q, bufs.logits, sm_scale, max_len, stream)
    fp16_pv_matvec(cache, bufs.logits, bufs.out, bufs.workspace, max_len, stream)
    return bufs.out


def fit_codebook(u: torch.Tensor, bits: int, iters: int, out: torch.Tensor | None = None,
                 workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_fit_codebook: float32 device activations (already divided by their scale) ->
    fp16 codebook of 2^bits entries (a float16 tensor)."""
    assert u.dtype == torch.float32 and u.is_contiguous()
    lib = load_library()
    if out is None:
        out = torch.empty(1 << bits, dtype=torch.float16, device=u.device)
    if workspace is None:
        workspace = torch.empty(int(lib.kvq_fit_workspace_bytes()), dtype=torch.uint8, device=u.device)
    st = lib.kvq_fit_codebook(u.data_ptr() if u.numel() else None, u.numel(), int(bits), int(iters), out.data_ptr(),
                              workspace.data_ptr(), workspace.numel() * workspace.element_size(), _stream(stream))
    _check("kvq_fit_codebook", st)
    return out


def key_scale(cfg: CacheConfig, keys: torch.Tensor, exclude_outliers: bool = False,
              out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_key_scale: calibration keys fp16 [B][n][Hkv][D] -> float32 [Hkv][D] per-channel
    scale (max |x|, over each vector's dense part with exclude_outliers)."""
    assert keys.dtype == torch.float16 and keys.is_contiguous() and keys.dim() == 4
    assert keys.shape[0] == cfg.batch and keys.shape[2] == cfg.n_kv_heads and keys.shape[3] == cfg.head_dim
    if out is None:
        out = torch.empty(cfg.n_kv_heads, cfg.head_dim, dtype=torch.float32, device=keys.device)
    st = load_library().kvq_key_scale(ctypes.byref(cfg.shape()), keys.data_ptr() if keys.numel() else None,
                                      keys.shape[1], 1 if exclude_outliers else 0, out.data_ptr(), _stream(stream))
    _check("kvq_key_scale", st)
    return out


def key_threshold_workspace_bytes(cfg: CacheConfig, n_tokens: int) -> int:
    return int(load_library().kvq_key_threshold_workspace_bytes(ctypes.byref(cfg.shape()), int(n_tokens)))


def key_threshold(cfg: CacheConfig, keys: torch.Tensor, outlier_frac: float, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """kvq_key_threshold: calibration keys fp16 [B][n][Hkv][D] -> float32 [Hkv][D] per-channel
    threshold for the per-channel outlier rule (the (m+1)-th largest |x_c|, m = floor(f N))."""
    assert keys.dtype == torch.float16 and keys.is_contiguous() and keys.dim() == 4
    assert keys.shape[0] == cfg.batch and keys.shape[2] == cfg.n_kv_heads and keys.shape[3] == cfg.head_dim
    if out is None:
        out = torch.empty(cfg.n_kv_heads, cfg.head_dim, dtype=torch.float32, device=keys.device)
    need = key_threshold_workspace_bytes(cfg, keys.shape[1])
    if workspace is None and need > 0:
        workspace = torch.empty((need + 3) // 4, dtype=torch.int32, device=keys.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    st = load_library().kvq_key_threshold(ctypes.byref(cfg.shape()), keys.data_ptr() if keys.numel() else None,
                                          keys.shape[1], float(outlier_frac), out.data_ptr(), ws_ptr, ws_bytes,
                                          _stream(stream))
    _check("kvq_key_threshold", st)
    return out


def stream_read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """kvq_stream_read: read every byte of a contiguous device tensor once (measurement)."""
    assert buf.is_contiguous() and sink.dtype == torch.int32 and sink.numel() >= 1
    nbytes = buf.numel() * buf.element_size()
    _check("kvq_stream_read", load_library().kvq_stream_read(buf.data_ptr() if nbytes else None, nbytes,
                                                             sink.data_ptr(), _stream(stream)))
