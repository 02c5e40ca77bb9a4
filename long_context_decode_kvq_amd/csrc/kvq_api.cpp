// C ABI of libkvq.so: argument validation, sizing, and kernel dispatch.
// Every check that the host can make is made before anything is enqueued.
#include "../../include/kvq.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstring>
#include <mutex>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace {

bool bits_ok(int b) { return b == 2 || b == 3 || b == 4; }
bool group_ok(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

int check_shape(const kvq_shape* s) {
  if (!s) return KVQ_ERR_INVALID;
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->max_seq < 1) return KVQ_ERR_INVALID;
  if (s->max_seq % kvq::kTile != 0 || s->max_seq > kvq::kMaxSeqLimit) return KVQ_ERR_INVALID;
  if (s->n_q_heads % s->n_kv_heads != 0) return KVQ_ERR_INVALID;
  if (s->n_outliers < 0) return KVQ_ERR_INVALID;
  if (!(s->rope_base > 1.0f) || !std::isfinite(s->rope_base)) return KVQ_ERR_INVALID;
  if (s->head_dim != kvq::kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (s->n_outliers > s->head_dim) return KVQ_ERR_INVALID;
  if (!bits_ok(s->k_bits) || !bits_ok(s->v_bits)) return KVQ_ERR_UNSUPPORTED;
  if (!group_ok(s->n_q_heads / s->n_kv_heads)) return KVQ_ERR_UNSUPPORTED;
  if (s->key_outliers != 0 && s->key_outliers != 1) return KVQ_ERR_INVALID;
  return KVQ_OK;
}

int check_cache_common(const kvq_shape* s, const kvq_cache* c) {
  if (!c) return KVQ_ERR_INVALID;
  if (!c->seq_len) return KVQ_ERR_INVALID;
  if (s->n_outliers > 0) {
    if (!c->k_out_idx || !c->k_out_val || !c->v_out_idx || !c->v_out_val) return KVQ_ERR_INVALID;
  }
  return KVQ_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? KVQ_OK : KVQ_ERR_HIP; }

// Split partials of kvq_pv_matvec_noalloc: a device array of the library, so that the call
// allocates nothing.  Each device holds its own copy at its own address, found once per
// device with hipGetSymbolAddress (host code never passes the array's name itself).
__device__ __align__(256) unsigned char scratch[KVQ_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::atomic<void*> scratch_ptr[kMaxDevices];
std::mutex scratch_mu;

// The current device's address of `scratch`.
int scratch_for_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return KVQ_ERR_HIP;
  void* p = scratch_ptr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(scratch_mu);
    p = scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return KVQ_ERR_HIP;
      scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return KVQ_OK;
}

size_t n_chunks_for(int32_t max_len) { return (static_cast<size_t>(max_len) + kvq::kPvChunk - 1) / kvq::kPvChunk; }

kvq::QkArgs make_qk_args(const kvq_shape* s, const kvq_cache* c, const void* q, int32_t q_is_fp16, float sm_scale,
                         float* logits, int32_t max_len) {
  kvq::QkArgs a;
  std::memset(&a, 0, sizeof(a));
  a.n_q_heads = s->n_q_heads;
  a.n_kv_heads = s->n_kv_heads;
  a.max_seq = s->max_seq;
  a.n_outliers = s->n_outliers;
  a.max_len = max_len;
  a.q_is_fp16 = q_is_fp16;
  a.sm_scale = sm_scale;
  // theta_i = base^(-2i/D); stored in revolutions so that the kernels reduce phases exactly
  const double theta_log2 = std::log2(static_cast<double>(s->rope_base)) * 2.0 / s->head_dim;
  for (int i = 0; i < kvq::kHalf; ++i) {
    a.theta_rev[i] = std::exp2(-i * theta_log2) / (2.0 * M_PI);
    int e = 0;
    const double m = std::frexp(a.theta_rev[i], &e);  // theta_rev = m 2^e, m in [0.5, 1)
    a.th_hi[i] = static_cast<float>(std::ldexp(std::nearbyint(std::ldexp(m, 15)), e - 15));
    a.th_lo[i] = static_cast<float>(a.theta_rev[i] - static_cast<double>(a.th_hi[i]));
  }
  a.q = q;
  a.k_codes = c->k_codes;
  a.k_idx = c->k_out_idx;
  a.k_val = c->k_out_val;
  a.k_scale = c->k_scale;
  a.k_cb = c->k_codebook;
  a.seq_len = c->seq_len;
  a.logits = logits;
  return a;
}

kvq::PvArgs make_pv_args(const kvq_shape* s, const kvq_cache* c, const float* logits, float* out, void* workspace,
                         int32_t max_len) {
  kvq::PvArgs a;
  std::memset(&a, 0, sizeof(a));
  a.n_q_heads = s->n_q_heads;
  a.n_kv_heads = s->n_kv_heads;
  a.max_seq = s->max_seq;
  a.n_outliers = s->n_outliers;
  a.max_len = max_len;
  a.logits = logits;
  a.v_codes = c->v_codes;
  a.v_idx = c->v_out_idx;
  a.v_val = c->v_out_val;
  a.v_scale = c->v_scale;
  a.v_cb = c->v_codebook;
  a.seq_len = c->seq_len;
  a.partial = static_cast<float*>(workspace);
  a.out = out;
  return a;
}

}  // namespace

namespace kvq {

int device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace kvq

extern "C" {

int kvq_abi_version(void) { return KVQ_ABI_VERSION; }

const char* kvq_status_string(int status) {
  switch (status) {
    case KVQ_OK: return "ok";
    case KVQ_ERR_INVALID: return "invalid argument";
    case KVQ_ERR_UNSUPPORTED: return "unsupported shape or bit width";
    case KVQ_ERR_CAPACITY: return "append exceeds cache capacity";
    case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
    case KVQ_ERR_HIP: return "HIP launch or runtime error";
    default: return "unknown status";
  }
}

int kvq_cache_sizes(const kvq_shape* s, kvq_sizes* out) {
  int st = check_shape(s);
  if (st != KVQ_OK) return st;
  if (!out) return KVQ_ERR_INVALID;
  const size_t streams = static_cast<size_t>(s->batch) * s->n_kv_heads;
  const size_t slots = streams * s->max_seq;
  const size_t D = s->head_dim;
  kvq_sizes z;
  std::memset(&z, 0, sizeof(z));
  z.k_codes = slots * D * s->k_bits / 8;
  z.v_codes = slots * D * s->v_bits / 8;
  z.k_out_idx = slots * s->n_outliers;
  z.k_out_val = slots * s->n_outliers * 2;
  z.v_out_idx = slots * s->n_outliers;
  z.v_out_val = slots * s->n_outliers * 2;
  z.v_scale = slots * 2;
  z.k_scale = static_cast<size_t>(s->n_kv_heads) * D * 4;
  z.k_codebook = (static_cast<size_t>(1) << s->k_bits) * 2;
  z.v_codebook = (static_cast<size_t>(1) << s->v_bits) * 2;
  z.seq_len = static_cast<size_t>(s->batch) * 4;
  z.total = z.k_codes + z.v_codes + z.k_out_idx + z.k_out_val + z.v_out_idx + z.v_out_val + z.v_scale +
            z.k_scale + z.k_codebook + z.v_codebook + z.seq_len;
  *out = z;
  return KVQ_OK;
}

size_t kvq_workspace_bytes(const kvq_shape* s, int32_t max_len) {
  if (check_shape(s) != KVQ_OK || max_len < 1) return 0;
  return static_cast<size_t>(s->batch) * s->n_q_heads * n_chunks_for(max_len) * (kvq::kHeadDim + 2) * sizeof(float);
}

int kvq_quantize_append(const kvq_shape* s, const kvq_cache* c, const uint16_t* k_new, const uint16_t* v_new,
                        int32_t n_max, const int32_t* n_new_host, const int32_t* seq_len_host,
                        hipStream_t stream) {
  int st = check_shape(s);
  if (st != KVQ_OK) return st;
  st = check_cache_common(s, c);
  if (st != KVQ_OK) return st;
  if (!c->k_codes || !c->v_codes || !c->v_scale || !c->k_scale || !c->k_codebook || !c->v_codebook)
    return KVQ_ERR_INVALID;
  if (n_max < 0) return KVQ_ERR_INVALID;
  if (n_max > 0 && (!k_new || !v_new)) return KVQ_ERR_INVALID;
  const bool device_positions = seq_len_host == nullptr;
  if (device_positions && s->n_kv_heads > kvq::kMaxKvHeadsDevicePos) return KVQ_ERR_UNSUPPORTED;
  for (int b = 0; b < s->batch; ++b) {
    const int32_t n = n_new_host ? n_new_host[b] : n_max;
    if (n < 0 || n > n_max) return KVQ_ERR_INVALID;
    if (!device_positions) {
      if (seq_len_host[b] < 0) return KVQ_ERR_INVALID;
      if (static_cast<int64_t>(seq_len_host[b]) + n > s->max_seq) return KVQ_ERR_CAPACITY;
    }
  }
  const size_t H = s->n_kv_heads, S = s->max_seq, D = s->head_dim, k = s->n_outliers;
  for (int b0 = 0; b0 < s->batch; b0 += kvq::kMaxBatchPerLaunch) {
    const int nb = s->batch - b0 < kvq::kMaxBatchPerLaunch ? s->batch - b0 : kvq::kMaxBatchPerLaunch;
    kvq::AppendArgs a;
    std::memset(&a, 0, sizeof(a));
    const size_t slot0 = static_cast<size_t>(b0) * H * S;
    a.n_kv_heads = s->n_kv_heads;
    a.max_seq = s->max_seq;
    a.n_outliers = s->n_outliers;
    a.n_max = n_max;
    a.n_batch = nb;
    a.device_positions = device_positions ? 1 : 0;
    a.key_per_channel = s->key_outliers;
    a.k_new = k_new ? k_new + static_cast<size_t>(b0) * n_max * H * D : nullptr;
    a.v_new = v_new ? v_new + static_cast<size_t>(b0) * n_max * H * D : nullptr;
    a.k_codes = c->k_codes + slot0 * D * s->k_bits / 8;
    a.v_codes = c->v_codes + slot0 * D * s->v_bits / 8;
    a.k_idx = c->k_out_idx ? c->k_out_idx + slot0 * k : nullptr;
    a.k_val = c->k_out_val ? c->k_out_val + slot0 * k : nullptr;
    a.v_idx = c->v_out_idx ? c->v_out_idx + slot0 * k : nullptr;
    a.v_val = c->v_out_val ? c->v_out_val + slot0 * k : nullptr;
    a.v_scale = c->v_scale + slot0;
    a.k_scale = c->k_scale;
    a.k_cb = c->k_codebook;
    a.v_cb = c->v_codebook;
    a.seq_len = c->seq_len + b0;
    for (int b = 0; b < nb; ++b) {
      a.start[b] = device_positions ? 0 : seq_len_host[b0 + b];
      a.count[b] = n_new_host ? n_new_host[b0 + b] : n_max;
    }
    hipError_t e = kvq::launch_append(s->k_bits, s->v_bits, a, stream);
    if (e != hipSuccess) return KVQ_ERR_HIP;
  }
  return KVQ_OK;
}

int kvq_qk_matvec(const kvq_shape* s, const kvq_cache* c, const void* q, int32_t q_is_fp16, float sm_scale,
                  float* logits, int32_t max_len, hipStream_t stream) {
  int st = check_shape(s);
  if (st != KVQ_OK) return st;
  st = check_cache_common(s, c);
  if (st != KVQ_OK) return st;
  if (!c->k_codes || !c->k_scale || !c->k_codebook || !q || !logits) return KVQ_ERR_INVALID;
  if (q_is_fp16 != 0 && q_is_fp16 != 1) return KVQ_ERR_INVALID;
  if (max_len < 1 || max_len > s->max_seq || !std::isfinite(sm_scale)) return KVQ_ERR_INVALID;
  const kvq::QkArgs a = make_qk_args(s, c, q, q_is_fp16, sm_scale, logits, max_len);
  // One query head per kv head: the table kernel (qk_lut; 4-bit keys with separable rows);
  // grouped heads: the matrix-core table kernel (qk_mfma) for 2/3-bit keys, the general
  // kernel (qk) for 4-bit keys.
  if (s->n_q_heads == s->n_kv_heads) return hip_status(kvq::launch_qk_lut(s->k_bits, s->batch, a, stream));
  if (s->k_bits <= 3) return hip_status(kvq::launch_qk_mfma(s->k_bits, s->n_q_heads / s->n_kv_heads, s->batch, a, stream));
  return hip_status(kvq::launch_qk(s->k_bits, s->n_q_heads / s->n_kv_heads, s->batch, a, stream));
}

int kvq_pv_matvec(const kvq_shape* s, const kvq_cache* c, const float* logits, float* out, void* workspace,
                  size_t workspace_bytes, int32_t max_len, hipStream_t stream) {
  int st = check_shape(s);
  if (st != KVQ_OK) return st;
  st = check_cache_common(s, c);
  if (st != KVQ_OK) return st;
  if (!c->v_codes || !c->v_scale || !c->v_codebook || !logits || !out) return KVQ_ERR_INVALID;
  if (max_len < 1 || max_len > s->max_seq) return KVQ_ERR_INVALID;
  if (!workspace || workspace_bytes < kvq_workspace_bytes(s, max_len)) return KVQ_ERR_WORKSPACE;
  const kvq::PvArgs a = make_pv_args(s, c, logits, out, workspace, max_len);
  return hip_status(kvq::launch_pv(s->v_bits, s->n_q_heads / s->n_kv_heads, s->batch, a, stream));
}

int kvq_pv_matvec_noalloc(const kvq_shape* s, const kvq_cache* c, const float* logits, float* out, int32_t max_len,
                          hipStream_t stream) {
  int st = check_shape(s);
  if (st != KVQ_OK) return st;
  st = check_cache_common(s, c);
  if (st != KVQ_OK) return st;
  if (!c->v_codes || !c->v_scale || !c->v_codebook || !logits || !out) return KVQ_ERR_INVALID;
  if (max_len < 1 || max_len > s->max_seq) return KVQ_ERR_INVALID;
  if (kvq_workspace_bytes(s, max_len) > KVQ_NOALLOC_SCRATCH_BYTES) return KVQ_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_for_current_device(&ws);
  if (st != KVQ_OK) return st;
  const kvq::PvArgs a = make_pv_args(s, c, logits, out, ws, max_len);
  return hip_status(kvq::launch_pv(s->v_bits, s->n_q_heads / s->n_kv_heads, s->batch, a, stream));
}

int kvq_decode_attention(const kvq_shape* s, const kvq_cache* c, const void* q, int32_t q_is_fp16, float sm_scale,
                         float* out, void* workspace, size_t workspace_bytes, int32_t max_len, hipStream_t stream) {
  int st = check_shape(s);
  if (st != KVQ_OK) return st;
  st = check_cache_common(s, c);
  if (st != KVQ_OK) return st;
  if (!c->k_codes || !c->k_scale || !c->k_codebook || !c->v_codes || !c->v_scale || !c->v_codebook || !q || !out)
    return KVQ_ERR_INVALID;
  if (q_is_fp16 != 0 && q_is_fp16 != 1) return KVQ_ERR_INVALID;
  if (max_len < 1 || max_len > s->max_seq || !std::isfinite(sm_scale)) return KVQ_ERR_INVALID;
  if (s->n_q_heads != s->n_kv_heads || s->k_bits > 3) return KVQ_ERR_UNSUPPORTED;
  if (!workspace || workspace_bytes < kvq_workspace_bytes(s, max_len)) return KVQ_ERR_WORKSPACE;
  const kvq::QkArgs a = make_qk_args(s, c, q, q_is_fp16, sm_scale, nullptr, max_len);
  const kvq::PvArgs p = make_pv_args(s, c, nullptr, out, workspace, max_len);
  return hip_status(kvq::launch_fused(s->k_bits, s->v_bits, s->batch, a, p, stream));
}

// ---- calibration ----------------------------------------------------------------------

int kvq_key_scale(const kvq_shape* s, const uint16_t* keys, int32_t n_tokens, int32_t exclude_outliers,
                  float* k_scale_out, hipStream_t stream) {
  int st = check_shape(s);
  if (st != KVQ_OK) return st;
  if (n_tokens < 0 || !k_scale_out || (n_tokens > 0 && !keys)) return KVQ_ERR_INVALID;
  if (exclude_outliers != 0 && exclude_outliers != 1) return KVQ_ERR_INVALID;
  return hip_status(kvq::launch_key_scale(keys, s->batch, n_tokens, s->n_kv_heads,
                                          exclude_outliers ? s->n_outliers : 0, k_scale_out, stream));
}

size_t kvq_key_threshold_workspace_bytes(const kvq_shape* s, int32_t n_tokens) {
  if (check_shape(s) != KVQ_OK || n_tokens < 0) return 0;
  if (static_cast<long long>(s->batch) * n_tokens >= (1LL << 31)) return 0;
  return kvq::key_threshold_workspace_bytes(s->batch, n_tokens, s->n_kv_heads);
}

int kvq_key_threshold(const kvq_shape* s, const uint16_t* keys, int32_t n_tokens, double outlier_frac,
                      float* k_scale_out, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  int st = check_shape(s);
  if (st != KVQ_OK) return st;
  if (n_tokens < 0 || !k_scale_out || (n_tokens > 0 && !keys)) return KVQ_ERR_INVALID;
  if (!(outlier_frac >= 0.0 && outlier_frac <= 1.0)) return KVQ_ERR_INVALID;  // NaN fails too
  const long long n_vec = static_cast<long long>(s->batch) * n_tokens;
  if (n_vec >= (1LL << 31)) return KVQ_ERR_INVALID;
  const size_t need = kvq::key_threshold_workspace_bytes(s->batch, n_tokens, s->n_kv_heads);
  if (need > 0 && (!workspace || workspace_bytes < need)) return KVQ_ERR_WORKSPACE;
  // the exceed budget floor(f N), the product formed in double precision
  const long long budget = static_cast<long long>(std::floor(outlier_frac * static_cast<double>(n_vec)));
  return hip_status(kvq::launch_key_threshold(keys, s->batch, n_tokens, s->n_kv_heads, budget, k_scale_out,
                                              workspace, stream));
}

// ---- measurement ----------------------------------------------------------------------

int kvq_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream) {
  if (bytes % 16 != 0 || (bytes > 0 && (!buf || !sink))) return KVQ_ERR_INVALID;
  if (reinterpret_cast<uintptr_t>(buf) % 16 != 0) return KVQ_ERR_INVALID;
  return hip_status(kvq::launch_stream_read(buf, bytes, sink, stream));
}

// ---- codebook fitting ---------------------------------------------------------------

size_t kvq_fit_workspace_bytes(void) { return kvq::fit_workspace_bytes(); }

int kvq_fit_codebook(const float* u, int64_t n, int32_t bits, int32_t iters, uint16_t* codebook_out, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  if (!bits_ok(bits)) return KVQ_ERR_UNSUPPORTED;
  if (n < 0 || n >= (static_cast<int64_t>(1) << 33) || iters < 0 || !codebook_out) return KVQ_ERR_INVALID;
  if (n > 0 && !u) return KVQ_ERR_INVALID;
  if (!workspace || workspace_bytes < kvq::fit_workspace_bytes()) return KVQ_ERR_WORKSPACE;
  return hip_status(kvq::launch_fit_codebook(bits, u, n, iters, codebook_out, workspace, stream));
}

// ---- uncompressed fp16 baseline --------------------------------------------------------

static int check_fp16_shape(const kvq_shape* s) {
  if (!s) return KVQ_ERR_INVALID;
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1 || s->max_seq < 1) return KVQ_ERR_INVALID;
  if (s->max_seq % kvq::kTile != 0 || s->max_seq > kvq::kMaxSeqLimit) return KVQ_ERR_INVALID;
  if (s->n_q_heads % s->n_kv_heads != 0) return KVQ_ERR_INVALID;
  if (s->head_dim != kvq::kHeadDim) return KVQ_ERR_UNSUPPORTED;
  if (!group_ok(s->n_q_heads / s->n_kv_heads)) return KVQ_ERR_UNSUPPORTED;
  return KVQ_OK;
}

int kvq_fp16_qk_matvec(const kvq_shape* s, const uint16_t* k_fp16, const int32_t* seq_len, const void* q,
                       int32_t q_is_fp16, float sm_scale, float* logits, int32_t max_len, hipStream_t stream) {
  int st = check_fp16_shape(s);
  if (st != KVQ_OK) return st;
  if (!k_fp16 || !seq_len || !q || !logits) return KVQ_ERR_INVALID;
  if (q_is_fp16 != 0 && q_is_fp16 != 1) return KVQ_ERR_INVALID;
  if (max_len < 1 || max_len > s->max_seq || !std::isfinite(sm_scale)) return KVQ_ERR_INVALID;
  kvq::Fp16Args a;
  std::memset(&a, 0, sizeof(a));
  a.n_q_heads = s->n_q_heads;
  a.n_kv_heads = s->n_kv_heads;
  a.max_seq = s->max_seq;
  a.max_len = max_len;
  a.q_is_fp16 = q_is_fp16;
  a.sm_scale = sm_scale;
  a.q = q;
  a.k = k_fp16;
  a.seq_len = seq_len;
  a.logits = logits;
  return hip_status(kvq::launch_fp16_qk(s->n_q_heads / s->n_kv_heads, s->batch, a, stream));
}

int kvq_fp16_pv_matvec(const kvq_shape* s, const uint16_t* v_fp16, const int32_t* seq_len, const float* logits,
                       float* out, void* workspace, size_t workspace_bytes, int32_t max_len, hipStream_t stream) {
  int st = check_fp16_shape(s);
  if (st != KVQ_OK) return st;
  if (!v_fp16 || !seq_len || !logits || !out) return KVQ_ERR_INVALID;
  if (max_len < 1 || max_len > s->max_seq) return KVQ_ERR_INVALID;
  const size_t need = static_cast<size_t>(s->batch) * s->n_q_heads * n_chunks_for(max_len) * (kvq::kHeadDim + 2) * sizeof(float);
  if (!workspace || workspace_bytes < need) return KVQ_ERR_WORKSPACE;
  kvq::Fp16Args a;
  std::memset(&a, 0, sizeof(a));
  a.n_q_heads = s->n_q_heads;
  a.n_kv_heads = s->n_kv_heads;
  a.max_seq = s->max_seq;
  a.max_len = max_len;
  a.v = v_fp16;
  a.seq_len = seq_len;
  a.logits = const_cast<float*>(logits);
  a.partial = static_cast<float*>(workspace);
  a.out = out;
  return hip_status(kvq::launch_fp16_pv(s->n_q_heads / s->n_kv_heads, s->batch, a, stream));
}

}  // extern "C"
