// Kernel argument blocks and launchers shared between the kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kMaxBatchPerLaunch = 128;  // per-sequence starts/counts travel in kernel args
constexpr int kQkTokensPerBlock = 1024;  // 4 waves x 4 tiles of 64 tokens
constexpr int kPvChunk = 1024;           // tokens per split of the softmax.V pass
constexpr int kMaxSeqLimit = (1 << 24) - 64;  // lengths live in the low 24 bits of seq_len
constexpr int kMaxKvHeadsDevicePos = 127;     // arrival counter width of a device-positioned append

struct AppendArgs {
  int32_t n_kv_heads, max_seq, n_outliers, n_max, n_batch;  // n_batch: sequences in this launch
  int32_t device_positions;  // 1: start positions come from seq_len on the device
  int32_t key_per_channel;   // 1: key outliers by the per-channel rule (|x_c| > s_c, at most k)
  const uint16_t* k_new;  // [n_batch][n_max][Hkv][D] (already offset to the first sequence)
  const uint16_t* v_new;
  uint8_t* k_codes;  // cache buffers offset to the first sequence of this launch
  uint8_t* v_codes;
  uint8_t* k_idx;
  uint16_t* k_val;
  uint8_t* v_idx;
  uint16_t* v_val;
  uint16_t* v_scale;
  const float* k_scale;
  const uint16_t* k_cb;  // fp16 codebooks
  const uint16_t* v_cb;
  int32_t* seq_len;  // offset to the first sequence of this launch
  int32_t start[kMaxBatchPerLaunch];  // host positions (unused with device_positions)
  int32_t count[kMaxBatchPerLaunch];
};

struct QkArgs {
  int32_t n_q_heads, n_kv_heads, max_seq, n_outliers, max_len, q_is_fp16;
  int32_t tiles_per_wave;  // set by the launcher
  float sm_scale;
  double theta_rev[kHalf];  // theta_i / 2pi for the 64 rotary pairs, from the host in float64
  float th_hi[kHalf];       // theta_rev rounded to 15 significant bits: tau * th_hi is exact for tau < 512
  float th_lo[kHalf];       // theta_rev - th_hi
  const void* q;
  const uint8_t* k_codes;
  const uint8_t* k_idx;
  const uint16_t* k_val;
  const float* k_scale;
  const uint16_t* k_cb;  // fp16 codebook
  const int32_t* seq_len;
  float* logits;
};

struct PvArgs {
  int32_t n_q_heads, n_kv_heads, max_seq, n_outliers, max_len;
  int32_t tiles_per_block, n_parts;  // set by the launcher: split of each stream into parts
  const float* logits;
  const uint8_t* v_codes;
  const uint8_t* v_idx;
  const uint16_t* v_val;
  const uint16_t* v_scale;
  const uint16_t* v_cb;  // fp16 codebook
  const int32_t* seq_len;
  float* partial;  // [B][Hq][n_parts][D + 2]: o[D], m, l
  float* out;      // [B][Hq][D]
};

struct Fp16Args {
  int32_t n_q_heads, n_kv_heads, max_seq, max_len, q_is_fp16;
  int32_t tokens_per_block;          // set by the q.K^T launcher
  int32_t tiles_per_block, n_parts;  // set by the softmax.V launcher
  float sm_scale;
  const void* q;
  const uint16_t* k;  // fp16 [B][Hkv][S][D], keys after the rotary embedding
  const uint16_t* v;  // fp16 [B][Hkv][S][D]
  const int32_t* seq_len;
  float* logits;   // [B][Hq][S]
  float* partial;  // [B][Hq][n_parts][D + 2], as PvArgs
  float* out;      // [B][Hq][D]
};

// Compute units of the current device (queried once per device, then cached).
int device_cu_count();

// Resident blocks of `kernel` per CU at `threads` per block (queried once, then cached by
// the caller), at least 1.
inline int blocks_per_cu(const void* kernel, int threads) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

hipError_t launch_append(int k_bits, int v_bits, const AppendArgs& a, hipStream_t s);
hipError_t launch_qk(int k_bits, int group, int batch, const QkArgs& a, hipStream_t s);
hipError_t launch_qk_lut(int k_bits, int batch, const QkArgs& a, hipStream_t s);
// 2/3-bit keys, 2, 4 or 8 query heads per kv head: the head contraction on the matrix cores.
hipError_t launch_qk_mfma(int k_bits, int group, int batch, const QkArgs& a, hipStream_t s);
hipError_t launch_pv(int v_bits, int group, int batch, const PvArgs& a, hipStream_t s);
// Log-sum-exp merge of the (o, m, l) partials in a.partial into a.out (used by launch_pv).
hipError_t launch_pv_combine(int batch, const PvArgs& a, hipStream_t s);
// Single-pass q.K^T + softmax.V for one query head per kv head, 2/3-bit keys: QkArgs
// supplies the key side (logits unused), PvArgs the value side and the workspace.
hipError_t launch_fused(int k_bits, int v_bits, int batch, const QkArgs& a, const PvArgs& p, hipStream_t s);
hipError_t launch_fp16_qk(int group, int batch, const Fp16Args& a, hipStream_t s);
// Per-channel key scale (max |x| over calibration keys, optionally their dense parts).
hipError_t launch_key_scale(const uint16_t* keys, int batch, int n_tokens, int n_kv_heads, int k, float* out,
                            hipStream_t s);
// Per-channel key threshold (the (budget+1)-th largest |x| per channel over calibration
// keys, 0 when budget >= batch * n_tokens): workspace size and launcher.
size_t key_threshold_workspace_bytes(int batch, int n_tokens, int n_kv_heads);
hipError_t launch_key_threshold(const uint16_t* keys, int batch, int n_tokens, int n_kv_heads, long long budget,
                                float* out, void* workspace, hipStream_t s);
// Codebook fitting (k-means over normalised activations): workspace size and launcher.
size_t fit_workspace_bytes();
hipError_t launch_fit_codebook(int bits, const float* u, long long n, int iters, uint16_t* out, void* workspace,
                               hipStream_t s);
hipError_t launch_fp16_pv(int group, int batch, const Fp16Args& a, hipStream_t s);
// Streaming-read probe: reads bytes / 16 16-byte words of buf once.
hipError_t launch_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

}  // namespace kvq
