/*
 * kvq.h - C ABI of the quantized-KV decode-attention library (libkvq.so), gfx950.
 *
 * The library implements the decode hot path of KVQuant ("KVQuant: Towards 10 Million
 * Context Length LLM Inference with KV Cache Quantization", study.space summary,
 * abstract paragraph; and the phantomic12 paper note, "Four components" paragraph):
 *   (i)   keys are quantized per channel,
 *   (ii)  keys are quantized before the rotary embedding, which is applied after
 *         dequantization at each cached token's own position,
 *   (iii) every entry is mapped to the nearest entry of a sorted per-layer
 *         non-uniform codebook of 2^b values in [-1, 1],
 *   (iv)  each (token, kv head) vector keeps its k largest-magnitude entries aside in
 *         fp16 (dense-and-sparse split), the rest is quantized.
 * Decode is memory-bound (summary page, same paragraph): every kernel here streams the
 * compressed cache once.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller; the library
 *     allocates nothing and keeps no state between calls.
 *   - fp16 data is passed as uint16_t bit patterns.
 *   - Work is enqueued on `stream` and returns without synchronising.  Host-checkable
 *     errors return a negative kvq_status and enqueue nothing.  A failed launch returns
 *     KVQ_ERR_HIP.  Faults inside a kernel surface at the caller's next synchronisation.
 *   - Inputs must be finite (no NaN/Inf keys or values).
 *
 * Storage layout of the compressed cache (B = batch, H = n_kv_heads, S = max_seq, a
 * multiple of 64, D = head_dim = 128, k = n_outliers):
 *   k_codes   uint8 [B][H][S][D*k_bits/8]      one record per token.  Field f (b bits)
 *             holds channel f/2 + (D/2)*(f%2), i.e. the two halves of each rotary pair
 *             side by side; bit i of field f is stream bit f*b+i; stream bit p is bit
 *             p%8 of byte p/8 (little-endian bitstream).
 *   v_codes   uint8 [B][H][S/64][D*8*v_bits]   channel-major 64-token tiles: inside a
 *             tile, channel c owns bytes [c*8*b, (c+1)*8*b): its 64 codes in token order
 *             as a little-endian bitstream.
 *   k_out_idx uint8  [B][H][S][k]  outlier channels of each key vector, strictly
 *                                  ascending (under the per-channel key rule, unused
 *                                  slots after them hold channel 255)
 *   k_out_val uint16 [B][H][S][k]  their fp16 values, unchanged
 *   v_out_idx, v_out_val           the same for values: always k distinct channels,
 *                                  strictly ascending.  The value pass sums a tile's
 *                                  outlier terms in 32-bit fixed point and relies on
 *                                  this (at most one term per channel and token); a
 *                                  cache with repeated value channels is outside the
 *                                  contract (its outputs are undefined, nothing faults)
 *   v_scale   uint16 [B][H][S]     fp16 per-vector value scale (max |dense entry|)
 *   k_scale   float  [H][D]        frozen per-channel key scale (caller calibrated)
 *   k_codebook, v_codebook  fp16 [2^bits] (uint16_t bits), strictly ascending, in [-1, 1];
 *             the quantizer compares against their exact float32 values
 *   seq_len   int32 [B]            tokens held per sequence (device copy; the length is
 *                                  the low 24 bits, the high bits are zero between calls)
 * Bits of tokens at or beyond seq_len[b] are never read.  A cache whose buffers start
 * zero-filled holds zero bits there, which makes the packed buffers comparable byte for
 * byte.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KVQ_OK = 0,
  KVQ_ERR_INVALID = -1,      /* null pointer, negative or inconsistent size */
  KVQ_ERR_UNSUPPORTED = -2,  /* head_dim != 128, bits not in {2,3,4}, group not in {1,2,4,8} */
  KVQ_ERR_CAPACITY = -3,     /* an append would pass max_seq */
  KVQ_ERR_WORKSPACE = -4,    /* workspace null or smaller than kvq_workspace_bytes() */
  KVQ_ERR_HIP = -5           /* a HIP launch or runtime call failed */
} kvq_status;

typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t n_q_heads;   /* Hq, a multiple of n_kv_heads; q head h reads kv head h / (Hq/Hkv) */
  int32_t n_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;    /* D, must be 128 */
  int32_t max_seq;     /* S, cache capacity in tokens, a positive multiple of 64, < 2^24 */
  int32_t k_bits;      /* 2, 3 or 4 */
  int32_t v_bits;      /* 2, 3 or 4 */
  int32_t n_outliers;  /* k per (token, kv head) vector, 0 <= k <= D */
  float rope_base;     /* rotary base (10000 for LLaMA-family models), > 1 */
  int32_t key_outliers; /* rule choosing each key vector's outliers (values always use 0):
                           0  per vector: its k largest |x_c| (ties to the lower channel);
                           1  per channel (keys are quantized per channel): the candidates
                              |x_c| > k_scale[c] (so the dense part stays within its
                              channel's scale), at most k of them, largest float32
                              |x_c| / k_scale[c] first (+inf where the scale is 0), ties to
                              the lower channel; unused slots hold channel 255 and value 0.
                           The pages quantize keys per channel and isolate outliers per
                           vector (summary page, techniques (i) and (iv); paper note, items
                           (1) and (4)) without fixing whose standard makes an outlier; 1
                           is the per-channel reading.  Other values: KVQ_ERR_INVALID. */
} kvq_shape;

typedef struct {
  uint8_t *k_codes, *v_codes;
  uint8_t *k_out_idx;
  uint16_t *k_out_val;
  uint8_t *v_out_idx;
  uint16_t *v_out_val;
  uint16_t *v_scale;
  const float *k_scale;
  const uint16_t *k_codebook, *v_codebook;
  int32_t *seq_len;
} kvq_cache;

/* Byte sizes of each cache buffer for `shape` (host only, no device work). */
typedef struct {
  size_t k_codes, v_codes, k_out_idx, k_out_val, v_out_idx, v_out_val, v_scale;
  size_t k_scale, k_codebook, v_codebook, seq_len;
  size_t total;  /* sum of all of the above */
} kvq_sizes;

int kvq_cache_sizes(const kvq_shape* shape, kvq_sizes* out);

/* Workspace bytes kvq_pv_matvec needs for caches of at most `max_len` tokens.
 * Returns 0 for an invalid shape or max_len < 1. */
size_t kvq_workspace_bytes(const kvq_shape* shape, int32_t max_len);

/*
 * Quantize and append new keys/values (summary page, techniques (i)-(iv)).
 *   k_new, v_new   fp16 [B][n_max][Hkv][D], keys BEFORE the rotary embedding.
 *   n_max          tokens per sequence in k_new / v_new (>= 0).
 *   n_new_host     host int32 [B]: tokens of sequence b to append (its first n_new_host[b]
 *                  rows, 0 <= n_new_host[b] <= n_max); NULL appends n_max for every b.
 *   seq_len_host   host int32 [B]: current length of every sequence (must equal the
 *                  device seq_len).  Token j of sequence b goes to position
 *                  seq_len_host[b] + j.
 *                  NULL selects device positions: each sequence's start is read from the
 *                  device seq_len inside the kernel, so the call can be recorded once in a
 *                  HIP graph and replayed every decode step.  The host cannot check
 *                  capacity then: a sequence without room for its new tokens appends
 *                  nothing and keeps its length (visible in seq_len).  Requires
 *                  n_kv_heads <= 127.
 * Per new vector: its outliers (values and, with key_outliers = 0, keys: the k largest
 * |x| entries, ties to the lower channel; keys with key_outliers = 1: the per-channel rule
 * of kvq_shape) go to the outlier store in ascending channel order with their fp16 bits;
 * the dense rest (outlier slots zeroed) is divided in float32 by the key's per-channel
 * scale or by the value vector's own max |dense| (0 -> all-zero u) and coded as the lowest
 * j minimising |u - cb_j| (a key entry beyond its scale lands on an end code).
 * Afterwards seq_len[b] = old length + n_new (device), enqueued on `stream`.
 * Errors: KVQ_ERR_CAPACITY if any seq_len_host[b] + n_new > max_seq (host positions).
 * Calls that overlap on one cache (e.g. on two streams) race.
 */
int kvq_quantize_append(const kvq_shape* shape, const kvq_cache* cache, const uint16_t* k_new,
                        const uint16_t* v_new, int32_t n_max, const int32_t* n_new_host,
                        const int32_t* seq_len_host, hipStream_t stream);

/*
 * Decode-time q.K^T over the compressed key cache (paper note, item (2): RoPE after
 * dequantization).
 *   q          [B][Hq][D], float32 (q_is_fp16 = 0) or fp16 bits (q_is_fp16 = 1), already
 *              rotated at the query's own position.
 *   logits     float32 [B][Hq][max_seq]; for every t < seq_len[b]:
 *              logits[b][h][t] = sm_scale * q[b][h] . RoPE_t(k~[b][h/g][t]),
 *              k~ = cb_K[code] * k_scale (dense channels) or the fp16 outlier value;
 *              RoPE_t rotates pair (i, i+D/2) by t * rope_base^(-2i/D).
 *              Entries at t >= seq_len[b] are not written.
 *   max_len    host bound, >= every seq_len[b] and <= max_seq; sizes the grid.
 */
int kvq_qk_matvec(const kvq_shape* shape, const kvq_cache* cache, const void* q, int32_t q_is_fp16,
                  float sm_scale, float* logits, int32_t max_len, hipStream_t stream);

/*
 * softmax(logits) . V over the compressed value cache plus the value outliers, as a
 * split over the sequence (chunks of tokens) followed by a log-sum-exp combine.  Values
 * are decoded as the append stored them (summary page, abstract paragraph, techniques
 * (iii) and (iv); paper note, items (3) and (4)): the per-layer codebook entry of each
 * code times the vector's own scale (values take the per-token axis, keys the
 * per-channel one of technique (i)), except at the vector's outlier channels, which take
 * their stored fp16 values.
 *   logits     float32 [B][Hq][max_seq] as written by kvq_qk_matvec.
 *   out        float32 [B][Hq][D]: sum_t p_t v~[b][h/g][t], p = softmax over t < seq_len[b];
 *              a sequence of length 0 gives zeros.
 *   workspace  device scratch of at least kvq_workspace_bytes(shape, max_len) bytes.
 */
int kvq_pv_matvec(const kvq_shape* shape, const kvq_cache* cache, const float* logits, float* out,
                  void* workspace, size_t workspace_bytes, int32_t max_len, hipStream_t stream);

/*
 * kvq_pv_matvec without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Arguments and results as for kvq_pv_matvec; the split partials go to a
 * device array of the library of KVQ_NOALLOC_SCRATCH_BYTES bytes (each device holds its
 * own copy until the process ends; the call itself allocates nothing).
 * Errors: as kvq_pv_matvec, and KVQ_ERR_WORKSPACE when kvq_workspace_bytes(shape, max_len)
 * exceeds KVQ_NOALLOC_SCRATCH_BYTES (for example 32 query heads of one sequence up to
 * about 2M tokens, or 16 sequences of 32 query heads up to about 126K tokens).  All calls
 * on one device share the array: calls that overlap on one device (several streams, or
 * several threads) race and must be serialised by the caller.
 */
#define KVQ_NOALLOC_SCRATCH_BYTES (32u << 20)
int kvq_pv_matvec_noalloc(const kvq_shape* shape, const kvq_cache* cache, const float* logits, float* out,
                          int32_t max_len, hipStream_t stream);

/*
 * Single-pass decode attention: kvq_qk_matvec followed by kvq_pv_matvec in one kernel
 * pass (plus the combine), without writing the logits (summary page, abstract paragraph:
 * decode is bandwidth-bound, and the logits are the one intermediate both passes move).
 *   q, sm_scale, out, workspace, max_len  as for kvq_qk_matvec and kvq_pv_matvec; out
 *   equals kvq_pv_matvec's output after kvq_qk_matvec (up to float rounding order).
 * Supported: one query head per kv head (n_q_heads == n_kv_heads) and 2- or 3-bit keys;
 * other shapes return KVQ_ERR_UNSUPPORTED and enqueue nothing (use the two calls).
 */
int kvq_decode_attention(const kvq_shape* shape, const kvq_cache* cache, const void* q, int32_t q_is_fp16,
                         float sm_scale, float* out, void* workspace, size_t workspace_bytes, int32_t max_len,
                         hipStream_t stream);

/*
 * Per-channel key scale from a bulk of calibration keys (summary page, abstract paragraph,
 * technique (i); paper note, item (1)): k_scale[h][c] = max |x_c| over every vector of kv
 * head h in `keys`, e.g. a prompt before its prefill append.
 *   keys              fp16 [B][n_tokens][Hkv][D], before the rotary embedding (the layout
 *                     kvq_quantize_append takes).
 *   exclude_outliers  0: over all entries; 1: over each vector's dense part, its
 *                     shape->n_outliers largest-magnitude entries (ties to the lower
 *                     channel, as the quantizer selects them) left out.
 *   k_scale_out       device float32 [Hkv][D]; overwritten (zeros for n_tokens = 0).
 * The max is exact: the result is bit-for-bit the maximum fp16 magnitude.
 */
int kvq_key_scale(const kvq_shape* shape, const uint16_t* keys, int32_t n_tokens, int32_t exclude_outliers,
                  float* k_scale_out, hipStream_t stream);

/*
 * Per-channel key threshold for the per-channel outlier rule (key_outliers = 1), from a
 * bulk of calibration keys, e.g. a prompt before its prefill append.  The pages quantize
 * keys per channel and isolate outliers per vector (summary page, abstract paragraph,
 * techniques (i) and (iv); paper note, items (1) and (4)) but give no calibration for a
 * per-channel threshold; this one leaves a chosen share of each channel's calibration
 * entries above it.  With N = B * n_tokens vectors and m = floor(outlier_frac * N) (the
 * product in double precision), k_scale[h][c] = the (m+1)-th largest |x_c| over the
 * vectors of kv head h, so at most m of them exceed it; 0 when m >= N (also for N = 0).
 * Magnitudes are compared as fp16 bit patterns with the sign cleared (numeric order for
 * finite keys; a NaN ranks above +inf); the result is that fp16 magnitude, exact.
 *   keys              fp16 [B][n_tokens][Hkv][D], before the rotary embedding.
 *   outlier_frac      share of entries allowed above the threshold, 0 <= f <= 1 (0 gives
 *                     the channel maximum, as kvq_key_scale without exclusion).
 *   k_scale_out       device float32 [Hkv][D]; overwritten.
 *   workspace         device scratch of kvq_key_threshold_workspace_bytes(shape, n_tokens)
 *                     bytes (NULL allowed when that is 0); its contents are not kept.
 * Errors: KVQ_ERR_INVALID for f outside [0, 1] or NaN, n_tokens < 0, B * n_tokens >= 2^31,
 * null pointers; KVQ_ERR_WORKSPACE for a missing or short workspace.  Six kernels are
 * enqueued on `stream` (histograms of the magnitudes' high and low bits, their sums and
 * the selections); calls sharing one workspace must not overlap.
 */
size_t kvq_key_threshold_workspace_bytes(const kvq_shape* shape, int32_t n_tokens);
int kvq_key_threshold(const kvq_shape* shape, const uint16_t* keys, int32_t n_tokens, double outlier_frac,
                      float* k_scale_out, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Per-layer codebook fitting (summary page, abstract paragraph, technique (iii); paper
 * note, item (3)): unweighted 1-D k-means over normalised calibration activations (keys
 * divided by their per-channel scale, values by their per-vector scale), the input of a
 * layer's k_codebook or v_codebook.  The pages weight the fit by each activation's
 * sensitivity, which needs a trained model; this is the unweighted version.
 *   u             device float32 [n] (n < 2^33; NULL allowed for n = 0), clamped to [-1, 1].
 *   bits          2, 3 or 4: 2^bits entries.
 *   iters         Lloyd iterations (>= 0), starting from the midpoints -1 + (2j+1)/2^bits.
 *                 Each iteration assigns every input to its nearest entry by the quantizer's
 *                 own rule (smallest j minimising the float32 |u - c_j|) and moves each entry
 *                 with inputs to their mean, formed exactly from the inputs rounded to the
 *                 grid 2^-30 (so the result does not depend on the order of summation):
 *                 c_j = float32(sum / (count * 2^30)); an entry without inputs stays.
 *   codebook_out  device fp16 bits [2^bits]: the entries rounded to fp16, then raised where
 *                 needed to at least the next fp16 above their predecessor and, if the last
 *                 passes 1, lowered from the top: strictly ascending, within [-1, 1].
 *   workspace     device scratch of at least kvq_fit_workspace_bytes() bytes.
 * Errors as elsewhere; KVQ_ERR_UNSUPPORTED for bits outside {2, 3, 4}.
 */
size_t kvq_fit_workspace_bytes(void);
int kvq_fit_codebook(const float* u, int64_t n, int32_t bits, int32_t iters, uint16_t* codebook_out,
                     void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Uncompressed fp16 decode attention over a plain fp16 cache: the comparison point the
 * pages quote the compressed kernels against (summary page, abstract paragraph: custom
 * kernels faster than fp16 matrix-vector products).  Same logits and outputs as
 * kvq_qk_matvec / kvq_pv_matvec, over
 *   k_fp16, v_fp16  fp16 bits [B][Hkv][max_seq][D], token-major; the keys already rotated
 *                   at their own positions (an fp16 cache stores keys after RoPE), so
 *                   logits[b][h][t] = sm_scale * q[b][h] . k_fp16[b][h/g][t].
 *   seq_len         device int32 [B], tokens held per sequence (low 24 bits).
 * Only batch, n_q_heads, n_kv_heads, head_dim and max_seq of `shape` are used (and
 * checked: head_dim 128, max_seq a multiple of 64, group in {1, 2, 4, 8}).  The fp16 pv
 * workspace is sized like the compressed one: kvq_workspace_bytes of a valid shape with
 * the same heads and max_seq.  Errors and asynchrony as for the compressed calls.
 */
int kvq_fp16_qk_matvec(const kvq_shape* shape, const uint16_t* k_fp16, const int32_t* seq_len, const void* q,
                       int32_t q_is_fp16, float sm_scale, float* logits, int32_t max_len, hipStream_t stream);
int kvq_fp16_pv_matvec(const kvq_shape* shape, const uint16_t* v_fp16, const int32_t* seq_len,
                       const float* logits, float* out, void* workspace, size_t workspace_bytes,
                       int32_t max_len, hipStream_t stream);

/* Human-readable name of a kvq_status value (static string). */
const char* kvq_status_string(int status);

/* ABI version of this header (bumped on any incompatible change). */
int kvq_abi_version(void);

/*
 * Streaming-read probe (measurement only): reads every byte of a device buffer once with
 * 16-byte loads, so that bytes / time is the HBM read bandwidth a plain kernel reaches on
 * this device, the practical ceiling beside the quoted peak (the pages call decode memory-
 * and bandwidth-bound: summary page, abstract paragraph).
 *   buf    device buffer, 16-byte aligned; bytes a multiple of 16 (0 enqueues nothing).
 *   sink   device uint32; receives 0x9e3779b9 when a thread's XOR of the 32-bit words it
 *          read equals that value, and is untouched otherwise (the conditional store keeps
 *          the loads from being optimised away).
 * Errors: KVQ_ERR_INVALID for a misaligned buffer or size, or null pointers.
 */
int kvq_stream_read(const void* buf, size_t bytes, uint32_t* sink, hipStream_t stream);

#define KVQ_ABI_VERSION 4

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
