// Per-channel key scale from a bulk of calibration keys (e.g. the prompt of a prefill).
//
// KVQuant summary page, abstract paragraph, technique (i), and the paper note, "Four
// components" paragraph, item (1): keys are quantized per channel, so each channel needs
// its own range before any key is quantized.  s_c = max |x_c| over the given vectors of a
// kv head, optionally over each vector's dense part only (its k outliers, chosen as the
// quantizer chooses them, left out).
//
// A wave takes one (sequence, token, kv head) vector at a time, channels (2l, 2l + 1) in
// lane l (one 4-byte load, four vectors in flight); the outliers are found by k rounds of
// a wave maximum over (|x| bits, inverted channel), as the append finds them.  Each lane keeps the running maxima
// of its two channels and the block ends with one integer atomic maximum per channel
// (non-negative floats order as their bit patterns).
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kKsThreads = 256;
constexpr int kKsWaves = kKsThreads / kWave;

__global__ __launch_bounds__(kKsThreads) void key_scale_zero_kernel(float* out, int n) {
  const int i = blockIdx.x * kKsThreads + threadIdx.x;
  if (i < n) out[i] = 0.0f;
}

__global__ __launch_bounds__(kKsThreads) void key_scale_kernel(const uint16_t* __restrict__ keys, int n_tokens,
                                                              int n_kv_heads, int tokens_per_block, int k,
                                                              float* out) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int t_lo = blockIdx.x * tokens_per_block;
  const int t_hi = min(t_lo + tokens_per_block, n_tokens);
  float m0 = 0.0f, m1 = 0.0f;
  auto vec = [&](int t) {  // channels (2 lane, 2 lane + 1) of vector t: one 4-byte load
    return reinterpret_cast<const uint32_t*>(keys + ((static_cast<size_t>(b) * n_tokens + t) * n_kv_heads + h) * kHeadDim)[lane];
  };
  auto take = [&](uint32_t xx) {
    const uint32_t x0 = xx & 0xffffu, x1 = xx >> 16;
    bool sel0 = false, sel1 = false;
    if (k > 0) select_outliers(outlier_key(x0, 2 * lane), outlier_key(x1, 2 * lane + 1), k, sel0, sel1);
    if (!sel0) m0 = fmaxf(m0, fabsf(half_bits_to_float(x0)));
    if (!sel1) m1 = fmaxf(m1, fabsf(half_bits_to_float(x1)));
  };
  int t = t_lo + wave;
  for (; t + 3 * kKsWaves < t_hi; t += 4 * kKsWaves) {  // four vectors' loads in flight
    const uint32_t a0 = vec(t), a1 = vec(t + kKsWaves), a2 = vec(t + 2 * kKsWaves), a3 = vec(t + 3 * kKsWaves);
    take(a0);
    take(a1);
    take(a2);
    take(a3);
  }
  for (; t < t_hi; t += kKsWaves) take(vec(t));
  float* o = out + static_cast<size_t>(h) * kHeadDim;
  atomicMax(reinterpret_cast<unsigned int*>(o + 2 * lane), __builtin_bit_cast(unsigned int, m0));
  atomicMax(reinterpret_cast<unsigned int*>(o + 2 * lane + 1), __builtin_bit_cast(unsigned int, m1));
}

}  // namespace

hipError_t launch_key_scale(const uint16_t* keys, int batch, int n_tokens, int n_kv_heads, int k, float* out,
                            hipStream_t s) {
  const int n_out = n_kv_heads * kHeadDim;
  hipLaunchKernelGGL(key_scale_zero_kernel, dim3((n_out + kKsThreads - 1) / kKsThreads), dim3(kKsThreads), 0, s, out,
                     n_out);
  if (n_tokens <= 0) return hipGetLastError();
  // about four blocks per CU over all (sequence, kv head) pairs, whole waves of tokens
  const long streams = static_cast<long>(batch) * n_kv_heads;
  const long want = std::max(1L, (4L * device_cu_count() + streams - 1) / streams);
  const int per_block = static_cast<int>(std::max<long>(kKsWaves, ((n_tokens + want - 1) / want + kKsWaves - 1) / kKsWaves * kKsWaves));
  dim3 grid((n_tokens + per_block - 1) / per_block, n_kv_heads, batch);
  hipLaunchKernelGGL(key_scale_kernel, grid, dim3(kKsThreads), 0, s, keys, n_tokens, n_kv_heads, per_block, k, out);
  return hipGetLastError();
}

}  // namespace kvq
