// Device-side helpers shared by the kvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kHalf = kHeadDim / 2;  // rotary pairs per vector
constexpr int kTile = 64;            // tokens per value tile and per QK wave pass
constexpr int kWave = 64;
// seq_len words hold the length in their low 24 bits; the high bits are an arrival
// counter used only while a device-positioned append is in flight.
constexpr int32_t kLenMask = 0x00ffffff;

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint32_t o = __shfl_xor(v, off, kWave);
    v = v > o ? v : o;
  }
  return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// b-bit field starting at compile-time bit position POS of a little-endian stream held in
// 32-bit words (registers after full unrolling).
template <int BITS, int POS, int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N]) {
  constexpr int wi = POS / 32;
  constexpr int sh = POS % 32;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  static_assert(wi < N, "field outside the word array");
  if constexpr (sh + BITS <= 32) {
    return (w[wi] >> sh) & mask;
  } else {
    static_assert(wi + 1 < N, "straddling field outside the word array");
    return ((w[wi] >> sh) | (w[wi + 1] << (32 - sh))) & mask;
  }
}

// Compile-time loop: calls f(std::integral_constant<int, I>) for I in [0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Nearest codebook entry: the smallest j minimising the float32 |u - cb[j]|, scanned in
// ascending j with a strict '<' (ties go to the lower index).
template <int NC>
__device__ __forceinline__ uint32_t nearest_code(float u, const float* cb) {
  uint32_t best = 0;
  float bd = fabsf(u - cb[0]);
#pragma unroll
  for (int j = 1; j < NC; ++j) {
    float d = fabsf(u - cb[j]);
    if (d < bd) {
      bd = d;
      best = j;
    }
  }
  return best;
}

// Index of the codebook entry nearest to 0 (the code of every dense-zero entry, in
// particular of every outlier slot): smallest j minimising |0 - cb[j]|.
template <int NC>
__device__ __forceinline__ int zero_code_index(const float* cb) {
  int j0 = 0;
  float bd = fabsf(0.0f - cb[0]);
  for (int j = 1; j < NC; ++j) {
    const float d = fabsf(0.0f - cb[j]);
    if (d < bd) {
      bd = d;
      j0 = j;
    }
  }
  return j0;
}

// cos/sin of 2*pi*r for a revolution count r already reduced to [0, 1).
__device__ __forceinline__ void sincos_rev(float r, float* s, float* c) { sincospif(2.0f * r, s, c); }

// Fractional revolutions of angle t * theta, theta given as theta / (2*pi) in float64.
__device__ __forceinline__ float frac_rev(double t, double theta_over_2pi) {
  double r = t * theta_over_2pi;
  return static_cast<float>(r - floor(r));
}

}  // namespace kvq
