// softmax(P) . V over the compressed value cache plus the sparse value outliers, split
// over the sequence with a second-pass log-sum-exp combine.
//
// KVQuant summary page, abstract paragraph, techniques (iii) and (iv): values are decoded
// through the layer's codebook and their per-vector scale, and each vector's fp16
// outliers are added back.  The split over the sequence lets a single long sequence fill
// the GPU.
//
// pv_partial: one block per (sequence, kv head, chunk of 1024 tokens).  Pass 1 reads the
// chunk's logits (one thread per token) for every query head of the group, forms
// p_t = exp(l_t - m) and the per-token weight w_t = p_t * s_t, and scatters the outlier
// corrections p_t * (x_c - zc * s_t) into LDS.  Pass 2 walks the channel-major value
// tiles with one lane per channel pair, so each lane accumulates its two channels over
// the tile's 64 tokens in registers.  The chunk's (o, m, l) go to the workspace.
// pv_combine: one block per (sequence, query head) merges the chunks.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kTokPerThread = kPvChunk / kThreads;
constexpr int kTilesPerChunk = kPvChunk / kTile;

template <int VB, int G>
__global__ __launch_bounds__(256) void pv_partial_kernel(PvArgs a) {
  constexpr int kNc = 1 << VB;
  constexpr int kLaneWords = 4 * VB;
  constexpr int kChanBits = 64 * VB;

  __shared__ float cb[kNc];
  __shared__ float wt[G][kPvChunk];          // p_t * s_t
  __shared__ float osp[G][kHeadDim];         // outlier corrections
  __shared__ float part[kWaves][G][kHeadDim];
  __shared__ float red[kWaves][G];
  __shared__ float zc;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int chunk = blockIdx.x;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int H = a.n_kv_heads;
  const int S = a.max_seq;
  const int k = a.n_outliers;
  const int L = min(a.seq_len[seq], a.max_len);
  const int c0 = chunk * kPvChunk;
  const int n = min(L - c0, kPvChunk);
  const size_t part_stride = kHeadDim + 2;

  if (n <= 0) {
    for (int e = tid; e < G * (kHeadDim + 2); e += kThreads) {
      const int h = e / (kHeadDim + 2), c = e % (kHeadDim + 2);
      float* dst = a.partial + ((static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * a.n_chunks + chunk) * part_stride;
      dst[c] = (c == kHeadDim) ? -INFINITY : 0.0f;
    }
    return;
  }

  if (tid < kNc) cb[tid] = a.v_cb[tid];
  for (int e = tid; e < G * kHeadDim; e += kThreads) (&osp[0][0])[e] = 0.0f;
  if (tid == 0) {
    int j0 = 0;
    float bd = fabsf(0.0f - a.v_cb[0]);
    for (int j = 1; j < kNc; ++j) {
      const float d = fabsf(0.0f - a.v_cb[j]);
      if (d < bd) {
        bd = d;
        j0 = j;
      }
    }
    zc = a.v_cb[j0];
  }

  const size_t stream = static_cast<size_t>(seq) * H + kvh;

  // ---- pass 1: max, exp, weights, outlier scatter ----------------------------------
  float lg[G][kTokPerThread];
  float mloc[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float* lrow = a.logits + (static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * S + c0;
    mloc[h] = -INFINITY;
#pragma unroll
    for (int u = 0; u < kTokPerThread; ++u) {
      const int t = u * kThreads + tid;
      lg[h][u] = t < n ? lrow[t] : -INFINITY;
      mloc[h] = fmaxf(mloc[h], lg[h][u]);
    }
    mloc[h] = wave_max_f32(mloc[h]);
    if (lane == 0) red[wave][h] = mloc[h];
  }
  __syncthreads();
  float m[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = red[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) m[h] = fmaxf(m[h], red[w][h]);
  }
  __syncthreads();

  float lsum[G];
#pragma unroll
  for (int h = 0; h < G; ++h) lsum[h] = 0.0f;
#pragma unroll
  for (int u = 0; u < kTokPerThread; ++u) {
    const int t = u * kThreads + tid;
    const bool valid = t < n;
    const size_t slot = stream * S + c0 + t;
    const float s = valid ? half_bits_to_float(a.v_scale[slot]) : 0.0f;
    float p[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      p[h] = valid ? expf(lg[h][u] - m[h]) : 0.0f;
      lsum[h] += p[h];
      wt[h][t] = p[h] * s;
    }
    if (valid) {
      for (int j = 0; j < k; ++j) {
        const int c = a.v_idx[slot * k + j];
        const float dv = half_bits_to_float(a.v_val[slot * k + j]) - zc * s;
#pragma unroll
        for (int h = 0; h < G; ++h) atomicAdd(&osp[h][c], p[h] * dv);
      }
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    lsum[h] = wave_sum_f32(lsum[h]);
    if (lane == 0) red[wave][h] = lsum[h];
  }
  __syncthreads();

  // ---- pass 2: dense product over channel-major tiles -------------------------------
  float acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) acc[h][0] = acc[h][1] = 0.0f;
  const uint8_t* tiles = a.v_codes + (stream * (S / kTile) + c0 / kTile) * (1024 * VB);
  for (int tl = wave; tl < kTilesPerChunk; tl += kWaves) {
    if (tl * kTile >= n) break;
    uint32_t w[kLaneWords];
    const uint4* p = reinterpret_cast<const uint4*>(tiles + static_cast<size_t>(tl) * (1024 * VB) + lane * (16 * VB));
#pragma unroll
    for (int v = 0; v < VB; ++v) {
      const uint4 d = p[v];
      w[4 * v + 0] = d.x;
      w[4 * v + 1] = d.y;
      w[4 * v + 2] = d.z;
      w[4 * v + 3] = d.w;
    }
    const float* wrow = &wt[0][tl * kTile];
    static_for<0, kTile>([&](auto tc) {
      constexpr int tau = decltype(tc)::value;
      const float v0 = cb[field<VB, tau * VB>(w)];
      const float v1 = cb[field<VB, kChanBits + tau * VB>(w)];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float ww = wrow[h * kPvChunk + tau];
        acc[h][0] += ww * v0;
        acc[h][1] += ww * v1;
      }
    });
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    part[wave][h][2 * lane] = acc[h][0];
    part[wave][h][2 * lane + 1] = acc[h][1];
  }
  __syncthreads();

  for (int e = tid; e < G * kHeadDim; e += kThreads) {
    const int h = e / kHeadDim, c = e % kHeadDim;
    float o = osp[h][c];
#pragma unroll
    for (int w = 0; w < kWaves; ++w) o += part[w][h][c];
    float* dst = a.partial + ((static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * a.n_chunks + chunk) * part_stride;
    dst[c] = o;
    if (c == 0) {
      float l = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) l += red[w][h];
      dst[kHeadDim] = m[h];
      dst[kHeadDim + 1] = l;
    }
  }
}

__global__ __launch_bounds__(128) void pv_combine_kernel(PvArgs a) {
  const int c = threadIdx.x;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const size_t part_stride = kHeadDim + 2;
  const float* src = a.partial + (static_cast<size_t>(seq) * a.n_q_heads + h) * a.n_chunks * part_stride;
  const int L = min(a.seq_len[seq], a.max_len);
  const int nc = (L + kPvChunk - 1) / kPvChunk;
  float M = -INFINITY;
  for (int j = 0; j < nc; ++j) M = fmaxf(M, src[j * part_stride + kHeadDim]);
  float num = 0.0f, den = 0.0f;
  if (M > -INFINITY) {
    for (int j = 0; j < nc; ++j) {
      const float mj = src[j * part_stride + kHeadDim];
      const float wj = mj > -INFINITY ? expf(mj - M) : 0.0f;
      num += wj * src[j * part_stride + c];
      den += wj * src[j * part_stride + kHeadDim + 1];
    }
  }
  a.out[(static_cast<size_t>(seq) * a.n_q_heads + h) * kHeadDim + c] = den > 0.0f ? num / den : 0.0f;
}

template <int VB, int G>
hipError_t launch_pv_t(int batch, const PvArgs& a, hipStream_t s) {
  dim3 grid(a.n_chunks, a.n_kv_heads, batch);
  hipLaunchKernelGGL((pv_partial_kernel<VB, G>), grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pv_combine_kernel, dim3(a.n_q_heads, batch), dim3(kHeadDim), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_pv(int v_bits, int group, int batch, const PvArgs& a, hipStream_t s) {
#define KVQ_PV_CASE(VB, G) \
  if (v_bits == VB && group == G) return launch_pv_t<VB, G>(batch, a, s);
  KVQ_PV_CASE(2, 1) KVQ_PV_CASE(2, 2) KVQ_PV_CASE(2, 4) KVQ_PV_CASE(2, 8)
  KVQ_PV_CASE(3, 1) KVQ_PV_CASE(3, 2) KVQ_PV_CASE(3, 4) KVQ_PV_CASE(3, 8)
  KVQ_PV_CASE(4, 1) KVQ_PV_CASE(4, 2) KVQ_PV_CASE(4, 4) KVQ_PV_CASE(4, 8)
#undef KVQ_PV_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
