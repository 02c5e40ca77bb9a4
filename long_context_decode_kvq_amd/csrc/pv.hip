// softmax(P) . V over the compressed value cache plus the sparse value outliers, split
// over the sequence with a second-pass log-sum-exp combine.
//
// KVQuant summary page, abstract paragraph, techniques (iii) and (iv): values are decoded
// through the layer's codebook and their per-vector scale, and each vector's fp16
// outliers are added back.  The split over the sequence lets a single long sequence fill
// the GPU.
//
// pv_partial: one block per (sequence, kv head, chunk of 1024 tokens).  Every wave first
// issues the loads of its four value tiles, so they are in flight during pass 1, which
// reads the chunk's logits (one thread per token) for every query head of the group,
// forms p_t = exp(l_t - m) and the per-token weight w_t = p_t * s_t, and scatters the
// outlier corrections p_t * (x_c - zc * s_t) into LDS.  Pass 2 walks the channel-major
// tiles with one lane per channel pair: the 2b-bit field holding two consecutive tokens
// of one channel indexes a table of (cb[a], cb[b]), so one lookup decodes two tokens.
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
constexpr int kTilesPerWave = kTilesPerChunk / kWaves;

template <int VB, int G>
__global__ __launch_bounds__(256) void pv_partial_kernel(PvArgs a) {
  constexpr int kNc = 1 << VB;
  constexpr int kLaneWords = 4 * VB;
  constexpr int kChanBits = 64 * VB;
  constexpr int kPairEntries = 1 << (2 * VB);

  __shared__ float2 lut2[kPairEntries];      // (cb[a], cb[b]) for a token pair
  __shared__ float2 wt[G][kPvChunk / 2];     // (w_t, w_{t+1}), w = p * s
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
  const int L = min(a.seq_len[seq] & kLenMask, a.max_len);
  const int c0 = chunk * kPvChunk;
  const int n = min(L - c0, kPvChunk);
  const size_t part_stride = kHeadDim + 2;
  const size_t stream = static_cast<size_t>(seq) * H + kvh;

  if (n <= 0) {
    for (int e = tid; e < G * (kHeadDim + 2); e += kThreads) {
      const int h = e / (kHeadDim + 2), c = e % (kHeadDim + 2);
      float* dst = a.partial + ((static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * a.n_chunks + chunk) * part_stride;
      dst[c] = (c == kHeadDim) ? -INFINITY : 0.0f;
    }
    return;
  }

  // ---- issue this wave's value-tile loads first -------------------------------------
  const int wave_tile0 = wave * kTilesPerWave;  // tile index inside the chunk
  uint32_t w[kTilesPerWave][kLaneWords];
  const uint8_t* tiles = a.v_codes + (stream * (S / kTile) + c0 / kTile) * (1024 * VB);
#pragma unroll
  for (int tl = 0; tl < kTilesPerWave; ++tl) {
    if ((wave_tile0 + tl) * kTile < n) {
      const uint4* p = reinterpret_cast<const uint4*>(tiles + static_cast<size_t>(wave_tile0 + tl) * (1024 * VB) +
                                                      lane * (16 * VB));
#pragma unroll
      for (int v = 0; v < VB; ++v) {
        const uint4 d = p[v];
        w[tl][4 * v + 0] = d.x;
        w[tl][4 * v + 1] = d.y;
        w[tl][4 * v + 2] = d.z;
        w[tl][4 * v + 3] = d.w;
      }
    }
  }

  for (int e = tid; e < kPairEntries; e += kThreads) lut2[e] = make_float2(a.v_cb[e & (kNc - 1)], a.v_cb[e >> VB]);
  for (int e = tid; e < G * kHeadDim; e += kThreads) (&osp[0][0])[e] = 0.0f;
  if (tid == 0) zc = a.v_cb[zero_code_index<kNc>(a.v_cb)];

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
    for (int ww = 1; ww < kWaves; ++ww) m[h] = fmaxf(m[h], red[ww][h]);
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
      reinterpret_cast<float*>(&wt[h][0])[t] = p[h] * s;
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
#pragma unroll
  for (int tl = 0; tl < kTilesPerWave; ++tl) {
    if ((wave_tile0 + tl) * kTile < n) {
      const float2* wrow = &wt[0][(wave_tile0 + tl) * (kTile / 2)];
      static_for<0, kTile / 2>([&](auto mc) {
        constexpr int mm = decltype(mc)::value;
        const float2 v0 = lut2[field<2 * VB, 2 * VB * mm>(w[tl])];
        const float2 v1 = lut2[field<2 * VB, kChanBits + 2 * VB * mm>(w[tl])];
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float2 ww = wrow[h * (kPvChunk / 2) + mm];
          acc[h][0] = fmaf(ww.y, v0.y, fmaf(ww.x, v0.x, acc[h][0]));
          acc[h][1] = fmaf(ww.y, v1.y, fmaf(ww.x, v1.x, acc[h][1]));
        }
      });
    }
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
    for (int ww = 0; ww < kWaves; ++ww) o += part[ww][h][c];
    float* dst = a.partial + ((static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * a.n_chunks + chunk) * part_stride;
    dst[c] = o;
    if (c == 0) {
      float l = 0.0f;
#pragma unroll
      for (int ww = 0; ww < kWaves; ++ww) l += red[ww][h];
      dst[kHeadDim] = m[h];
      dst[kHeadDim + 1] = l;
    }
  }
}

// One block per (sequence, query head): 256 threads = 128 channels x 2 halves of the
// chunk list.  Loads are independent, so the chunk loop keeps several in flight.
__global__ __launch_bounds__(256) void pv_combine_kernel(PvArgs a) {
  __shared__ float red[4];
  __shared__ float acc_n[kHeadDim], acc_d[kHeadDim];
  const int tid = threadIdx.x;
  const int c = tid & (kHeadDim - 1);
  const int half = tid >> 7;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const size_t part_stride = kHeadDim + 2;
  const float* src = a.partial + (static_cast<size_t>(seq) * a.n_q_heads + h) * a.n_chunks * part_stride;
  const int L = min(a.seq_len[seq] & kLenMask, a.max_len);
  const int nc = (L + kPvChunk - 1) / kPvChunk;

  float M = -INFINITY;
  for (int j = tid; j < nc; j += 256) M = fmaxf(M, src[j * part_stride + kHeadDim]);
  M = wave_max_f32(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  float num = 0.0f, den = 0.0f;
  if (M > -INFINITY) {
#pragma unroll 4
    for (int j = half; j < nc; j += 2) {
      const float* pj = src + j * part_stride;
      const float mj = pj[kHeadDim];
      const float wj = mj > -INFINITY ? expf(mj - M) : 0.0f;
      num += wj * pj[c];
      den += wj * pj[kHeadDim + 1];
    }
  }
  if (half == 1) {
    acc_n[c] = num;
    acc_d[c] = den;
  }
  __syncthreads();
  if (half == 0) {
    num += acc_n[c];
    den += acc_d[c];
    a.out[(static_cast<size_t>(seq) * a.n_q_heads + h) * kHeadDim + c] = den > 0.0f ? num / den : 0.0f;
  }
}

template <int VB, int G>
hipError_t launch_pv_t(int batch, const PvArgs& a, hipStream_t s) {
  dim3 grid(a.n_chunks, a.n_kv_heads, batch);
  hipLaunchKernelGGL((pv_partial_kernel<VB, G>), grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(pv_combine_kernel, dim3(a.n_q_heads, batch), dim3(256), 0, s, a);
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
