// Uncompressed fp16 decode attention: the comparison point for the compressed kernels.
//
// KVQuant summary page, abstract paragraph: the method's custom kernels are reported as
// a speed-up over fp16 matrix-vector products.  These kernels are that baseline on this
// device, with the same logits and outputs as the compressed path, over a plain fp16
// cache whose keys are stored after the rotary embedding (so q . K^T is one dot product
// per cached token) and whose values are stored as they are.
//
// fp16_qk: 16 lanes cover one token's 128 channels, 8 channels (one 16-byte load) each,
// so a wave reads four tokens (1 KB) per load instruction, with eight such loads in
// flight per lane; four DPP steps sum each 16-lane row.
// fp16_pv_partial: lane = channel pair, one 4-byte load per token (a wave reads a whole
// token, 256 bytes, per instruction), the next 64-token tile in flight while the current
// one is accumulated.  Per tile, lane = token for the wave's online softmax (max, rescale,
// p_t), then p_t reaches every channel lane as a scalar operand.  The partial (o, m, l)
// of each block uses the compressed path's layout and combine kernel.
#include <algorithm>
#include <cstring>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kFpThreads = 256;
constexpr int kFpWaves = kFpThreads / kWave;
constexpr int kQkUnroll = 8;                        // 16-byte loads in flight per lane
constexpr int kQkStep = kFpWaves * 4 * kQkUnroll;   // tokens a block covers per loop step
constexpr int kPvMinTilesPerBlock = 16;             // as the compressed path: same workspace bound

// Sum over each 16-lane row; every lane of the row receives it.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_f32<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_f32<0x141>(v);  // row_half_mirror
  v += dpp_f32<0x140>(v);  // row_mirror
  return v;
}

template <int G>
__global__ __launch_bounds__(kFpThreads) void fp16_qk_kernel(Fp16Args a) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int S = a.max_seq;
  const int L = min(a.seq_len[seq] & kLenMask, a.max_len);
  const int t_lo = blockIdx.x * a.tokens_per_block;
  const int t_hi = min(t_lo + a.tokens_per_block, L);
  if (t_lo >= t_hi) return;
  const int cg = lane & 15;   // channels 8 cg .. 8 cg + 7
  const int sub = lane >> 4;  // token inside the wave's group of four

  float qv[G][8];
  const size_t qbase = (static_cast<size_t>(seq) * a.n_q_heads + static_cast<size_t>(kvh) * G) * kHeadDim + 8 * cg;
#pragma unroll
  for (int h = 0; h < G; ++h) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const size_t o = qbase + static_cast<size_t>(h) * kHeadDim + j;
      qv[h][j] = a.q_is_fp16 ? half_bits_to_float(static_cast<const uint16_t*>(a.q)[o]) : static_cast<const float*>(a.q)[o];
    }
  }
  const uint16_t* kb = a.k + (static_cast<size_t>(seq) * a.n_kv_heads + kvh) * static_cast<size_t>(S) * kHeadDim + 8 * cg;
  float* lg = a.logits + (static_cast<size_t>(seq) * a.n_q_heads + static_cast<size_t>(kvh) * G) * S;

  // Token of (step t0, slot u): t0 + 16 u + 4 wave + sub.  Loads past the range read the
  // range's last token (in bounds) and their results are not written.
  for (int t0 = t_lo; t0 < t_hi; t0 += kQkStep) {
    uint4 kk[kQkUnroll];
#pragma unroll
    for (int u = 0; u < kQkUnroll; ++u) {
      const int t = min(t0 + 16 * u + 4 * wave + sub, t_hi - 1);
      kk[u] = *reinterpret_cast<const uint4*>(kb + static_cast<size_t>(t) * kHeadDim);
    }
#pragma unroll
    for (int u = 0; u < kQkUnroll; ++u) {
      const int t = t0 + 16 * u + 4 * wave + sub;
      const uint32_t w[4] = {kk[u].x, kk[u].y, kk[u].z, kk[u].w};
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc[h] = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[h] = fmaf(half_bits_to_float(w[j] & 0xffffu), qv[h][2 * j], acc[h]);
          acc[h] = fmaf(half_bits_to_float(w[j] >> 16), qv[h][2 * j + 1], acc[h]);
        }
        acc[h] = row16_sum(acc[h]);
      }
      if (cg == 0 && t < t_hi) {
#pragma unroll
        for (int h = 0; h < G; ++h) lg[static_cast<size_t>(h) * S + t] = a.sm_scale * acc[h];
      }
    }
  }
}

template <int G>
__global__ __launch_bounds__(kFpThreads) void fp16_pv_partial_kernel(Fp16Args a) {
  __shared__ float wm[kFpWaves][G], wl[kFpWaves][G];
  __shared__ float wo[kFpWaves][G][kHeadDim];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int S = a.max_seq;
  const int L = min(a.seq_len[seq] & kLenMask, a.max_len);
  const int n_tiles = (L + kTile - 1) / kTile;
  const int tile_lo = blockIdx.x * a.tiles_per_block;
  const int tile_hi = min(tile_lo + a.tiles_per_block, n_tiles);
  const size_t part_stride = kHeadDim + 2;
  auto part_ptr = [&](int h) {
    return a.partial + ((static_cast<size_t>(seq) * a.n_q_heads + static_cast<size_t>(kvh) * G + h) * a.n_parts + blockIdx.x) * part_stride;
  };
  if (tile_lo >= tile_hi) {
    for (int e = tid; e < G * (kHeadDim + 2); e += kFpThreads) {
      const int h = e / (kHeadDim + 2), c = e % (kHeadDim + 2);
      part_ptr(h)[c] = (c == kHeadDim) ? -INFINITY : 0.0f;
    }
    return;
  }
  const int nt = tile_hi - tile_lo;
  const int w_lo = tile_lo + (nt * wave) / kFpWaves;
  const int w_hi = tile_lo + (nt * (wave + 1)) / kFpWaves;

  const uint32_t* vb = reinterpret_cast<const uint32_t*>(a.v + (static_cast<size_t>(seq) * a.n_kv_heads + kvh) * static_cast<size_t>(S) * kHeadDim) + lane;
  const float* lgb = a.logits + (static_cast<size_t>(seq) * a.n_q_heads + static_cast<size_t>(kvh) * G) * S;

  // A tile's values (token tt of the tile, channels 2 lane, 2 lane + 1) and the logit of
  // token `lane` for every head; tiles past the wave's run reload its last tile and tokens
  // past the length read the last token (in bounds; weights zero).
  struct Tile {
    uint32_t v[kTile];
    float lg[G];
  };
  auto load = [&](int tile, Tile& d) {
    tile = max(0, min(tile, w_hi - 1));
#pragma unroll
    for (int tt = 0; tt < kTile; ++tt) {
      const int t = min(tile * kTile + tt, L - 1);
      d.v[tt] = vb[static_cast<size_t>(t) * (kHeadDim / 2)];
    }
    const int t = min(tile * kTile + lane, L - 1);
#pragma unroll
    for (int h = 0; h < G; ++h) d.lg[h] = lgb[static_cast<size_t>(h) * S + t];
  };

  float m_run[G], lsum[G], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    lsum[h] = 0.0f;
    acc[h][0] = acc[h][1] = 0.0f;
  }
  auto compute = [&](int tile, const Tile& d) {
    const bool valid = tile * kTile + lane < L;
    float pr[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float lg = valid ? d.lg[h] : -INFINITY;
      const float mt = wave_max_f32(lg);
      if (mt > m_run[h]) {  // wave-uniform: rescale the running state to the new max
        const float sc = m_run[h] > -INFINITY ? expf(m_run[h] - mt) : 0.0f;
        m_run[h] = mt;
        acc[h][0] *= sc;
        acc[h][1] *= sc;
        lsum[h] *= sc;
      }
      pr[h] = valid ? expf(lg - m_run[h]) : 0.0f;
      lsum[h] += pr[h];
    }
    float part[G][2][2];
#pragma unroll
    for (int h = 0; h < G; ++h) part[h][0][0] = part[h][0][1] = part[h][1][0] = part[h][1][1] = 0.0f;
#pragma unroll
    for (int tt = 0; tt < kTile; ++tt) {
      const float va = half_bits_to_float(d.v[tt] & 0xffffu), vbh = half_bits_to_float(d.v[tt] >> 16);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, pr[h]), tt));
        part[h][0][tt & 1] = fmaf(va, w, part[h][0][tt & 1]);
        part[h][1][tt & 1] = fmaf(vbh, w, part[h][1][tt & 1]);
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      acc[h][0] += part[h][0][0] + part[h][0][1];
      acc[h][1] += part[h][1][0] + part[h][1][1];
    }
  };

  if (w_lo < w_hi) {
    Tile bufA, bufB;
    load(w_lo, bufA);
    for (int tile = w_lo; tile < w_hi; tile += 2) {
      load(tile + 1, bufB);
      compute(tile, bufA);
      if (tile + 1 >= w_hi) break;
      load(tile + 2, bufA);
      compute(tile + 1, bufB);
    }
  }

  // ---- merge the four waves' states -------------------------------------------------
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const float ls = wave_sum_f32(lsum[h]);
    if (lane == 0) {
      wm[wave][h] = m_run[h];
      wl[wave][h] = ls;
    }
    wo[wave][h][2 * lane] = acc[h][0];
    wo[wave][h][2 * lane + 1] = acc[h][1];
  }
  block_lds_barrier();
  for (int e = tid; e < G * kHeadDim; e += kFpThreads) {
    const int h = e / kHeadDim, c = e % kHeadDim;
    float M = wm[0][h];
#pragma unroll
    for (int w = 1; w < kFpWaves; ++w) M = fmaxf(M, wm[w][h]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kFpWaves; ++w) {
      const float f = wm[w][h] > -INFINITY ? expf(wm[w][h] - M) : 0.0f;
      o += f * wo[w][h][c];
      l += f * wl[w][h];
    }
    float* dst = part_ptr(h);
    dst[c] = o;
    if (c == 0) {
      dst[kHeadDim] = M;
      dst[kHeadDim + 1] = l;
    }
  }
}

template <int G>
hipError_t launch_fp16_qk_t(int batch, const Fp16Args& a0, hipStream_t s) {
  Fp16Args a = a0;
  // About eight blocks per CU over all streams, in whole loop steps.
  const long streams = static_cast<long>(batch) * a.n_kv_heads;
  const long want = std::max(1L, (8L * device_cu_count() + streams - 1) / streams);
  const long steps = (a.max_len + kQkStep - 1) / kQkStep;
  a.tokens_per_block = static_cast<int>(std::max(1L, (steps + want - 1) / want) * kQkStep);
  dim3 grid((a.max_len + a.tokens_per_block - 1) / a.tokens_per_block, a.n_kv_heads, batch);
  hipLaunchKernelGGL((fp16_qk_kernel<G>), grid, dim3(kFpThreads), 0, s, a);
  return hipGetLastError();
}

template <int G>
hipError_t launch_fp16_pv_t(int batch, const Fp16Args& a0, hipStream_t s) {
  Fp16Args a = a0;
  const int tiles = (a.max_len + kTile - 1) / kTile;
  const long streams = static_cast<long>(batch) * a.n_kv_heads;
  static const int resident = blocks_per_cu(reinterpret_cast<const void*>(&fp16_pv_partial_kernel<G>), kFpThreads);
  const long slots = static_cast<long>(device_cu_count()) * resident;
  const long per_stream = std::max(1L, std::min<long>((slots + streams - 1) / streams,
                                                      (tiles + kPvMinTilesPerBlock - 1) / kPvMinTilesPerBlock));
  a.tiles_per_block = static_cast<int>((tiles + per_stream - 1) / per_stream);
  a.n_parts = (tiles + a.tiles_per_block - 1) / a.tiles_per_block;
  dim3 grid(a.n_parts, a.n_kv_heads, batch);
  hipLaunchKernelGGL((fp16_pv_partial_kernel<G>), grid, dim3(kFpThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  PvArgs c;
  std::memset(&c, 0, sizeof(c));
  c.n_q_heads = a.n_q_heads;
  c.n_kv_heads = a.n_kv_heads;
  c.max_seq = a.max_seq;
  c.max_len = a.max_len;
  c.tiles_per_block = a.tiles_per_block;
  c.n_parts = a.n_parts;
  c.seq_len = a.seq_len;
  c.partial = a.partial;
  c.out = a.out;
  return launch_pv_combine(batch, c, s);
}

}  // namespace

hipError_t launch_fp16_qk(int group, int batch, const Fp16Args& a, hipStream_t s) {
  switch (group) {
    case 1: return launch_fp16_qk_t<1>(batch, a, s);
    case 2: return launch_fp16_qk_t<2>(batch, a, s);
    case 4: return launch_fp16_qk_t<4>(batch, a, s);
    case 8: return launch_fp16_qk_t<8>(batch, a, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_fp16_pv(int group, int batch, const Fp16Args& a, hipStream_t s) {
  switch (group) {
    case 1: return launch_fp16_pv_t<1>(batch, a, s);
    case 2: return launch_fp16_pv_t<2>(batch, a, s);
    case 4: return launch_fp16_pv_t<4>(batch, a, s);
    case 8: return launch_fp16_pv_t<8>(batch, a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvq
