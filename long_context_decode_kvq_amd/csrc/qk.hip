// Decode-time q . K^T over the compressed key cache, RoPE applied after dequantization.
//
// KVQuant paper note, "Four components" paragraph, item (2): keys are stored before the
// rotary embedding, so the rotation is applied to the dequantized key at each cached
// token's own position; items (1), (3), (4): per-channel scale, per-layer codebook,
// per-vector fp16 outliers.
//
// Mapping: one lane per cached token, one wave per 64-token tile, each wave walking a
// contiguous run of tiles.  The angle (t0 + tau) * theta_i is split into
//   * R(-t0), folded into the query once per tile (lane i rotates pair i of every query
//     of the group; the tile-base phase is formed once per wave from a float64 angle and
//     then advanced by the fixed step 64 * theta_i), and
//   * R(tau), tau = lane < 64, held in registers for the whole kernel.
// Dequantization is one LDS lookup per rotary pair: the record stores the two halves of
// pair i side by side, so their 2b-bit field indexes a per-kv-head table of
// (cb[a] * s_i, cb[b] * s_{i+64}).  Per (token, pair): 2 integer ops, 1 lookup, 4 FMA-class
// ops for the rotation, 2 per query head for the dot.  4-bit keys (256 entries per pair
// would not fit) look up the two channels separately in per-channel tables.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;

template <int KB, int G>
__global__ __launch_bounds__(256) void qk_kernel(QkArgs a) {
  constexpr int kNc = 1 << KB;
  constexpr int kRecWords = 4 * KB;
  constexpr bool kPairLut = KB <= 3;
  constexpr int kPairEntries = 1 << (2 * KB);

  __shared__ float2 et[kHalf][kTile];  // R(tau) for pair i: (cos, sin) of tau * theta_i
  __shared__ float2 lut[kPairLut ? kHalf * kPairEntries : 1];
  __shared__ float lutc[kPairLut ? 1 : kHeadDim * kNc];
  __shared__ float ks[kHeadDim];
  __shared__ float2 qr[kWaves][G][kHalf];  // per-wave tile-rotated query pairs
  __shared__ float zc;                     // codebook value every outlier slot decodes to

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int H = a.n_kv_heads;
  const int S = a.max_seq;
  const int k = a.n_outliers;
  const int L = min(a.seq_len[seq] & kLenMask, a.max_len);
  const int tiles_per_block = a.tiles_per_wave * kWaves;
  const int block_tile0 = blockIdx.x * tiles_per_block;
  if (block_tile0 * kTile >= L) return;

  // ---- per-block tables -----------------------------------------------------------
  const float* kscale = a.k_scale + kvh * kHeadDim;
  if (tid < kHeadDim) ks[tid] = kscale[tid];
  if constexpr (kPairLut) {
    for (int e = tid; e < kHalf * kPairEntries; e += 256) {
      const int i = e / kPairEntries, v = e % kPairEntries;
      lut[e] = make_float2(a.k_cb[v & (kNc - 1)] * kscale[i], a.k_cb[v >> KB] * kscale[i + kHalf]);
    }
  } else {
    for (int e = tid; e < kHeadDim * kNc; e += 256) lutc[e] = a.k_cb[e % kNc] * kscale[e / kNc];
  }
  const double inv2pi = 0.15915494309189533577;
  const double th_rev = exp2(-static_cast<double>(lane) * a.theta_log2) * inv2pi;  // theta_lane / 2pi
  {
    // 16 consecutive tau of pair `lane` per thread: one accurate seed angle, then steps by
    // the single-step rotation (<= 15 float32 rotations).
    const int tau0 = 16 * wave;
    float s0, c0, s1, c1;
    sincos_rev(frac_rev(static_cast<double>(tau0), th_rev), &s0, &c0);
    sincos_rev(frac_rev(1.0, th_rev), &s1, &c1);
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      et[lane][tau0 + u] = make_float2(c0, s0);
      const float cn = c0 * c1 - s0 * s1;
      const float sn = s0 * c1 + c0 * s1;
      c0 = cn;
      s0 = sn;
    }
  }
  if (tid == 0) zc = a.k_cb[zero_code_index<kNc>(a.k_cb)];
  // this lane's query pairs (lane = pair index when rotating the query)
  float qa[G], qb[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t qi = (static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * kHeadDim + lane;
    if (a.q_is_fp16) {
      const uint16_t* q16 = static_cast<const uint16_t*>(a.q);
      qa[h] = half_bits_to_float(q16[qi]);
      qb[h] = half_bits_to_float(q16[qi + kHalf]);
    } else {
      const float* q32 = static_cast<const float*>(a.q);
      qa[h] = q32[qi];
      qb[h] = q32[qi + kHalf];
    }
  }
  __syncthreads();

  // R(tau) for this lane's token, all 64 pairs, in registers.
  float er[kHalf], ei[kHalf];
#pragma unroll
  for (int i = 0; i < kHalf; ++i) {
    const float2 e = et[i][lane];
    er[i] = e.x;
    ei[i] = e.y;
  }

  const int wave_tile0 = block_tile0 + wave * a.tiles_per_wave;
  const int n_tiles = min(a.tiles_per_wave, (L - wave_tile0 * kTile + kTile - 1) / kTile);
  if (n_tiles <= 0) return;

  // tile-base phase of pair `lane` for the wave's first tile, and its per-tile step
  float bc, bs, sc, ss;
  sincos_rev(frac_rev(static_cast<double>(wave_tile0) * kTile, th_rev), &bs, &bc);
  sincos_rev(frac_rev(static_cast<double>(kTile), th_rev), &ss, &sc);

  const size_t stream = static_cast<size_t>(seq) * H + kvh;
  const uint8_t* recs = a.k_codes + stream * S * (16 * KB);

  auto load_rec = [&](int tile, uint32_t (&w)[kRecWords]) {
    const uint4* p = reinterpret_cast<const uint4*>(recs + (static_cast<size_t>(tile) * kTile + lane) * (16 * KB));
#pragma unroll
    for (int v = 0; v < KB; ++v) {
      const uint4 d = p[v];
      w[4 * v + 0] = d.x;
      w[4 * v + 1] = d.y;
      w[4 * v + 2] = d.z;
      w[4 * v + 3] = d.w;
    }
  };

  uint32_t r0[kRecWords], r1[kRecWords], r2[kRecWords];
  load_rec(wave_tile0, r0);
  if (n_tiles > 1) load_rec(wave_tile0 + 1, r1);

  for (int it = 0; it < n_tiles; ++it) {
    const int tile = wave_tile0 + it;
    if (it + 2 < n_tiles) load_rec(tile + 2, r2);

    // q' = R(-t0) q for every head of the group (lane = pair), then step the base phase.
#pragma unroll
    for (int h = 0; h < G; ++h) qr[wave][h][lane] = make_float2(qa[h] * bc + qb[h] * bs, qb[h] * bc - qa[h] * bs);
    {
      const float nc = bc * sc - bs * ss;
      const float ns = bs * sc + bc * ss;
      bc = nc;
      bs = ns;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    const int t = tile * kTile + lane;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0f;

    static_for<0, kHalf>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      float xa, xb;
      if constexpr (kPairLut) {
        const float2 x = lut[i * kPairEntries + field<2 * KB, 2 * KB * i>(r0)];
        xa = x.x;
        xb = x.y;
      } else {
        xa = lutc[i * kNc + field<KB, 2 * KB * i>(r0)];
        xb = lutc[(i + kHalf) * kNc + field<KB, 2 * KB * i + KB>(r0)];
      }
      const float ya = xa * er[i] - xb * ei[i];
      const float yb = xa * ei[i] + xb * er[i];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float2 qq = qr[wave][h][i];
        acc[h] = fmaf(qq.y, yb, fmaf(qq.x, ya, acc[h]));
      }
    });

    // Outliers: the record holds the zero code at each outlier channel; replace its
    // decoded value zc * s_c by the stored fp16 value.
    if (t < L) {
      const size_t o = (stream * S + t) * k;
      for (int j = 0; j < k; ++j) {
        const int c = a.k_idx[o + j];
        const float dv = half_bits_to_float(a.k_val[o + j]) - zc * ks[c];
        const int i = c & (kHalf - 1);
        const float2 e = et[i][lane];
        const bool upper = c >= kHalf;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float2 qq = qr[wave][h][i];
          acc[h] += dv * (upper ? (qq.y * e.x - qq.x * e.y) : (qq.x * e.x + qq.y * e.y));
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        a.logits[(static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * S + t] = a.sm_scale * acc[h];
      }
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int v = 0; v < kRecWords; ++v) {
      r0[v] = r1[v];
      r1[v] = r2[v];
    }
  }
}

template <int KB, int G>
hipError_t launch_qk_t(int batch, const QkArgs& a0, hipStream_t s) {
  QkArgs a = a0;
  const int tiles = (a.max_len + kTile - 1) / kTile;
  // Enough blocks to fill the GPU at two resident blocks per CU, up to 8 tiles per wave.
  const long streams = static_cast<long>(batch) * a.n_kv_heads;
  int tpw = 1;
  while (tpw < 8 && streams * ((tiles + kWaves * tpw * 2 - 1) / (kWaves * tpw * 2)) >= 1024) tpw *= 2;
  a.tiles_per_wave = tpw;
  dim3 grid((tiles + kWaves * tpw - 1) / (kWaves * tpw), a.n_kv_heads, batch);
  hipLaunchKernelGGL((qk_kernel<KB, G>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk(int k_bits, int group, int batch, const QkArgs& a, hipStream_t s) {
#define KVQ_QK_CASE(KB, G) \
  if (k_bits == KB && group == G) return launch_qk_t<KB, G>(batch, a, s);
  KVQ_QK_CASE(2, 1) KVQ_QK_CASE(2, 2) KVQ_QK_CASE(2, 4) KVQ_QK_CASE(2, 8)
  KVQ_QK_CASE(3, 1) KVQ_QK_CASE(3, 2) KVQ_QK_CASE(3, 4) KVQ_QK_CASE(3, 8)
  KVQ_QK_CASE(4, 1) KVQ_QK_CASE(4, 2) KVQ_QK_CASE(4, 4) KVQ_QK_CASE(4, 8)
#undef KVQ_QK_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
