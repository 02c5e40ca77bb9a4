// Decode-time q . K^T over the compressed key cache, RoPE applied after dequantization.
//
// KVQuant paper note, "Four components" paragraph, item (2): keys are stored before the
// rotary embedding, so the rotation is applied to the dequantized key at each cached
// token's own position; items (1), (3), (4): per-channel scale, per-layer codebook,
// per-vector fp16 outliers.
//
// Mapping: one lane per cached token, one wave per 64-token tile, the 64 rotary pairs of
// the record walked in registers.  The rotation angle (t0 + tau) * theta_i is split into
// a per-tile part, folded into the query once per tile (q' = R(-t0) q, formed from a
// float64 angle so positions up to 2^31 keep full phase accuracy), and a per-lane part
// R(tau), tau < 64, read from a table built once per block.  Logit:
//   l_t = sm_scale * q' . R(tau) k~_t,   k~ = cb[code] * s_c  (+ outlier corrections).
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWavesPerBlock = 4;
constexpr int kTilesPerWave = kQkTokensPerBlock / (kWavesPerBlock * kTile);

template <int KB, int G>
__global__ __launch_bounds__(256) void qk_kernel(QkArgs a) {
  constexpr int kNc = 1 << KB;
  constexpr int kRecWords = 4 * KB;

  __shared__ float cb[kNc];
  __shared__ float ks[kHeadDim];
  __shared__ float2 ksp[kHalf];            // (s_i, s_{i+64})
  __shared__ float2 et[kHalf][kTile];      // R(tau) for pair i: (cos, sin) of tau * theta_i
  __shared__ float qs[G][kHeadDim];        // the group's queries, float32
  __shared__ float2 qr[kWavesPerBlock][G][kHalf];  // per-wave tile-rotated query pairs
  __shared__ float zc;                     // codebook value every outlier slot decodes to

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int H = a.n_kv_heads;
  const int S = a.max_seq;
  const int k = a.n_outliers;
  const int L = min(a.seq_len[seq], a.max_len);
  const int block_t0 = blockIdx.x * kQkTokensPerBlock;
  if (block_t0 >= L) return;

  // ---- per-block tables -----------------------------------------------------------
  if (tid < kNc) cb[tid] = a.k_cb[tid];
  if (tid < kHeadDim) ks[tid] = a.k_scale[kvh * kHeadDim + tid];
  if (tid < kHalf) ksp[tid] = make_float2(a.k_scale[kvh * kHeadDim + tid], a.k_scale[kvh * kHeadDim + tid + kHalf]);
  for (int e = tid; e < G * kHeadDim; e += 256) {
    const int h = e / kHeadDim, c = e % kHeadDim;
    const size_t qi = (static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * kHeadDim + c;
    qs[h][c] = a.q_is_fp16 ? half_bits_to_float(static_cast<const uint16_t*>(a.q)[qi])
                           : static_cast<const float*>(a.q)[qi];
  }
  // theta_i / (2 pi) in float64 for pair i = lane
  const double inv2pi = 0.15915494309189533577;
  const double th = exp2(-static_cast<double>(lane) * a.theta_log2);
  const double th_rev = th * inv2pi;
  {
    // Each thread fills 16 consecutive tau of pair `lane`: one accurate seed angle, then
    // exact-enough steps by the single-step rotation (<= 15 float32 rotations).
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
  if (tid == 0) {
    int j0 = 0;
    float bd = fabsf(0.0f - a.k_cb[0]);
    for (int j = 1; j < kNc; ++j) {
      const float d = fabsf(0.0f - a.k_cb[j]);
      if (d < bd) {
        bd = d;
        j0 = j;
      }
    }
    zc = a.k_cb[j0];
  }
  __syncthreads();

  const size_t stream = static_cast<size_t>(seq) * H + kvh;
  const uint8_t* recs = a.k_codes + stream * S * (16 * KB);

  for (int it = 0; it < kTilesPerWave; ++it) {
    const int t0 = block_t0 + (it * kWavesPerBlock + wave) * kTile;
    if (t0 >= L) break;

    // q' = R(-t0) q for every head of the group; lane = pair.
    {
      float s, c;
      sincos_rev(frac_rev(static_cast<double>(t0), th_rev), &s, &c);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float qa = qs[h][lane], qb = qs[h][lane + kHalf];
        qr[wave][h][lane] = make_float2(qa * c + qb * s, qb * c - qa * s);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    const int t = t0 + lane;
    uint32_t w[kRecWords];
    {
      const uint4* p = reinterpret_cast<const uint4*>(recs + static_cast<size_t>(t) * (16 * KB));
#pragma unroll
      for (int v = 0; v < KB; ++v) {
        const uint4 d = p[v];
        w[4 * v + 0] = d.x;
        w[4 * v + 1] = d.y;
        w[4 * v + 2] = d.z;
        w[4 * v + 3] = d.w;
      }
    }

    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = 0.0f;

    static_for<0, kHalf>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const float xa = cb[field<KB, 2 * KB * i>(w)] * ksp[i].x;
      const float xb = cb[field<KB, 2 * KB * i + KB>(w)] * ksp[i].y;
      const float2 e = et[i][lane];
      const float ya = xa * e.x - xb * e.y;
      const float yb = xa * e.y + xb * e.x;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float2 qq = qr[wave][h][i];
        acc[h] += qq.x * ya + qq.y * yb;
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
  }
}

template <int KB, int G>
hipError_t launch_qk_t(int batch, const QkArgs& a, hipStream_t s) {
  dim3 grid((a.max_len + kQkTokensPerBlock - 1) / kQkTokensPerBlock, a.n_kv_heads, batch);
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
