// Decode-time q . K^T over the compressed key cache, RoPE applied after dequantization.
//
// KVQuant paper note, "Four components" paragraph, item (2): keys are stored before the
// rotary embedding, so the rotation is applied to the dequantized key at each cached
// token's own position; items (1), (3), (4): per-channel scale, per-layer codebook,
// per-vector fp16 outliers.
//
// Mapping: one lane per cached token, one wave per 64-token tile, each wave walking a
// contiguous run of tiles with the records of the next two tiles in flight.  The angle
// (t0 + tau) * theta_i is split into
//   * R(-t0), folded into the query once per tile (lane i handles rotary pair i; the
//     tile-base phase is formed once per wave from a float64 angle and then advanced by
//     the fixed step 64 * theta_i), and
//   * R(tau), tau = lane < 64, from a per-block table (the first KVQ_QK_REG_PAIRS pairs
//     copied into registers, the rest read from LDS).
// The record keeps the two halves of rotary pair i side by side, so one 2b-bit field
// indexes a small shared table of fp16 pairs (cb[a], cb[b]); the fp16 values feed
// mixed-precision FMAs directly (exact conversion).  With one query head per kv head the
// per-channel key scale is folded into four per-(tile, pair) coefficients of the rotated
// query:
//   l += cb[a] * (s_i q'_i E_r + s_i q'_{i+64} E_i) + cb[b] * (s_{i+64} q'_{i+64} E_r - s_{i+64} q'_i E_i)
// (8 VALU ops per token and pair); the four coefficients reach the lanes through DPP row
// broadcasts inside the multiplies, so the pair loop reads LDS only for the table lookup
// (and R(tau) when it is not in registers).  With g > 1 query heads the key is dequantized and rotated once and
// dotted with every head (8 + 2g ops).
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

#ifndef KVQ_QK_REG_PAIRS
#define KVQ_QK_REG_PAIRS 0
#endif

namespace kvq {
namespace {

// One rotary pair's contribution for g = 1, in a single block so that the scheduler
// keeps the six operations next to the table entry they consume:
//   P = alpha E_r + beta E_i,  Q = gamma E_r + ndelta E_i,  acc += cb_a P + cb_b Q.
// alpha, beta, gamma, ndelta are read from lane N of the lane's 16-lane row (DPP
// row_newbcast), so one register per coefficient serves 16 pairs.  e2 holds the fp16
// pair (cb_a, cb_b), consumed directly by the mixed-precision FMAs.  The DPP sources
// must have been written at least two wait states earlier (see the fence where the
// coefficients are formed).
template <int N>
__device__ __forceinline__ float pair_term(float acc, uint32_t e2, float er, float ei, float al, float be,
                                           float ga, float nd) {
  float p, q;
  asm("v_mul_f32_dpp %1, %4, %8 row_newbcast:%10 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %2, %6, %8 row_newbcast:%10 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %1, %5, %9 row_newbcast:%10 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %2, %7, %9 row_newbcast:%10 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fma_mix_f32 %0, %3, %1, %0 op_sel_hi:[1,0,0]\n\t"
      "v_fma_mix_f32 %0, %3, %2, %0 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
      : "+v"(acc), "=&v"(p), "=&v"(q)
      : "v"(e2), "v"(al), "v"(be), "v"(ga), "v"(nd), "v"(er), "v"(ei), "i"(N));
  return acc;
}

constexpr int kWaves = 4;
constexpr int kPartials = 4;  // partial sums per logit
constexpr int kRegPairs = KVQ_QK_REG_PAIRS;
static_assert(kRegPairs >= 0 && kRegPairs <= kHalf, "register pairs out of range");

template <int KB, int G>
__global__ __launch_bounds__(256) void qk_kernel(QkArgs a) {
  constexpr int kNc = 1 << KB;
  constexpr int kRecWords = 4 * KB;
  constexpr int kPairEntries = 1 << (2 * KB);
  constexpr bool kFoldScale = G == 1;

  __shared__ float2 et[kHalf][kTile];       // R(tau) for pair i: (cos, sin) of tau * theta_i
  __shared__ uint32_t lutp[kPairEntries];   // fp16 (cb[a], cb[b]) for a pair field a | b << KB
  __shared__ float ks[kHeadDim];
  __shared__ float2 ksp[kHalf];             // (s_i, s_{i+64})
  __shared__ float2 qr[kWaves][G][kHalf];   // per-wave tile-rotated query pairs
  __shared__ float cbs[kNc];
  __shared__ float zc;                      // value every outlier slot decodes to

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int H = a.n_kv_heads;
  const int S = a.max_seq;
  const int k = a.n_outliers;
  const int L = min(a.seq_len[seq] & kLenMask, a.max_len);
  const int block_tile0 = blockIdx.x * a.tiles_per_wave * kWaves;
  if (block_tile0 * kTile >= L) return;

  // ---- per-block tables -----------------------------------------------------------
  if (tid < kHeadDim) ks[tid] = a.k_scale[kvh * kHeadDim + tid];
  if (tid < kHalf) ksp[tid] = make_float2(a.k_scale[kvh * kHeadDim + tid], a.k_scale[kvh * kHeadDim + tid + kHalf]);
  if (tid < kNc) cbs[tid] = half_bits_to_float(a.k_cb[tid]);
  for (int e = tid; e < kPairEntries; e += 256)
    lutp[e] = static_cast<uint32_t>(a.k_cb[e & (kNc - 1)]) | (static_cast<uint32_t>(a.k_cb[e >> KB]) << 16);
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
  // Query pairs this lane rotates every tile.  Slot j holds rotary pair
  // (lane & 15) + 16 j, so lane n of every 16-lane row holds the pairs congruent to n mod
  // 16 and a row broadcast hands pair i's coefficient to all lanes.  The pair `lane` itself
  // (needed in LDS) is slot lane >> 4.
  constexpr int kSlots = kHalf / 16;
  float qa[kSlots][G], qb[kSlots][G];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int pr = (lane & 15) + 16 * j;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const size_t qi = (static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * kHeadDim + pr;
      if (a.q_is_fp16) {
        const uint16_t* q16 = static_cast<const uint16_t*>(a.q);
        qa[j][h] = half_bits_to_float(q16[qi]);
        qb[j][h] = half_bits_to_float(q16[qi + kHalf]);
      } else {
        const float* q32 = static_cast<const float*>(a.q);
        qa[j][h] = q32[qi];
        qb[j][h] = q32[qi + kHalf];
      }
    }
  }
  __syncthreads();
  if (tid == 0) zc = cbs[zero_code_index<kNc>(cbs)];
  float s_lo[kSlots], s_hi[kSlots];  // scales of the slot pairs
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    s_lo[j] = ks[(lane & 15) + 16 * j];
    s_hi[j] = ks[(lane & 15) + 16 * j + kHalf];
  }

  // R(tau) for this lane's token: the first kRegPairs pairs in registers.
  float er[kRegPairs > 0 ? kRegPairs : 1], ei[kRegPairs > 0 ? kRegPairs : 1];
#pragma unroll
  for (int i = 0; i < kRegPairs; ++i) {
    const float2 e = et[i][lane];
    er[i] = e.x;
    ei[i] = e.y;
  }
  __syncthreads();

  const int wave_tile0 = block_tile0 + wave * a.tiles_per_wave;
  const int n_tiles = min(a.tiles_per_wave, (L - wave_tile0 * kTile + kTile - 1) / kTile);
  if (n_tiles <= 0) return;

  // tile-base phase of every slot pair for the wave's first tile, and its per-tile step
  float bc[kSlots], bs[kSlots], sc[kSlots], ss[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const double thj = exp2(-static_cast<double>((lane & 15) + 16 * j) * a.theta_log2) * inv2pi;
    sincos_rev(frac_rev(static_cast<double>(wave_tile0) * kTile, thj), &bs[j], &bc[j]);
    sincos_rev(frac_rev(static_cast<double>(kTile), thj), &ss[j], &sc[j]);
  }
  const int my_slot = lane >> 4;
  static_assert(kSlots == 4, "four 16-lane rows");
  auto pick = [&](float v0, float v1, float v2, float v3) {
    return my_slot == 0 ? v0 : my_slot == 1 ? v1 : my_slot == 2 ? v2 : v3;
  };

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

  auto process = [&](int tile, const uint32_t (&r)[kRecWords]) {
    // q' = R(-t0) q for the slot pairs of every head, then step the base phases.
    float alp[kSlots], bet[kSlots], gam[kSlots], ndl[kSlots];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float pa[kSlots], pb[kSlots];
#pragma unroll
      for (int j = 0; j < kSlots; ++j) {
        pa[j] = qa[j][h] * bc[j] + qb[j][h] * bs[j];
        pb[j] = qb[j][h] * bc[j] - qa[j][h] * bs[j];
      }
      const float pa_l = pick(pa[0], pa[1], pa[2], pa[3]), pb_l = pick(pb[0], pb[1], pb[2], pb[3]);
      qr[wave][h][lane] = make_float2(pa_l, pb_l);
      if constexpr (kFoldScale) {
#pragma unroll
        for (int j = 0; j < kSlots; ++j) {
          alp[j] = s_lo[j] * pa[j];
          bet[j] = s_lo[j] * pb[j];
          gam[j] = s_hi[j] * pb[j];
          ndl[j] = -(s_hi[j] * pa[j]);
        }
        // at least two wait states between these VALU writes and their DPP reads
        asm volatile("s_nop 1"
                     : "+v"(alp[0]), "+v"(alp[1]), "+v"(alp[2]), "+v"(alp[3]), "+v"(bet[0]), "+v"(bet[1]),
                       "+v"(bet[2]), "+v"(bet[3]), "+v"(gam[0]), "+v"(gam[1]), "+v"(gam[2]), "+v"(gam[3]),
                       "+v"(ndl[0]), "+v"(ndl[1]), "+v"(ndl[2]), "+v"(ndl[3]));
      }
    }
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const float nc = bc[j] * sc[j] - bs[j] * ss[j];
      const float ns = bs[j] * sc[j] + bc[j] * ss[j];
      bc[j] = nc;
      bs[j] = ns;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");

    const int t = tile * kTile + lane;
    // Independent partial sums keep the FMA chains short, so the scheduler interleaves
    // pairs instead of computing every rotated pair before the first accumulation.
    float accp[G][kPartials];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int u = 0; u < kPartials; ++u) accp[h][u] = 0.0f;

    static_for<0, kHalf>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint32_t e2 = lutp[field<2 * KB, 2 * KB * i>(r)];
      float cr, ci;
      if constexpr (i < kRegPairs) {
        cr = er[i];
        ci = ei[i];
      } else {
        const float2 e = et[i][lane];
        cr = e.x;
        ci = e.y;
      }
      if constexpr (kFoldScale) {
        accp[0][i % kPartials] =
            pair_term<i % 16>(accp[0][i % kPartials], e2, cr, ci, alp[i / 16], bet[i / 16], gam[i / 16], ndl[i / 16]);
      } else {
        const float cb_a = half_bits_to_float(e2 & 0xffffu);
        const float cb_b = half_bits_to_float(e2 >> 16);
        const float2 sp = ksp[i];
        const float xa = cb_a * sp.x;
        const float xb = cb_b * sp.y;
        const float ya = xa * cr - xb * ci;
        const float yb = xa * ci + xb * cr;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float2 qq = qr[wave][h][i];
          accp[h][i % kPartials] = fmaf(qq.y, yb, fmaf(qq.x, ya, accp[h][i % kPartials]));
        }
      }
    });

    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      acc[h] = accp[h][0];
#pragma unroll
      for (int u = 1; u < kPartials; ++u) acc[h] += accp[h][u];
    }

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
  };

  // Three record buffers: the tiles it+1 and it+2 are in flight while tile it is used.
  uint32_t r0[kRecWords], r1[kRecWords], r2[kRecWords];
  load_rec(wave_tile0, r0);
  if (n_tiles > 1) load_rec(wave_tile0 + 1, r1);
  for (int it = 0; it < n_tiles; it += 3) {
    if (it + 2 < n_tiles) load_rec(wave_tile0 + it + 2, r2);
    process(wave_tile0 + it, r0);
    if (it + 1 >= n_tiles) break;
    if (it + 3 < n_tiles) load_rec(wave_tile0 + it + 3, r0);
    process(wave_tile0 + it + 1, r1);
    if (it + 2 >= n_tiles) break;
    if (it + 4 < n_tiles) load_rec(wave_tile0 + it + 4, r1);
    process(wave_tile0 + it + 2, r2);
  }
}

template <int KB, int G>
hipError_t launch_qk_t(int batch, const QkArgs& a0, hipStream_t s) {
  QkArgs a = a0;
  // One resident round: every (sequence, kv head) stream gets an equal share of the
  // device's block slots, and each block walks a contiguous run of tiles (4 waves x
  // tiles_per_wave), so the per-block tables are amortised over long runs.
  const int tiles = (a.max_len + kTile - 1) / kTile;
  const long streams = static_cast<long>(batch) * a.n_kv_heads;
  static const int resident = blocks_per_cu(reinterpret_cast<const void*>(&qk_kernel<KB, G>), 256);
  const long slots = static_cast<long>(device_cu_count()) * resident;
  const long per_stream = std::max(1L, std::min<long>((slots + streams - 1) / streams, (tiles + kWaves - 1) / kWaves));
  const int tpw = static_cast<int>((tiles + per_stream * kWaves - 1) / (per_stream * kWaves));
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
