// Decode-time q . K^T over the compressed key cache for one query head per kv head
// (g = 1), with RoPE applied to each dequantized key at its own position.
//
// KVQuant paper note, "Four components" paragraph, item (2): keys are cached before the
// rotary embedding; items (1), (3), (4): per-channel scale, per-layer codebook, per-vector
// fp16 outliers.
//
// With a single query the rotated-query coefficients and the codebook fold into one
// table per group of tiles.  For rotary pair i of a key at position t = T0 + tau (T0 the
// first token of a super-tile of kWaves x 64 tokens, tau < 64 kWaves) with codes a (channel
// i) and b (channel i + 64):
//   q . R(t) k = E_r(tau) A_i[a, b] + E_i(tau) B_i[a, b]
//   A_i = s_i cb[a] p_a + s_{i+64} cb[b] p_b,  B_i = s_i cb[a] p_b - s_{i+64} cb[b] p_a
// where (p_a, p_b) = R(-T0 theta_i) (q_i, q_{i+64}) and E(tau) = (cos, sin)(tau theta_i).
// Lane = token: each lane keeps E(tau) of its own tau for all 64 pairs in registers, so a
// pair costs one field extraction, one 8-byte table read and two FMAs.  The waves of a block
// share the table of the super-tile: they build the next one (double-buffered) while
// each computes its tile of the current one, with one block barrier per super-tile.
// Outliers replace the zero code decoded at their channel: their correction uses the
// hardware sine/cosine (argument in revolutions) at the outlier's pair.
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kLutWaves = 8;                 // waves per block = tiles per super-tile
constexpr int kLutThreads = 64 * kLutWaves;
constexpr int kLutPrefetchOutliers = 2;      // outliers per token fetched with the record

template <int KB>
struct LutShape {
  static constexpr int kNc = 1 << KB;
  static constexpr int kNe = kNc * kNc;               // code pairs (a | b << KB) per rotary pair
  static constexpr int kBufs = 2;                     // double-buffered (2- and 3-bit codes only)
  static constexpr int kBufBytes = kHalf * kNe * 8;   // 64 rows of (A, B) float pairs
};

template <int KB>
struct LutRec {
  uint32_t w[4 * KB];     // the token's key record
  uint32_t oi[2], ov[2];  // its first two outliers: channels and fp16 value bits
};

// kExtra: outliers beyond the first kLutPrefetchOutliers per token exist (read in a loop
// of their own); without them that loop is compiled out.
template <int KB, bool kExtra>
__global__ __launch_bounds__(kLutThreads) void qk_lut_kernel(QkArgs a) {
  using Sh = LutShape<KB>;
  constexpr int kNc = Sh::kNc;
  constexpr int kNe = Sh::kNe;

  extern __shared__ __align__(16) unsigned char lds[];
  float2* lut = reinterpret_cast<float2*>(lds);                            // [bufs][64][kNe] (A, B)
  float* ks = reinterpret_cast<float*>(lds + Sh::kBufs * Sh::kBufBytes);   // [128] key scales
  float2* pab = reinterpret_cast<float2*>(ks + kHeadDim);                  // [bufs][64] (p_a, p_b)
  float2* thl = pab + Sh::kBufs * kHalf;                                   // [64] theta_i/2pi split hi, lo

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int H = a.n_kv_heads;
  const int S = a.max_seq;
  const int k = a.n_outliers;
  const int L = min(a.seq_len[seq] & kLenMask, a.max_len);
  const int n_tiles = (L + kTile - 1) / kTile;
  const int n_super = (n_tiles + kLutWaves - 1) / kLutWaves;
  const int s_lo = blockIdx.x * a.tiles_per_wave;  // super-tiles per block, set by the launcher
  const int s_hi = min(s_lo + a.tiles_per_wave, n_super);
  if (s_lo >= s_hi) return;  // block-uniform

  const size_t stream = static_cast<size_t>(seq) * H + kvh;
  const uint8_t* recs = a.k_codes + stream * S * (16 * KB);
  const int tile_cap = S / kTile - 1;
  const int tau = kTile * wave + lane;  // position of this lane's token inside a super-tile

  // The first kLutPrefetchOutliers outliers of every token travel with its record; with
  // fewer outliers the spare loads repeat a real one or read the first code word, and
  // their results are ignored.
  const int kp = min(k, kLutPrefetchOutliers);
  const uint8_t* o_idx = kp > 0 ? a.k_idx : a.k_codes;
  const uint16_t* o_val = kp > 0 ? a.k_val : reinterpret_cast<const uint16_t*>(a.k_codes);
  const size_t o_stride = kp > 0 ? k : 0;
  const int o_second = kp > 1 ? 1 : 0;

  // Every call issues the same loads at valid addresses (super-tile clamped to the block's
  // range, tile to the buffer), so the compiler counts the loads in flight exactly.  The
  // loads go through buffer descriptors rebuilt per tile at the tile's first token (scalar
  // arithmetic), with fixed per-lane offsets, so they cost no vector instructions.
  const uint32_t rec_off = static_cast<uint32_t>(lane) * (16 * KB);
  const uint32_t out_off = static_cast<uint32_t>(lane * o_stride);  // outlier entries before this lane's
  const uint32_t second_off = out_off + o_second;
  const uint32_t tile_outs = static_cast<uint32_t>(kTile * o_stride);  // outlier entries of a tile
  auto load_rec = [&](int s, LutRec<KB>& d) {
    s = min(s, s_hi - 1);
    const int tile = min(kLutWaves * s + wave, tile_cap);  // wave-uniform
    const size_t tok0 = static_cast<size_t>(tile) * kTile;
    const __amdgpu_buffer_rsrc_t rr = make_rsrc(recs + tok0 * (16 * KB), kTile * 16 * KB);
#pragma unroll
    for (int v = 0; v < KB; ++v) {
      const u32x4 q = buf_load_b128(rr, rec_off + 16 * v);
      d.w[4 * v + 0] = q.x;
      d.w[4 * v + 1] = q.y;
      d.w[4 * v + 2] = q.z;
      d.w[4 * v + 3] = q.w;
    }
    const size_t slot0 = (stream * S + tok0) * o_stride;
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(o_idx + slot0, tile_outs + 1);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(o_val + slot0, 2 * tile_outs + 2);
    d.oi[0] = buf_load_u8(ri, out_off);
    d.oi[1] = buf_load_u8(ri, second_off);
    d.ov[0] = buf_load_u16(rv, 2 * out_off);
    d.ov[1] = buf_load_u16(rv, 2 * second_off);
  };

  // ---- set-up inputs, then the first two records ---------------------------------------
  // Lane l of wave w prepares the table coefficients of one of the eight pairs w + 8 m
  // whose rows the wave fills, placed for the DPP row broadcasts of the build: 3-bit rows,
  // m = l & 7 (lane m of every 16-lane row holds pair w + 8 m); 2-bit rows, lane 16 r + f
  // prepares m = 4 f + r (fill step f finds its row's pair at lane f of the row).
  const int P = KB == 3 ? wave + kLutWaves * (lane & 7) : wave + kLutWaves * ((lane >> 4) + 4 * (lane & 1));
  const bool writes_pab = KB == 3 ? lane < 8 : (lane & 14) == 0;  // one lane per pair
  const size_t qbase = (static_cast<size_t>(seq) * a.n_q_heads + kvh) * kHeadDim;
  uint32_t qraw[2];
  if (a.q_is_fp16) {  // wave-uniform; both paths issue the same loads
    const uint16_t* q16 = static_cast<const uint16_t*>(a.q) + qbase;
    qraw[0] = q16[P];
    qraw[1] = q16[P + kHalf];
  } else {
    const uint32_t* q32 = static_cast<const uint32_t*>(a.q) + qbase;
    qraw[0] = q32[P];
    qraw[1] = q32[P + kHalf];
  }
  const float ks_own = a.k_scale[kvh * kHeadDim + (tid & (kHeadDim - 1))];
  const uint32_t cb_lane = a.k_cb[lane & (kNc - 1)];
  const double th_P = a.theta_rev[P];
  const float2 th_split = make_float2(a.th_hi[lane], a.th_lo[lane]);

  LutRec<KB> r0, r1, r2;
  load_rec(s_lo, r0);
  load_rec(s_lo + 1, r1);

  ks[tid & (kHeadDim - 1)] = ks_own;  // threads sharing an entry write the same value
  thl[lane] = th_split;
  float qv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) qv[j] = a.q_is_fp16 ? half_bits_to_float(qraw[j]) : __builtin_bit_cast(float, qraw[j]);
  const float zc = zero_code_value<kNc>(cb_lane, lane);  // value every outlier slot decodes to
  // codebook values this lane's table entries use: entry e = a | b << KB
  float cba[1], cbb;
  {
    const int e0 = KB == 3 ? lane : (lane & 15);
#pragma unroll
    for (int j = 0; j < 1; ++j) cba[j] = half_bits_to_float(__shfl(static_cast<int>(cb_lane), (e0 + j) & (kNc - 1)) & 0xffffu);
    cbb = half_bits_to_float(__shfl(static_cast<int>(cb_lane), (e0 >> KB) & (kNc - 1)) & 0xffffu);
  }

  // E(tau) for all 64 pairs: the argument tau theta_i / 2pi is formed exactly (tau < 512
  // times the 15-bit leading part of theta_i / 2pi) plus the small remainder term.
  float er[kHalf], ei[kHalf];
  const float tauf = static_cast<float>(tau);
#pragma unroll
  for (int i = 0; i < kHalf; ++i) {
    const float ph = fmaf(tauf, a.th_lo[i], __builtin_amdgcn_fractf(tauf * a.th_hi[i]));
    er[i] = __builtin_amdgcn_cosf(ph);
    ei[i] = __builtin_amdgcn_sinf(ph);
  }
  block_lds_barrier();  // ks, thl visible
  const float sP_lo = ks[P], sP_hi = ks[P + kHalf];

  // ---- table build for super-tile s into buffer b -------------------------------------
  auto build = [&](int s, int b) {
    const double t0 = static_cast<double>(s) * (kLutWaves * kTile);
    float2* T = lut + b * (Sh::kBufBytes / 8);
    auto coef = [&](double th, float qa, float qb, float s_lo, float s_hi, float4& c, float2& p) {
      const float r = frac_rev(t0, th);
      const float cs = __builtin_amdgcn_cosf(r), sn = __builtin_amdgcn_sinf(r);
      const float pa = qa * cs + qb * sn;  // R(-t0 theta) q
      const float pb = qb * cs - qa * sn;
      c = make_float4(s_lo * pa, s_lo * pb, s_hi * pb, -(s_hi * pa));  // alpha, beta, gamma, -delta
      p = make_float2(pa, pb);
    };
    float4 c1;
    float2 p1;
    coef(th_P, qv[0], qv[1], sP_lo, sP_hi, c1, p1);
    if (writes_pab) pab[b * kHalf + P] = p1;
    static_assert(KB == 2 || KB == 3, "2- and 3-bit keys");
    if constexpr (KB == 3) {
      // wave w fills the rows of pairs w + 8 m, m < 8; lane m of every 16-lane row holds
      // their coefficients (lane l prepares pair w + 8 (l & 7)) and hands them over by DPP
      // row broadcast inside the multiplies
      float4 cc = c1;
      // at least two wait states between these VALU writes and their DPP reads
      asm volatile("s_nop 1" : "+v"(cc.x), "+v"(cc.y), "+v"(cc.z), "+v"(cc.w));
      static_for<0, 8>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        T[(wave + kLutWaves * m) * kNe + lane] = lut_entry_bcast<m>(cc.x, cc.y, cc.z, cc.w, cba[0], cbb);
      });
    } else {
      // 16 entries per row: fill step f covers the rows of 4 pairs, m = 4 f + (lane >> 4),
      // whose coefficients lane f of each 16-lane row holds (DPP row broadcast).
      float4 cc = c1;
      // at least two wait states between these VALU writes and their DPP reads
      asm volatile("s_nop 1" : "+v"(cc.x), "+v"(cc.y), "+v"(cc.z), "+v"(cc.w));
      static_for<0, 2>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        const int i = wave + kLutWaves * (4 * f + (lane >> 4));
        T[i * kNe + (lane & 15)] = lut_entry_bcast<f>(cc.x, cc.y, cc.z, cc.w, cba[0], cbb);
      });
    }
  };

  // ---- one tile of super-tile s from buffer b ------------------------------------------
  auto compute = [&](int s, int b, const LutRec<KB>& d) {
    const uint32_t T = lds_address(lut + b * (Sh::kBufBytes / 8));
    const unsigned char* lb = lds - lds_address(lds);  // LDS address -> pointer
    // Software-pipelined over batches of kBatch pairs: the table reads of batch j + 1 are
    // issued before the FMAs of batch j, so each read's latency is covered by a batch of
    // arithmetic (the scheduling barriers keep the compiler from re-serializing them).
    constexpr int kBatch = 8;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float va[2][kBatch], vb[2][kBatch];
    auto issue = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      static_for<0, kBatch>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int i = j * kBatch + u;
        const float2 v = *reinterpret_cast<const float2*>(lb + field_addr<2 * KB, 2 * KB * i, 3>(d.w, T) + i * kNe * 8);
        va[j & 1][u] = v.x;
        vb[j & 1][u] = v.y;
      });
    };
    auto consume = [&](auto jc) {
      constexpr int j = decltype(jc)::value;
      static_for<0, kBatch>([&](auto uc) {
        constexpr int u = decltype(uc)::value;
        constexpr int i = j * kBatch + u;
        acc[u & 3] = fmaf(er[i], va[j & 1][u], fmaf(ei[i], vb[j & 1][u], acc[u & 3]));
      });
    };
    issue(std::integral_constant<int, 0>{});
    static_for<1, kHalf / kBatch>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      issue(jc);
      __builtin_amdgcn_sched_barrier(0);
      consume(std::integral_constant<int, j - 1>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    consume(std::integral_constant<int, kHalf / kBatch - 1>{});
    float l = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    // Outliers: the record holds the zero code at each outlier channel; replace its decoded
    // value zc * s_c by the stored fp16 value at the channel's rotated query coefficient.
    auto add_outlier = [&](uint32_t c, uint32_t vbits) {
      const bool used = c != kNoOutlier;  // an unused slot (per-channel rule) adds nothing
      c &= kHeadDim - 1;                  // a token past the length may hold stale bytes
      const int i = c & (kHalf - 1);
      const float dv = used ? half_bits_to_float(vbits) - zc * ks[c] : 0.0f;
      const float2 th = thl[i];
      const float ph = fmaf(tauf, th.y, __builtin_amdgcn_fractf(tauf * th.x));
      const float cs = __builtin_amdgcn_cosf(ph), sn = __builtin_amdgcn_sinf(ph);
      const float2 p = pab[b * kHalf + i];
      l += dv * (c < kHalf ? (p.x * cs + p.y * sn) : (p.y * cs - p.x * sn));
    };
    if (kp >= 1) add_outlier(d.oi[0], d.ov[0]);
    if (kp >= 2) add_outlier(d.oi[1], d.ov[1]);
    const int t0 = (kLutWaves * s + wave) * kTile;  // wave-uniform
    const int t = t0 + lane;
    if (t < L) {
      if constexpr (kExtra) {
        const size_t o = (stream * S + t) * k;
        for (int j = kLutPrefetchOutliers; j < k; ++j) add_outlier(a.k_idx[o + j], a.k_val[o + j]);
      }
      (a.logits + (static_cast<size_t>(seq) * a.n_q_heads + kvh) * S + t0)[lane] = a.sm_scale * l;
    }
  };

  // ---- main loop -----------------------------------------------------------------------
  build(s_lo, 0);
  block_lds_barrier();
  auto step = [&](int s, LutRec<KB>& cur, LutRec<KB>& next2) {
    const int b = (s - s_lo) & 1;
    load_rec(s + 2, next2);
    if (s + 1 < s_hi) build(s + 1, b ^ 1);
    compute(s, b, cur);
    block_lds_barrier();
  };
  for (int s = s_lo; s < s_hi; s += 3) {
    step(s, r0, r2);
    if (s + 1 >= s_hi) break;
    step(s + 1, r1, r0);
    if (s + 2 >= s_hi) break;
    step(s + 2, r2, r1);
  }
}

template <int KB, bool kExtra>
hipError_t launch_qk_lut_t(int batch, const QkArgs& a0, hipStream_t st) {
  using Sh = LutShape<KB>;
  QkArgs a = a0;
  const size_t lds = Sh::kBufs * Sh::kBufBytes + kHeadDim * 4 + Sh::kBufs * kHalf * 8 + kHalf * 8;
  static const bool attr_ok = hipFuncSetAttribute(reinterpret_cast<const void*>(&qk_lut_kernel<KB, kExtra>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  static_cast<int>(lds)) == hipSuccess;
  if (!attr_ok) return hipErrorInvalidValue;
  // One resident round: the device's block slots shared equally among the streams, each
  // block walking a contiguous run of super-tiles.
  const int tiles = (a.max_len + kTile - 1) / kTile;
  const int supers = (tiles + kLutWaves - 1) / kLutWaves;
  const long streams = static_cast<long>(batch) * a.n_kv_heads;
  static const int resident = [&] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&qk_lut_kernel<KB, kExtra>),
                                                     kLutThreads, lds) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  const long slots = static_cast<long>(device_cu_count()) * resident;
  const long per_stream = std::max(1L, std::min<long>((slots + streams - 1) / streams, supers));
  a.tiles_per_wave = static_cast<int>((supers + per_stream - 1) / per_stream);  // super-tiles per block
  dim3 grid((supers + a.tiles_per_wave - 1) / a.tiles_per_wave, a.n_kv_heads, batch);
  hipLaunchKernelGGL((qk_lut_kernel<KB, kExtra>), grid, dim3(kLutThreads), lds, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_lut(int k_bits, int batch, const QkArgs& a, hipStream_t s) {
  const bool extra = a.n_outliers > kLutPrefetchOutliers;
  if (k_bits == 2) return extra ? launch_qk_lut_t<2, true>(batch, a, s) : launch_qk_lut_t<2, false>(batch, a, s);
  if (k_bits == 3) return extra ? launch_qk_lut_t<3, true>(batch, a, s) : launch_qk_lut_t<3, false>(batch, a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
