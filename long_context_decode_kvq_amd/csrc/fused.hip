// Single-pass decode attention for one query head per kv head: q . K^T, online softmax
// and softmax . V over the compressed cache in one kernel, split over the sequence and
// merged by the log-sum-exp combine.
//
// KVQuant paper note, "Four components" paragraph, items (1)-(4), and the summary page,
// abstract paragraph: keys are dequantized through the per-layer codebook and per-channel
// scale and rotated at their own positions, values through the codebook and per-vector
// scale, and both add back their fp16 outliers.  The logits never leave the chip: each
// wave turns the logits of its own 64-token tile into softmax weights and accumulates the
// tile's values at once.
//
// Key side as the table-driven q . K^T kernel: 8 waves, super-tiles of 8 tiles, a table of
// (A, B) per rotary pair and code pair for each super-tile (double-buffered, built by all
// waves while they compute the current one), lane = token with E(tau) in registers.
// Value side as the softmax . V kernel: lane = token for the wave's running (max, sum) and
// the token weights, lane = channel pair for the packed fp16 dot products against the
// codebook-pair table; the first two value outliers of each token summed per tile in
// fixed point with integer LDS atomics.  Records and value tiles of the next super-tile
// are in flight while the current one is computed.  At the end the 8 waves merge their
// (max, sum, o) and the block writes one partial.
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kFuseWaves = 8;  // waves per block = tiles per super-tile
constexpr int kFuseThreads = kWave * kFuseWaves;
constexpr int kFuseOutliers = 2;  // outliers per token fetched with its record / tile

template <int KB>
struct FuseShape {
  static constexpr int kNc = 1 << KB;
  static constexpr int kNe = kNc * kNc;              // code pairs (a | b << KB) per rotary pair
  static constexpr int kBufBytes = kHalf * kNe * 8;  // 64 rows of (A, B) float pairs
};

template <int KB>
struct KeyRec {
  uint32_t w[4 * KB];     // the token's key record
  uint32_t oi[2], ov[2];  // its first two key outliers: channels and fp16 value bits
};

template <int VB>
struct ValRec {
  uint32_t w[4 * VB];     // this lane's value-tile words (channels 2l, 2l+1)
  uint32_t sv;            // fp16 value scale of token `lane`
  uint32_t oi[2], ov[2];  // its first two value outliers
};

template <int KB, int VB>
__global__ __launch_bounds__(kFuseThreads) void fused_decode_kernel(QkArgs a, PvArgs pa) {
  using Sh = FuseShape<KB>;
  constexpr int kNc = Sh::kNc;
  constexpr int kNe = Sh::kNe;
  constexpr int kNcV = 1 << VB;
  constexpr int kChanBits = 64 * VB;
  constexpr int kPairEntries = 1 << (2 * VB);

  extern __shared__ __align__(16) unsigned char lds[];
  float2* lut = reinterpret_cast<float2*>(lds);                         // [2][64][kNe] (A, B)
  float* ks = reinterpret_cast<float*>(lds + 2 * Sh::kBufBytes);        // [128] key scales
  float2* pab = reinterpret_cast<float2*>(ks + kHeadDim);               // [2][64] (p_a, p_b)
  float2* thl = pab + 2 * kHalf;                                        // [64] theta_i/2pi split hi, lo
  uint32_t* lut2 = reinterpret_cast<uint32_t*>(thl + kHalf);            // fp16 (cb[a], cb[b]) per token pair
  int* osi = reinterpret_cast<int*>(lut2 + kPairEntries);               // [8][128] fixed-point outlier sums
  float* wo = reinterpret_cast<float*>(osi + kFuseWaves * kHeadDim);    // [8][128] per-wave sums
  float* wml = wo + kFuseWaves * kHeadDim;                              // [8][2] per-wave max, sum

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
  const int n_super = (n_tiles + kFuseWaves - 1) / kFuseWaves;
  const int s_lo = blockIdx.x * a.tiles_per_wave;  // super-tiles per block, set by the launcher
  const int s_hi = min(s_lo + a.tiles_per_wave, n_super);
  if (s_lo >= s_hi) {  // block-uniform: an empty part (m = -inf), as the combine reads every part
    if (threadIdx.x < kHeadDim + 2) {
      float* dst = pa.partial + ((static_cast<size_t>(seq) * a.n_q_heads + kvh) * pa.n_parts + blockIdx.x) * (kHeadDim + 2);
      dst[threadIdx.x] = threadIdx.x == kHeadDim ? -INFINITY : 0.0f;
    }
    return;
  }

  const size_t stream = static_cast<size_t>(seq) * H + kvh;
  const uint8_t* recs = a.k_codes + stream * S * (16 * KB);
  const uint8_t* vtiles = pa.v_codes + stream * (S / kTile) * (1024 * VB);
  const int tile_cap = S / kTile - 1;
  const int tau = kTile * wave + lane;  // position of this lane's token inside a super-tile
  const float tauf = static_cast<float>(tau);

  // The first two outliers of every token travel with its data; with fewer outliers the
  // spare loads repeat a real one or read the first code word, and are ignored.
  const int kp = min(k, kFuseOutliers);
  const size_t o_stride = kp > 0 ? k : 0;
  const int o_second = kp > 1 ? 1 : 0;
  const uint8_t* ko_idx = kp > 0 ? a.k_idx : a.k_codes;
  const uint16_t* ko_val = kp > 0 ? a.k_val : reinterpret_cast<const uint16_t*>(a.k_codes);
  const uint8_t* vo_idx = kp > 0 ? pa.v_idx : pa.v_codes;
  const uint16_t* vo_val = kp > 0 ? pa.v_val : reinterpret_cast<const uint16_t*>(pa.v_codes);

  // Every call issues the same loads at valid addresses (super-tile clamped to the block's
  // range, tile to the buffer), so the compiler counts the loads in flight exactly.
  auto load = [&](int s, KeyRec<KB>& r, ValRec<VB>& v) {
    s = min(s, s_hi - 1);
    const int tile = min(kFuseWaves * s + wave, tile_cap);
    const size_t tok = static_cast<size_t>(tile) * kTile + lane;
    const uint4* p = reinterpret_cast<const uint4*>(recs + tok * (16 * KB));
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const uint4 q = p[i];
      r.w[4 * i + 0] = q.x;
      r.w[4 * i + 1] = q.y;
      r.w[4 * i + 2] = q.z;
      r.w[4 * i + 3] = q.w;
    }
    const uint4* pv = reinterpret_cast<const uint4*>(vtiles + static_cast<size_t>(tile) * (1024 * VB) + lane * (16 * VB));
#pragma unroll
    for (int i = 0; i < VB; ++i) {
      const uint4 q = pv[i];
      v.w[4 * i + 0] = q.x;
      v.w[4 * i + 1] = q.y;
      v.w[4 * i + 2] = q.z;
      v.w[4 * i + 3] = q.w;
    }
    const size_t slot = stream * S + tok;
    r.oi[0] = ko_idx[slot * o_stride];
    r.oi[1] = ko_idx[slot * o_stride + o_second];
    r.ov[0] = ko_val[slot * o_stride];
    r.ov[1] = ko_val[slot * o_stride + o_second];
    v.sv = pa.v_scale[slot];
    v.oi[0] = vo_idx[slot * o_stride];
    v.oi[1] = vo_idx[slot * o_stride + o_second];
    v.ov[0] = vo_val[slot * o_stride];
    v.ov[1] = vo_val[slot * o_stride + o_second];
  };

  // ---- set-up inputs, then the first super-tile's data --------------------------------
  // Lane l of wave w prepares the table coefficients of one of the eight pairs w + 8 m
  // whose rows the wave fills, placed for the DPP row broadcasts of the build: 3-bit rows,
  // m = l & 7 (lane m of every 16-lane row holds pair w + 8 m); 2-bit rows, lane 16 r + f
  // prepares m = 4 f + r (fill step f finds its row's pair at lane f of the row).
  const int P = KB == 3 ? wave + kFuseWaves * (lane & 7) : wave + kFuseWaves * ((lane >> 4) + 4 * (lane & 1));
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
  const uint32_t vcb_a = pa.v_cb[tid & (kNcV - 1)];
  const uint32_t vcb_b = pa.v_cb[(tid >> VB) & (kNcV - 1)];
  const uint32_t vcb_lo = pa.v_cb[lane & (kNcV - 1)];
  const double th_P = a.theta_rev[P];
  const float2 th_split = make_float2(a.th_hi[lane], a.th_lo[lane]);

  KeyRec<KB> r0, r1;
  ValRec<VB> v0, v1;
  load(s_lo, r0, v0);

  static_assert(kPairEntries <= kFuseThreads, "one value-table entry per thread");
  ks[tid & (kHeadDim - 1)] = ks_own;  // threads sharing an entry write the same value
  thl[lane] = th_split;
  lut2[tid & (kPairEntries - 1)] = vcb_a | (vcb_b << 16);
  for (int e = tid; e < kFuseWaves * kHeadDim; e += kFuseThreads) osi[e] = 0;
  float qv[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) qv[j] = a.q_is_fp16 ? half_bits_to_float(qraw[j]) : __builtin_bit_cast(float, qraw[j]);
  const float zc = zero_code_value<kNc>(cb_lane, lane);    // key value every outlier slot decodes to
  const float zv = zero_code_value<kNcV>(vcb_lo, lane);    // value value every outlier slot decodes to
  // codebook values this lane's table entries use: entry e = a | b << KB
  float cba, cbb;
  {
    const int e0 = KB == 3 ? lane : (lane & 15);
    cba = half_bits_to_float(__shfl(static_cast<int>(cb_lane), e0 & (kNc - 1)) & 0xffffu);
    cbb = half_bits_to_float(__shfl(static_cast<int>(cb_lane), (e0 >> KB) & (kNc - 1)) & 0xffffu);
  }

  // E(tau) for all 64 pairs: the argument tau theta_i / 2pi is formed exactly (tau < 512
  // times the 15-bit leading part of theta_i / 2pi) plus the small remainder term.
  float er[kHalf], ei[kHalf];
#pragma unroll
  for (int i = 0; i < kHalf; ++i) {
    const float ph = fmaf(tauf, a.th_lo[i], __builtin_amdgcn_fractf(tauf * a.th_hi[i]));
    er[i] = __builtin_amdgcn_cosf(ph);
    ei[i] = __builtin_amdgcn_sinf(ph);
  }
  block_lds_barrier();  // ks, thl, lut2, cleared outlier rows visible
  const float sP_lo = ks[P], sP_hi = ks[P + kHalf];

  // ---- key table build for super-tile s into buffer b ----------------------------------
  auto build = [&](int s, int b) {
    const double t0 = static_cast<double>(s) * (kFuseWaves * kTile);
    float2* T = lut + b * (Sh::kBufBytes / 8);
    const float r = frac_rev(t0, th_P);
    const float cs = __builtin_amdgcn_cosf(r), sn = __builtin_amdgcn_sinf(r);
    const float pa_ = qv[0] * cs + qv[1] * sn;  // R(-t0 theta) q
    const float pb_ = qv[1] * cs - qv[0] * sn;
    const float4 c1 = make_float4(sP_lo * pa_, sP_lo * pb_, sP_hi * pb_, -(sP_hi * pa_));  // alpha, beta, gamma, -delta
    if (writes_pab) pab[b * kHalf + P] = make_float2(pa_, pb_);
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
        T[(wave + kFuseWaves * m) * kNe + lane] = lut_entry_bcast<m>(cc.x, cc.y, cc.z, cc.w, cba, cbb);
      });
    } else {
      // 16 entries per row: fill step f covers the rows of 4 pairs, m = 4 f + (lane >> 4),
      // whose coefficients lane f of each 16-lane row holds (DPP row broadcast)
      float4 cc = c1;
      // at least two wait states between these VALU writes and their DPP reads
      asm volatile("s_nop 1" : "+v"(cc.x), "+v"(cc.y), "+v"(cc.z), "+v"(cc.w));
      static_for<0, 2>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        const int i = wave + kFuseWaves * (4 * f + (lane >> 4));
        T[i * kNe + (lane & 15)] = lut_entry_bcast<f>(cc.x, cc.y, cc.z, cc.w, cba, cbb);
      });
    }
  };

  // ---- logit of token `lane` of this wave's tile of super-tile s (table buffer b) --------
  auto logit = [&](int s, int b, const KeyRec<KB>& d) -> float {
    const uint32_t T = lds_address(lut + b * (Sh::kBufBytes / 8));
    const unsigned char* lb = lds - lds_address(lds);  // LDS address -> pointer
    // Software-pipelined over batches of kBatch pairs: the table reads of batch j + 1 are
    // issued before the FMAs of batch j.
    constexpr int kBatch = 4;
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
    // Key outliers: replace the decoded zero code zc * s_c at the channel by the stored
    // fp16 value, at the channel's rotated query coefficient.
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
    const int t = (kFuseWaves * s + wave) * kTile + lane;
    if (t < L) {
      const size_t o = (stream * S + t) * k;
      for (int j = kFuseOutliers; j < k; ++j) add_outlier(a.k_idx[o + j], a.k_val[o + j]);
    }
    return t < L ? a.sm_scale * l : -INFINITY;
  };

  // ---- softmax . V of this wave's tile, running state per wave --------------------------
  float m_run = -INFINITY, lsum = 0.0f, acc0 = 0.0f, acc1 = 0.0f;
  int* my_osi = osi + wave * kHeadDim;
  auto accumulate = [&](int s, float lg, const ValRec<VB>& d) {
    const int t = (kFuseWaves * s + wave) * kTile + lane;
    const bool valid = t < L;
    const float sv = half_bits_to_float(d.sv);
    const float mt = wave_max_f32(lg);
    if (mt > m_run) {  // wave-uniform: rescale the running state to the new max
      const float sc = m_run > -INFINITY ? expf(m_run - mt) : 0.0f;
      m_run = mt;
      acc0 *= sc;
      acc1 *= sc;
      lsum *= sc;
    }
    const float pr = valid ? __expf(lg - m_run) : 0.0f;  // hardware exp2 of x log2(e): relative error < 4e-6 for x >= -100
    lsum += pr;
    const float wts = pr * sv;
    wave_lds_sync();
    // Value outliers: channel c gets p_t (x_c - zv s_t), summed in 32-bit fixed point with
    // integer atomics (scale 2^(23 - e), 2^e above the tile's largest term over all of the
    // token's outliers; at most one term per channel and token, so the sums fit and do not
    // depend on the order the atomics land).  Outliers past the first two are read twice,
    // for the scale and for the sums.
    float unscale = 0.0f;
    bool have_fixed = false;
    {
      const float dv0 = half_bits_to_float(d.ov[0]) - zv * sv;
      const float dv1 = half_bits_to_float(d.ov[1]) - zv * sv;
      const int c0 = d.oi[0] & (kHeadDim - 1), c1 = d.oi[1] & (kHeadDim - 1);  // stale bytes past the length
      const bool more = k > kFuseOutliers && valid;
      const size_t slot = (stream * S + t) * k;
      float dmax = fmaxf(kp >= 1 ? fabsf(dv0) : 0.0f, kp >= 2 ? fabsf(dv1) : 0.0f);
      if (more) {
        for (int j = kFuseOutliers; j < k; ++j) dmax = fmaxf(dmax, fabsf(half_bits_to_float(pa.v_val[slot + j]) - zv * sv));
      }
      const float m = wave_max_f32(pr * dmax);
      have_fixed = m > 0.0f;  // wave-uniform
      if (have_fixed) {
        const int e = min(max(static_cast<int>((__builtin_bit_cast(uint32_t, m) >> 23) & 0xffu) - 126, -100), 100);
        const float sc = __builtin_bit_cast(float, static_cast<uint32_t>(23 - e + 127) << 23);  // 2^(23-e)
        unscale = __builtin_bit_cast(float, static_cast<uint32_t>(e - 23 + 127) << 23);       // 2^(e-23)
        if (kp >= 1) atomicAdd(my_osi + c0, static_cast<int>(rintf(pr * dv0 * sc)));
        if (kp >= 2) atomicAdd(my_osi + c1, static_cast<int>(rintf(pr * dv1 * sc)));
        if (more) {
          for (int j = kFuseOutliers; j < k; ++j) {
            const int c = pa.v_idx[slot + j] & (kHeadDim - 1);
            const float dv = half_bits_to_float(pa.v_val[slot + j]) - zv * sv;
            atomicAdd(my_osi + c, static_cast<int>(rintf(pr * dv * sc)));
          }
        }
      }
    }
    wave_lds_sync();
    if (have_fixed) {  // this tile's fixed-point sums of channels (2l, 2l+1), read and cleared by one LDS exchange
      unsigned long long* cell = reinterpret_cast<unsigned long long*>(my_osi + 2 * lane);
      const unsigned long long q = __hip_atomic_exchange(cell, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
      acc0 = fmaf(static_cast<float>(static_cast<int>(static_cast<uint32_t>(q))), unscale, acc0);
      acc1 = fmaf(static_cast<float>(static_cast<int>(static_cast<uint32_t>(q >> 32))), unscale, acc1);
    }
    // Dense part: fp16 weight pairs (w_t, w_t+1) as one scalar operand per two tokens of a
    // packed dot product with the codebook pair; the weights scaled by the power of two
    // that puts the tile's largest in [2^13, 2^14), undone exactly after the tile.
    const float wmax = wave_max_f32(wts);
    const int ex = wmax > 0.0f ? static_cast<int>((__builtin_bit_cast(uint32_t, wmax) >> 23) & 0xffu) - 127 : 0;
    const int sh = min(max(13 - ex, -100), 100);
    const float unsc = __builtin_bit_cast(float, static_cast<uint32_t>(127 - sh) << 23);
    const float ws = wts * __builtin_bit_cast(float, static_cast<uint32_t>(127 + sh) << 23);
    const uint32_t wh = __builtin_bit_cast(uint16_t, static_cast<_Float16>(ws));
    const uint32_t wn = dpp_u32<0xF5>(wh);  // quad_perm [1,1,3,3]: lane 2m gets lane 2m + 1
    const uint32_t wpair = wh | (wn << 16);
    typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
    float p00 = 0.0f, p01 = 0.0f, p10 = 0.0f, p11 = 0.0f;
    static_for<0, kTile / 2>([&](auto mc) {
      constexpr int mm = decltype(mc)::value;
      const half2_t e0 = __builtin_bit_cast(half2_t, lut2[field<2 * VB, 2 * VB * mm>(d.w)]);
      const half2_t e1 = __builtin_bit_cast(half2_t, lut2[field<2 * VB, kChanBits + 2 * VB * mm>(d.w)]);
      const half2_t wp = __builtin_bit_cast(half2_t, __builtin_amdgcn_readlane(static_cast<int>(wpair), 2 * mm));
      if constexpr (mm & 1) {
        p01 = __builtin_amdgcn_fdot2(e0, wp, p01, false);
        p11 = __builtin_amdgcn_fdot2(e1, wp, p11, false);
      } else {
        p00 = __builtin_amdgcn_fdot2(e0, wp, p00, false);
        p10 = __builtin_amdgcn_fdot2(e1, wp, p10, false);
      }
    });
    acc0 = fmaf(p00 + p01, unsc, acc0);
    acc1 = fmaf(p10 + p11, unsc, acc1);
    wave_lds_sync();  // the cleared cells are written before the next tile's atomics
  };

  // ---- main loop -----------------------------------------------------------------------
  build(s_lo, 0);
  block_lds_barrier();
  auto step = [&](int s, const KeyRec<KB>& rc, const ValRec<VB>& vc, KeyRec<KB>& rn, ValRec<VB>& vn) {
    const int b = (s - s_lo) & 1;
    load(s + 1, rn, vn);
    if (s + 1 < s_hi) build(s + 1, b ^ 1);
    const float lg = logit(s, b, rc);
    accumulate(s, lg, vc);
    block_lds_barrier();
  };
  for (int s = s_lo; s < s_hi; s += 2) {
    step(s, r0, v0, r1, v1);
    if (s + 1 >= s_hi) break;
    step(s + 1, r1, v1, r0, v0);
  }

  // ---- merge the eight waves' states into the block's partial ---------------------------
  const float ls = wave_sum_f32(lsum);
  if (lane == 0) {
    wml[2 * wave] = m_run;
    wml[2 * wave + 1] = ls;
  }
  wo[wave * kHeadDim + 2 * lane] = acc0;
  wo[wave * kHeadDim + 2 * lane + 1] = acc1;
  block_lds_barrier();
  if (tid < kHeadDim) {
    const int c = tid;
    float M = wml[0];
#pragma unroll
    for (int w = 1; w < kFuseWaves; ++w) M = fmaxf(M, wml[2 * w]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kFuseWaves; ++w) {
      const float f = wml[2 * w] > -INFINITY ? expf(wml[2 * w] - M) : 0.0f;
      o += f * wo[w * kHeadDim + c];
      l += f * wml[2 * w + 1];
    }
    float* dst = pa.partial + ((static_cast<size_t>(seq) * a.n_q_heads + kvh) * pa.n_parts + blockIdx.x) * (kHeadDim + 2);
    dst[c] = o;
    if (c == 0) {
      dst[kHeadDim] = M;
      dst[kHeadDim + 1] = l;
    }
  }
}

template <int KB, int VB>
hipError_t launch_fused_t(int batch, const QkArgs& a0, const PvArgs& p0, hipStream_t st) {
  using Sh = FuseShape<KB>;
  QkArgs a = a0;
  PvArgs pa = p0;
  constexpr int kPairEntries = 1 << (2 * VB);
  const size_t lds = 2 * Sh::kBufBytes + kHeadDim * 4 + 2 * kHalf * 8 + kHalf * 8 + kPairEntries * 4 +
                     2 * kFuseWaves * kHeadDim * 4 + 2 * kFuseWaves * 4;
  static const bool attr_ok = hipFuncSetAttribute(reinterpret_cast<const void*>(&fused_decode_kernel<KB, VB>),
                                                  hipFuncAttributeMaxDynamicSharedMemorySize,
                                                  static_cast<int>(lds)) == hipSuccess;
  if (!attr_ok) return hipErrorInvalidValue;
  // One resident round: the block slots shared equally among the streams, each block a
  // contiguous run of super-tiles; at most one part per 1024 tokens (the workspace bound).
  const int tiles = (a.max_len + kTile - 1) / kTile;
  const int supers = (tiles + kFuseWaves - 1) / kFuseWaves;
  const long streams = static_cast<long>(batch) * a.n_kv_heads;
  static const int resident = [&] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&fused_decode_kernel<KB, VB>),
                                                     kFuseThreads, lds) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  const long slots = static_cast<long>(device_cu_count()) * resident;
  const long max_parts = (a.max_len + kPvChunk - 1) / kPvChunk;
  const long per_stream = std::max(1L, std::min<long>(std::min<long>((slots + streams - 1) / streams, supers), max_parts));
  a.tiles_per_wave = static_cast<int>((supers + per_stream - 1) / per_stream);  // super-tiles per block
  const int n_blocks = (supers + a.tiles_per_wave - 1) / a.tiles_per_wave;
  pa.n_parts = n_blocks;
  dim3 grid(n_blocks, a.n_kv_heads, batch);
  hipLaunchKernelGGL((fused_decode_kernel<KB, VB>), grid, dim3(kFuseThreads), lds, st, a, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_pv_combine(batch, pa, st);
}

}  // namespace

hipError_t launch_fused(int k_bits, int v_bits, int batch, const QkArgs& a, const PvArgs& p, hipStream_t s) {
#define KVQ_FUSED_CASE(KB, VB) \
  if (k_bits == KB && v_bits == VB) return launch_fused_t<KB, VB>(batch, a, p, s);
  KVQ_FUSED_CASE(2, 2) KVQ_FUSED_CASE(2, 3) KVQ_FUSED_CASE(2, 4)
  KVQ_FUSED_CASE(3, 2) KVQ_FUSED_CASE(3, 3) KVQ_FUSED_CASE(3, 4)
#undef KVQ_FUSED_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
