// Decode-time q . K^T for several query heads per kv head (g = 2, 4, 8) with 2- or 3-bit
// keys: RoPE applied to each dequantized key at its own position, the contraction over the
// head dimension on the matrix cores.
//
// KVQuant paper note, "Four components" paragraph, item (2): keys are cached before the
// rotary embedding; items (1), (3), (4): per-channel scale, per-layer codebook, per-vector
// fp16 outliers.
//
// For a key at position t = T0 + tau (T0 the first token of a super-tile of kMfWaves x 64
// tokens, tau < 64 kMfWaves) and rotary pair i with codes a (channel i) and b (i + 64):
//   y_i = R(t theta_i) (cb[a] s_i, cb[b] s_{i+64}) = R(tau theta_i) X_i[a, b],
//   X_i[a, b] = R(T0 theta_i) (cb[a] s_i, cb[b] s_{i+64}),
// X a per-super-tile table of 64 rows of 2^(2b) float pairs (rows filled by every wave
// between block barriers, as in the one-head table kernel: two buffers and a barrier per
// step for 3-bit keys, eight buffers and a barrier every fourth step for 2-bit keys), E(tau) =
// R(tau theta_i) in 128 registers (lane = token).  A key and pair cost the table address (a
// shift and a mask), one 8-byte read, the rotation (four operations) and one conversion of
// the rotated pair to fp16, independent of the number of heads.  The fp16 rotated keys are
// the B operand of v_mfma_f32_4x4x4_16b_f16 (16 blocks of 4 tokens: block b takes lanes
// 4b..4b+3, a lane's 4 values are 4 channels of its token), the fp16 queries of 4 heads the A
// operand (the same in every block), so one MFMA adds 4 channels of all 64 tokens for 4 heads
// and a lane ends with its token's logits of those heads.  The channel order inside the
// contraction is (2j, 2j + 64, 2j + 1, 2j + 65) for step j, so one rotated pair is one packed
// register.
//
// Precision: the rotated key is formed in fp32 and rounded once to fp16; a power-of-two
// prescale 2^e (from the largest scale and codebook magnitude) keeps every dense element
// below 2^15 and far above fp16's subnormal range, so each element's rounding error is at
// most 2^-11 of itself.  fp16 x fp16 products are exact in fp32 and summed in fp32, so the
// logit error is at most 2^-11 sm sum_c |q_c y_c| plus fp32 rounding.  fp32 queries are
// prescaled per head and split into two fp16 parts (hi + lo, two MFMAs per step), leaving a
// 2^-22 relative error.  Outliers replace the zero code decoded at their channel; their
// correction is computed in fp32 per head from the query rotated by R(-T0 theta) and the
// hardware sine/cosine of tau theta at the outlier's pair.
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kMfWaves = 8;                  // waves per block = tiles per super-tile
constexpr int kMfThreads = 64 * kMfWaves;
constexpr int kMfSuper = kMfWaves * kTile;   // tokens per super-tile
constexpr int kMfPrefetchOutliers = 2;       // outliers per token fetched with the record
constexpr int kMfAhead = 6;                  // table reads in flight ahead of their rotation

typedef _Float16 mf_half2 __attribute__((ext_vector_type(2)));
typedef _Float16 mf_half4 __attribute__((ext_vector_type(4)));
typedef float mf_float4 __attribute__((ext_vector_type(4)));

template <int KB, int G, bool kSplit>
struct MfShape {
  static constexpr int kNc = 1 << KB;
  static constexpr int kNe = kNc * kNc;               // code pairs (a | b << KB) per rotary pair
  static constexpr int kRowBytes = kNe * 8;           // X float pairs of one rotary pair
  static constexpr int kBufBytes = kHalf * kRowBytes; // 64 rows
  static constexpr int kGroups = G > 4 ? G / 4 : 1;   // MFMA row blocks of 4 heads
  static constexpr int kParts = kSplit ? 2 : 1;       // fp16 parts of the query
  static constexpr int kSteps = kHalf / 2;            // MFMA steps of 4 channels
  // LDS layout (byte offsets): tables [kNB][64][kNe] float2; build coefficients [kCR][64]
  // float4; rotated query pairs [kPR][G][64] float2; A operands [group][part][row][step] of 4
  // fp16; query pairs [G][64] float2; per-head output scales [8]; key scales [128]; split
  // frequencies [64] float2
  // Steps per block barrier (kSB): 2-bit tables are small enough for eight buffers (a
  // barrier every fourth step) except where the extra record set would spill (eight heads,
  // split fp32 queries); 3-bit tables (32 KB) keep two buffers and a barrier per step.
  static constexpr int kSB = KB == 2 && !(G == 8 && kSplit) ? 4 : 1;
  static constexpr int kNB = 2 * kSB;  // table buffers
  static constexpr int kCR = 2 * kSB;  // build-coefficient ring
  static constexpr int kPR = 4 * kSB;  // rotated-query ring
  static constexpr int kTab = 0;
  static constexpr int kCoef = kNB * kBufBytes;
  static constexpr int kCpab = kCoef + kCR * kHalf * 16;
  static constexpr int kQa = kCpab + kPR * G * kHalf * 8;
  static constexpr int kQf = kQa + kGroups * kParts * 4 * kSteps * 8;
  static constexpr int kQsc = kQf + G * kHalf * 8;
  static constexpr int kKs = kQsc + 8 * 4;
  static constexpr int kThl = kKs + kHeadDim * 4;
  static constexpr int kLdsBytes = kThl + kHalf * 8;
  static_assert(kLdsBytes <= 160 * 1024, "LDS of one block");
};

template <int KB>
struct MfRec {
  uint32_t w[4 * KB];     // the token's key record
  uint32_t oi[2], ov[2];  // its first two outliers: channels and fp16 value bits
};

__device__ __forceinline__ float pow2f(int e) {  // 2^e for -126 <= e <= 127
  return __builtin_bit_cast(float, static_cast<uint32_t>(e + 127) << 23);
}

template <int KB, int G, bool kSplit>
__global__ __launch_bounds__(kMfThreads) void qk_mfma_kernel(QkArgs a) {
  using Sh = MfShape<KB, G, kSplit>;
  constexpr int kNc = Sh::kNc;
  constexpr int kNe = Sh::kNe;
  constexpr int kGroups = Sh::kGroups;
  constexpr int kParts = Sh::kParts;
  static_assert(KB == 2 || KB == 3, "2- and 3-bit keys");
  static_assert(G == 2 || G == 4 || G == 8, "2, 4 or 8 query heads per kv head");

  // statically sized, so that table offsets are compile-time LDS addresses (immediate
  // offsets of the reads)
  __shared__ __align__(16) unsigned char lds[Sh::kLdsBytes];
  float2* tab = reinterpret_cast<float2*>(lds + Sh::kTab);
  float4* coef = reinterpret_cast<float4*>(lds + Sh::kCoef);
  float2* cpab = reinterpret_cast<float2*>(lds + Sh::kCpab);
  float2* qf = reinterpret_cast<float2*>(lds + Sh::kQf);
  float* qsc = reinterpret_cast<float*>(lds + Sh::kQsc);
  float* ks = reinterpret_cast<float*>(lds + Sh::kKs);
  float2* thl = reinterpret_cast<float2*>(lds + Sh::kThl);

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
  const int n_super = (n_tiles + kMfWaves - 1) / kMfWaves;
  const int s_lo = blockIdx.x * a.tiles_per_wave;  // super-tiles per block, set by the launcher
  const int s_hi = min(s_lo + a.tiles_per_wave, n_super);
  if (s_lo >= s_hi) return;  // block-uniform

  const size_t stream = static_cast<size_t>(seq) * H + kvh;
  const uint8_t* recs = a.k_codes + stream * S * (16 * KB);
  const int tile_cap = S / kTile - 1;
  const int tau = kTile * wave + lane;  // position of this lane's token inside a super-tile

  // The first kMfPrefetchOutliers outliers of every token travel with its record; with
  // fewer outliers the spare loads repeat a real one or read the first code word, and
  // their results are ignored.
  const int kp = min(k, kMfPrefetchOutliers);
  const uint8_t* o_idx = kp > 0 ? a.k_idx : a.k_codes;
  const uint16_t* o_val = kp > 0 ? a.k_val : reinterpret_cast<const uint16_t*>(a.k_codes);
  const size_t o_stride = kp > 0 ? k : 0;
  const int o_second = kp > 1 ? 1 : 0;

  // Every call issues the same loads at valid addresses (super-tile clamped to the block's
  // range, tile to the buffer), through buffer descriptors rebuilt per tile at the tile's
  // first token with fixed per-lane offsets.
  const uint32_t rec_off = static_cast<uint32_t>(lane) * (16 * KB);
  const uint32_t out_off = static_cast<uint32_t>(lane * o_stride);
  const uint32_t second_off = out_off + o_second;
  const uint32_t tile_outs = static_cast<uint32_t>(kTile * o_stride);
  auto load_rec = [&](int s, MfRec<KB>& d) __attribute__((always_inline)) {
    s = min(s, s_hi - 1);
    const int tile = min(kMfWaves * s + wave, tile_cap);  // wave-uniform
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
  // Thread (h, i) = (tid >> 6, tid & 63), h < G, stages head h's query pair i; lane l of
  // wave w distributes the build coefficients of pair P (as in the one-head table kernel:
  // 3-bit rows, lane m of every 16-lane row holds pair w + 8 m; 2-bit rows, lane 16 r + f
  // holds pair w + 8 (4 f + r)).
  const int P = KB == 3 ? wave + kMfWaves * (lane & 7) : wave + kMfWaves * ((lane >> 4) + 4 * (lane & 1));
  const int hq = min(tid >> 6, G - 1);
  const size_t qbase = (static_cast<size_t>(seq) * a.n_q_heads + static_cast<size_t>(kvh) * G + hq) * kHeadDim;
  uint32_t qraw[2];
  if (a.q_is_fp16) {  // wave-uniform; both paths issue the same loads
    const uint16_t* q16 = static_cast<const uint16_t*>(a.q) + qbase;
    qraw[0] = q16[lane];
    qraw[1] = q16[lane + kHalf];
  } else {
    const uint32_t* q32 = static_cast<const uint32_t*>(a.q) + qbase;
    qraw[0] = q32[lane];
    qraw[1] = q32[lane + kHalf];
  }
  const float s_lo_c = a.k_scale[kvh * kHeadDim + lane];  // pair `lane`: s_i, s_{i+64}
  const float s_hi_c = a.k_scale[kvh * kHeadDim + lane + kHalf];
  const double th_l = a.theta_rev[lane];
  const uint32_t cb_lane = a.k_cb[lane & (kNc - 1)];

  MfRec<KB> r0, r1, r2, r3;  // r3 only with several steps per barrier
  load_rec(s_lo, r0);
  load_rec(s_lo + 1, r1);

  // Prescale 2^pe: |y| <= sqrt(2) max|cb| max s, so 1.5 max|cb| max s 2^pe < 2^15.
  const float smax = wave_max_f32(fmaxf(fabsf(s_lo_c), fabsf(s_hi_c)));
  const float cbmax = wave_max_f32(lane < kNc ? fabsf(half_bits_to_float(cb_lane & 0xffffu)) : 0.0f);
  const float ybound = 1.5f * smax * cbmax;
  const int pe = ybound > 0.0f ? min(max(14 - (static_cast<int>((__builtin_bit_cast(uint32_t, ybound) >> 23) & 0xffu) - 127), -100), 100) : 0;
  const float pre = pow2f(pe);

  {
    float qv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) qv[j] = a.q_is_fp16 ? half_bits_to_float(qraw[j]) : __builtin_bit_cast(float, qraw[j]);
    // fp32 queries: a per-head power of two puts the head's largest |q| below 2^15 before
    // the split (fp16 queries are used as they are)
    int qe = 0;
    if constexpr (kSplit) {
      const float qm = wave_max_f32(fmaxf(fabsf(qv[0]), fabsf(qv[1])));  // the wave holds one head
      qe = qm > 0.0f ? min(max(14 - (static_cast<int>((__builtin_bit_cast(uint32_t, qm) >> 23) & 0xffu) - 127), -100), 100) : 0;
    }
    const int row = tid >> 6;  // MFMA row (head) this thread's wave stages, < 4 kGroups
    if (row < 4 * kGroups) {
      const bool real = row < G;
      const float qs = pow2f(qe);
      const float x0 = real ? qv[0] * qs : 0.0f, x1 = real ? qv[1] * qs : 0.0f;
      const _Float16 h0 = static_cast<_Float16>(x0), h1 = static_cast<_Float16>(x1);
      // step j = lane >> 1 holds (2j, 2j + 64, 2j + 1, 2j + 65): this pair is half lane & 1
      uint32_t* qa = reinterpret_cast<uint32_t*>(lds + Sh::kQa);
      const int g = row >> 2, m = row & 3;
      const int word = (((g * kParts + 0) * 4 + m) * Sh::kSteps + (lane >> 1)) * 2 + (lane & 1);
      qa[word] = __builtin_bit_cast(uint32_t, mf_half2{h0, h1});
      if constexpr (kSplit) {
        const _Float16 l0 = static_cast<_Float16>(x0 - static_cast<float>(h0));
        const _Float16 l1 = static_cast<_Float16>(x1 - static_cast<float>(h1));
        qa[word + 4 * Sh::kSteps * 2] = __builtin_bit_cast(uint32_t, mf_half2{l0, l1});
      }
      if (real) {
        qf[row * kHalf + lane] = make_float2(qv[0], qv[1]);
        if (lane == 0) qsc[row] = pow2f(-qe);
      }
    }
  }
  if (tid < kHalf) {
    thl[tid] = make_float2(a.th_hi[tid], a.th_lo[tid]);
    ks[tid] = s_lo_c;
    ks[tid + kHalf] = s_hi_c;
  }
  const float zc = zero_code_value<kNc>(cb_lane, lane);  // value every outlier slot decodes to
  // codebook values this lane's table entries use: entry e = a | b << KB
  const int e0 = KB == 3 ? lane : (lane & 15);
  const float cba = half_bits_to_float(__shfl(static_cast<int>(cb_lane), e0 & (kNc - 1)) & 0xffffu);
  const float cbb = half_bits_to_float(__shfl(static_cast<int>(cb_lane), (e0 >> KB) & (kNc - 1)) & 0xffffu);

  // E(tau) for all 64 pairs: the argument tau theta_i / 2pi is formed exactly (tau < 512
  // times the 15-bit leading part of theta_i / 2pi) plus the small remainder term.  The
  // sine is kept negated, so that both products of the rotation are plain two-operand
  // multiplies (the other sign rides on the mixed FMA's operand modifier).
  float er[kHalf], en[kHalf];
  const float tauf = static_cast<float>(tau);
#pragma unroll
  for (int i = 0; i < kHalf; ++i) {
    const float ph = fmaf(tauf, a.th_lo[i], __builtin_amdgcn_fractf(tauf * a.th_hi[i]));
    er[i] = __builtin_amdgcn_cosf(ph);
    en[i] = -__builtin_amdgcn_sinf(ph);
    asm volatile("" : "+v"(en[i]));  // stored negated: the compiler would fold the sign back
  }

  // ---- table coefficients and rotated query pairs of super-tile x (one wave, lane = pair) -
  // X_i[a, b] = (cb[a] c s_i - cb[b] n s_{i+64}, cb[a] n s_i + cb[b] c s_{i+64}) 2^pe with
  // (c, n) = (cos, sin)(T0 theta_i); the outlier correction uses R(-T0 theta_i) q per head.
  auto coefs = [&](int x) __attribute__((always_inline)) {
    const double t0 = static_cast<double>(x) * kMfSuper;
    const float r = frac_rev(t0, th_l);
    const float cs = __builtin_amdgcn_cosf(r), sn = __builtin_amdgcn_sinf(r);
    const float sa = s_lo_c * pre, sb = s_hi_c * pre;
    coef[(x & (Sh::kCR - 1)) * kHalf + lane] = make_float4(cs * sa, sn * sa, -(sn * sb), cs * sb);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float2 qq = qf[h * kHalf + lane];
      cpab[((x & (Sh::kPR - 1)) * G + h) * kHalf + lane] = make_float2(qq.x * cs + qq.y * sn, qq.y * cs - qq.x * sn);
    }
  };

  // ---- this wave's rows of the table of a super-tile into buffer B ---------------------
  auto build = [&](auto bc, float4 cc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    float2* T = tab + B * (Sh::kBufBytes / 8);
    asm volatile("s_nop 1" : "+v"(cc.x), "+v"(cc.y), "+v"(cc.z), "+v"(cc.w));  // DPP read wait states
    if constexpr (KB == 3) {
      static_for<0, 8>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        T[(wave + kMfWaves * m) * kNe + lane] = lut_entry_bcast<m>(cc.x, cc.y, cc.z, cc.w, cba, cbb);
      });
    } else {
      static_for<0, 2>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        const int i = wave + kMfWaves * (4 * f + (lane >> 4));
        T[i * kNe + (lane & 15)] = lut_entry_bcast<f>(cc.x, cc.y, cc.z, cc.w, cba, cbb);
      });
    }
  };

  // Outlier slot operands, requested from LDS before the pair loop; the arithmetic on them
  // waits for out_add, after it (used at once, the channel's scale would make the step wait
  // for every LDS read in flight).
  struct OutOps {
    uint32_t vbits;  // the stored fp16 value; above 0xffff for an unused slot (per-channel rule)
    float sc;        // its channel's key scale
    float2 th;       // theta/2pi of its pair (hi, lo)
    int i;           // its pair
    bool lo_half;    // channel < 64
  };
  // Channel c of pair i rotated by tau theta_i meets the rotated query pair (p_a, p_b) as
  // p_a cos + p_b sin (c = i) or p_b cos - p_a sin (c = i + 64): both are p_a u + p_b v
  // with (u, v) chosen once per outlier and scaled by its value, two FMAs per head.
  auto out_ops = [&](uint32_t c, uint32_t vbits) __attribute__((always_inline)) {
    OutOps o;
    o.vbits = c != kNoOutlier ? vbits : 0xffffffffu;  // an unused slot adds nothing
    c &= kHeadDim - 1;                                // a token past the length may hold stale bytes
    o.i = c & (kHalf - 1);
    o.sc = ks[c];
    o.th = thl[o.i];
    o.lo_half = c < kHalf;
    return o;
  };
  auto out_add = [&](const OutOps& o, const float2* pab, float (&ol)[G]) __attribute__((always_inline)) {
    const float dv = o.vbits <= 0xffffu ? half_bits_to_float(o.vbits) - zc * o.sc : 0.0f;  // minus the decoded zero code
    const float ph = fmaf(tauf, o.th.y, __builtin_amdgcn_fractf(tauf * o.th.x));
    const float cs = __builtin_amdgcn_cosf(ph), sn = __builtin_amdgcn_sinf(ph);
    const float u = dv * (o.lo_half ? cs : -sn);
    const float v = dv * (o.lo_half ? sn : cs);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float2 p = pab[h * kHalf + o.i];
      ol[h] = fmaf(p.x, u, fmaf(p.y, v, ol[h]));
    }
  };

  // per-head factor of the MFMA sums: sm_scale 2^-pe (and the query's 2^-qe)
  float osc[G];

  // this lane's A operand rows: row lane & 3 of every group and part
  const unsigned char* qa_lane = lds + Sh::kQa + (lane & 3) * (Sh::kSteps * 8);

  // ---- one tile of super-tile s from table buffer B, and the rows of s + 1 -------------
  auto step = [&](auto bc, int s, const MfRec<KB>& d, MfRec<KB>& ahead) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    constexpr int kSB = Sh::kSB, kNB = Sh::kNB, kCR = Sh::kCR, kPR = Sh::kPR;
    constexpr bool kBuild = B % kSB == 0;
    float4 cc[kSB];  // build coefficients of super-tiles s + kSB + j
    if constexpr (kSB == 1) cc[0] = coef[((s + 1) & (kCR - 1)) * kHalf + P];
    const float2* pab = cpab + (s & (kPR - 1)) * G * kHalf;
    OutOps o0, o1;
    if (kp >= 1) o0 = out_ops(d.oi[0], d.ov[0]);
    if (kp >= 2) o1 = out_ops(d.oi[1], d.ov[1]);

    const unsigned char* tb = lds + B * Sh::kBufBytes;
    mf_float4 acc[kGroups];
#pragma unroll
    for (int g = 0; g < kGroups; ++g) acc[g] = mf_float4{0.0f, 0.0f, 0.0f, 0.0f};
    float va[kMfAhead + 1], vb[kMfAhead + 1];
    auto issue = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      const float2 v = *reinterpret_cast<const float2*>(tb + i * Sh::kRowBytes + pair_entry_offset<KB, i>(d.w));
      va[i % (kMfAhead + 1)] = v.x;
      vb[i % (kMfAhead + 1)] = v.y;
    };
    // With one A operand per step (g <= 4, fp16 queries) the query row of MFMA step j + 1 is
    // requested right after the products of step j: read just before its own product, its
    // wait would also drain the table reads issued ahead (LDS reads complete in order).  With
    // two or four per step the extra live registers cost spills, and each row is read just
    // before its product.
    constexpr bool kEarlyA = kGroups * kParts == 1;
    auto a_row = [&](int gp, int j) __attribute__((always_inline)) {
      return *reinterpret_cast<const uint2*>(qa_lane + (gp * 4 * Sh::kSteps + j) * 8);
    };
    uint2 aw_next = kEarlyA ? a_row(0, 0) : make_uint2(0u, 0u);
    static_for<0, kMfAhead>([&](auto ic) { issue(ic); });
    uint32_t hp[2];
    static_for<0, kHalf>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + kMfAhead < kHalf) issue(std::integral_constant<int, i + kMfAhead>{});
      // the next records' loads and their scalar address arithmetic, issued inside the loop so
      // that they overlap the other wave's arithmetic rather than lengthen the step's start
      if constexpr (i == 8) load_rec(s + 2, ahead);
      if constexpr (kSB > 1 && kBuild && i == 40) {
#pragma unroll
        for (int j = 0; j < kSB; ++j) cc[j] = coef[((s + kSB + j) & (kCR - 1)) * kHalf + P];
      }
      const float xa = va[i % (kMfAhead + 1)], xb = vb[i % (kMfAhead + 1)];
      const float ya = fmaf(xa, er[i], xb * en[i]);
      const float yb = fmaf(xa, -en[i], xb * er[i]);
      hp[i & 1] = __builtin_bit_cast(uint32_t, mf_half2{static_cast<_Float16>(ya), static_cast<_Float16>(yb)});
      if constexpr ((i & 1) == 1) {
        constexpr int j = i >> 1;
        const mf_half4 bop = __builtin_bit_cast(mf_half4, make_uint2(hp[0], hp[1]));
#pragma unroll
        for (int g = 0; g < kGroups; ++g)
#pragma unroll
          for (int part = 0; part < kParts; ++part) {
            const uint2 aw = kEarlyA ? aw_next : a_row(g * kParts + part, j);
            acc[g] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(mf_half4, aw), bop, acc[g], 0, 0, 0);
            // keeps the product here, so that the rotated pairs die at once instead of the
            // compiler sinking every MFMA to the end of the loop
            asm volatile("" : "+v"(acc[g]));
          }
        if constexpr (kEarlyA && j + 1 < Sh::kSteps) aw_next = a_row(0, j + 1);
      }
      if constexpr ((i & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    });
    float ol[G];
#pragma unroll
    for (int h = 0; h < G; ++h) ol[h] = 0.0f;
    if (kp >= 1) out_add(o0, pab, ol);
    if (kp >= 2) out_add(o1, pab, ol);
    const int t0 = (kMfWaves * s + wave) * kTile;  // wave-uniform
    const int t = t0 + lane;
    if (t < L) {
      const size_t o = (stream * S + t) * k;
      for (int j = kMfPrefetchOutliers; j < k; ++j) out_add(out_ops(a.k_idx[o + j], a.k_val[o + j]), pab, ol);
      float* lg = a.logits + (static_cast<size_t>(seq) * a.n_q_heads + static_cast<size_t>(kvh) * G) * S + t0;
#pragma unroll
      for (int h = 0; h < G; ++h) lg[static_cast<size_t>(h) * S + lane] = fmaf(acc[h >> 2][h & 3], osc[h], a.sm_scale * ol[h]);
    }
    if constexpr (kBuild) {
      static_for<0, kSB>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if (s + kSB + j < s_hi) build(std::integral_constant<int, (B + kSB + j) % kNB>{}, cc[j]);
      });
#pragma unroll
      for (int j = 0; j < kSB; ++j)
        if (wave == ((s + j) & (kMfWaves - 1)) && s + 2 * kSB + j < s_hi) coefs(s + 2 * kSB + j);
    }
    if constexpr (B % kSB == kSB - 1) block_lds_barrier();
  };

  // ---- main loop -----------------------------------------------------------------------
  block_lds_barrier();  // query pairs, A operands, scales, frequencies visible
#pragma unroll
  for (int h = 0; h < G; ++h) osc[h] = a.sm_scale * pow2f(-pe) * (kSplit ? qsc[h] : 1.0f);
  constexpr int kSB = Sh::kSB;
  if (wave < 2 * kSB && s_lo + wave < s_hi) coefs(s_lo + wave);
  block_lds_barrier();  // the coefficients of the first 2 kSB super-tiles visible
  static_for<0, kSB>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if (s_lo + j < s_hi) build(std::integral_constant<int, j>{}, coef[((s_lo + j) & (Sh::kCR - 1)) * kHalf + P]);
  });
  block_lds_barrier();
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  if constexpr (kSB == 1) {
    // six steps per round: three record sets (two super-tiles in flight) by two table buffers
    for (int s = s_lo; s < s_hi; s += 6) {
      step(I0{}, s, r0, r2);
      if (s + 1 >= s_hi) break;
      step(I1{}, s + 1, r1, r0);
      if (s + 2 >= s_hi) break;
      step(I0{}, s + 2, r2, r1);
      if (s + 3 >= s_hi) break;
      step(I1{}, s + 3, r0, r2);
      if (s + 4 >= s_hi) break;
      step(I0{}, s + 4, r1, r0);
      if (s + 5 >= s_hi) break;
      step(I1{}, s + 5, r2, r1);
    }
  } else {
    // eight steps per round: four record sets by eight table buffers
    using I4 = std::integral_constant<int, 4>;
    using I5 = std::integral_constant<int, 5>;
    using I6 = std::integral_constant<int, 6>;
    using I7 = std::integral_constant<int, 7>;
    for (int s = s_lo; s < s_hi; s += 8) {
      step(I0{}, s, r0, r2);
      if (s + 1 >= s_hi) break;
      step(I1{}, s + 1, r1, r3);
      if (s + 2 >= s_hi) break;
      step(I2{}, s + 2, r2, r0);
      if (s + 3 >= s_hi) break;
      step(I3{}, s + 3, r3, r1);
      if (s + 4 >= s_hi) break;
      step(I4{}, s + 4, r0, r2);
      if (s + 5 >= s_hi) break;
      step(I5{}, s + 5, r1, r3);
      if (s + 6 >= s_hi) break;
      step(I6{}, s + 6, r2, r0);
      if (s + 7 >= s_hi) break;
      step(I7{}, s + 7, r3, r1);
    }
  }
}

template <int KB, int G, bool kSplit>
hipError_t launch_qk_mfma_t(int batch, const QkArgs& a0, hipStream_t st) {
  QkArgs a = a0;
  // One resident round: the device's block slots shared equally among the streams, each
  // block walking a contiguous run of super-tiles.
  const int tiles = (a.max_len + kTile - 1) / kTile;
  const int supers = (tiles + kMfWaves - 1) / kMfWaves;
  const long streams = static_cast<long>(batch) * a.n_kv_heads;
  static const int resident = blocks_per_cu(reinterpret_cast<const void*>(&qk_mfma_kernel<KB, G, kSplit>), kMfThreads);
  const long slots = static_cast<long>(device_cu_count()) * resident;
  const long per_stream = std::max(1L, std::min<long>((slots + streams - 1) / streams, supers));
  a.tiles_per_wave = static_cast<int>((supers + per_stream - 1) / per_stream);  // super-tiles per block
  dim3 grid((supers + a.tiles_per_wave - 1) / a.tiles_per_wave, a.n_kv_heads, batch);
  hipLaunchKernelGGL((qk_mfma_kernel<KB, G, kSplit>), grid, dim3(kMfThreads), 0, st, a);
  return hipGetLastError();
}

template <int KB, int G>
hipError_t launch_qk_mfma_g(int batch, const QkArgs& a, hipStream_t st) {
  return a.q_is_fp16 ? launch_qk_mfma_t<KB, G, false>(batch, a, st) : launch_qk_mfma_t<KB, G, true>(batch, a, st);
}

}  // namespace

hipError_t launch_qk_mfma(int k_bits, int group, int batch, const QkArgs& a, hipStream_t s) {
#define KVQ_QK_MFMA_CASE(KB, G) \
  if (k_bits == KB && group == G) return launch_qk_mfma_g<KB, G>(batch, a, s);
  KVQ_QK_MFMA_CASE(2, 2) KVQ_QK_MFMA_CASE(2, 4) KVQ_QK_MFMA_CASE(2, 8)
  KVQ_QK_MFMA_CASE(3, 2) KVQ_QK_MFMA_CASE(3, 4) KVQ_QK_MFMA_CASE(3, 8)
#undef KVQ_QK_MFMA_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
