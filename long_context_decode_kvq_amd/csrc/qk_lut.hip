// Decode-time q . K^T over the compressed key cache for one query head per kv head
// (g = 1), with RoPE applied to each dequantized key at its own position.
//
// KVQuant paper note, "Four components" paragraph, item (2): keys are cached before the
// rotary embedding; items (1), (3), (4): per-channel scale, per-layer codebook, per-vector
// fp16 outliers.
//
// With a single query the rotated-query coefficients and the codebook fold into one
// table per group of tiles.  For rotary pair i of a key at position t = T0 + tau (T0 the
// first token of a super-tile of kLutWaves x 64 tokens, tau < 64 kLutWaves) with codes a
// (channel i) and b (channel i + 64):
//   q . R(t) k = E_r(tau) A_i[a, b] + E_i(tau) B_i[a, b]
//   A_i = s_i cb[a] p_a + s_{i+64} cb[b] p_b,  B_i = s_i cb[a] p_b - s_{i+64} cb[b] p_a
// where (p_a, p_b) = R(-T0 theta_i) (q_i, q_{i+64}) and E(tau) = (cos, sin)(tau theta_i).
// Lane = token: each lane keeps E(tau) of its own tau for all 64 pairs in 128 registers,
// so a pair costs one 8-byte table read, two FMAs and the table address.  The address is
// the pair's code field times 8: 1.5 integer operations per pair for 2-bit codes (a word's
// fields spread into bytes by two operations shared by four pairs, then one byte taken),
// a shift and a mask for 3-bit codes; the row of the pair and the table buffer are
// immediate offsets of the read (the main loop is unrolled over the buffers).
//
// 4-bit codes would need 256 entries per row; A and B are linear in cb[a] and cb[b], so
// the row is stored separably instead: U[a] = cb[a] (s_i p_a, s_i p_b) and V[b] =
// cb[b] (s_{i+64} p_b, -s_{i+64} p_a), 16 entries each, (A, B) = U[a] + V[b].  A pair then
// costs two table reads, four FMAs and three address operations (byte i of the record is
// the pair's field, its two nibbles spread as with 2-bit codes).  Its 16-register records
// leave room for two record sets only, loaded one super-tile ahead.
//
// The waves of a block share the table of a super-tile.  With 3-bit keys, between two
// block barriers every wave computes its tile of super-tile s and fills its rows of the
// table of s + 1 (two buffers), and one wave (a different one each step) forms the
// rotated-query coefficients of all 64 pairs for s + 2.  2-bit tables (8 KB) are small
// enough for eight buffers: a barrier every fourth step, the first of the four filling the
// rows of s + 4 .. s + 7 and forming the coefficients of s + 8 .. s + 11; 4-bit tables
// (16 KB) take four buffers and a barrier every second step in the same way.  The
// coefficients reach the lanes by DPP row broadcasts.  Operands that come from LDS (the
// build coefficients, each outlier's scale, frequency and rotated-query pair) are
// requested before or early in the pair loop and consumed after it, so their latency
// hides behind the loop.  Outliers replace the zero code decoded at
// their channel: their correction uses the hardware sine/cosine (argument in revolutions)
// at the outlier's pair.
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kLutWaves = 8;                 // waves per block = tiles per super-tile
constexpr int kLutThreads = 64 * kLutWaves;
constexpr int kLutSuper = kLutWaves * kTile; // tokens per super-tile
constexpr int kLutPrefetchOutliers = 2;      // outliers per token fetched with the record
constexpr int kLutRows = kHalf / kLutWaves;  // table rows (rotary pairs) each wave fills
static_assert(kLutRows >= 4 && kLutRows <= 16, "a wave's rows are broadcast from lanes 0..15 of a DPP row");

template <int KB>
struct LutShape {
  static constexpr int kNc = 1 << KB;
  // entries per row: one per code pair (a | b << KB) with 2/3-bit codes; with 4-bit codes
  // the row is separable, 16 entries U[a] then 16 entries V[b]
  static constexpr int kNe = KB == 4 ? 2 * kNc : kNc * kNc;
  static constexpr int kRowBytes = kNe * 8;           // (A, B) float pairs of one rotary pair
  static constexpr int kBufBytes = kHalf * kRowBytes; // 64 rows
  // tables, build coefficients, rotated-query pairs, key scales, frequencies (split and
  // float64), query and scales per pair
  // Steps per block barrier: 2-bit tables (8 KB) in eight buffers, a barrier every fourth
  // step; 4-bit separable tables (16 KB) in four buffers, every second step; 3-bit tables
  // (32 KB) in two buffers, a barrier per step.
  static constexpr int kSB = KB == 3 ? 1 : (KB == 4 ? 2 : 4);
  static constexpr int kNB = 2 * kSB;      // table buffers
  static constexpr int kCR = 2 * kSB;      // build-coefficient ring
  static constexpr int kPR = 4 * kSB;      // rotated-query ring of the outlier terms
  static constexpr int kLdsBytes = kNB * kBufBytes + kCR * kHalf * 16 + kPR * kHalf * 8 + kHeadDim * 4 +
                                   kHalf * 8 + kHalf * 16 + kHalf * 8;
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
  static_assert(KB >= 2 && KB <= 4, "2-, 3- and 4-bit keys");
  // 4-bit records are 16 registers: two record sets, loaded one super-tile ahead
  constexpr int kRecAhead = KB == 4 ? 1 : 2;

  // statically sized, so that table offsets are compile-time LDS addresses (immediate
  // offsets of the reads)
  __shared__ __align__(16) unsigned char lds[Sh::kLdsBytes];
  constexpr int kSB = Sh::kSB, kNB = Sh::kNB, kCR = Sh::kCR, kPR = Sh::kPR;
  float2* lut = reinterpret_cast<float2*>(lds);                           // [kNB][64][kNe] (A, B)
  float4* coef = reinterpret_cast<float4*>(lds + kNB * Sh::kBufBytes);    // [kCR][64] (alpha, beta, gamma, -delta)
  float2* cpab = reinterpret_cast<float2*>(coef + kCR * kHalf);           // [kPR][64] (p_a, p_b)
  float* ks = reinterpret_cast<float*>(cpab + kPR * kHalf);               // [128] key scales
  float2* thl = reinterpret_cast<float2*>(ks + kHeadDim);                 // [64] theta_i/2pi split hi, lo
  float4* qsl = reinterpret_cast<float4*>(thl + kHalf);                   // [64] (q_i, q_{i+64}, s_i, s_{i+64})
  double* thd = reinterpret_cast<double*>(qsl + kHalf);                   // [64] theta_i/2pi

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
  auto load_rec = [&](int s, LutRec<KB>& d) __attribute__((always_inline)) {
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
  // Thread i < 64 stages rotary pair i's query, key scales and frequency in LDS.  Lane l of
  // wave w distributes the build coefficients of one of the kLutRows pairs w + W m (W waves)
  // whose rows the wave fills, placed for the DPP row broadcasts of the build: 3-bit rows,
  // m = l mod kLutRows (lane m of every 16-lane row holds pair w + W m); 2-bit rows, lane
  // 16 r + f holds m = 4 f + r (fill step f finds its row's pair at lane f of the row).
  // 4-bit rows: lane 16 R + m holds pair 2 m + R / 2 (m < 4), U coefficients in even DPP
  // rows R and V coefficients in odd ones.
  const int P = KB == 3   ? wave + kLutWaves * (lane & (kLutRows - 1))
                : KB == 2 ? wave + kLutWaves * ((lane >> 4) + 4 * (lane & (kLutRows / 4 - 1)))
                          : wave + kLutWaves * ((2 * (lane & 15) + (lane >> 5)) & (kLutRows - 1));
  const int ip = tid & (kHalf - 1);
  const size_t qbase = (static_cast<size_t>(seq) * a.n_q_heads + kvh) * kHeadDim;
  uint32_t qraw[2];
  if (a.q_is_fp16) {  // wave-uniform; both paths issue the same loads
    const uint16_t* q16 = static_cast<const uint16_t*>(a.q) + qbase;
    qraw[0] = q16[ip];
    qraw[1] = q16[ip + kHalf];
  } else {
    const uint32_t* q32 = static_cast<const uint32_t*>(a.q) + qbase;
    qraw[0] = q32[ip];
    qraw[1] = q32[ip + kHalf];
  }
  const float s_ip_lo = a.k_scale[kvh * kHeadDim + ip];
  const float s_ip_hi = a.k_scale[kvh * kHeadDim + ip + kHalf];
  const double th_ip = a.theta_rev[ip];
  const uint32_t cb_lane = a.k_cb[lane & (kNc - 1)];

  LutRec<KB> r0, r1, r2, r3;  // r2 and r3 only with several record sets
  load_rec(s_lo, r0);
  if constexpr (kRecAhead == 2) load_rec(s_lo + 1, r1);

  if (tid < kHalf) {
    float qv[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) qv[j] = a.q_is_fp16 ? half_bits_to_float(qraw[j]) : __builtin_bit_cast(float, qraw[j]);
    qsl[tid] = make_float4(qv[0], qv[1], s_ip_lo, s_ip_hi);
    thd[tid] = th_ip;
    thl[tid] = make_float2(a.th_hi[tid], a.th_lo[tid]);
    ks[tid] = s_ip_lo;
    ks[tid + kHalf] = s_ip_hi;
  }
  const float zc = zero_code_value<kNc>(cb_lane, lane);  // value every outlier slot decodes to
  // codebook values this lane's table entries use: entry e = a | b << KB
  const int e0 = KB == 3 ? lane : (lane & 15);  // 4-bit: cba = cb[lane & 15], the lane's U or V entry
  const float cba = half_bits_to_float(__shfl(static_cast<int>(cb_lane), e0 & (kNc - 1)) & 0xffffu);
  const float cbb = half_bits_to_float(__shfl(static_cast<int>(cb_lane), (e0 >> KB) & (kNc - 1)) & 0xffffu);

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

  // ---- rotated-query coefficients of all 64 pairs for super-tile x (one wave) ---------
  auto coefs = [&](int x) __attribute__((always_inline)) {
    const float4 qs = qsl[lane];  // (q_i, q_{i+64}, s_i, s_{i+64}), lane = pair i
    const double t0 = static_cast<double>(x) * kLutSuper;
    const float r = frac_rev(t0, thd[lane]);
    const float cs = __builtin_amdgcn_cosf(r), sn = __builtin_amdgcn_sinf(r);
    const float pa = qs.x * cs + qs.y * sn;  // R(-t0 theta) q
    const float pb = qs.y * cs - qs.x * sn;
    coef[(x & (kCR - 1)) * kHalf + lane] = make_float4(qs.z * pa, qs.z * pb, qs.w * pb, -(qs.w * pa));
    cpab[(x & (kPR - 1)) * kHalf + lane] = make_float2(pa, pb);
  };

  // ---- this wave's rows of the table of a super-tile into buffer B ---------------------
  // cc: the coefficients of pair P (read from LDS before the step's pair loop).
  auto build = [&](auto bc, float4 cc) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    float2* T = lut + B * (Sh::kBufBytes / 8);
    if constexpr (KB == 3) {
      // wave w fills the rows of pairs w + W m, m < kLutRows; lane m of every 16-lane row
      // holds their coefficients and hands them over by DPP row broadcast inside the multiplies
      asm volatile("s_nop 1" : "+v"(cc.x), "+v"(cc.y), "+v"(cc.z), "+v"(cc.w));  // DPP read wait states
      static_for<0, kLutRows>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        T[(wave + kLutWaves * m) * kNe + lane] = lut_entry_bcast<m>(cc.x, cc.y, cc.z, cc.w, cba, cbb);
      });
    } else if constexpr (KB == 2) {
      // 16 entries per row: fill step f covers the rows of 4 pairs, m = 4 f + (lane >> 4),
      // whose coefficients lane f of each 16-lane row holds (DPP row broadcast).
      asm volatile("s_nop 1" : "+v"(cc.x), "+v"(cc.y), "+v"(cc.z), "+v"(cc.w));  // DPP read wait states
      static_for<0, kLutRows / 4>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        const int i = wave + kLutWaves * (4 * f + (lane >> 4));
        T[i * kNe + (lane & 15)] = lut_entry_bcast<f>(cc.x, cc.y, cc.z, cc.w, cba, cbb);
      });
    } else {
      // separable rows: U[a] = cb[a] (alpha, beta), V[b] = cb[b] (gamma, -delta).  Fill
      // step f covers pairs 2 f (lanes 0..31) and 2 f + 1 (lanes 32..63); a 16-lane row
      // holds U or V entries only, so lane f of the row broadcasts the one coefficient pair
      // it needs.
      const bool v_row = (lane >> 4) & 1;
      float c0 = v_row ? cc.z : cc.x, c1 = v_row ? cc.w : cc.y;
      asm volatile("s_nop 1" : "+v"(c0), "+v"(c1));  // DPP read wait states
      static_for<0, kLutRows / 2>([&](auto fc) {
        constexpr int f = decltype(fc)::value;
        const int i = wave + kLutWaves * (2 * f + (lane >> 5));
        T[i * kNe + (lane & 31)] = lut_sep_bcast<f>(c0, c1, cba);
      });
    }
  };

  // Outlier slot operands, requested from LDS before the pair loop.
  // Only the reads happen here; the arithmetic on them waits for out_term, after the pair
  // loop (used at once, the channel's scale would make the step wait for every LDS read).
  struct OutOps {
    uint32_t vbits;  // the stored fp16 value
    float sc;        // its channel's key scale
    bool used;       // false for an unused slot (per-channel rule): adds nothing
    float2 th;       // theta/2pi of its pair (hi, lo)
    float2 p;        // rotated query pair of its pair
    bool lo_half;    // channel < 64
  };
  auto out_ops = [&](uint32_t c, uint32_t vbits, const float2* pab) __attribute__((always_inline)) {
    OutOps o;
    o.used = c != kNoOutlier;
    c &= kHeadDim - 1;  // a token past the length may hold stale bytes
    const int i = c & (kHalf - 1);
    o.vbits = vbits;
    o.sc = ks[c];
    o.th = thl[i];
    o.p = pab[i];
    o.lo_half = c < kHalf;
    return o;
  };
  auto out_term = [&](const OutOps& o) __attribute__((always_inline)) {
    // stored value minus the decoded zero code, at the channel's rotated query coefficient
    const float dv = o.used ? half_bits_to_float(o.vbits) - zc * o.sc : 0.0f;
    const float ph = fmaf(tauf, o.th.y, __builtin_amdgcn_fractf(tauf * o.th.x));
    const float cs = __builtin_amdgcn_cosf(ph), sn = __builtin_amdgcn_sinf(ph);
    return dv * (o.lo_half ? (o.p.x * cs + o.p.y * sn) : (o.p.y * cs - o.p.x * sn));
  };

  // ---- one tile of super-tile s from table buffer B --------------------------------------
  // Every kSB-th step (B % kSB == 0) builds the tables of super-tiles s + kSB .. s + 2 kSB - 1
  // and computes the coefficients of the kSB super-tiles after those; every step with
  // B % kSB == kSB - 1 ends in the block barrier.  A table is thus finished one barrier before
  // it is read, and a buffer or ring slot is rewritten only after a barrier that follows its
  // last read.
  auto step = [&](auto bc, int s, const LutRec<KB>& d, LutRec<KB>& ahead) __attribute__((always_inline)) {
    constexpr int B = decltype(bc)::value;
    constexpr bool kBuild = B % kSB == 0;
    float4 cc[kSB];  // build coefficients of super-tiles s + kSB + j
    if constexpr (kSB == 1) cc[0] = coef[((s + 1) & (kCR - 1)) * kHalf + P];
    const float2* pab = cpab + (s & (kPR - 1)) * kHalf;
    OutOps o0, o1;
    if (kp >= 1) o0 = out_ops(d.oi[0], d.ov[0], pab);
    if (kp >= 2) o1 = out_ops(d.oi[1], d.ov[1], pab);

    // The 64 pairs in groups of four: the table reads of the group kAhead pairs further on
    // are issued before the FMAs of this group, and those FMAs take the group's last read
    // first, so one LDS wait covers the group's four reads (a wait before every pair's FMAs
    // measured 2-5 % slower).  The scheduling barriers keep that order.
    const unsigned char* tb = lds + B * Sh::kBufBytes;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // pairs read ahead: 4-bit pairs take two reads each, and eight more registers would spill
    constexpr int kAhead = KB == 4 ? 4 : 8;
    constexpr int kRing = kAhead + 4;
    float va[kRing], vb[kRing];
    float wa[KB == 4 ? kRing : 1], wb[KB == 4 ? kRing : 1];  // 4-bit: V[b]
    auto issue = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (KB == 4) {
        uint32_t oa, ob;
        pair_offsets_sep4<i>(d.w, oa, ob);
        const float2 u = *reinterpret_cast<const float2*>(tb + i * Sh::kRowBytes + oa);
        const float2 v = *reinterpret_cast<const float2*>(tb + i * Sh::kRowBytes + 8 * kNc + ob);
        va[i % kRing] = u.x;
        vb[i % kRing] = u.y;
        wa[i % kRing] = v.x;
        wb[i % kRing] = v.y;
      } else {
        const float2 v = *reinterpret_cast<const float2*>(tb + i * Sh::kRowBytes + pair_entry_offset<KB, i>(d.w));
        va[i % kRing] = v.x;
        vb[i % kRing] = v.y;
      }
    };
    auto consume = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      constexpr int r = i % kRing;
      if constexpr (KB == 4) {
        acc[0] = fmaf(er[i], va[r], acc[0]);
        acc[1] = fmaf(ei[i], vb[r], acc[1]);
        acc[2] = fmaf(er[i], wa[r], acc[2]);
        acc[3] = fmaf(ei[i], wb[r], acc[3]);
      } else {
        acc[i & 3] = fmaf(er[i], va[r], fmaf(ei[i], vb[r], acc[i & 3]));
      }
    };
    static_for<0, kAhead>([&](auto ic) { issue(ic); });
    static_for<0, kHalf / 4>([&](auto gc) {
      constexpr int g = decltype(gc)::value;
      static_for<0, 4>([&](auto jc) {
        constexpr int i = 4 * g + kAhead + decltype(jc)::value;
        if constexpr (i < kHalf) issue(std::integral_constant<int, i>{});
      });
      // The record loads of super-tile s + 2 go out here rather than at the step start: their
      // scalar address arithmetic then overlaps the other wave's FMAs on this SIMD instead of
      // adding to the start of a step that both waves begin together after the barrier.
      if constexpr (g == 2) load_rec(s + kRecAhead, ahead);
      if constexpr (kSB > 1 && kBuild && g == 10) {
#pragma unroll
        for (int j = 0; j < kSB; ++j) cc[j] = coef[((s + kSB + j) & (kCR - 1)) * kHalf + P];
      }
      consume(std::integral_constant<int, 4 * g + 3>{});
      consume(std::integral_constant<int, 4 * g>{});
      consume(std::integral_constant<int, 4 * g + 1>{});
      consume(std::integral_constant<int, 4 * g + 2>{});
      __builtin_amdgcn_sched_barrier(0);
    });
    float l = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    // Outliers: the record holds the zero code at each outlier channel; replace its decoded
    // value zc * s_c by the stored fp16 value at the channel's rotated query coefficient.
    if (kp >= 1) l += out_term(o0);
    if (kp >= 2) l += out_term(o1);
    const int t0 = (kLutWaves * s + wave) * kTile;  // wave-uniform
    const int t = t0 + lane;
    if (t < L) {
      if constexpr (kExtra) {
        const size_t o = (stream * S + t) * k;
        for (int j = kLutPrefetchOutliers; j < k; ++j) l += out_term(out_ops(a.k_idx[o + j], a.k_val[o + j], pab));
      }
      (a.logits + (static_cast<size_t>(seq) * a.n_q_heads + kvh) * S + t0)[lane] = a.sm_scale * l;
    }
    if constexpr (kBuild) {
      static_for<0, kSB>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        if (s + kSB + j < s_hi) build(std::integral_constant<int, (B + kSB + j) % kNB>{}, cc[j]);
      });
#pragma unroll
      for (int j = 0; j < kSB; ++j)
        if (wave == ((s + j) & (kLutWaves - 1)) && s + 2 * kSB + j < s_hi) coefs(s + 2 * kSB + j);
    }
    if constexpr (B % kSB == kSB - 1) block_lds_barrier();
  };

  // ---- main loop -----------------------------------------------------------------------
  block_lds_barrier();  // qsl, thd, ks, thl visible
  if (wave < 2 * kSB && s_lo + wave < s_hi) coefs(s_lo + wave);
  block_lds_barrier();  // the coefficients of the first 2 kSB super-tiles visible
  static_for<0, kSB>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    if (s_lo + j < s_hi) build(std::integral_constant<int, j>{}, coef[((s_lo + j) & (kCR - 1)) * kHalf + P]);
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
  } else if constexpr (kRecAhead == 1) {
    static_assert(kNB == 4, "buffer count");
    // four steps per round: two record sets by four table buffers
    for (int s = s_lo; s < s_hi; s += 4) {
      step(I0{}, s, r0, r1);
      if (s + 1 >= s_hi) break;
      step(I1{}, s + 1, r1, r0);
      if (s + 2 >= s_hi) break;
      step(I2{}, s + 2, r0, r1);
      if (s + 3 >= s_hi) break;
      step(I3{}, s + 3, r1, r0);
    }
  } else {
    // eight steps per round: four record sets by eight table buffers
    static_assert(kNB == 8, "buffer count");
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

template <int KB, bool kExtra>
hipError_t launch_qk_lut_t(int batch, const QkArgs& a0, hipStream_t st) {
  QkArgs a = a0;
  // One resident round: the device's block slots shared equally among the streams, each
  // block walking a contiguous run of super-tiles.
  const int tiles = (a.max_len + kTile - 1) / kTile;
  const int supers = (tiles + kLutWaves - 1) / kLutWaves;
  const long streams = static_cast<long>(batch) * a.n_kv_heads;
  static const int resident = [&] {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(&qk_lut_kernel<KB, kExtra>),
                                                     kLutThreads, 0) != hipSuccess || n < 1)
      n = 1;
    return n;
  }();
  const long slots = static_cast<long>(device_cu_count()) * resident;
  const long per_stream = std::max(1L, std::min<long>((slots + streams - 1) / streams, supers));
  a.tiles_per_wave = static_cast<int>((supers + per_stream - 1) / per_stream);  // super-tiles per block
  dim3 grid((supers + a.tiles_per_wave - 1) / a.tiles_per_wave, a.n_kv_heads, batch);
  hipLaunchKernelGGL((qk_lut_kernel<KB, kExtra>), grid, dim3(kLutThreads), 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_qk_lut(int k_bits, int batch, const QkArgs& a, hipStream_t s) {
  const bool extra = a.n_outliers > kLutPrefetchOutliers;
  if (k_bits == 2) return extra ? launch_qk_lut_t<2, true>(batch, a, s) : launch_qk_lut_t<2, false>(batch, a, s);
  if (k_bits == 3) return extra ? launch_qk_lut_t<3, true>(batch, a, s) : launch_qk_lut_t<3, false>(batch, a, s);
  if (k_bits == 4) return extra ? launch_qk_lut_t<4, true>(batch, a, s) : launch_qk_lut_t<4, false>(batch, a, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
