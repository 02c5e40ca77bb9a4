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
//   * R(tau), tau = lane < 64, from a per-block LDS table (with all 64 pairs in registers
//     the kernel would drop to two waves per SIMD; 16 or 32 of them measured no faster).
// The record keeps the two halves of rotary pair i side by side, so one 2b-bit field
// indexes a small shared table of fp16 pairs (cb[a], cb[b]).  With g > 1 query heads the
// key is dequantized (the fp16 codebook pair scaled by the pair's two channel scales),
// rotated once and dotted with every head.  This kernel serves 4-bit keys with grouped
// heads; one head per kv head goes to the table kernel (qk_lut.hip, every bit width) and
// 2/3-bit grouped heads to the matrix-core kernel (qk_mfma.hip).
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kWaves = 4;
constexpr int kPrefetchOutliers = 2;  // outliers per token fetched with the record

template <int KB>
struct Rec {
  uint32_t w[4 * KB];  // the token's key record
  uint32_t oi[2], ov[2];  // its first two outliers: channels and fp16 value bits
};
constexpr int kPartials = 4;  // partial sums per logit

template <int KB, int G>
__global__ __launch_bounds__(256) void qk_kernel(QkArgs a) {
  constexpr int kNc = 1 << KB;
  constexpr int kPairEntries = 1 << (2 * KB);
  static_assert(KB == 4 && G > 1, "4-bit keys, grouped heads (the table kernels serve the rest)");

  __shared__ float2 et[kHalf][kTile];       // R(tau) for pair i: (cos, sin) of tau * theta_i
  using Tab = RepTable<kPairEntries>;
  __shared__ uint32_t lutp[Tab::kWords];  // fp16 (cb[a], cb[b]) for a pair field a | b << KB, replicated
  __shared__ float ks[kHeadDim];
  __shared__ float2 ksp[kHalf];             // (s_i, s_{i+64})
  __shared__ float2 qr[kWaves][G][kHalf];   // per-wave tile-rotated query pairs
  __shared__ float2 tb[kWaves][kHalf];      // per wave: R(t0 theta_i) at its first tile
  __shared__ float2 tstep[kHalf];           // R(64 theta_i), the step between tiles

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int H = a.n_kv_heads;
  const int S = a.max_seq;
  const int k = a.n_outliers;
  const int L = min(a.seq_len[seq] & kLenMask, a.max_len);
  const int block_tile0 = blockIdx.x * a.tiles_per_wave * kWaves;
  if (block_tile0 * kTile >= L) return;

  const int wave_tile0 = block_tile0 + wave * a.tiles_per_wave;
  const int n_tiles = min(a.tiles_per_wave, (L - wave_tile0 * kTile + kTile - 1) / kTile);
  const size_t stream = static_cast<size_t>(seq) * H + kvh;
  const uint8_t* recs = a.k_codes + stream * S * (16 * KB);
  // last tile a prefetch may touch; a wave without tiles reads tile 0 (always valid)
  const int last_tile = n_tiles > 0 ? wave_tile0 + n_tiles - 1 : 0;
  // The first kPrefetchOutliers outliers of every token travel with its record; with
  // fewer outliers the spare loads repeat a real one or read the first code word, and
  // their results are ignored.
  const int kp = min(k, kPrefetchOutliers);
  const uint8_t* o_idx = kp > 0 ? a.k_idx : a.k_codes;
  const uint16_t* o_val = kp > 0 ? a.k_val : reinterpret_cast<const uint16_t*>(a.k_codes);
  const size_t o_stride = kp > 0 ? k : 0;
  const int o_second = kp > 1 ? 1 : 0;

  // Loads through buffer descriptors rebuilt per tile at the tile's first token (scalar
  // arithmetic) with fixed per-lane offsets: no vector address arithmetic per tile.
  const uint32_t rec_off = static_cast<uint32_t>(lane) * (16 * KB);
  const uint32_t out_off = static_cast<uint32_t>(lane * o_stride);  // outlier entries before this lane's
  const uint32_t second_off = out_off + o_second;
  const uint32_t tile_outs = static_cast<uint32_t>(kTile * o_stride);
  auto load_rec = [&](int tile, Rec<KB>& d) {
    tile = min(tile, last_tile);  // past the run: reload the last tile (cache hit), keeps the load count fixed
    const size_t tok0 = static_cast<size_t>(tile) * kTile;  // wave-uniform
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

  // Query pairs this lane rotates every tile.  Slot j holds rotary pair
  // (lane & 15) + 16 j, so lane n of every 16-lane row holds the pairs congruent to n mod
  // 16 and a row broadcast hands pair i's coefficient to all lanes.  The pair `lane` itself
  // (needed in LDS) is slot lane >> 4.
  constexpr int kSlots = kHalf / 16;
  // Raw query words (fp16 or fp32 bits), converted only after the tile prefetch is issued.
  uint32_t ra[kSlots][G], rb[kSlots][G];
  const size_t q0 = (static_cast<size_t>(seq) * a.n_q_heads + kvh * G) * kHeadDim + (lane & 15);
  if (a.q_is_fp16) {  // wave-uniform; both paths issue the same loads
    const uint16_t* q16 = static_cast<const uint16_t*>(a.q) + q0;
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        ra[j][h] = q16[h * kHeadDim + 16 * j];
        rb[j][h] = q16[h * kHeadDim + 16 * j + kHalf];
      }
  } else {
    const uint32_t* q32 = static_cast<const uint32_t*>(a.q) + q0;
#pragma unroll
    for (int j = 0; j < kSlots; ++j)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        ra[j][h] = q32[h * kHeadDim + 16 * j];
        rb[j][h] = q32[h * kHeadDim + 16 * j + kHalf];
      }
  }
  // Set-up inputs, loaded ahead of the tile prefetch so that waiting for them never
  // waits for the prefetch (global loads complete in issue order).
  // Every thread writes its table entries (indices masked, so threads that share an entry
  // write the same value): no load is guarded by a branch the compiler could sink it into.
  const float ks_own = a.k_scale[kvh * kHeadDim + (tid & (kHeadDim - 1))];
  const float ks_lo = a.k_scale[kvh * kHeadDim + (tid & (kHalf - 1))];
  const float ks_hi = a.k_scale[kvh * kHeadDim + (tid & (kHalf - 1)) + kHalf];
  const uint32_t cb_lo = a.k_cb[lane & (kNc - 1)];
  static_assert(kPairEntries <= 256, "one table entry per thread");
  const double th_rev = a.theta_rev[lane];

  // The first two tiles are requested before the tables are built, so their memory
  // latency overlaps the set-up.
  // Every load here is unconditional (clamped addresses), so the compiler can count the
  // loads in flight exactly and wait only for the ones it needs.
  Rec<KB> r0, r1, r2;
  load_rec(wave_tile0, r0);
  load_rec(wave_tile0 + 1, r1);

  // ---- per-block tables -----------------------------------------------------------
  ks[tid & (kHeadDim - 1)] = ks_own;
  ksp[tid & (kHalf - 1)] = make_float2(ks_lo, ks_hi);
  for (int wd = tid; wd < Tab::kWords; wd += 256) {  // word wd holds entry wd / copies
    const int e = wd / Tab::kCopies;                 // codebook entries from the lanes holding them
    const uint32_t lo = static_cast<uint32_t>(__shfl(static_cast<int>(cb_lo), e & (kNc - 1))) & 0xffffu;
    const uint32_t hi = static_cast<uint32_t>(__shfl(static_cast<int>(cb_lo), e >> KB)) & 0xffffu;
    lutp[wd] = lo | (hi << 16);
  }
  float qa[kSlots][G], qb[kSlots][G];
#pragma unroll
  for (int j = 0; j < kSlots; ++j)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      qa[j][h] = a.q_is_fp16 ? half_bits_to_float(ra[j][h]) : __builtin_bit_cast(float, ra[j][h]);
      qb[j][h] = a.q_is_fp16 ? half_bits_to_float(rb[j][h]) : __builtin_bit_cast(float, rb[j][h]);
    }
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
  {
    // pair `lane`: its phase at the wave's first tile, and the per-tile step
    float sb, cb, sst, cst;
    sincos_rev(frac_rev(static_cast<double>(wave_tile0) * kTile, th_rev), &sb, &cb);
    sincos_rev(frac_rev(static_cast<double>(kTile), th_rev), &sst, &cst);
    tb[wave][lane] = make_float2(cb, sb);
    tstep[lane] = make_float2(cst, sst);  // every wave writes the same value
  }
  // value every outlier slot decodes to: the codebook entry nearest zero
  const float zc = zero_code_value<kNc>(cb_lo, lane);
  block_lds_barrier();
  float bc[kSlots], bs[kSlots], sc[kSlots], ss[kSlots];  // slot pairs' tile-base phase and per-tile step
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int pr = (lane & 15) + 16 * j;
    const float2 b = tb[wave][pr], st = tstep[pr];
    bc[j] = b.x;
    bs[j] = b.y;
    sc[j] = st.x;
    ss[j] = st.y;
  }

  if (n_tiles <= 0) return;  // after the block's last barrier

  const int my_slot = lane >> 4;
  const uint32_t tab_base = Tab::lane_base(lane);
  static_assert(kSlots == 4, "four 16-lane rows");
  auto pick = [&](float v0, float v1, float v2, float v3) {
    return my_slot == 0 ? v0 : my_slot == 1 ? v1 : my_slot == 2 ? v2 : v3;
  };

  auto process = [&](int tile, const Rec<KB>& d) {
    // q' = R(-t0) q for the slot pairs of every head, then step the base phases.
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
    }
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const float nc = bc[j] * sc[j] - bs[j] * ss[j];
      const float ns = bs[j] * sc[j] + bc[j] * ss[j];
      bc[j] = nc;
      bs[j] = ns;
    }
    wave_lds_sync();

    const int t = tile * kTile + lane;
    // Independent partial sums keep the FMA chains short, so the scheduler interleaves
    // pairs instead of computing every rotated pair before the first accumulation.
    float accp[G][kPartials];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int u = 0; u < kPartials; ++u) accp[h][u] = 0.0f;

    // Per pair: the table entry (fp16 codebook pair), R(tau) and the heads' query pairs are
    // read from LDS beside their use.
    static_for<0, kHalf>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      const uint32_t e2 = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const unsigned char*>(lutp) +
                                                             Tab::at(field<2 * KB, 2 * KB * i>(d.w), tab_base));
      const float2 e = et[i][lane];  // R(tau) of pair i for this lane's token
      const float2 sp = ksp[i];
      const float xa = half_bits_to_float(e2 & 0xffffu) * sp.x;
      const float xb = half_bits_to_float(e2 >> 16) * sp.y;
      const float ya = xa * e.x - xb * e.y;
      const float yb = xa * e.y + xb * e.x;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float2 qq = qr[wave][h][i];
        accp[h][i % kPartials] = fmaf(qq.y, yb, fmaf(qq.x, ya, accp[h][i % kPartials]));
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
    auto add_outlier = [&](int c, uint32_t vbits) {
      const bool used = c != static_cast<int>(kNoOutlier);  // an unused slot (per-channel rule) adds nothing
      c &= kHeadDim - 1;                                     // a token past the length may hold stale bytes
      const float dv = used ? half_bits_to_float(vbits) - zc * ks[c] : 0.0f;
      const int i = c & (kHalf - 1);
      const float2 e = et[i][lane];
      const bool upper = c >= kHalf;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float2 qq = qr[wave][h][i];
        acc[h] += dv * (upper ? (qq.y * e.x - qq.x * e.y) : (qq.x * e.x + qq.y * e.y));
      }
    };
    if (kp >= 1) add_outlier(d.oi[0], d.ov[0]);
    if (kp >= 2) add_outlier(d.oi[1], d.ov[1]);
    if (t < L) {
      const size_t o = (stream * S + t) * k;
      for (int j = kPrefetchOutliers; j < k; ++j) add_outlier(a.k_idx[o + j], a.k_val[o + j]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        a.logits[(static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * S + t] = a.sm_scale * acc[h];
      }
    }
    __builtin_amdgcn_wave_barrier();
  };

  // Three buffers: the tiles it+1 and it+2 are in flight while tile it is used.
  for (int it = 0; it < n_tiles; it += 3) {
    load_rec(wave_tile0 + it + 2, r2);
    process(wave_tile0 + it, r0);
    if (it + 1 >= n_tiles) break;
    load_rec(wave_tile0 + it + 3, r0);
    process(wave_tile0 + it + 1, r1);
    if (it + 2 >= n_tiles) break;
    load_rec(wave_tile0 + it + 4, r1);
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
  // 4-bit keys with grouped heads; the table kernels (qk_lut.hip, qk_mfma.hip) serve the rest
  KVQ_QK_CASE(4, 2) KVQ_QK_CASE(4, 4) KVQ_QK_CASE(4, 8)
#undef KVQ_QK_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
