// softmax(P) . V over the compressed value cache plus the sparse value outliers, split
// over the sequence with a second-pass log-sum-exp combine.
//
// KVQuant summary page, abstract paragraph, techniques (iii) and (iv): values are decoded
// through the layer's codebook and their per-vector scale, and each vector's fp16
// outliers are added back.  The split over the sequence lets a single long sequence fill
// the GPU.
//
// pv_partial: the device's block slots are shared equally among the (sequence, kv head)
// streams; a block owns a contiguous run of 64-token tiles of one stream and each of its
// four waves walks its own share of that run independently, with its own running
// (max, sum) softmax state and the next tile's data already in flight.  Per tile:
//   * lane = token: the tile's max logit per query head raises the running max m (with
//     one head, only a logit more than 16 above m), rescaling the running state;
//     p_t = exp(l_t - m), w_t = p_t * s_t, and the outlier corrections
//     p_t * (x_c - zc * s_t) are summed per channel in fixed point (integer atomics on
//     the wave's own LDS rows, so the sums do not depend on the order the atomics land);
//   * lane = channel pair (2l, 2l+1): the 2b-bit field holding two consecutive tokens of
//     one channel indexes a small table of fp16 pairs (cb[a], cb[b]).  With one query head
//     w_t reaches every lane as a scalar operand (read from lane t) of a packed fp16 dot
//     product; with several, the fp16 weights of 4 heads are the A operand and the fp16
//     codebook values of 4 tokens of a channel the B operand of v_mfma_f32_4x4x4_16b_f16.
// The four waves merge their states once at the end; each block writes one (o, m, l).
// pv_combine: one block per (sequence, query head) merges the block partials.
#include <algorithm>
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

typedef _Float16 pv_half4 __attribute__((ext_vector_type(4)));
typedef float pv_float4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMinTilesPerBlock = 16;   // parts never outnumber ceil(max_len / 1024)
constexpr int kPrefetchOutliers = 2;    // outliers per token held in registers
// How far a logit may exceed the running max of a single query head before the max is
// raised: weights stay below e^16 (about 8.9e6), far inside fp32 and the per-tile
// rescaling of the dense and outlier sums, and a tile's max is computed only when the max
// moves (1-2 % fewer cycles).
constexpr float kRunSlack = 16.0f;

template <int VB, int G>
struct TileData {
  uint32_t w[4 * VB];  // this lane's value-tile words (channels 2l, 2l+1)
  float lg[G];         // logit of token `lane` for every query head of the group
  uint32_t sv;         // fp16 value scale of token `lane`
  uint32_t oi[2], ov[2];  // its first two outliers: channels and fp16 value bits
};

template <int VB, int G>
__global__ __launch_bounds__(256) void pv_partial_kernel(PvArgs a) {
  constexpr int kNc = 1 << VB;
  constexpr int kChanBits = 64 * VB;
  constexpr int kPairEntries = 1 << (2 * VB);

  // With 2-bit values one byte (four consecutive tokens of a channel) indexes a 256-entry
  // table of the four fp16 codebook values; otherwise a field of two tokens indexes a table
  // of fp16 pairs.  (A 4096-entry quad table for 3-bit values measured slower: its 32 KB
  // cost resident blocks and its random reads conflict.)
  constexpr bool kQuad = VB == 2;
  constexpr int kQuadEntries = kQuad ? 1 << (4 * VB) : 1;
  __shared__ uint32_t lut2[kPairEntries];         // fp16 (cb[a], cb[b]) for a token pair
  __shared__ uint2 lut4[kQuadEntries];            // fp16 (cb[a], cb[b], cb[c], cb[d]) for a token quad
  __shared__ uint32_t cbs[kNc];                   // fp16 codebook (for building lut4)
  __shared__ __align__(16) int osi[kWaves][G][kHeadDim];  // per-wave, per-tile fixed-point outlier sums (64-bit exchanges)
  __shared__ float wm[kWaves][G], wl[kWaves][G];  // per-wave max and sum
  __shared__ float wo[kWaves][G][kHeadDim];       // per-wave weighted sums
  // With several query heads the tile's fp16 weight pairs are staged in LDS and read back
  // at wave-uniform addresses (broadcast), four pairs per read, instead of one lane read
  // (a VALU instruction) per pair and head; with one head the lane reads measured faster.
  // Several query heads: the dense part runs on the matrix cores, with this wave's fp16
  // weights staged in LDS as [head][token] rows (rows past G stay zero).  With one head the
  // packed dot products measured faster (1M 2-bit layer: 294 against 353 us; 128K 4-bit:
  // 74 against 83 us): three of the four MFMA rows would carry nothing.
  constexpr bool kMfma = G > 1;
  constexpr int kGroups = G > 4 ? G / 4 : 1;
  __shared__ _Float16 wsh[kMfma ? kWaves : 1][kMfma ? 4 * kGroups : 1][kMfma ? kTile : 1];
  constexpr bool kStageW = G > 1 && !kMfma;
  __shared__ uint4 wst[kStageW ? kWaves : 1][G][kTile / 8];  // (w_2m, w_2m+1) at word m

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, kept in an SGPR
  const int kvh = blockIdx.y;
  const int seq = blockIdx.z;
  const int H = a.n_kv_heads;
  const int S = a.max_seq;
  const int k = a.n_outliers;
  const int L = min(a.seq_len[seq] & kLenMask, a.max_len);
  const int n_tiles = (L + kTile - 1) / kTile;
  const int tile_lo = blockIdx.x * a.tiles_per_block;
  const int tile_hi = min(tile_lo + a.tiles_per_block, n_tiles);
  const size_t part_stride = kHeadDim + 2;
  const size_t stream = static_cast<size_t>(seq) * H + kvh;
  auto part_ptr = [&](int h) {
    return a.partial + ((static_cast<size_t>(seq) * a.n_q_heads + kvh * G + h) * a.n_parts + blockIdx.x) * part_stride;
  };

  if (tile_lo >= tile_hi) {
    for (int e = tid; e < G * (kHeadDim + 2); e += kThreads) {
      const int h = e / (kHeadDim + 2), c = e % (kHeadDim + 2);
      part_ptr(h)[c] = (c == kHeadDim) ? -INFINITY : 0.0f;
    }
    return;
  }

  // This wave's share of the block's tiles.
  const int nt = tile_hi - tile_lo;
  const int w_lo = tile_lo + (nt * wave) / kWaves;
  const int w_hi = tile_lo + (nt * (wave + 1)) / kWaves;

  const uint8_t* vtiles = a.v_codes + stream * (S / kTile) * (1024 * VB);
  const float* lbase = a.logits + (static_cast<size_t>(seq) * a.n_q_heads + kvh * G) * S;
  // The first kPrefetchOutliers outliers of every token travel with its tile data; with
  // fewer outliers the spare loads repeat a real one or read the first code word, and
  // their results are ignored.
  const int kp = min(k, kPrefetchOutliers);
  const uint8_t* o_idx = kp > 0 ? a.v_idx : a.v_codes;
  const uint16_t* o_val = kp > 0 ? a.v_val : reinterpret_cast<const uint16_t*>(a.v_codes);
  const size_t o_stride = kp > 0 ? k : 0;
  const int o_second = kp > 1 ? 1 : 0;

  // Every call issues the same loads (a tile past the wave's run reloads its last tile,
  // a cache hit), so the compiler can wait for exactly the tile being consumed.  The loads
  // go through buffer descriptors rebuilt per tile at the tile's first token (scalar
  // arithmetic) with fixed per-lane offsets, so they cost no vector instructions.
  const uint32_t val_off = static_cast<uint32_t>(lane) * (16 * VB);
  const uint32_t out_off = static_cast<uint32_t>(lane * o_stride);  // outlier entries before this lane's
  const uint32_t second_off = out_off + o_second;
  const uint32_t tile_outs = static_cast<uint32_t>(kTile * o_stride);
  auto load = [&](int tile, TileData<VB, G>& d) {
    tile = max(0, min(tile, w_hi - 1));  // a wave without tiles reads tile 0 (always valid)
    const size_t t0 = static_cast<size_t>(tile) * kTile;  // wave-uniform; t0 + 64 <= max_seq
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(vtiles + static_cast<size_t>(tile) * (1024 * VB), 1024 * VB);
#pragma unroll
    for (int v = 0; v < VB; ++v) {
      const u32x4 q = buf_load_b128(rt, val_off + 16 * v);
      d.w[4 * v + 0] = q.x;
      d.w[4 * v + 1] = q.y;
      d.w[4 * v + 2] = q.z;
      d.w[4 * v + 3] = q.w;
    }
    const __amdgpu_buffer_rsrc_t rl = make_rsrc(lbase + t0, static_cast<uint32_t>(((G - 1) * static_cast<size_t>(S) + kTile) * 4));
#pragma unroll
    for (int h = 0; h < G; ++h)
      d.lg[h] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rl, 4u * lane, static_cast<uint32_t>(h * static_cast<size_t>(S) * 4), 0));
    const size_t slot0 = stream * S + t0;
    d.sv = buf_load_u16(make_rsrc(a.v_scale + slot0, 2 * kTile), 2u * lane);
    const __amdgpu_buffer_rsrc_t ri = make_rsrc(o_idx + slot0 * o_stride, tile_outs + 1);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(o_val + slot0 * o_stride, 2 * tile_outs + 2);
    d.oi[0] = buf_load_u8(ri, out_off);
    d.oi[1] = buf_load_u8(ri, second_off);
    d.ov[0] = buf_load_u16(rv, 2 * out_off);
    d.ov[1] = buf_load_u16(rv, 2 * second_off);
  };

  // Set-up inputs first, then the wave's first tile, so that the tile's memory latency
  // overlaps the set-up and waiting for the inputs never waits for the tile (global loads
  // complete in issue order).
  static_assert(kPairEntries <= kThreads, "one table entry per thread");
  const uint32_t cb_a = a.v_cb[tid & (kNc - 1)];
  const uint32_t cb_b = a.v_cb[(tid >> VB) & (kNc - 1)];
  const uint32_t cb_lo = a.v_cb[lane & (kNc - 1)];
  TileData<VB, G> bufA, bufB;
  load(w_lo, bufA);  // unconditional, so the compiler counts the loads in flight exactly

  lut2[tid & (kPairEntries - 1)] = cb_a | (cb_b << 16);  // threads sharing an entry write the same value
  if (kQuad && tid < kNc) cbs[tid] = cb_a;               // cb_a = cb[tid] for tid < 2^VB
  for (int e = tid; e < kWaves * G * kHeadDim; e += kThreads) (&osi[0][0][0])[e] = 0;
  if constexpr (kMfma) {
    for (int e = tid; e < kWaves * 4 * kGroups * kTile; e += kThreads) (&wsh[0][0][0])[e] = static_cast<_Float16>(0.0f);
  }
  const float zc = zero_code_value<kNc>(cb_lo, lane);  // value every outlier slot decodes to
  block_lds_barrier();
  if constexpr (kQuad) {
    constexpr uint32_t m = kNc - 1;
    for (int e = tid; e < kQuadEntries; e += kThreads) {
      const uint32_t c0 = cbs[e & m], c1 = cbs[(e >> VB) & m], c2 = cbs[(e >> (2 * VB)) & m], c3 = cbs[(e >> (3 * VB)) & m];
      lut4[e] = make_uint2(c0 | (c1 << 16), c2 | (c3 << 16));
    }
    block_lds_barrier();
  }


  float m_run[G], lsum[G], acc[G][2];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m_run[h] = -INFINITY;
    lsum[h] = 0.0f;
    acc[h][0] = acc[h][1] = 0.0f;
  }

  auto compute = [&](int tile, const TileData<VB, G>& d) {
    const int t = tile * kTile + lane;
    const bool valid = t < L;
    const float s = half_bits_to_float(d.sv);
    float pr[G], wts[G], lgv[G], mtv[G], wmaxv[G];
    // With one query head the running max is raised only when a logit of the tile exceeds
    // it by more than kRunSlack (always on the wave's first tile with a valid token): the
    // tile's max then takes one DPP pass, and weights exp(l - m) stay below e^kRunSlack
    // otherwise.  Several heads share one fixed-point outlier scale, set by the largest
    // p * |dv| of the group; that bounds each head's rounding only while every head's
    // weights are at most 1, so they raise the max on every tile.
    bool over = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      lgv[h] = valid ? d.lg[h] : -INFINITY;
      over |= lgv[h] > m_run[h] + kRunSlack;
    }
    if (G > 1 || __builtin_amdgcn_ballot_w64(over) != 0) {  // wave-uniform
      wave_max_n_f32<G>(lgv, mtv);  // the tile's max logit of every head, in one pass
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float mt = mtv[h];
        if (mt > m_run[h]) {  // wave-uniform: rescale the running state to the new max
          const float sc = m_run[h] > -INFINITY ? expf(m_run[h] - mt) : 0.0f;
          m_run[h] = mt;
          acc[h][0] *= sc;
          acc[h][1] *= sc;
          lsum[h] *= sc;
        }
      }
    }
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float lg = lgv[h];
      pr[h] = valid ? __expf(lg - m_run[h]) : 0.0f;  // hardware exp2 of x log2(e): relative error < 4e-6 measured on [-100, 0]; smaller argument rounding on (0, 16]
      lsum[h] += pr[h];
      wts[h] = pr[h] * s;
    }
    wave_lds_sync();
    // Outliers: the dense code at an outlier channel is the zero code, so channel c gets
    // p_t * (x_c - zc * s_t).  These are summed per tile in 32-bit fixed point with integer
    // LDS atomics (float atomics on LDS are slow on this device, about 190 cycles per wave
    // instruction, and their sums would depend on the order they land): the scale
    // 2^(23 - e), with 2^e above the tile's largest |contribution| over every outlier and
    // head, keeps each term below 2^23, and a channel receives at most one term per token
    // (a vector's outlier channels are distinct), so a tile's sum stays below 2^29.  Each
    // term is rounded to 2^-24 of 2^e.  The first two outliers of every token travel with
    // the tile data; further ones are read twice from global memory (cache hits the second
    // time), once for the scale and once for the sums.  Each channel lane folds its two
    // channels into its accumulators after the atomics.
    float unscale = 0.0f;
    bool have_fixed = false;
    {
      const float dv0 = half_bits_to_float(d.ov[0]) - zc * s;
      const float dv1 = half_bits_to_float(d.ov[1]) - zc * s;
      const int c0 = d.oi[0] & (kHeadDim - 1), c1 = d.oi[1] & (kHeadDim - 1);  // stale bytes past the length
      const bool more = k > kPrefetchOutliers && valid;
      const size_t slot = (stream * S + t) * k;
      float dmax = fmaxf(kp >= 1 ? fabsf(dv0) : 0.0f, kp >= 2 ? fabsf(dv1) : 0.0f);
      if (more) {
        for (int j = kPrefetchOutliers; j < k; ++j) dmax = fmaxf(dmax, fabsf(half_bits_to_float(a.v_val[slot + j]) - zc * s));
      }
      float mloc = 0.0f;
#pragma unroll
      for (int h = 0; h < G; ++h) mloc = fmaxf(mloc, pr[h] * dmax);
      // one outlier scale for every head of the group; with it, the tile's largest weight of
      // every head (the dense part's prescale)
      float m;
      if constexpr (G == 1) {
        wave_max2_f32(wts[0], mloc, wmaxv[0], m);
      } else {
        wave_max_n_f32<G>(wts, wmaxv);
        m = wave_max_f32(mloc);
      }
      have_fixed = m > 0.0f;               // wave-uniform
      if (have_fixed) {
        const int e = min(max(static_cast<int>((__builtin_bit_cast(uint32_t, m) >> 23) & 0xffu) - 126, -100), 100);
        const float sc = __builtin_bit_cast(float, static_cast<uint32_t>(23 - e + 127) << 23);  // 2^(23-e)
        unscale = __builtin_bit_cast(float, static_cast<uint32_t>(e - 23 + 127) << 23);       // 2^(e-23)
#pragma unroll
        for (int h = 0; h < G; ++h) {
          int* row = &osi[wave][h][0];
          if (kp >= 1) atomicAdd(row + c0, static_cast<int>(rintf(pr[h] * dv0 * sc)));
          if (kp >= 2) atomicAdd(row + c1, static_cast<int>(rintf(pr[h] * dv1 * sc)));
        }
        if (more) {
          for (int j = kPrefetchOutliers; j < k; ++j) {
            const int c = a.v_idx[slot + j] & (kHeadDim - 1);
            const float dv = half_bits_to_float(a.v_val[slot + j]) - zc * s;
#pragma unroll
            for (int h = 0; h < G; ++h) atomicAdd(&osi[wave][h][c], static_cast<int>(rintf(pr[h] * dv * sc)));
          }
        }
      }
    }
    wave_lds_sync();
    // This tile's fixed-point outlier sums of channels (2l, 2l+1), read and cleared by one
    // LDS exchange (one instruction instead of a read and a write: 1M value pass 291.7 ->
    // 284.8 us).
    if (have_fixed) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        unsigned long long* cell = reinterpret_cast<unsigned long long*>(&osi[wave][h][2 * lane]);
        const unsigned long long q = __hip_atomic_exchange(cell, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WAVEFRONT);
        acc[h][0] = fmaf(static_cast<float>(static_cast<int>(static_cast<uint32_t>(q))), unscale, acc[h][0]);
        acc[h][1] = fmaf(static_cast<float>(static_cast<int>(static_cast<uint32_t>(q >> 32))), unscale, acc[h][1]);
      }
    }
    // Dense part: lane = channel pair, the token weights in fp16 against fp16 codebook
    // values (products exact in fp32, fp32 accumulation).  Each tile's weights are scaled by
    // 2^sh, which puts the tile's largest weight in [2^13, 2^14): every weight whose rounding
    // matters is then a normal fp16 number, so its relative error is at most 2^-11 and the
    // output's at most 2^-11 sum_t p_t |v~_t,c|; 2^-sh is undone exactly after the tile.
    if constexpr (kMfma) {
      // Dense part on the matrix cores: v_mfma_f32_4x4x4_16b_f16 with the tile's fp16
      // weights of 4 heads as the A operand (row m = head, the same in all 16 blocks, read
      // back from this wave's LDS rows) and the fp16 codebook values of 4 consecutive tokens
      // of one channel as the B operand (block b, column n = lane 4b + n: channel 2l + half
      // of lane l), so one MFMA adds 4 tokens of 64 channels for 4 heads and lane l ends
      // with o[h][2l + half] in row h of its result.  Weights are prescaled per tile and
      // head as in the packed-dot path (largest in [2^13, 2^14), relative rounding error
      // at most 2^-11).
      float unsc[G];
      _Float16* wrow = &wsh[kMfma ? wave : 0][0][0];
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float wmax = wmaxv[h];
        const int ex = wmax > 0.0f ? static_cast<int>((__builtin_bit_cast(uint32_t, wmax) >> 23) & 0xffu) - 127 : 0;
        const int sh = min(max(13 - ex, -100), 100);  // 2^sh * wmax in [2^13, 2^14)
        unsc[h] = __builtin_bit_cast(float, static_cast<uint32_t>(127 - sh) << 23);
        wrow[h * kTile + lane] = static_cast<_Float16>(wts[h] * __builtin_bit_cast(float, static_cast<uint32_t>(127 + sh) << 23));
      }
      wave_lds_sync();
      const unsigned char* wa = reinterpret_cast<const unsigned char*>(wrow) + (lane & 3) * (kTile * 2);
      pv_float4 dacc[kGroups][2];
#pragma unroll
      for (int g = 0; g < kGroups; ++g) dacc[g][0] = dacc[g][1] = pv_float4{0.0f, 0.0f, 0.0f, 0.0f};
      // The operands of step j + 1 (table lookups and weight rows) are requested before the
      // products of step j, so the wait before each step's products leaves the next step's
      // reads in flight instead of draining every LDS read (they complete in order).
      uint2 bq[2][2], aw[2][kGroups];
      auto fetch = [&](auto jc) __attribute__((always_inline)) {
        constexpr int j = decltype(jc)::value;
        constexpr int b = j & 1;
        if constexpr (kQuad) {
          bq[b][0] = lut4[field<4 * VB, 4 * VB * j>(d.w)];
          bq[b][1] = lut4[field<4 * VB, kChanBits + 4 * VB * j>(d.w)];
        } else {
          bq[b][0] = make_uint2(lut2[field<2 * VB, 4 * VB * j>(d.w)], lut2[field<2 * VB, 4 * VB * j + 2 * VB>(d.w)]);
          bq[b][1] = make_uint2(lut2[field<2 * VB, kChanBits + 4 * VB * j>(d.w)],
                                lut2[field<2 * VB, kChanBits + 4 * VB * j + 2 * VB>(d.w)]);
        }
#pragma unroll
        for (int g = 0; g < kGroups; ++g) aw[b][g] = *reinterpret_cast<const uint2*>(wa + g * (4 * kTile * 2) + j * 8);
      };
      fetch(std::integral_constant<int, 0>{});
      static_for<0, kTile / 4>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int b = j & 1;
        if constexpr (j + 1 < kTile / 4) fetch(std::integral_constant<int, j + 1>{});
#pragma unroll
        for (int g = 0; g < kGroups; ++g) {
#pragma unroll
          for (int hf = 0; hf < 2; ++hf) {
            dacc[g][hf] = __builtin_amdgcn_mfma_f32_4x4x4f16(__builtin_bit_cast(pv_half4, aw[b][g]),
                                                             __builtin_bit_cast(pv_half4, bq[b][hf]), dacc[g][hf], 0, 0, 0);
            asm volatile("" : "+a"(dacc[g][hf]));  // keeps each product next to its operands
          }
        }
      });
#pragma unroll
      for (int h = 0; h < G; ++h) {
        acc[h][0] = fmaf(dacc[h >> 2][0][h & 3], unsc[h], acc[h][0]);
        acc[h][1] = fmaf(dacc[h >> 2][1][h & 3], unsc[h], acc[h][1]);
      }
    } else {
      // One head: the weights enter as fp16 pairs (w_t, w_t+1), one scalar operand per two
      // tokens of a packed dot product with the fp16 codebook pair (cb[a], cb[b]).
      float unsc[G];
      uint32_t wpair[G];
  #pragma unroll
      for (int h = 0; h < G; ++h) {
        const float wmax = wmaxv[h];
        const int ex = wmax > 0.0f ? static_cast<int>((__builtin_bit_cast(uint32_t, wmax) >> 23) & 0xffu) - 127 : 0;
        const int sh = min(max(13 - ex, -100), 100);  // 2^sh * wmax in [2^13, 2^14)
        unsc[h] = __builtin_bit_cast(float, static_cast<uint32_t>(127 - sh) << 23);
        const float ws = wts[h] * __builtin_bit_cast(float, static_cast<uint32_t>(127 + sh) << 23);
        const uint32_t wh = __builtin_bit_cast(uint16_t, static_cast<_Float16>(ws));
        const uint32_t wn = dpp_u32<0xF5>(wh);  // quad_perm [1,1,3,3]: lane 2m gets lane 2m + 1
        wpair[h] = wh | (wn << 16);             // in lane 2m: (w_2m, w_2m+1)
        if (kStageW && (lane & 1) == 0) reinterpret_cast<uint32_t*>(&wst[kStageW ? wave : 0][h][0])[lane >> 1] = wpair[h];
      }
      if constexpr (kStageW) wave_lds_sync();
      // the weight pair of tokens (2m, 2m + 1) for head h, the same in every lane
      auto wpair_of = [&](int h, auto mc) {
        constexpr int m = decltype(mc)::value;
        if constexpr (kStageW) {
          const uint4 wq = wst[kStageW ? wave : 0][h][m / 4];
          return (m & 3) == 0 ? wq.x : (m & 3) == 1 ? wq.y : (m & 3) == 2 ? wq.z : wq.w;
        } else {
          return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(wpair[h]), 2 * m));
        }
      };
      typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
      float accp[G][2][2];
  #pragma unroll
      for (int h = 0; h < G; ++h) accp[h][0][0] = accp[h][0][1] = accp[h][1][0] = accp[h][1][1] = 0.0f;
      // A step is the tokens one table entry covers (four with 2-bit values, else two) for
      // both channels of the lane.  Table reads go in groups of two steps (four reads),
      // issued four steps ahead, and a group's products take its last read first, so one
      // LDS wait covers the group (a wait per read measured slower).
      constexpr int kSteps = kQuad ? kTile / 4 : kTile / 2;
      constexpr int kGS = 2;
      constexpr int kAheadS = 4;
      constexpr int kRingS = kAheadS + kGS;
      uint2 r0[kRingS], r1[kRingS];
      auto issue = [&](auto sc) __attribute__((always_inline)) {
        constexpr int q = decltype(sc)::value;
        if constexpr (kQuad) {
          r0[q % kRingS] = lut4[field<4 * VB, 4 * VB * q>(d.w)];
          r1[q % kRingS] = lut4[field<4 * VB, kChanBits + 4 * VB * q>(d.w)];
        } else {
          r0[q % kRingS].x = lut2[field<2 * VB, 2 * VB * q>(d.w)];
          r1[q % kRingS].x = lut2[field<2 * VB, kChanBits + 2 * VB * q>(d.w)];
        }
      };
      // weight pairs of a group, read one group ahead (a lane read's result needs wait
      // states before a VALU instruction can use it)
      constexpr int kWG = kQuad ? 2 * kGS : kGS;  // weight pairs per group
      uint32_t wr[G][2 * kWG];
      auto wload = [&](auto gc) __attribute__((always_inline)) {
        constexpr int g = decltype(gc)::value;
        static_for<0, kWG>([&](auto jc) {
          constexpr int m = kWG * g + decltype(jc)::value;
  #pragma unroll
          for (int h = 0; h < G; ++h) wr[h][m % (2 * kWG)] = wpair_of(h, std::integral_constant<int, m>{});
        });
      };
      // channel half hf of step q
      auto consume = [&](auto sc, auto hc) __attribute__((always_inline)) {
        constexpr int q = decltype(sc)::value;
        constexpr int hf = decltype(hc)::value;
        const uint2 e = hf ? r1[q % kRingS] : r0[q % kRingS];
  #pragma unroll
        for (int h = 0; h < G; ++h) {
          if constexpr (kQuad) {
            const half2_t wlo = __builtin_bit_cast(half2_t, wr[h][(2 * q) % (2 * kWG)]);
            const half2_t whi = __builtin_bit_cast(half2_t, wr[h][(2 * q + 1) % (2 * kWG)]);
            accp[h][hf][0] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, e.x), wlo, accp[h][hf][0], false);
            accp[h][hf][1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, e.y), whi, accp[h][hf][1], false);
          } else {
            const half2_t wp = __builtin_bit_cast(half2_t, wr[h][q % (2 * kWG)]);
            accp[h][hf][q & 1] = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, e.x), wp, accp[h][hf][q & 1], false);
          }
        }
      };
      using Z = std::integral_constant<int, 0>;
      using O = std::integral_constant<int, 1>;
      static_for<0, kAheadS>([&](auto sc) { issue(sc); });
      wload(Z{});
      static_for<0, kSteps / kGS>([&](auto gc) {
        constexpr int g = decltype(gc)::value;
        static_for<0, kGS>([&](auto jc) {
          constexpr int q = kGS * g + kAheadS + decltype(jc)::value;
          if constexpr (q < kSteps) issue(std::integral_constant<int, q>{});
        });
        if constexpr (g + 1 < kSteps / kGS) wload(std::integral_constant<int, g + 1>{});
        consume(std::integral_constant<int, kGS * g + kGS - 1>{}, O{});
        consume(std::integral_constant<int, kGS * g + kGS - 1>{}, Z{});
        static_for<0, kGS - 1>([&](auto jc) {
          consume(std::integral_constant<int, kGS * g + decltype(jc)::value>{}, Z{});
          consume(std::integral_constant<int, kGS * g + decltype(jc)::value>{}, O{});
        });
        __builtin_amdgcn_sched_barrier(0);
      });
  #pragma unroll
      for (int h = 0; h < G; ++h) {
        acc[h][0] = fmaf(accp[h][0][0] + accp[h][0][1], unsc[h], acc[h][0]);
        acc[h][1] = fmaf(accp[h][1][0] + accp[h][1][1], unsc[h], acc[h][1]);
      }
    }
    wave_lds_sync();  // the cleared cells are written before the next tile's atomics
  };

  if (w_lo < w_hi) {
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
  for (int e = tid; e < G * kHeadDim; e += kThreads) {
    const int h = e / kHeadDim, c = e % kHeadDim;
    float M = wm[0][h];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) M = fmaxf(M, wm[w][h]);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
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

// One block per (sequence, query head): 256 threads = 128 channels x 2 halves of the part
// list.  Each thread loads every (m, l, o[c]) of its parts in one pass (independent loads,
// up to kCombineRegs parts in registers), so the merge waits for a single round trip.
constexpr int kCombineRegs = 32;  // parts per half held in registers; more fall back to a second pass
__global__ __launch_bounds__(256) void pv_combine_kernel(PvArgs a) {
  __shared__ float red[4];
  __shared__ float acc_n[kHeadDim], acc_d[kHeadDim];
  const int tid = threadIdx.x;
  const int c = tid & (kHeadDim - 1);
  const int half = tid >> 7;
  const int h = blockIdx.x;
  const int seq = blockIdx.y;
  const size_t part_stride = kHeadDim + 2;
  const float* src = a.partial + (static_cast<size_t>(seq) * a.n_q_heads + h) * a.n_parts * part_stride;
  // Every block of the partial pass writes its part (m = -inf for a block past the
  // sequence's length), so all n_parts parts are read without waiting for the length.
  const int np = a.n_parts;

  float mj[kCombineRegs], lj[kCombineRegs], oj[kCombineRegs];
#pragma unroll
  for (int r = 0; r < kCombineRegs; ++r) {
    const int j = half + 2 * r;
    const bool ok = j < np;
    const float* pj = src + static_cast<size_t>(ok ? j : 0) * part_stride;
    mj[r] = ok ? pj[kHeadDim] : -INFINITY;
    lj[r] = pj[kHeadDim + 1];
    oj[r] = pj[c];
  }
  float M = -INFINITY;
#pragma unroll
  for (int r = 0; r < kCombineRegs; ++r) M = fmaxf(M, mj[r]);
  for (int j = half + 2 * kCombineRegs; j < np; j += 2) M = fmaxf(M, src[j * part_stride + kHeadDim]);
  M = wave_max_f32(M);
  if ((tid & 63) == 0) red[tid >> 6] = M;
  __syncthreads();
  M = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));

  float num = 0.0f, den = 0.0f;
  if (M > -INFINITY) {
#pragma unroll
    for (int r = 0; r < kCombineRegs; ++r) {
      const float wj = mj[r] > -INFINITY ? expf(mj[r] - M) : 0.0f;
      num += wj * oj[r];
      den += wj * lj[r];
    }
    for (int j = half + 2 * kCombineRegs; j < np; j += 2) {
      const float* pj = src + j * part_stride;
      const float m = pj[kHeadDim];
      const float wj = m > -INFINITY ? expf(m - M) : 0.0f;
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
hipError_t launch_pv_t(int batch, const PvArgs& a0, hipStream_t s) {
  PvArgs a = a0;
  // One resident round, equal share of block slots per stream, tile-granular runs of at
  // least kMinTilesPerBlock tiles.
  const int tiles = (a.max_len + kTile - 1) / kTile;
  const long streams = static_cast<long>(batch) * a.n_kv_heads;
  static const int resident = blocks_per_cu(reinterpret_cast<const void*>(&pv_partial_kernel<VB, G>), kThreads);
  const long slots = static_cast<long>(device_cu_count()) * resident;
  const long per_stream = std::max(1L, std::min<long>((slots + streams - 1) / streams,
                                                      (tiles + kMinTilesPerBlock - 1) / kMinTilesPerBlock));
  a.tiles_per_block = static_cast<int>((tiles + per_stream - 1) / per_stream);
  a.n_parts = (tiles + a.tiles_per_block - 1) / a.tiles_per_block;
  dim3 grid(a.n_parts, a.n_kv_heads, batch);
  hipLaunchKernelGGL((pv_partial_kernel<VB, G>), grid, dim3(kThreads), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_pv_combine(batch, a, s);
}

}  // namespace

hipError_t launch_pv_combine(int batch, const PvArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(pv_combine_kernel, dim3(a.n_q_heads, batch), dim3(256), 0, s, a);
  return hipGetLastError();
}

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
