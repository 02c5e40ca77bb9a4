// Online quantize-append of new key/value vectors into the compressed cache.
//
// KVQuant summary page, abstract paragraph, techniques (i)-(iv): per-channel key scale,
// keys taken before the rotary embedding, nearest entry of a sorted per-layer
// non-uniform codebook, and per-vector dense-and-sparse outlier isolation.
//
// A block is two waves: wave 0 quantizes keys, wave 1 values, of one (sequence, kv head)
// for the new tokens that fall into one 64-token tile (host positions) or into all tiles
// the step touches (device positions).  Inside a wave a vector's 128 channels sit two per
// lane: keys as (l, l + 64) -- the two halves of rotary pair l, adjacent in the key
// record -- and values as (2l, 2l + 1), which is how the value tile stores them.  Each
// value tile has exactly one writer wave per call: a bulk append copies the tile through
// LDS and writes it back; a decode step's few tokens instead clear and set their code
// fields in place with global and/or atomics, which saves the dependent read of the tile.
//
// Device positions: each block reads its sequence's start from seq_len with an atomic
// that also counts the block's arrival in the word's high bits; the last block to arrive
// advances the length and clears the count, after every block has read the start.
#include <type_traits>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kInPlaceTokens = 4;  // new tokens per tile written with atomics instead of a tile copy

template <int KB, int VB>
__global__ __launch_bounds__(128) void append_kernel(AppendArgs a) {
  constexpr int kNcK = 1 << KB;
  constexpr int kNcV = 1 << VB;
  constexpr int kRecWords = 4 * KB;    // key record: D*KB/8 bytes
  constexpr int kLaneWords = 4 * VB;   // value tile bytes owned by one lane (2 channels)
  constexpr int kChanWords = 2 * VB;   // one channel's 64 codes

  __shared__ float cbk[kNcK];
  __shared__ float cbv[kNcV];
  __shared__ uint32_t rec[kRecWords];
  __shared__ uint32_t vt[kWave * kLaneWords];
  __shared__ int s_start;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const bool is_key_wave = tid < 64;
  const int seq = blockIdx.z;
  const int kvh = blockIdx.y;
  const int count = a.count[seq];
  const int H = a.n_kv_heads;
  const int S = a.max_seq;
  const int k = a.n_outliers;

  // The block's first new token is known before its position is: token 0 with device
  // positions (one block per sequence and head), else the first token of this block's tile.
  // Its input vectors and the key scales are requested before the position atomic's
  // round trip, so the two latencies overlap.
  const int j_first = a.device_positions ? 0 : max(0, (a.start[seq] / kTile + static_cast<int>(blockIdx.x)) * kTile - a.start[seq]);
  const size_t src_first = ((static_cast<size_t>(seq) * a.n_max + min(j_first, max(a.n_max - 1, 0))) * H + kvh) * kHeadDim;
  const bool have_first = j_first < count && a.n_max > 0;
  uint32_t pre0 = 0u, pre1 = 0u;
  if (have_first) {
    if (is_key_wave) {
      pre0 = a.k_new[src_first + lane];
      pre1 = a.k_new[src_first + lane + kHalf];
    } else {
      pre0 = reinterpret_cast<const uint32_t*>(a.v_new + src_first)[lane];
    }
  }
  const float ks0 = a.k_scale[kvh * kHeadDim + lane];
  const float ks1 = a.k_scale[kvh * kHeadDim + lane + kHalf];

  if (tid == 0) {
    if (a.device_positions) {
      const int nblk = gridDim.x * gridDim.y;
      const int old = atomicAdd(&a.seq_len[seq], 1 << 24);
      const int st = old & kLenMask;
      const bool fits = st + count <= S;
      if ((old >> 24) + 1 == nblk) atomicAdd(&a.seq_len[seq], (fits ? count : 0) - (nblk << 24));
      s_start = fits ? st : -1;
    } else {
      s_start = a.start[seq];
      if (blockIdx.x == 0 && kvh == 0) a.seq_len[seq] = a.start[seq] + count;
    }
  }
  if (tid < kNcK) cbk[tid] = half_bits_to_float(a.k_cb[tid]);
  if (tid < kNcV) cbv[tid] = half_bits_to_float(a.v_cb[tid]);
  __syncthreads();
  const int start = s_start;
  if (start < 0 || count <= 0) return;

  const size_t stream = static_cast<size_t>(seq) * H + kvh;
  const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int first_tile = start / kTile;
  const int last_tile = (start + count - 1) / kTile;

  for (int tile = first_tile + blockIdx.x; tile <= last_tile; tile += gridDim.x) {
    const int lo = max(start, tile * kTile);
    const int hi = min(start + count, (tile + 1) * kTile);
    uint32_t* vtile = reinterpret_cast<uint32_t*>(a.v_codes + (stream * (S / kTile) + tile) * (1024 * VB));
    // A few tokens update their code fields in place with global atomics (disjoint bits of
    // shared words), so the tile is never read; more read-modify-write it through LDS.
    const bool in_place = hi - lo <= kInPlaceTokens;
    if (!is_key_wave && !in_place) {
      for (int i = lane; i < kWave * kLaneWords; i += kWave) vt[i] = vtile[i];
      wave_lds_sync();
    }
    for (int t = lo; t < hi; ++t) {
      const int j = t - start;  // row of this token in the new-token block
      const size_t src = ((static_cast<size_t>(seq) * a.n_max + j) * H + kvh) * kHeadDim;
      const size_t slot = stream * S + t;
      const bool use_pre = j == j_first && have_first;
      if (is_key_wave) {
        // ---- key: channels (lane, lane + 64), per-channel scale ----------------------
        const uint32_t x0 = use_pre ? pre0 : a.k_new[src + lane];
        const uint32_t x1 = use_pre ? pre1 : a.k_new[src + lane + kHalf];
        bool sel0, sel1;
        if (a.key_per_channel)  // launch-uniform
          select_outliers_by_scale(x0, x1, ks0, ks1, lane, k, sel0, sel1);
        else
          select_outliers(outlier_key(x0, lane), outlier_key(x1, lane + kHalf), k, sel0, sel1);
        const uint64_t b0 = __ballot(sel0);
        const uint64_t b1 = __ballot(sel1);
        if (sel0) {
          const int r = __popcll(b0 & lt);
          a.k_idx[slot * k + r] = static_cast<uint8_t>(lane);
          a.k_val[slot * k + r] = static_cast<uint16_t>(x0);
        }
        if (sel1) {
          const int r = __popcll(b0) + __popcll(b1 & lt);
          a.k_idx[slot * k + r] = static_cast<uint8_t>(lane + kHalf);
          a.k_val[slot * k + r] = static_cast<uint16_t>(x1);
        }
        // slots past the kept outliers (per-channel rule only): the sentinel channel, value 0
        for (int r = __popcll(b0) + __popcll(b1) + lane; r < k; r += kWave) {
          a.k_idx[slot * k + r] = static_cast<uint8_t>(kNoOutlier);
          a.k_val[slot * k + r] = 0;
        }
        const float d0 = sel0 ? 0.0f : half_bits_to_float(x0);
        const float d1 = sel1 ? 0.0f : half_bits_to_float(x1);
        const float u0 = ks0 > 0.0f ? d0 / ks0 : 0.0f;
        const float u1 = ks1 > 0.0f ? d1 / ks1 : 0.0f;
        const uint32_t pair = nearest_code<kNcK>(u0, cbk) | (nearest_code<kNcK>(u1, cbk) << KB);
        if (lane < kRecWords) rec[lane] = 0u;
        wave_lds_sync();
        const int bit = 2 * KB * lane;
        const int w = bit >> 5;
        const int sh = bit & 31;
        atomicOr(&rec[w], pair << sh);
        if (sh + 2 * KB > 32) atomicOr(&rec[w + 1], pair >> (32 - sh));
        wave_lds_sync();
        if (lane < kRecWords) reinterpret_cast<uint32_t*>(a.k_codes + slot * (16 * KB))[lane] = rec[lane];
        wave_lds_sync();
      } else {
        // ---- value: channels (2 lane, 2 lane + 1), one scale per vector --------------
        const uint32_t xx = use_pre ? pre0 : reinterpret_cast<const uint32_t*>(a.v_new + src)[lane];
        const uint32_t x0 = xx & 0xffffu;
        const uint32_t x1 = xx >> 16;
        bool sel0, sel1;
        select_outliers(outlier_key(x0, 2 * lane), outlier_key(x1, 2 * lane + 1), k, sel0, sel1);
        const uint64_t b0 = __ballot(sel0);
        const uint64_t b1 = __ballot(sel1);
        const int r0 = __popcll(b0 & lt) + __popcll(b1 & lt);
        if (sel0) {
          a.v_idx[slot * k + r0] = static_cast<uint8_t>(2 * lane);
          a.v_val[slot * k + r0] = static_cast<uint16_t>(x0);
        }
        if (sel1) {
          const int r1 = r0 + (sel0 ? 1 : 0);
          a.v_idx[slot * k + r1] = static_cast<uint8_t>(2 * lane + 1);
          a.v_val[slot * k + r1] = static_cast<uint16_t>(x1);
        }
        const uint32_t m0 = sel0 ? 0u : (x0 & 0x7fffu);
        const uint32_t m1 = sel1 ? 0u : (x1 & 0x7fffu);
        const uint32_t sbits = wave_max_u32(m0 > m1 ? m0 : m1);
        const float s = half_bits_to_float(sbits);
        if (lane == 0) a.v_scale[slot] = static_cast<uint16_t>(sbits);
        const float d0 = sel0 ? 0.0f : half_bits_to_float(x0);
        const float d1 = sel1 ? 0.0f : half_bits_to_float(x1);
        const float u0 = s > 0.0f ? d0 / s : 0.0f;
        const float u1 = s > 0.0f ? d1 / s : 0.0f;
        const uint32_t c0 = nearest_code<kNcV>(u0, cbv);
        const uint32_t c1 = nearest_code<kNcV>(u1, cbv);
        const int bit = (t - tile * kTile) * VB;
        const int w = bit >> 5;
        const int sh = bit & 31;
        constexpr uint32_t mask = (1u << VB) - 1u;
        uint32_t* seg = (in_place ? vtile : vt) + lane * kLaneWords;
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const uint32_t code = ch ? c1 : c0;
          uint32_t* cw = seg + ch * kChanWords;
          if (in_place) {
            atomicAnd(cw + w, ~(mask << sh));
            atomicOr(cw + w, code << sh);
            if (sh + VB > 32) {
              atomicAnd(cw + w + 1, ~(mask >> (32 - sh)));
              atomicOr(cw + w + 1, code >> (32 - sh));
            }
          } else {
            cw[w] = (cw[w] & ~(mask << sh)) | (code << sh);
            if (sh + VB > 32) cw[w + 1] = (cw[w + 1] & ~(mask >> (32 - sh))) | (code >> (32 - sh));
          }
        }
      }
    }
    if (!is_key_wave && !in_place) {
      wave_lds_sync();
      for (int i = lane; i < kWave * kLaneWords; i += kWave) vtile[i] = vt[i];
      wave_lds_sync();
    }
  }
}

template <int KB, int VB>
hipError_t launch_append_t(const AppendArgs& a, hipStream_t s) {
  int grid_x = 1;
  if (!a.device_positions) {
    for (int b = 0; b < a.n_batch; ++b) {
      if (a.count[b] > 0) {
        const int first = a.start[b] / kTile;
        const int last = (a.start[b] + a.count[b] - 1) / kTile;
        grid_x = max(grid_x, last - first + 1);
      }
    }
  }
  dim3 grid(grid_x, a.n_kv_heads, a.n_batch);
  hipLaunchKernelGGL((append_kernel<KB, VB>), grid, dim3(2 * kWave), 0, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int k_bits, int v_bits, const AppendArgs& a, hipStream_t s) {
#define KVQ_APPEND_CASE(KB, VB) \
  if (k_bits == KB && v_bits == VB) return launch_append_t<KB, VB>(a, s);
  KVQ_APPEND_CASE(2, 2) KVQ_APPEND_CASE(2, 3) KVQ_APPEND_CASE(2, 4)
  KVQ_APPEND_CASE(3, 2) KVQ_APPEND_CASE(3, 3) KVQ_APPEND_CASE(3, 4)
  KVQ_APPEND_CASE(4, 2) KVQ_APPEND_CASE(4, 3) KVQ_APPEND_CASE(4, 4)
#undef KVQ_APPEND_CASE
  return hipErrorInvalidValue;
}

}  // namespace kvq
