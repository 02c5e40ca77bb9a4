// Device-side helpers shared by the kvq kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace kvq {

constexpr int kHeadDim = 128;
constexpr int kHalf = kHeadDim / 2;  // rotary pairs per vector
constexpr int kTile = 64;            // tokens per value tile and per QK wave pass
constexpr int kWave = 64;
// seq_len words hold the length in their low 24 bits; the high bits are an arrival
// counter used only while a device-positioned append is in flight.
constexpr int32_t kLenMask = 0x00ffffff;

__device__ __forceinline__ float half_bits_to_float(uint32_t h) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(h)));
}

// Orders this wave's LDS writes before its later LDS reads of other lanes' entries.  A
// wave's LDS operations execute in order, so wavefront-scope fences suffice: they emit
// no wait on outstanding global loads, which keeps prefetched tiles in flight.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One 3-bit table entry (A, B) = (al cba + ga cbb, be cba + nd cbb) whose four
// coefficients come from lane N of the lane's 16-lane row, by DPP row broadcasts inside
// the multiplies (no separate lane reads).  The DPP sources must have been written at
// least two wait states earlier.
template <int N>
__device__ __forceinline__ float2 lut_entry_bcast(float al, float be, float ga, float nd, float cba, float cbb) {
  float A, B;
  asm("v_mul_f32_dpp %0, %4, %6 row_newbcast:%8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %1, %5, %6 row_newbcast:%8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %0, %2, %7 row_newbcast:%8 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_fmac_f32_dpp %1, %3, %7 row_newbcast:%8 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=&v"(A), "=&v"(B)
      : "v"(al), "v"(be), "v"(ga), "v"(nd), "v"(cbb), "v"(cba), "i"(N));
  return make_float2(A, B);
}

// Byte offset of rotary pair I's entry in a table row of 8-byte entries indexed by the
// pair's 2KB-bit code field (a | b << KB): the field times 8.  W is the token's key record.
//  - 2-bit codes (4-bit fields, eight to a word): the word's even fields times 8 are the
//    bytes of (w << 3) & 0x78787878 and its odd fields times 8 those of (w >> 1) &
//    0x78787878, two operations each shared by four pairs; a byte is then one AND (byte 0),
//    one bit-field extract (bytes 1 and 2) or one shift (byte 3): 1.5 operations per pair.
//  - 3-bit codes (6-bit fields): a shift and a mask per pair (an align-bit first for a
//    field that straddles two words).
template <int KB, int I, int N>
__device__ __forceinline__ uint32_t pair_entry_offset(const uint32_t (&w)[N]) {
  constexpr int kBits = 2 * KB;
  constexpr int pos = kBits * I;
  constexpr int wi = pos / 32;
  constexpr int sh = pos % 32;
  static_assert(wi < N, "field outside the record");
  uint32_t r;
  if constexpr (KB == 2) {
    constexpr int nib = I % 8;
    constexpr int j = nib / 2;
    const uint32_t src = (nib & 1) ? ((w[wi] >> 1) & 0x78787878u) : ((w[wi] << 3) & 0x78787878u);
    if constexpr (j == 0)
      asm("v_and_b32_e32 %0, 0xff, %1" : "=v"(r) : "v"(src));
    else if constexpr (j == 3)
      asm("v_lshrrev_b32_e32 %0, 24, %1" : "=v"(r) : "v"(src));
    else
      asm("v_bfe_u32 %0, %1, %2, 8" : "=v"(r) : "v"(src), "n"(8 * j));
    return r;
  }
  constexpr uint32_t mask = ((1u << kBits) - 1u) << 3;
  if constexpr (sh + kBits <= 32) {
    if constexpr (sh >= 3) {
      asm("v_lshrrev_b32_e32 %0, %2, %1\n\tv_and_b32_e32 %0, %3, %0" : "=&v"(r) : "v"(w[wi]), "n"(sh - 3), "n"(mask));
    } else {
      asm("v_lshlrev_b32_e32 %0, %2, %1\n\tv_and_b32_e32 %0, %3, %0" : "=&v"(r) : "v"(w[wi]), "n"(3 - sh), "n"(mask));
    }
  } else {
    static_assert(wi + 1 < N, "straddling field outside the record");
    asm("v_alignbit_b32 %0, %1, %2, %3\n\tv_and_b32_e32 %0, %4, %0"
        : "=&v"(r)
        : "v"(w[wi + 1]), "v"(w[wi]), "n"(sh - 3), "n"(mask));
  }
  return r;
}

// One separable 4-bit table entry (c0 cbv, c1 cbv), the coefficients from lane N of the
// lane's 16-lane row by DPP row broadcast (sources written at least two wait states earlier).
template <int N>
__device__ __forceinline__ float2 lut_sep_bcast(float c0, float c1, float cbv) {
  float A, B;
  asm("v_mul_f32_dpp %0, %2, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
      "v_mul_f32_dpp %1, %3, %4 row_newbcast:%5 row_mask:0xf bank_mask:0xf bound_ctrl:1"
      : "=&v"(A), "=&v"(B)
      : "v"(c0), "v"(c1), "v"(cbv), "i"(N));
  return make_float2(A, B);
}

// 4-bit codes: byte I of the record is pair I's field a | b << 4.  The even nibbles times 8
// are the bytes of (w << 3) & 0x78787878, the odd ones those of (w >> 1) & 0x78787878; a
// byte is one AND, bit-field extract or shift.  oa = 8 a, ob = 8 b.
template <int I, int N>
__device__ __forceinline__ void pair_offsets_sep4(const uint32_t (&w)[N], uint32_t& oa, uint32_t& ob) {
  constexpr int wi = I / 4;
  constexpr int j = I % 4;
  static_assert(wi < N, "field outside the record");
  const uint32_t lo = (w[wi] << 3) & 0x78787878u, hi = (w[wi] >> 1) & 0x78787878u;
  if constexpr (j == 0) {
    asm("v_and_b32_e32 %0, 0xff, %1" : "=v"(oa) : "v"(lo));
    asm("v_and_b32_e32 %0, 0xff, %1" : "=v"(ob) : "v"(hi));
  } else if constexpr (j == 3) {
    asm("v_lshrrev_b32_e32 %0, 24, %1" : "=v"(oa) : "v"(lo));
    asm("v_lshrrev_b32_e32 %0, 24, %1" : "=v"(ob) : "v"(hi));
  } else {
    asm("v_bfe_u32 %0, %1, %2, 8" : "=v"(oa) : "v"(lo), "n"(8 * j));
    asm("v_bfe_u32 %0, %1, %2, 8" : "=v"(ob) : "v"(hi), "n"(8 * j));
  }
}

// Wave reductions: four DPP steps combine the 16 lanes of each row (xor 1, xor 2, half-row
// mirror, row mirror), then the four row results are read into scalar registers.  Every
// lane gets the result; no LDS round trips.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(static_cast<int>(v), static_cast<int>(v), CTRL, 0xf, 0xf, false));
}
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __builtin_bit_cast(float, dpp_u32<CTRL>(__builtin_bit_cast(uint32_t, v)));
}
__device__ __forceinline__ uint32_t lane_u32(uint32_t v, int l) {
  return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
}
__device__ __forceinline__ float lane_f32(float v, int l) {
  return __builtin_bit_cast(float, lane_u32(__builtin_bit_cast(uint32_t, v), l));
}
// Wave maxima: each step is one max in DPP form (the four row steps above, then lane 15 of
// each row into the next row and lane 31 into the upper half), so lane 63 ends with the
// maximum, read into a scalar register: seven VALU instructions, where max over separately
// moved DPP values costs two or three per step (the float form also re-canonicalises).
// Each DPP read follows the write of its source by two wait states (s_nop 1).  The float
// form is for finite or infinite inputs (no NaN), as a maximum of logits, weights or
// magnitudes is.
#define KVQ_WAVE_MAX_STEPS(OP)                                                       \
  "s_nop 1\n\t" OP "_dpp %0, %1, %1 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n\t" \
  "s_nop 1\n\t" OP "_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n\t" \
  "s_nop 1\n\t" OP "_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n\t"      \
  "s_nop 1\n\t" OP "_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n\t"           \
  "s_nop 1\n\t" OP "_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n\t"         \
  "s_nop 1\n\t" OP "_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf"
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  uint32_t r;
  asm(KVQ_WAVE_MAX_STEPS("v_max_u32") : "=&v"(r) : "v"(v));
  return lane_u32(r, 63);
}
__device__ __forceinline__ float wave_max_f32(float v) {
  float r;
  asm(KVQ_WAVE_MAX_STEPS("v_max_f32") : "=&v"(r) : "v"(v));
  return lane_f32(r, 63);
}
#undef KVQ_WAVE_MAX_STEPS
// Two or four independent float wave maxima in one pass, the same six DPP steps with the
// chains interleaved: with four, each DPP read follows the write of its source by three
// other instructions; with two, by one instruction and an s_nop 0.  One s_nop 1 covers the
// inputs' writes before the block.
#define KVQ_MAX_DPP(D, S, CTL) "v_max_f32_dpp %" #D ", %" #S ", %" #S " " CTL "\n\t"
#define KVQ_CTL1 "quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
#define KVQ_CTL2 "quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf"
#define KVQ_CTL3 "row_half_mirror row_mask:0xf bank_mask:0xf"
#define KVQ_CTL4 "row_mirror row_mask:0xf bank_mask:0xf"
#define KVQ_CTL5 "row_bcast:15 row_mask:0xa bank_mask:0xf"
#define KVQ_CTL6 "row_bcast:31 row_mask:0xc bank_mask:0xf"
#define KVQ_MAX2_STEP(CTL) "s_nop 0\n\t" KVQ_MAX_DPP(0, 0, CTL) KVQ_MAX_DPP(1, 1, CTL)
#define KVQ_MAX4_STEP(CTL) KVQ_MAX_DPP(0, 0, CTL) KVQ_MAX_DPP(1, 1, CTL) KVQ_MAX_DPP(2, 2, CTL) KVQ_MAX_DPP(3, 3, CTL)
__device__ __forceinline__ void wave_max2_f32(float a, float b, float& ma, float& mb) {
  float r0, r1;
  asm("s_nop 1\n\t" KVQ_MAX_DPP(0, 2, KVQ_CTL1) KVQ_MAX_DPP(1, 3, KVQ_CTL1)
      KVQ_MAX2_STEP(KVQ_CTL2) KVQ_MAX2_STEP(KVQ_CTL3) KVQ_MAX2_STEP(KVQ_CTL4) KVQ_MAX2_STEP(KVQ_CTL5)
      KVQ_MAX2_STEP(KVQ_CTL6)
      : "=&v"(r0), "=&v"(r1)
      : "v"(a), "v"(b));
  ma = lane_f32(r0, 63);
  mb = lane_f32(r1, 63);
}
__device__ __forceinline__ void wave_max4_f32(const float (&v)[4], float (&m)[4]) {
  float r0, r1, r2, r3;
  asm("s_nop 1\n\t" KVQ_MAX_DPP(0, 4, KVQ_CTL1) KVQ_MAX_DPP(1, 5, KVQ_CTL1) KVQ_MAX_DPP(2, 6, KVQ_CTL1)
      KVQ_MAX_DPP(3, 7, KVQ_CTL1) KVQ_MAX4_STEP(KVQ_CTL2) KVQ_MAX4_STEP(KVQ_CTL3) KVQ_MAX4_STEP(KVQ_CTL4)
      KVQ_MAX4_STEP(KVQ_CTL5) KVQ_MAX4_STEP(KVQ_CTL6)
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(v[0]), "v"(v[1]), "v"(v[2]), "v"(v[3]));
  m[0] = lane_f32(r0, 63);
  m[1] = lane_f32(r1, 63);
  m[2] = lane_f32(r2, 63);
  m[3] = lane_f32(r3, 63);
}
// G wave maxima (G = 1, 2, 4, 8), in as few interleaved passes as that allows.
template <int G>
__device__ __forceinline__ void wave_max_n_f32(const float (&v)[G], float (&m)[G]) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "one, two, four or eight maxima");
  if constexpr (G == 1) {
    m[0] = wave_max_f32(v[0]);
  } else if constexpr (G == 2) {
    wave_max2_f32(v[0], v[1], m[0], m[1]);
  } else if constexpr (G == 4) {
    wave_max4_f32(v, m);
  } else {
    wave_max4_f32(*reinterpret_cast<const float(*)[4]>(&v[0]), *reinterpret_cast<float(*)[4]>(&m[0]));
    wave_max4_f32(*reinterpret_cast<const float(*)[4]>(&v[4]), *reinterpret_cast<float(*)[4]>(&m[4]));
  }
}
#undef KVQ_MAX4_STEP
#undef KVQ_MAX2_STEP
#undef KVQ_CTL1
#undef KVQ_CTL2
#undef KVQ_CTL3
#undef KVQ_CTL4
#undef KVQ_CTL5
#undef KVQ_CTL6
#undef KVQ_MAX_DPP
__device__ __forceinline__ float wave_sum_f32(float v) {
  v += dpp_f32<0xB1>(v);
  v += dpp_f32<0x4E>(v);
  v += dpp_f32<0x141>(v);
  v += dpp_f32<0x140>(v);
  return (lane_f32(v, 0) + lane_f32(v, 16)) + (lane_f32(v, 32) + lane_f32(v, 48));
}

// b-bit field starting at compile-time bit position POS of a little-endian stream held in
// 32-bit words (registers after full unrolling).
template <int BITS, int POS, int N>
__device__ __forceinline__ uint32_t field(const uint32_t (&w)[N]) {
  constexpr int wi = POS / 32;
  constexpr int sh = POS % 32;
  constexpr uint32_t mask = (1u << BITS) - 1u;
  static_assert(wi < N, "field outside the word array");
  if constexpr (sh + BITS <= 32) {
    return (w[wi] >> sh) & mask;
  } else {
    static_assert(wi + 1 < N, "straddling field outside the word array");
    return ((w[wi] >> sh) | (w[wi + 1] << (32 - sh))) & mask;
  }
}

// base + (field<BITS, POS>(w) << SHIFT): the LDS byte address of entry `field` of a table
// of (1 << SHIFT)-byte entries at `base` (wave-uniform).  Written as a bit-field extract
// and a shift-add: the compiler otherwise forms a shift, a mask and an add.
template <int BITS, int POS, int SHIFT, int N>
__device__ __forceinline__ uint32_t field_addr(const uint32_t (&w)[N], uint32_t base) {
  constexpr int wi = POS / 32;
  constexpr int sh = POS % 32;
  static_assert(wi < N, "field outside the word array");
  uint32_t r;
  if constexpr (sh + BITS <= 32) {
    asm("v_bfe_u32 %0, %1, %2, %3\n\tv_lshl_add_u32 %0, %0, %4, %5"
        : "=&v"(r)
        : "v"(w[wi]), "n"(sh), "n"(BITS), "n"(SHIFT), "s"(base));
  } else {
    static_assert(wi + 1 < N, "straddling field outside the word array");
    asm("v_alignbit_b32 %0, %1, %2, %3\n\tv_bfe_u32 %0, %0, 0, %4\n\tv_lshl_add_u32 %0, %0, %5, %6"
        : "=&v"(r)
        : "v"(w[wi + 1]), "v"(w[wi]), "n"(sh), "n"(BITS), "n"(SHIFT), "s"(base));
  }
  return r;
}

// Compile-time loop: calls f(std::integral_constant<int, I>) for I in [0, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// Nearest codebook entry: the smallest j minimising the float32 |u - cb[j]|, scanned in
// ascending j with a strict '<' (ties go to the lower index).
template <int NC>
__device__ __forceinline__ uint32_t nearest_code(float u, const float* cb) {
  uint32_t best = 0;
  float bd = fabsf(u - cb[0]);
#pragma unroll
  for (int j = 1; j < NC; ++j) {
    float d = fabsf(u - cb[j]);
    if (d < bd) {
      bd = d;
      best = j;
    }
  }
  return best;
}

// Index of the codebook entry nearest to 0 (the code of every dense-zero entry, in
// particular of every outlier slot): smallest j minimising |0 - cb[j]|.
// Small lookup tables indexed by per-lane codes are read with random indices, and bank
// conflicts make such reads several times slower than conflict-free ones.  The table is
// therefore stored in kCopies interleaved copies: entry e of copy r at word e * kCopies + r,
// lane l reading copy l % kCopies, so every lane reads its own bank.  Tables of more than 64
// entries stay single (a 256-entry table would take 64 KB).
template <int ENTRIES>
struct RepTable {
  static constexpr int kCopies = ENTRIES <= 64 ? 64 : 1;
  static constexpr int kWords = ENTRIES * kCopies;
  // byte offset of this lane's copy of entry 0
  __device__ static __forceinline__ uint32_t lane_base(int lane) {
    return kCopies > 1 ? static_cast<uint32_t>(lane & (kCopies - 1)) * 4u : 0u;
  }
  // byte offset of entry e for a lane whose lane_base is `base`
  __device__ static __forceinline__ uint32_t at(uint32_t e, uint32_t base) { return e * (4u * kCopies) + base; }
};

// Block barrier for data exchanged through LDS only.  It waits for this wave's LDS
// operations and then for every wave of the block, but not for outstanding global loads
// (a workgroup-scope fence, as in __syncthreads, drains those too), so prefetched tiles
// stay in flight across it.  The empty asm statements keep the compiler from moving
// memory accesses across the barrier.
__device__ __forceinline__ void block_lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Value of the codebook entry nearest zero (the lowest index among equal magnitudes):
// the dense value stored at an outlier's channel.  Lane j < NC passes the fp16 bits of
// entry j; fp16 magnitudes order as integers like the numbers they encode.  Every lane of
// the wave gets the value.
template <int NC>
__device__ __forceinline__ float zero_code_value(uint32_t cb_bits, int lane) {
  const uint32_t key = lane < NC ? ((cb_bits & 0x7fffu) << 8) | static_cast<uint32_t>(lane) : 0xffffffffu;
  const uint32_t m = ~wave_max_u32(~key);  // wave minimum
  return half_bits_to_float(static_cast<uint32_t>(__shfl(static_cast<int>(cb_bits), static_cast<int>(m & 0xffu))) & 0xffffu);
}

// Selection key: fp16 magnitude bits above the inverted channel index, so the unsigned
// maximum is the largest |x| and, among equal magnitudes, the lowest channel.
__device__ __forceinline__ uint32_t outlier_key(uint32_t xbits, uint32_t c) {
  return ((xbits & 0x7fffu) << 16) | (0xffffu - c);
}

// Marks the k largest-magnitude channels of the wave's vector (k <= 128).
__device__ __forceinline__ void select_outliers(uint32_t key0, uint32_t key1, int k, bool& sel0,
                                                bool& sel1) {
  sel0 = false;
  sel1 = false;
  for (int r = 0; r < k; ++r) {
    uint32_t m0 = sel0 ? 0u : key0;
    uint32_t m1 = sel1 ? 0u : key1;
    uint32_t m = wave_max_u32(m0 > m1 ? m0 : m1);
    if (!sel0 && key0 == m) {
      sel0 = true;
    } else if (!sel1 && key1 == m) {
      sel1 = true;
    }
  }
}

// Per-channel key outliers: channel c (fp16 bits x, frozen scale s >= 0) is a candidate
// iff |x| > s; the wave keeps at most k, the largest float32 |x| / s first (+inf where
// s = 0), ties toward the lower channel.  Lane l holds channels l (x0, s0) and l + 64
// (x1, s1).  A candidate's ratio is positive, so its bits order as unsigned integers.
__device__ __forceinline__ void select_outliers_by_scale(uint32_t x0, uint32_t x1, float s0, float s1, int lane,
                                                         int k, bool& sel0, bool& sel1) {
  const float m0 = fabsf(half_bits_to_float(x0)), m1 = fabsf(half_bits_to_float(x1));
  const uint32_t r0 = m0 > s0 ? __builtin_bit_cast(uint32_t, s0 > 0.0f ? m0 / s0 : INFINITY) : 0u;
  const uint32_t r1 = m1 > s1 ? __builtin_bit_cast(uint32_t, s1 > 0.0f ? m1 / s1 : INFINITY) : 0u;
  sel0 = false;
  sel1 = false;
  for (int r = 0; r < k; ++r) {
    const uint32_t e0 = sel0 ? 0u : r0, e1 = sel1 ? 0u : r1;
    const uint32_t best = wave_max_u32(e0 > e1 ? e0 : e1);
    if (best == 0u) break;  // no candidate left (wave-uniform)
    const uint32_t ch = e0 == best ? static_cast<uint32_t>(lane) : e1 == best ? static_cast<uint32_t>(lane + 64) : 255u;
    const uint32_t lowest = ~wave_max_u32(~ch);  // wave minimum
    if (lowest == static_cast<uint32_t>(lane)) {
      sel0 = true;
    } else if (lowest == static_cast<uint32_t>(lane + 64)) {
      sel1 = true;
    }
  }
}

// Channel index of an unused key-outlier slot (per-channel rule): it adds nothing.
constexpr uint32_t kNoOutlier = 255;

// LDS byte address of a pointer into shared memory.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}

// Raw buffer access for streaming loads: a descriptor over the wave-uniform range
// [base, base + bytes) (bytes < 2^32; base and size in scalar registers) read at a per-lane
// 32-bit byte offset.  A kernel that rebuilds the descriptor for every tile at the tile's
// first byte keeps its per-lane offsets fixed, so a load costs no vector arithmetic; a read
// past the range returns zero instead of faulting.  0x00020000 is the gfx9-family third
// descriptor word (raw, untyped dwords).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 buf_load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_b32(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_u16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ uint32_t buf_load_u8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b8(r, off, 0, 0);
}

// cos/sin of 2*pi*r for a revolution count r already reduced to [0, 1).
__device__ __forceinline__ void sincos_rev(float r, float* s, float* c) { sincospif(2.0f * r, s, c); }

// Fractional revolutions of angle t * theta, theta given as theta / (2*pi) in float64.
__device__ __forceinline__ float frac_rev(double t, double theta_over_2pi) {
  double r = t * theta_over_2pi;
  return static_cast<float>(r - floor(r));
}

}  // namespace kvq
