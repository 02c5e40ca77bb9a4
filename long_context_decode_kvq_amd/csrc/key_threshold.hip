// Per-channel key threshold for the per-channel outlier rule, from a bulk of calibration
// keys (e.g. the prompt of a prefill).
//
// KVQuant summary page, abstract paragraph, techniques (i) and (iv), and the paper note,
// "Four components" paragraph, items (1) and (4): keys are quantized per channel and
// outliers are held aside per vector.  Under the per-channel reading of the outlier rule
// an entry is a candidate when |x_c| exceeds its channel's scale, so the scale is also a
// threshold.  The pages give no calibration for it; this one keeps a chosen share of
// each channel's calibration entries above it: with N vectors and m = floor(f N), s_c is
// the (m+1)-th largest |x_c| (0 when m >= N), exact.
//
// An exact order statistic by radix selection over the 15-bit fp16 magnitude (sign
// cleared; numeric order for finite numbers):
//   pass A  every block histograms the high 8 bits of its vectors' magnitudes per
//           channel in LDS (256 bins x 128 channels), and writes the histogram out;
//   reduce  the blocks' histograms of a kv head are summed (one thread per bin and
//           channel, no atomics, so the result does not depend on timing);
//   select  per channel, the bin holding the (m+1)-th largest magnitude and the rank
//           inside it, scanning from the top bin;
//   pass B, reduce, select  the same over the low 7 bits of the magnitudes that fall in
//           the chosen bin, giving the magnitude itself.
// LDS histogram layout: word bin * 128 + j, with channel 2j' in j = j' and channel
// 2j' + 1 in j = 64 + j', so lane l's two channels (one 4-byte load of the vector) land in
// bank l for every bin: the 64 lanes of an atomic add never share a bank.
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kThrThreads = 1024;
constexpr int kThrWaves = kThrThreads / kWave;
constexpr int kHiBins = 256;  // magnitude bits 14..7
constexpr int kLoBins = 128;  // magnitude bits 6..0
constexpr int kSelThreads = 512;

// Histogram blocks per kv head: about 256 blocks in all, at least 64 vectors each.
int thr_chunks(long long n_vec, int n_kv_heads) {
  const long long want = std::max(1LL, (256LL + n_kv_heads - 1) / n_kv_heads);
  const long long most = std::max(1LL, (n_vec + 63) / 64);
  return static_cast<int>(std::min(want, most));
}

__global__ __launch_bounds__(256) void thr_zero_kernel(float* out, int n) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i < n) out[i] = 0.0f;
}

// kLo false: pass A over the high bits of every magnitude.  kLo true: pass B over the low
// bits of the magnitudes whose high bits equal the channel's selected bin.
template <bool kLo>
__global__ __launch_bounds__(kThrThreads) void thr_hist_kernel(const uint16_t* __restrict__ keys, long long n_vec,
                                                               int n_kv_heads, long long per_block, int chunks,
                                                               const uint2* __restrict__ sel,
                                                               uint32_t* __restrict__ part) {
  constexpr int kBins = kLo ? kLoBins : kHiBins;
  extern __shared__ uint32_t hist[];  // [kBins][128]
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = blockIdx.y;
  const int blk = blockIdx.x;
  for (int i = tid; i < kBins * kHeadDim; i += kThrThreads) hist[i] = 0u;
  uint32_t sel0 = 0, sel1 = 0;
  if constexpr (kLo) {
    sel0 = sel[h * kHeadDim + 2 * lane].x;
    sel1 = sel[h * kHeadDim + 2 * lane + 1].x;
  }
  __syncthreads();
  const long long v_lo = blk * per_block;
  const long long v_hi = min(v_lo + per_block, n_vec);
  auto vec = [&](long long v) {  // channels (2 lane, 2 lane + 1) of vector v: one 4-byte load
    return reinterpret_cast<const uint32_t*>(keys + (static_cast<size_t>(v) * n_kv_heads + h) * kHeadDim)[lane];
  };
  auto take = [&](uint32_t xx) {
    const uint32_t a0 = xx & 0x7fffu, a1 = (xx >> 16) & 0x7fffu;
    if constexpr (kLo) {
      if ((a0 >> 7) == sel0) atomicAdd(&hist[(a0 & 127u) * kHeadDim + lane], 1u);
      if ((a1 >> 7) == sel1) atomicAdd(&hist[(a1 & 127u) * kHeadDim + 64 + lane], 1u);
    } else {
      atomicAdd(&hist[(a0 >> 7) * kHeadDim + lane], 1u);
      atomicAdd(&hist[(a1 >> 7) * kHeadDim + 64 + lane], 1u);
    }
  };
  long long v = v_lo + wave;
  for (; v + 3 * kThrWaves < v_hi; v += 4 * kThrWaves) {  // four vectors' loads in flight
    const uint32_t x0 = vec(v), x1 = vec(v + kThrWaves), x2 = vec(v + 2 * kThrWaves), x3 = vec(v + 3 * kThrWaves);
    take(x0);
    take(x1);
    take(x2);
    take(x3);
  }
  for (; v < v_hi; v += kThrWaves) take(vec(v));
  __syncthreads();
  // part [Hkv][chunks][kBins][128 channels], channel order restored
  uint32_t* out = part + (static_cast<size_t>(h) * chunks + blk) * (kBins * kHeadDim);
  for (int o = tid; o < kBins * kHeadDim; o += kThrThreads) {
    const int bin = o >> 7, c = o & 127;
    const int j = (c & 1) ? 64 + (c >> 1) : (c >> 1);
    out[o] = hist[bin * kHeadDim + j];
  }
}

// hist[h][o] = sum over the head's blocks of part[h][p][o], o = bin * 128 + channel.
__global__ __launch_bounds__(256) void thr_reduce_kernel(const uint32_t* __restrict__ part, int chunks, int used,
                                                         int words, uint32_t* __restrict__ hist) {
  const int o = blockIdx.x * 256 + threadIdx.x;
  const int h = blockIdx.y;
  if (o >= words) return;
  const uint32_t* p = part + static_cast<size_t>(h) * chunks * words + o;
  uint32_t s = 0;
  for (int i = 0; i < used; ++i) s += p[static_cast<size_t>(i) * words];
  hist[static_cast<size_t>(h) * words + o] = s;
}

// One block per kv head: the head's histogram is staged in LDS, then thread c scans
// channel c from the top bin.  kLo false: rank r (1-based from the largest) -> sel[c] =
// (bin, rank inside the bin).  kLo true: sel -> the magnitude, written as float32.
template <bool kLo>
__global__ __launch_bounds__(kSelThreads) void thr_select_kernel(const uint32_t* __restrict__ hist, uint32_t rank,
                                                                 uint2* __restrict__ sel, float* __restrict__ out) {
  constexpr int kBins = kLo ? kLoBins : kHiBins;
  extern __shared__ uint32_t col[];  // [kBins][128]
  const int h = blockIdx.x;
  const uint4* src = reinterpret_cast<const uint4*>(hist + static_cast<size_t>(h) * kBins * kHeadDim);
  uint4* dst = reinterpret_cast<uint4*>(col);
  for (int i = threadIdx.x; i < kBins * kHeadDim / 4; i += kSelThreads) dst[i] = src[i];
  __syncthreads();
  const int c = threadIdx.x;
  if (c >= kHeadDim) return;
  const uint32_t r = kLo ? sel[h * kHeadDim + c].y : rank;
  uint32_t acc = 0;
  int found = 0;
  uint32_t inside = 1;
  for (int bin = kBins - 1; bin >= 0; --bin) {
    const uint32_t n = col[bin * kHeadDim + c];
    if (acc + n >= r) {
      found = bin;
      inside = r - acc;
      break;
    }
    acc += n;
  }
  if constexpr (kLo) {
    const uint32_t bits = (sel[h * kHeadDim + c].x << 7) | static_cast<uint32_t>(found);
    out[h * kHeadDim + c] = half_bits_to_float(bits);
  } else {
    sel[h * kHeadDim + c] = make_uint2(static_cast<uint32_t>(found), inside);
  }
}

template <typename K>
bool allow_lds(K kernel, size_t bytes) {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                             static_cast<int>(bytes)) == hipSuccess;
}

}  // namespace

size_t key_threshold_workspace_bytes(int batch, int n_tokens, int n_kv_heads) {
  const long long n_vec = static_cast<long long>(batch) * n_tokens;
  if (n_vec <= 0) return 0;
  const size_t chunks = static_cast<size_t>(thr_chunks(n_vec, n_kv_heads));
  const size_t words = static_cast<size_t>(kHiBins) * kHeadDim;
  return 4 * (static_cast<size_t>(n_kv_heads) * chunks * words + static_cast<size_t>(n_kv_heads) * words) +
         sizeof(uint2) * n_kv_heads * kHeadDim;
}

hipError_t launch_key_threshold(const uint16_t* keys, int batch, int n_tokens, int n_kv_heads, long long budget,
                                float* out, void* workspace, hipStream_t s) {
  const long long n_vec = static_cast<long long>(batch) * n_tokens;
  const int n_out = n_kv_heads * kHeadDim;
  if (budget >= n_vec) {  // every entry may exceed (also no vectors at all): threshold 0
    hipLaunchKernelGGL(thr_zero_kernel, dim3((n_out + 255) / 256), dim3(256), 0, s, out, n_out);
    return hipGetLastError();
  }
  static const bool lds_ok = allow_lds(thr_hist_kernel<false>, kHiBins * kHeadDim * 4) &&
                             allow_lds(thr_hist_kernel<true>, kLoBins * kHeadDim * 4) &&
                             allow_lds(thr_select_kernel<false>, kHiBins * kHeadDim * 4) &&
                             allow_lds(thr_select_kernel<true>, kLoBins * kHeadDim * 4);
  if (!lds_ok) return hipErrorInvalidValue;
  const int chunks = thr_chunks(n_vec, n_kv_heads);
  const long long per_block = ((n_vec + chunks - 1) / chunks + kThrWaves - 1) / kThrWaves * kThrWaves;
  const int used = static_cast<int>((n_vec + per_block - 1) / per_block);
  const size_t hi_words = static_cast<size_t>(kHiBins) * kHeadDim;
  uint32_t* part = static_cast<uint32_t*>(workspace);
  uint32_t* hist = part + static_cast<size_t>(n_kv_heads) * chunks * hi_words;
  uint2* sel = reinterpret_cast<uint2*>(hist + static_cast<size_t>(n_kv_heads) * hi_words);
  const uint32_t rank = static_cast<uint32_t>(budget + 1);

  hipLaunchKernelGGL(thr_hist_kernel<false>, dim3(used, n_kv_heads), dim3(kThrThreads), kHiBins * kHeadDim * 4, s,
                     keys, n_vec, n_kv_heads, per_block, chunks, static_cast<const uint2*>(nullptr), part);
  hipLaunchKernelGGL(thr_reduce_kernel, dim3(kHiBins * kHeadDim / 256, n_kv_heads), dim3(256), 0, s, part, chunks,
                     used, kHiBins * kHeadDim, hist);
  hipLaunchKernelGGL(thr_select_kernel<false>, dim3(n_kv_heads), dim3(kSelThreads), kHiBins * kHeadDim * 4, s, hist,
                     rank, sel, out);
  hipLaunchKernelGGL(thr_hist_kernel<true>, dim3(used, n_kv_heads), dim3(kThrThreads), kLoBins * kHeadDim * 4, s, keys,
                     n_vec, n_kv_heads, per_block, chunks, sel, part);
  hipLaunchKernelGGL(thr_reduce_kernel, dim3(kLoBins * kHeadDim / 256, n_kv_heads), dim3(256), 0, s, part, chunks,
                     used, kLoBins * kHeadDim, hist);
  hipLaunchKernelGGL(thr_select_kernel<true>, dim3(n_kv_heads), dim3(kSelThreads), kLoBins * kHeadDim * 4, s, hist,
                     rank, sel, out);
  return hipGetLastError();
}

}  // namespace kvq
