// Per-layer codebook fitting: unweighted 1-D k-means (Lloyd iterations) over normalised
// calibration activations.
//
// KVQuant summary page, abstract paragraph, technique (iii), and the paper note, "Four
// components" paragraph, item (3): one non-uniform datatype per layer, derived offline
// from calibration activations.  This is the unweighted fit (the pages weight it by each
// activation's sensitivity, which needs a trained model's gradients).
//
// One iteration is two launches.  fit_assign: a grid-stride pass (about two blocks per
// CU, four loads in flight per thread) where every input,
// clamped to [-1, 1], goes to its nearest centroid by the quantizer's rule (smallest j
// minimising the float32 |u - c_j|) and adds round(u 2^30) to that cluster's integer sum
// held in registers; the block folds its threads' sums in LDS and adds them to the
// global sums with one 64-bit integer atomic per cluster.  Integer sums make the result
// independent of the order of accumulation.  fit_update: c_j = float32(sum_j /
// (count_j 2^30)) in one float64 division, unchanged for an empty cluster; it clears the
// sums for the next pass.  fit_finalize rounds to fp16 and makes the codebook strictly
// ascending inside [-1, 1].
#include <algorithm>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

constexpr int kFitThreads = 256;
constexpr int kFitMaxK = 16;
constexpr double kFitScale = 1073741824.0;  // 2^30

struct FitWorkspace {
  float c[kFitMaxK];
  int32_t pad[kFitMaxK];
  unsigned long long sum[kFitMaxK];  // two's-complement int64 sums
  unsigned long long cnt[kFitMaxK];
};

template <int K>
__global__ __launch_bounds__(kFitThreads) void fit_init_kernel(FitWorkspace* ws) {
  const int j = threadIdx.x;
  if (j < K) {
    ws->c[j] = static_cast<float>(-1.0 + static_cast<double>(2 * j + 1) / K);
    ws->sum[j] = 0ull;
    ws->cnt[j] = 0ull;
  }
}

template <int K>
__global__ __launch_bounds__(kFitThreads) void fit_assign_kernel(const float* __restrict__ u, long long n, FitWorkspace* ws) {
  __shared__ unsigned long long bsum[K], bcnt[K];
  const int tid = threadIdx.x;
  if (tid < K) {
    bsum[tid] = 0ull;
    bcnt[tid] = 0ull;
  }
  float c[K];
#pragma unroll
  for (int j = 0; j < K; ++j) c[j] = ws->c[j];
  long long s[K];
  unsigned int cn[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    s[j] = 0;
    cn[j] = 0;
  }
  const long long stride = static_cast<long long>(gridDim.x) * kFitThreads;
  auto add = [&](float xin) {
    const float x = fminf(fmaxf(xin, -1.0f), 1.0f);
    int best = 0;
    float bd = fabsf(x - c[0]);
#pragma unroll
    for (int j = 1; j < K; ++j) {
      const float d = fabsf(x - c[j]);
      if (d < bd) {
        bd = d;
        best = j;
      }
    }
    const long long q = __float2ll_rn(x * 1073741824.0f);  // x 2^30 is exact in float
#pragma unroll
    for (int j = 0; j < K; ++j) {
      s[j] += best == j ? q : 0;
      cn[j] += best == j ? 1u : 0u;
    }
  };
  // four independent loads in flight per thread, then the remainder
  long long i = static_cast<long long>(blockIdx.x) * kFitThreads + tid;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const float x0 = u[i], x1 = u[i + stride], x2 = u[i + 2 * stride], x3 = u[i + 3 * stride];
    add(x0);
    add(x1);
    add(x2);
    add(x3);
  }
  for (; i < n; i += stride) add(u[i]);
  __syncthreads();
#pragma unroll
  for (int j = 0; j < K; ++j) {
    if (cn[j]) {
      atomicAdd(&bsum[j], static_cast<unsigned long long>(s[j]));
      atomicAdd(&bcnt[j], static_cast<unsigned long long>(cn[j]));
    }
  }
  __syncthreads();
  if (tid < K && bcnt[tid]) {
    atomicAdd(&ws->sum[tid], bsum[tid]);
    atomicAdd(&ws->cnt[tid], bcnt[tid]);
  }
}

template <int K>
__global__ __launch_bounds__(kFitThreads) void fit_update_kernel(FitWorkspace* ws) {
  const int j = threadIdx.x;
  if (j < K) {
    const unsigned long long cnt = ws->cnt[j];
    if (cnt > 0ull) {
      const long long sum = static_cast<long long>(ws->sum[j]);
      ws->c[j] = static_cast<float>(static_cast<double>(sum) / (static_cast<double>(cnt) * kFitScale));
    }
    ws->sum[j] = 0ull;
    ws->cnt[j] = 0ull;
  }
}

// Next fp16 value above (up = true) or below a finite fp16 value, as bits.
__device__ uint16_t half_step(uint16_t h, bool up) {
  const bool neg = (h & 0x8000u) != 0;
  if ((h & 0x7fffu) == 0) return up ? 0x0001u : 0x8001u;  // from +-0 to the smallest subnormal
  return (up != neg) ? static_cast<uint16_t>(h + 1) : static_cast<uint16_t>(h - 1);
}

template <int K>
__global__ __launch_bounds__(64) void fit_finalize_kernel(const FitWorkspace* ws, uint16_t* out) {
  if (threadIdx.x != 0) return;
  float h[K];
  uint16_t hb[K];
#pragma unroll
  for (int j = 0; j < K; ++j) {
    const _Float16 v = static_cast<_Float16>(ws->c[j]);  // round to nearest even
    hb[j] = __builtin_bit_cast(uint16_t, v);
    h[j] = static_cast<float>(v);
  }
  for (int j = 1; j < K; ++j) {
    const uint16_t fb = half_step(hb[j - 1], true);
    const float f = half_bits_to_float(fb);
    if (h[j] < f) {
      hb[j] = fb;
      h[j] = f;
    }
  }
  if (h[K - 1] > 1.0f) {
    hb[K - 1] = 0x3c00u;  // 1.0
    h[K - 1] = 1.0f;
    for (int j = K - 2; j >= 0; --j) {
      const uint16_t cb = half_step(hb[j + 1], false);
      const float cf = half_bits_to_float(cb);
      if (h[j] > cf) {
        hb[j] = cb;
        h[j] = cf;
      }
    }
  }
  for (int j = 0; j < K; ++j) out[j] = hb[j];
}

template <int K>
hipError_t launch_fit_t(const float* u, long long n, int iters, uint16_t* out, void* workspace, hipStream_t s) {
  FitWorkspace* ws = static_cast<FitWorkspace*>(workspace);
  hipLaunchKernelGGL((fit_init_kernel<K>), dim3(1), dim3(kFitThreads), 0, s, ws);
  // About two blocks per CU with at least 64 inputs per thread: the per-block reduction
  // (LDS and global 64-bit atomics) then stays small against the pass over the inputs.
  const long long want = (n + kFitThreads * 64LL - 1) / (kFitThreads * 64LL);
  const int blocks = static_cast<int>(std::max(1LL, std::min<long long>(want, 2LL * device_cu_count())));
  for (int it = 0; it < iters; ++it) {
    hipLaunchKernelGGL((fit_assign_kernel<K>), dim3(blocks), dim3(kFitThreads), 0, s, u, n, ws);
    hipLaunchKernelGGL((fit_update_kernel<K>), dim3(1), dim3(kFitThreads), 0, s, ws);
  }
  hipLaunchKernelGGL((fit_finalize_kernel<K>), dim3(1), dim3(64), 0, s, ws, out);
  return hipGetLastError();
}

}  // namespace

size_t fit_workspace_bytes() { return (sizeof(FitWorkspace) + 255) / 256 * 256; }

hipError_t launch_fit_codebook(int bits, const float* u, long long n, int iters, uint16_t* out, void* workspace,
                               hipStream_t s) {
  if (bits == 2) return launch_fit_t<4>(u, n, iters, out, workspace, s);
  if (bits == 3) return launch_fit_t<8>(u, n, iters, out, workspace, s);
  if (bits == 4) return launch_fit_t<16>(u, n, iters, out, workspace, s);
  return hipErrorInvalidValue;
}

}  // namespace kvq
