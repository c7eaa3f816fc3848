// Merge of partial attention states into the final output.
//
// Minima-KV summary (brainszone.ai), "Como os resultados parciais sao
// combinados": the per-format partial states are combined by a globally
// normalised online-softmax merge.  For query head h of sequence b with
// partial states (m_i, l_i, acc_i):
//   M = max_i m_i,  L = sum_i l_i exp(m_i - M),
//   O = sum_i acc_i exp(m_i - M) / L,  LSE = M + ln L.
// A chunk with l == 0 holds no token and is skipped.
#include <hip/hip_runtime.h>

#include "mkv_device.hpp"

namespace mkv {

namespace {

constexpr int kMergeThreads = 64;

// One wave per (b, h); lanes split head_dim.  Partial maxima are in the
// base-2 domain (see the partial kernels): scores there are s * log2(e).
__global__ void __launch_bounds__(kMergeThreads) merge_kernel(DecodeArgs a) {
  const int b = blockIdx.x / a.Hq;
  const int h = blockIdx.x % a.Hq;
  const int lane = threadIdx.x;
  const int c0 = a.chunk_base[b], c1 = a.chunk_base[b + 1];
  const int d = a.pv.d;
  float M = -INFINITY;
  for (int c = c0; c < c1; ++c) {
    const int64_t i = int64_t(c) * a.Hq + h;
    if (a.pl[i] > 0.0f) M = fmaxf(M, a.pm[i]);
  }
  float L = 0.0f;
  float o[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int c = c0; c < c1; ++c) {
    const int64_t i = int64_t(c) * a.Hq + h;
    const float l = a.pl[i];
    if (!(l > 0.0f)) continue;
    const float w = exp2f(a.pm[i] - M);
    L += l * w;
    const float* acc = a.pacc + i * d;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int j = lane + 64 * u;
      if (j < d) o[u] += acc[j] * w;
    }
  }
  const float inv = 1.0f / L;
  float* out = a.out + (int64_t(b) * a.Hq + h) * d;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = lane + 64 * u;
    if (j < d) out[j] = o[u] * inv;
  }
  if (lane == 0) a.lse[int64_t(b) * a.Hq + h] = (M + log2f(L)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(merge_kernel, dim3(unsigned(a.B * a.Hq)), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace mkv
