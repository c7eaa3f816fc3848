// Merge of partial attention states into the final output.
//
// Minima-KV summary (brainszone.ai), "Como os resultados parciais sao
// combinados": the per-format partial states are combined by a globally
// normalised online-softmax merge.  For query head h of sequence b with
// partial states (m_i, l_i, acc_i) in the base-2 domain:
//   M = max_i m_i,  L = sum_i l_i 2^(m_i - M),
//   O = sum_i acc_i 2^(m_i - M) / L,  LSE = (M + log2 L) * ln 2.
// A chunk with l == 0 holds no token and is skipped.
//
// One block per (b, h, 32-dim slice); its threads take one chunk each (looping
// when there are more chunks than threads) and the block reduces.
#include <hip/hip_runtime.h>

#include "mkv_device.hpp"

namespace mkv {

namespace {

constexpr int kMergeThreads = 256;
constexpr int kSlice = 32;

__global__ void __launch_bounds__(kMergeThreads) merge_kernel(DecodeArgs a) {
  __shared__ float red[kMergeThreads / 64][kSlice + 1];
  __shared__ float redm[kMergeThreads / 64];
  const int d = a.pv.d;
  const int nslices = d / kSlice;
  const int bh = blockIdx.x / nslices;
  const int slice = blockIdx.x % nslices;
  const int b = bh / a.Hq, h = bh % a.Hq;
  const int c0 = a.chunk_base[b], c1 = a.chunk_base[b + 1];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;

  // global reference maximum over the live chunks
  float M = -INFINITY;
  for (int c = c0 + threadIdx.x; c < c1; c += kMergeThreads) {
    const int64_t i = int64_t(c) * a.Hq + h;
    if (a.pl[i] > 0.0f) M = fmaxf(M, a.pm[i]);
  }
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
  if (lane == 0) redm[wave] = M;
  __syncthreads();
  M = redm[0];
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, redm[w]);

  float L = 0.0f;
  float o[kSlice];
#pragma unroll
  for (int j = 0; j < kSlice; ++j) o[j] = 0.0f;
  for (int c = c0 + threadIdx.x; c < c1; c += kMergeThreads) {
    const int64_t i = int64_t(c) * a.Hq + h;
    const float l = a.pl[i];
    if (!(l > 0.0f)) continue;
    const float w = exp2f(a.pm[i] - M);
    L += l * w;
    const float4* src = reinterpret_cast<const float4*>(a.pacc + i * d + slice * kSlice);
#pragma unroll
    for (int j = 0; j < kSlice / 4; ++j) {
      const float4 v = src[j];
      o[4 * j] += v.x * w;
      o[4 * j + 1] += v.y * w;
      o[4 * j + 2] += v.z * w;
      o[4 * j + 3] += v.w * w;
    }
  }
  // reduce over the block: within each wave by shuffles, then across waves
  for (int off = 32; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
#pragma unroll
  for (int j = 0; j < kSlice; ++j)
    for (int off = 32; off > 0; off >>= 1) o[j] += __shfl_xor(o[j], off, 64);
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < kSlice; ++j) red[wave][j] = o[j];
    red[wave][kSlice] = L;
  }
  __syncthreads();
  if (threadIdx.x < kSlice + 1) {
    float t = 0.0f;
    for (int w = 0; w < kMergeThreads / 64; ++w) t += red[w][threadIdx.x];
    red[0][threadIdx.x] = t;
  }
  __syncthreads();
  const float Ltot = red[0][kSlice];
  if (threadIdx.x < kSlice)
    a.out[(int64_t(b) * a.Hq + h) * d + slice * kSlice + threadIdx.x] = red[0][threadIdx.x] / Ltot;
  if (threadIdx.x == 0 && slice == 0)
    a.lse[int64_t(b) * a.Hq + h] = (M + log2f(Ltot)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
  const int nslices = a.pv.d / kSlice;
  hipLaunchKernelGGL(merge_kernel, dim3(unsigned(a.B * a.Hq * nslices)), dim3(kMergeThreads), 0,
                     s, a);
  return hipGetLastError();
}

}  // namespace mkv
