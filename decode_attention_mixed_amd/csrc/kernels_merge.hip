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
// Two variants.  Wide (many chunks per sequence): one wave per (b, h, 16-dim
// slice).  Lane (j, k) owns dims 4j..4j+3 of the slice for chunks k, k+16,
// ...; it loads a batch of up to U of them (max, denominator and a float4 of
// the accumulator) at once, so a batch of 16 * U chunks costs one memory
// round trip (U = 16 when a sequence has more than 128 chunks, else 8, so
// short lists do not pay for redundant loads).  The batch maximum is reduced over the wave, the lane
// accumulates its chunks with weights 2^(m_i - M) (rescaling earlier batches
// if M rose), and the 16 chunk lanes are summed with shuffles at the end (no
// LDS, no workgroup barrier).  Narrow (few chunks per sequence, as
// in large batches): one wave per 256/d query heads, d/4 lanes per head; a
// lane owns dims 4j..4j+3 of its head and walks all of the head's chunks
// itself in batches of kUnroll, so it needs no cross-lane reduction.
#include <hip/hip_runtime.h>

#include "mkv_device.hpp"

namespace mkv {

namespace {

constexpr int kMergeThreads = 64;
constexpr int kSlice = 16;                         // dims per wave
constexpr int kVecLanes = kSlice / 4;              // lanes per chunk (float4 each)
constexpr int kChunkLanes = kMergeThreads / kVecLanes;
constexpr int kUnroll = 8;

// Cross-lane steps without the LDS permute unit (each ds_bpermute is a round
// trip through the LDS pipeline; these are ALU operations): DPP moves within a
// row of 16 lanes and the row swaps of permlane16/32.
constexpr int kDppXor1 = 0xB1;      // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;      // quad_perm [2, 3, 0, 1]
constexpr int kDppRor4 = 0x124;     // row_ror:4
constexpr int kDppRor8 = 0x128;     // row_ror:8
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
// permlane16_swap (permlane32_swap) of a register with itself leaves, in the
// two results, the even and the odd row of each pair of 16-lane rows (the
// lower and the upper 32 lanes): combining the two gives every lane the
// combination of its row (half) and the partner row (half), the same bits in
// both.
__device__ __forceinline__ float pair16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float pair32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Maximum over the 64 lanes.
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  x = fmaxf(x, dpp<kDppRor4>(x));
  x = fmaxf(x, dpp<kDppRor8>(x));
  return pair32_max(pair16_max(x));
}

// Sum over the 16 lanes of the wave with the same lane index mod 4 (the
// rotations by 4 and 8 within a row reach the row's lanes of that residue).
__device__ __forceinline__ float sum_mod4(float x) {
  x += dpp<kDppRor4>(x);
  x += dpp<kDppRor8>(x);
  return pair32_sum(pair16_sum(x));
}

// The arguments the first state loads need come first, so the kernel can
// receive them preloaded in scalar registers (built with a kernel-argument
// preload count of 12): pm, pl, pacc, chunk_base, Hq, d, B, the largest
// chunk count per entry.
struct MergeArgs {
  const float* pm;
  const float* pl;
  const float* pacc;
  const int32_t* chunk_base;
  int32_t Hq, d, B, max_seq_chunks;
  float* out;
  float* lse;
};

template <int U>
__global__ void __launch_bounds__(kMergeThreads)
merge_kernel(const float* __restrict__ pm, const float* __restrict__ pl, const float* __restrict__ pacc,
             const int32_t* __restrict__ chunk_base, int32_t Hq, int32_t d, int32_t B, int32_t max_seq_chunks,
             float* __restrict__ out, float* __restrict__ lse) {
  const MergeArgs a{pm, pl, pacc, chunk_base, Hq, d, B, max_seq_chunks, out, lse};
  const int nslices = d / kSlice;
  const int bh = blockIdx.x / nslices;
  const int slice = blockIdx.x % nslices;
  const int b = bh / a.Hq, h = bh % a.Hq;
  // one batch entry: its chunks are 0 .. max_seq_chunks - 1 (no dependent load)
  const int c0 = a.B == 1 ? 0 : a.chunk_base[b];
  const int c1 = a.B == 1 ? a.max_seq_chunks : a.chunk_base[b + 1];
  const int t = threadIdx.x;
  const int j = t % kVecLanes, k = t / kVecLanes;

  float M = -INFINITY;                 // running maximum over live chunks
  float L = 0.0f;                      // this thread's share of the denominator
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int cb = c0; cb < c1; cb += kChunkLanes * U) {
    float m[U], l[U];
    float4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = cb + k + kChunkLanes * u;
      const bool ok = c < c1;
      const int64_t i = int64_t(ok ? c : c0) * a.Hq + h;
      m[u] = a.pm[i];
      l[u] = ok ? a.pl[i] : 0.0f;
      v[u] = *reinterpret_cast<const float4*>(a.pacc + i * d + slice * kSlice + 4 * j);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (l[u] > 0.0f) bm = fmaxf(bm, m[u]);
    bm = wave_max(bm);
    if (bm > M) {                      // rescale what earlier batches accumulated
      const float r = exp2f(M - bm);   // 0 on the first live batch
      L *= r;
      acc.x *= r;
      acc.y *= r;
      acc.z *= r;
      acc.w *= r;
      M = bm;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (!(l[u] > 0.0f)) continue;
      const float w = exp2f(m[u] - M);
      L += l[u] * w;
      acc.x += v[u].x * w;
      acc.y += v[u].y * w;
      acc.z += v[u].z * w;
      acc.w += v[u].w * w;
    }
  }
  // sum over the chunk lanes (lanes j + 4k')
  float r5[5] = {acc.x, acc.y, acc.z, acc.w, L};
  static_assert(kVecLanes == 4, "chunk lanes are the lanes of one residue mod 4");
#pragma unroll
  for (int e = 0; e < 5; ++e) r5[e] = sum_mod4(r5[e]);
  if (t < kVecLanes) {
    const float inv = 1.0f / r5[4];
    *reinterpret_cast<float4*>(a.out + (int64_t(b) * a.Hq + h) * d + slice * kSlice + 4 * t) =
        make_float4(r5[0] * inv, r5[1] * inv, r5[2] * inv, r5[3] * inv);
    if (t == 0 && slice == 0) a.lse[int64_t(b) * a.Hq + h] = (M + log2f(r5[4])) * 0.69314718055994531f;
  }
}

__global__ void __launch_bounds__(64)
merge_narrow_kernel(const float* __restrict__ pm, const float* __restrict__ pl, const float* __restrict__ pacc,
                    const int32_t* __restrict__ chunk_base, int32_t Hq, int32_t d, int32_t B,
                    int32_t max_seq_chunks, float* __restrict__ out, float* __restrict__ lse) {
  const MergeArgs a{pm, pl, pacc, chunk_base, Hq, d, B, max_seq_chunks, out, lse};
  const int lanes_per_head = d / 4;                // 8 .. 64
  const int lane = threadIdx.x;
  const int row = blockIdx.x * (64 / lanes_per_head) + lane / lanes_per_head;   // b * Hq + h
  const int j = lane % lanes_per_head;
  if (row >= a.B * a.Hq) return;
  const int b = row / a.Hq, h = row % a.Hq;
  const int c0 = a.B == 1 ? 0 : a.chunk_base[b];
  const int c1 = a.B == 1 ? a.max_seq_chunks : a.chunk_base[b + 1];
  float M = -INFINITY;
  float L = 0.0f;
  float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  for (int cb = c0; cb < c1; cb += kUnroll) {
    float m[kUnroll], l[kUnroll];
    float4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int c = cb + u;
      const bool ok = c < c1;
      const int64_t i = int64_t(ok ? c : c0) * a.Hq + h;
      m[u] = a.pm[i];
      l[u] = ok ? a.pl[i] : 0.0f;
      v[u] = *reinterpret_cast<const float4*>(a.pacc + i * d + 4 * j);
    }
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
      if (l[u] > 0.0f) bm = fmaxf(bm, m[u]);
    if (bm > M) {
      const float r = exp2f(M - bm);
      L *= r;
      acc.x *= r;
      acc.y *= r;
      acc.z *= r;
      acc.w *= r;
      M = bm;
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (!(l[u] > 0.0f)) continue;
      const float w = exp2f(m[u] - M);
      L += l[u] * w;
      acc.x += v[u].x * w;
      acc.y += v[u].y * w;
      acc.z += v[u].z * w;
      acc.w += v[u].w * w;
    }
  }
  const float inv = 1.0f / L;
  *reinterpret_cast<float4*>(a.out + int64_t(row) * d + 4 * j) =
      make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  if (j == 0) a.lse[row] = (M + log2f(L)) * 0.69314718055994531f;
}

}  // namespace

hipError_t launch_merge(const DecodeArgs& a, int narrow_max, hipStream_t s) {
  const MergeArgs M{a.pm, a.pl, a.pacc, a.chunk_base, a.Hq, a.pv.d, a.B, a.max_seq_chunks, a.out, a.lse};
  if (a.max_seq_chunks <= narrow_max) {
    const int heads_per_wave = 256 / a.pv.d;
    const int rows = a.B * a.Hq;
    hipLaunchKernelGGL(merge_narrow_kernel, dim3(unsigned((rows + heads_per_wave - 1) / heads_per_wave)),
                       dim3(64), 0, s, M.pm, M.pl, M.pacc, M.chunk_base, M.Hq, M.d, M.B, M.max_seq_chunks, M.out,
                       M.lse);
    return hipGetLastError();
  }
  const int nslices = a.pv.d / kSlice;
  const dim3 grid(unsigned(a.B * a.Hq * nslices));
  if (a.max_seq_chunks > kChunkLanes * 8)
    hipLaunchKernelGGL(merge_kernel<16>, grid, dim3(kMergeThreads), 0, s, M.pm, M.pl, M.pacc, M.chunk_base, M.Hq,
                       M.d, M.B, M.max_seq_chunks, M.out, M.lse);
  else
    hipLaunchKernelGGL(merge_kernel<8>, grid, dim3(kMergeThreads), 0, s, M.pm, M.pl, M.pacc, M.chunk_base, M.Hq,
                       M.d, M.B, M.max_seq_chunks, M.out, M.lse);
  return hipGetLastError();
}

}  // namespace mkv
