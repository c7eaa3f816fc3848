// Straightforward per-format partial-attention kernels (VALU, fp32 LDS tiles).
//
// Minima-KV summary (brainszone.ai), "Como os resultados parciais sao
// combinados": each format's pages are reduced by their own kernel to a
// partial state (running max m, denominator l, unnormalised accumulator acc),
// working directly on the stored format.  States are kept in the base-2
// domain: with t2 = softmax_scale * log2(e) and s2 = t2 * <q, k>,
//   m = max s2, l = sum 2^(s2 - m), acc = sum 2^(s2 - m) v.
//
// One wave per (work item, kv-head).  Each 16-token tile of a page is
// dequantised into LDS as fp32, scores for the G query heads of the kv-head
// are dot products over LDS, and the online-softmax update rescales the
// accumulator whenever the running max rises.
#include <hip/hip_runtime.h>

#include "mkv_device.hpp"

namespace mkv {

namespace {

constexpr int kRefThreads = 64;

template <int FMT>
__device__ __forceinline__ float load_elem(const PoolView& pv, const uint8_t* page, int h, int kv,
                                           int t, int j) {
  if constexpr (FMT == 0) {
    const float sigma = *reinterpret_cast<const float*>(page + fp8_scale_off(pv, h, kv));
    return e4m3_to_f32(page[fp8_codes_off(pv, h, kv) + int64_t(t) * pv.d + j]) * sigma;
  } else {
    const uint8_t* row = page + tq3_codes_off(pv, h, kv) + int64_t(t) * (3 * pv.d / 8);
    const int bit = 3 * j;
    const uint32_t two = uint32_t(row[bit >> 3]) | (uint32_t(row[(bit >> 3) + 1]) << 8);
    const uint32_t c = (two >> (bit & 7)) & 7u;
    const uint16_t sb = reinterpret_cast<const uint16_t*>(page + tq3_scale_off(pv, h, kv))
        [t * (pv.d / 32) + j / 32];
    return (float(c) - 3.5f) * f16_bits_to_f32(sb);
  }
}

template <int FMT>
__global__ void __launch_bounds__(kRefThreads) partial_ref_kernel(DecodeArgs a) {
  extern __shared__ float smem[];
  const WorkItem it = a.items[blockIdx.x];
  const int hk = blockIdx.y;
  const PoolView& pv = a.pv;
  const int d = pv.d;
  const int G = a.Hq / pv.Hkv;
  const int lane = threadIdx.x;
  float* Kf = smem;              // [16][d]
  float* Vf = Kf + 16 * d;       // [16][d]
  float* Qs = Vf + 16 * d;       // [G][d]
  float* acc = Qs + G * d;       // [G][d]
  float* S = acc + G * d;        // [G][16]
  float* corr = S + G * 16;      // [G]

  const float t2 = a.scale * 1.4426950408889634f;
  const uint16_t* qb = a.q + (int64_t(it.b) * a.Hq + int64_t(hk) * G) * d;
  for (int i = lane; i < G * d; i += kRefThreads) {
    Qs[i] = bf16_to_f32(qb[i]);
    acc[i] = 0.0f;
  }
  float m = -INFINITY, l = 0.0f;  // lanes < G own one query head each

  const int32_t* pt_row = pv.pt + int64_t(it.seq) * pv.pt_stride;
  for (int p = 0; p < it.npages; ++p) {
    const int32_t lp = a.pages[it.list_off + p];
    const uint8_t* page = page_address(pv, pt_row[lp]);
    const int ntok = (p == it.npages - 1) ? it.last_ntok : pv.P;
    for (int t0 = 0; t0 < ntok; t0 += 16) {
      const int nt = min(16, ntok - t0);
      __syncthreads();
      for (int i = lane; i < 16 * d; i += kRefThreads) {
        const int t = i / d, j = i % d;
        const bool ok = t < nt;
        Kf[i] = ok ? load_elem<FMT>(pv, page, hk, 0, t0 + t, j) : 0.0f;
        Vf[i] = ok ? load_elem<FMT>(pv, page, hk, 1, t0 + t, j) : 0.0f;
      }
      __syncthreads();
      for (int i = lane; i < G * 16; i += kRefThreads) {
        const int g = i / 16, t = i % 16;
        float s = -INFINITY;
        if (t < nt) {
          float dot = 0.0f;
          for (int j = 0; j < d; ++j) dot += Qs[g * d + j] * Kf[t * d + j];
          s = t2 * dot;
        }
        S[i] = s;
      }
      __syncthreads();
      if (lane < G) {
        float mx = -INFINITY;
        for (int t = 0; t < 16; ++t) mx = fmaxf(mx, S[lane * 16 + t]);
        const float m_new = fmaxf(m, mx);
        const float c = exp2f(m - m_new);
        float sum = 0.0f;
        for (int t = 0; t < 16; ++t) {
          const float pr = exp2f(S[lane * 16 + t] - m_new);
          S[lane * 16 + t] = pr;
          sum += pr;
        }
        l = l * c + sum;
        m = m_new;
        corr[lane] = c;
      }
      __syncthreads();
      for (int i = lane; i < G * d; i += kRefThreads) {
        const int g = i / d, j = i % d;
        float o = acc[i] * corr[g];
        for (int t = 0; t < 16; ++t) o += S[g * 16 + t] * Vf[t * d + j];
        acc[i] = o;
      }
    }
  }
  __syncthreads();
  const int64_t base = int64_t(it.chunk) * a.Hq + int64_t(hk) * G;
  if (lane < G) {
    a.pm[base + lane] = m;
    a.pl[base + lane] = l;
  }
  for (int i = lane; i < G * d; i += kRefThreads) a.pacc[base * d + i] = acc[i];
}

template <int FMT>
hipError_t launch_ref(const DecodeArgs& a, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  const int G = a.Hq / a.pv.Hkv;
  const size_t lds = sizeof(float) * (32 * a.pv.d + 2 * G * a.pv.d + 17 * G);
  hipLaunchKernelGGL(partial_ref_kernel<FMT>, dim3(unsigned(a.n_items), unsigned(a.pv.Hkv)),
                     dim3(kRefThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partial_fp8(const DecodeArgs& a, hipStream_t s) { return launch_ref<0>(a, s); }
hipError_t launch_partial_tq3(const DecodeArgs& a, hipStream_t s) { return launch_ref<1>(a, s); }

}  // namespace mkv
