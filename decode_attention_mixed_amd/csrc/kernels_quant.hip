// Kernels that write the cache: FP8 append, FP8 -> TQ3 demote, the BF16
// append of control pools, and the record gather used to check placement and
// packing.
//
// Every floating-point step here decides a stored code, so this file is built
// with -ffp-contract=off and relies on IEEE fp32 division and round-to-nearest-
// even fp16 conversion; the results are bit-identical to the CPU definitions.
#include <hip/hip_runtime.h>

#include "mkv_device.hpp"

namespace mkv {

namespace {

constexpr int kThreads = 256;

__device__ float block_max(float v, float* red) {
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  float r = red[0];
  for (int i = 1; i < kThreads / 64; ++i) r = fmaxf(r, red[i]);
  __syncthreads();
  return r;
}

// ---------------------------------------------------------------------------
// Append: one block per (touched page, kv-head, K-or-V).
// Minima-KV summary (brainszone.ai), "Ancoras em FP8, arquivo em TQ3": recent
// pages are FP8.  Scale sigma = amax / 448 per page-head; when new rows raise
// the running amax the earlier rows of the page are re-encoded from their
// dequantised values, so a page filled in one call equals one-shot encoding.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void append_fp8_block(const PoolView& pv, const AppendPage& ap,
                                                 const float* __restrict__ k,
                                                 const float* __restrict__ v) {
  __shared__ float red[kThreads / 64];
  const int h = (blockIdx.x / 2) % pv.Hkv;
  const int kv = blockIdx.x % 2;
  const int d = pv.d;
  const float* src = kv ? v : k;
  uint8_t* page = pv.fp8 + int64_t(ap.phys) * pv.fp8_stride;
  uint8_t* codes = page + fp8_codes_off(pv, h, kv);
  float* scale_p = reinterpret_cast<float*>(page + fp8_scale_off(pv, h, kv));
  float* amax_p = reinterpret_cast<float*>(page + fp8_amax_off(pv, h, kv));

  if (ap.pt_slot >= 0 && h == 0 && kv == 0 && threadIdx.x == 0)
    const_cast<int32_t*>(pv.pt)[ap.pt_slot] = ap.pt_entry;   // a page the step opened
  const int n_new = ap.nrows * d;
  float local = 0.0f;
  for (int i = threadIdx.x; i < n_new; i += kThreads) {
    const int r = i / d, j = i % d;
    local = fmaxf(local, fabsf(src[(int64_t(ap.src_row + r) * pv.Hkv + h) * d + j]));
  }
  const float new_amax = block_max(local, red);
  const float old_amax = ap.row0 > 0 ? *amax_p : 0.0f;
  const float old_sigma = ap.row0 > 0 ? *scale_p : 1.0f;
  const bool grown = new_amax > old_amax;
  const float amax = grown ? new_amax : old_amax;
  const float sigma = amax == 0.0f ? 1.0f : amax / 448.0f;
  __syncthreads();  // everyone has read the old scale and amax

  if (grown && ap.row0 > 0) {
    for (int i = threadIdx.x; i < ap.row0 * d; i += kThreads) {
      const float x = e4m3_to_f32(codes[i]) * old_sigma;
      codes[i] = uint8_t(f32_to_e4m3(x / sigma));
    }
  }
  for (int i = threadIdx.x; i < n_new; i += kThreads) {
    const int r = i / d, j = i % d;
    const float x = src[(int64_t(ap.src_row + r) * pv.Hkv + h) * d + j];
    codes[int64_t(ap.row0) * d + i] = uint8_t(f32_to_e4m3(x / sigma));
  }
  if (threadIdx.x == 0) {
    *scale_p = sigma;
    *amax_p = amax;
  }
}

__global__ void __launch_bounds__(kThreads)
append_fp8_kernel(PoolView pv, const AppendPage* __restrict__ plan, const float* __restrict__ k,
                  const float* __restrict__ v) {
  append_fp8_block(pv, plan[blockIdx.x / (pv.Hkv * 2)], k, v);
}

// ---------------------------------------------------------------------------
// Demote: one block per (page, kv-head); each thread encodes 32-element groups.
// Minima-KV summary, "Ancoras em FP8, arquivo em TQ3": older non-anchor pages
// are converted to packed TQ3.  x = fp32(e4m3(c) * sigma); s = fp16(fp32(a/3.5))
// clamped to 65504; c = #{b in -3..3 : x >= b*s} (4 when s == 0); the 32 codes
// form a 96-bit little-endian stream, code j at bit 3j.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
demote_tq3_kernel(PoolView pv, const DemotePage* __restrict__ plan) {
  const DemotePage dp = plan[blockIdx.x / pv.Hkv];
  const int h = blockIdx.x % pv.Hkv;
  const int d = pv.d, ng = d / 32, row_bytes = 3 * d / 8;
  const uint8_t* src = pv.fp8 + int64_t(dp.src_phys) * pv.fp8_stride;
  uint8_t* dst = pv.tq3 + int64_t(dp.dst_phys) * pv.tq3_stride;
  const int tasks = 2 * dp.ntok * ng;
  for (int task = threadIdx.x; task < tasks; task += kThreads) {
    const int kv = task / (dp.ntok * ng);
    const int rem = task % (dp.ntok * ng);
    const int t = rem / ng, g = rem % ng;
    const float sigma = *reinterpret_cast<const float*>(src + fp8_scale_off(pv, h, kv));
    const uint8_t* c8 = src + fp8_codes_off(pv, h, kv) + int64_t(t) * d + 32 * g;
    float x[32];
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      x[j] = e4m3_to_f32(c8[j]) * sigma;
      a = fmaxf(a, fabsf(x[j]));
    }
    const float q = fminf(a / 3.5f, 65504.0f);
    const _Float16 s16 = _Float16(q);          // round to nearest even
    const float s = float(s16);
    uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      uint32_t c = 4u;
      if (s != 0.0f) {
        c = 0u;
#pragma unroll
        for (int b = -3; b <= 3; ++b) c += (x[j] >= float(b) * s) ? 1u : 0u;
      }
      const int bit = 3 * j;
      w[bit >> 5] |= c << (bit & 31);
      if ((bit & 31) > 29) w[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
    }
    uint32_t* out = reinterpret_cast<uint32_t*>(dst + tq3_codes_off(pv, h, kv) +
                                                int64_t(t) * row_bytes + 12 * g);
    out[0] = w[0];
    out[1] = w[1];
    out[2] = w[2];
    reinterpret_cast<uint16_t*>(dst + tq3_scale_off(pv, h, kv))[t * ng + g] =
        __builtin_bit_cast(uint16_t, s16);
  }
}

// ---------------------------------------------------------------------------
// Gather: copy page records in logical order through the device page table.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
gather_kernel(PoolView pv, int32_t seq, int32_t first, uint8_t* __restrict__ dst, int64_t slot) {
  const int32_t entry = pv.pt[int64_t(seq) * pv.pt_stride + first + blockIdx.x];
  const uint8_t* src = page_address(pv, entry);
  const int64_t rec = pv.kind == kKindBf16 ? 4ll * pv.Hkv * pv.P * pv.d
                     : entry < 0         ? int64_t(pv.Hkv) * pv.P * pv.d * 7 / 8
                                         : 2ll * pv.Hkv * pv.P * pv.d + 16ll * pv.Hkv;
  const uint32_t* s32 = reinterpret_cast<const uint32_t*>(src);
  uint32_t* d32 = reinterpret_cast<uint32_t*>(dst + int64_t(blockIdx.x) * slot);
  for (int64_t i = threadIdx.x; i < slot / 4; i += kThreads) d32[i] = i < rec / 4 ? s32[i] : 0u;
}

// ---------------------------------------------------------------------------
// Control-pool append: one block per (touched page, kv-head, K-or-V); rows are
// stored as bf16 at [h][kv][row][d] of the page record.  bf16 is the upper
// half of the fp32 pattern; adding 0x7FFF plus the kept part's lowest bit
// carries into the kept half exactly when the dropped half is above one half
// unit, or equal to it with an odd kept part (round to nearest, ties to
// even), in integer arithmetic independent of the floating-point mode.
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
  const uint32_t u = __float_as_uint(x);
  return uint16_t((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ void append_bf16_block(const PoolView& pv, const AppendPage& ap,
                                                  const float* __restrict__ k,
                                                  const float* __restrict__ v) {
  const int h = (blockIdx.x / 2) % pv.Hkv;
  const int kv = blockIdx.x % 2;
  const int d = pv.d;
  const float* src = kv ? v : k;
  uint16_t* rows = reinterpret_cast<uint16_t*>(pv.fp8 + int64_t(ap.phys) * pv.fp8_stride) +
                   (int64_t(h * 2 + kv) * pv.P + ap.row0) * d;
  if (ap.pt_slot >= 0 && h == 0 && kv == 0 && threadIdx.x == 0)
    const_cast<int32_t*>(pv.pt)[ap.pt_slot] = ap.pt_entry;   // a page the step opened
  const int n = ap.nrows * d;
  for (int i = threadIdx.x; i < n; i += kThreads) {
    const int r = i / d, j = i % d;
    rows[i] = f32_to_bf16_rne(src[(int64_t(ap.src_row + r) * pv.Hkv + h) * d + j]);
  }
}

__global__ void __launch_bounds__(kThreads)
append_bf16_kernel(PoolView pv, const AppendPage* __restrict__ plan, const float* __restrict__ k,
                   const float* __restrict__ v) {
  append_bf16_block(pv, plan[blockIdx.x / (pv.Hkv * 2)], k, v);
}

// Append with the plan in the kernel arguments (one block per (page, kv-head,
// K-or-V) as above); the first block also applies the plan's patches.
template <bool kBf16>
__global__ void __launch_bounds__(kThreads)
append_inline_kernel(PoolView pv, InlinePlan plan, const float* __restrict__ k,
                     const float* __restrict__ v) {
  if (blockIdx.x == 0 && int(threadIdx.x) < plan.n_patch)
    plan.patch_base[plan.patch_off[threadIdx.x]] = plan.patch_val[threadIdx.x];
  const AppendPage ap = plan.pages[blockIdx.x / (pv.Hkv * 2)];
  if constexpr (kBf16)
    append_bf16_block(pv, ap, k, v);
  else
    append_fp8_block(pv, ap, k, v);
}

// ---------------------------------------------------------------------------
// Materialising profile (Minima-KV summary, "Qualidade em contexto longo": the
// hybrid pages expanded into dense tensors; a diagnostic, never on the decode
// path): one block per (page, kv-head, K-or-V).  Each valid element becomes
// the fp32 value the decode kernels work with -- fp32(e4m3(c) * sigma) for an
// FP8 page, (c - 3.5) * s for a TQ3 page (exact) -- rounded to bf16 into the
// control pool's record [h][kv][row][d].
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads)
materialise_kernel(PoolView src, PoolView dst, const MaterialisePage* __restrict__ plan) {
  const int per_page = src.Hkv * 2;
  const MaterialisePage mp = plan[blockIdx.x / per_page];
  const int h = (blockIdx.x / 2) % src.Hkv;
  const int kv = blockIdx.x % 2;
  const int d = src.d;
  const uint8_t* rec = page_address(src, mp.src_entry);
  uint16_t* rows = reinterpret_cast<uint16_t*>(dst.fp8 + int64_t(mp.dst_phys) * dst.fp8_stride) +
                   int64_t(h * 2 + kv) * dst.P * d;
  // eight consecutive elements of one row per step (they share a 32-group);
  // d is a multiple of 32, so a row holds whole steps
  const int n8 = mp.ntok * d / 8;
  for (int e = threadIdx.x; e < n8; e += kThreads) {
    const int i = 8 * e, t = i / d, j = i % d;
    float x[8];
    if (mp.src_entry < 0) {
      // codes j .. j+7 of the group: 24 bits starting at byte 3 (j % 32) / 8
      const uint8_t* grp = rec + tq3_codes_off(src, h, kv) + t * (3 * d / 8) + 12 * (j / 32) + 3 * (j % 32) / 8;
      const uint32_t u = uint32_t(grp[0]) | uint32_t(grp[1]) << 8 | uint32_t(grp[2]) << 16;
      const float s = f16_bits_to_f32(
          reinterpret_cast<const uint16_t*>(rec + tq3_scale_off(src, h, kv))[t * (d / 32) + j / 32]);
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = (float((u >> (3 * k)) & 7u) - 3.5f) * s;
    } else {
      const uint8_t* c = rec + fp8_codes_off(src, h, kv) + i;
      const float sigma = *reinterpret_cast<const float*>(rec + fp8_scale_off(src, h, kv));
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = e4m3_to_f32(c[k]) * sigma;
    }
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k)
      w[k] = uint32_t(f32_to_bf16_rne(x[2 * k])) | uint32_t(f32_to_bf16_rne(x[2 * k + 1])) << 16;
    *reinterpret_cast<uint4*>(rows + i) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

}  // namespace

hipError_t launch_materialise(const PoolView& src, const PoolView& dst, const MaterialisePage* plan,
                              int32_t n_pages, hipStream_t s) {
  if (n_pages <= 0) return hipSuccess;
  hipLaunchKernelGGL(materialise_kernel, dim3(unsigned(n_pages * src.Hkv * 2)), dim3(kThreads), 0, s,
                     src, dst, plan);
  return hipGetLastError();
}

hipError_t launch_append_bf16(const PoolView& pv, const AppendPage* plan, int32_t n_pages,
                              const float* k, const float* v, hipStream_t s) {
  if (n_pages <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_bf16_kernel, dim3(unsigned(n_pages * pv.Hkv * 2)), dim3(kThreads), 0,
                     s, pv, plan, k, v);
  return hipGetLastError();
}

hipError_t launch_append(const PoolView& pv, const AppendPage* plan, int32_t n_pages,
                         const float* k, const float* v, hipStream_t s) {
  if (n_pages <= 0) return hipSuccess;
  hipLaunchKernelGGL(append_fp8_kernel, dim3(unsigned(n_pages * pv.Hkv * 2)), dim3(kThreads), 0,
                     s, pv, plan, k, v);
  return hipGetLastError();
}

__global__ void __launch_bounds__(kThreads) upload_kernel(UploadSet u) {
  const uint32_t stride = gridDim.x * kThreads;
  for (int g = 0; g < u.nseg; ++g) {
    const uint32_t* __restrict__ src = u.src + u.src_word[g];
    uint32_t* __restrict__ dst = u.dst[g];
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < u.words[g]; i += stride) dst[i] = src[i];
  }
}

hipError_t launch_upload(const UploadSet& u, hipStream_t s) {
  if (u.nseg <= 0) return hipSuccess;
  if (u.nseg > kUploadSegs) return hipErrorInvalidValue;
  uint32_t most = 0;
  for (int g = 0; g < u.nseg; ++g) most = u.words[g] > most ? u.words[g] : most;
  if (most == 0) return hipSuccess;
  const uint32_t blocks = (most + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(upload_kernel, dim3(blocks < 128 ? blocks : 128), dim3(kThreads), 0, s, u);
  return hipGetLastError();
}

hipError_t launch_append_inline(const PoolView& pv, const InlinePlan& plan, int32_t n_pages,
                                const float* k, const float* v, hipStream_t s) {
  if (n_pages <= 0 || n_pages > kInlinePages || plan.n_patch < 0 || plan.n_patch > kInlinePages)
    return hipErrorInvalidValue;
  const dim3 grid(unsigned(n_pages * pv.Hkv * 2));
  if (pv.kind == kKindBf16)
    hipLaunchKernelGGL(append_inline_kernel<true>, grid, dim3(kThreads), 0, s, pv, plan, k, v);
  else
    hipLaunchKernelGGL(append_inline_kernel<false>, grid, dim3(kThreads), 0, s, pv, plan, k, v);
  return hipGetLastError();
}

hipError_t launch_demote(const PoolView& pv, const DemotePage* plan, int32_t n_pages,
                         hipStream_t s) {
  if (n_pages <= 0) return hipSuccess;
  hipLaunchKernelGGL(demote_tq3_kernel, dim3(unsigned(n_pages * pv.Hkv)), dim3(kThreads), 0, s,
                     pv, plan);
  return hipGetLastError();
}

hipError_t launch_gather(const PoolView& pv, int32_t seq, int32_t first, int32_t n,
                         uint8_t* dst, int64_t slot_bytes, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(gather_kernel, dim3(unsigned(n)), dim3(kThreads), 0, s, pv, seq, first, dst,
                     slot_bytes);
  return hipGetLastError();
}

}  // namespace mkv
