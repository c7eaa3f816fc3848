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
  // the page's scale and amax so far, loaded while the new rows arrive
  const float old_amax = ap.row0 > 0 ? *amax_p : 0.0f;
  const float old_sigma = ap.row0 > 0 ? *scale_p : 1.0f;
  // new rows as 16-byte vectors (d is a multiple of 32, rows 16-byte aligned),
  // kept in registers from the amax pass to the encoding
  constexpr int kVec = 4;
  const int n4 = ap.nrows * d / 4;
  auto row_vec = [&](int i) {
    const int e = 4 * i, r = e / d, j = e % d;
    return *reinterpret_cast<const float4*>(src + (int64_t(ap.src_row + r) * pv.Hkv + h) * d + j);
  };
  float4 val[kVec];
  float local = 0.0f;
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int i = int(threadIdx.x) + u * kThreads;
    if (i < n4) {
      val[u] = row_vec(i);
      local = fmaxf(local, fmaxf(fmaxf(fabsf(val[u].x), fabsf(val[u].y)), fmaxf(fabsf(val[u].z), fabsf(val[u].w))));
    }
  }
  for (int i = int(threadIdx.x) + kVec * kThreads; i < n4; i += kThreads) {   // pages past kVec vectors a lane
    const float4 x = row_vec(i);
    local = fmaxf(local, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
  }
  const float new_amax = block_max(local, red);
  const bool grown = new_amax > old_amax;
  const float amax = grown ? new_amax : old_amax;
  const float sigma = amax == 0.0f ? 1.0f : amax / 448.0f;

  auto enc4 = [&](const float4 x) {
    return uint32_t(f32_to_e4m3(x.x / sigma)) | (uint32_t(f32_to_e4m3(x.y / sigma)) << 8) |
           (uint32_t(f32_to_e4m3(x.z / sigma)) << 16) | (uint32_t(f32_to_e4m3(x.w / sigma)) << 24);
  };
  if (grown && ap.row0 > 0) {
    // earlier rows re-encoded from their dequantised values, four codes a word
    uint32_t* old = reinterpret_cast<uint32_t*>(codes);
    for (int i = threadIdx.x; i < ap.row0 * d / 4; i += kThreads) {
      const uint32_t w = old[i];
      float4 x;
      x.x = e4m3_to_f32(uint8_t(w)) * old_sigma;
      x.y = e4m3_to_f32(uint8_t(w >> 8)) * old_sigma;
      x.z = e4m3_to_f32(uint8_t(w >> 16)) * old_sigma;
      x.w = e4m3_to_f32(uint8_t(w >> 24)) * old_sigma;
      old[i] = enc4(x);
    }
  }
  uint32_t* out = reinterpret_cast<uint32_t*>(codes + int64_t(ap.row0) * d);
#pragma unroll
  for (int u = 0; u < kVec; ++u) {
    const int i = int(threadIdx.x) + u * kThreads;
    if (i < n4) out[i] = enc4(val[u]);
  }
  for (int i = int(threadIdx.x) + kVec * kThreads; i < n4; i += kThreads) out[i] = enc4(row_vec(i));
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
// Demote: one thread per 32-element group of a converted page.
// Minima-KV summary, "Ancoras em FP8, arquivo em TQ3": older non-anchor pages
// are converted to packed TQ3.  x = fp32(e4m3(c) * sigma); s = fp16(fp32(a/3.5))
// clamped to 65504; c = #{b in -3..3 : x >= b*s} (4 when s == 0); the 32 codes
// form a 96-bit little-endian stream, code j at bit 3j.
// Threads of a page walk its groups with the group fastest, then the token,
// then (kv-head, K or V), so consecutive lanes read consecutive 32-byte runs
// of codes and write consecutive 12-byte runs and fp16 scales.  The count of
// thresholds at or below x is floor(x / s) + 4 clamped to 0..7 in exact
// arithmetic.  t = x * (1 / s) is far less than one step from x / s, so with
// k = rint(t), x / s lies in (k - 1, k + 1) and floor(x / s) is k when
// x >= k * s and k - 1 otherwise: one comparison with an exact product
// (k * s is exact in fp32 for the small integers k), and the codes equal
// those of the seven comparisons.  The +4 rides along: k' = rint(x / s + 4)
// from one fma, compared with k' * s - 4 s (also exact).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int demote_groups(const PoolView& pv) { return pv.Hkv * 2 * pv.P * (pv.d / 32); }

// NG groups a row and PP tokens a page when known at compile time (0: the
// pool's values), so that the lane's (kv-head, K or V, token, group) comes
// from shifts and constant divisions.
template <int NG = 0, int PP = 0>
__device__ __forceinline__ void demote_group(const PoolView& pv, const DemotePage& dp, int rem) {
  const int ng = NG ? NG : pv.d / 32, P = PP ? PP : pv.P, d = 32 * ng, row_bytes = 12 * ng;
  const int g = rem % ng, t = (rem / ng) % P, hk = rem / (ng * P);
  const int h = hk >> 1, kv = hk & 1;
  if (t >= dp.ntok) return;
  const uint8_t* src = pv.fp8 + int64_t(dp.src_phys) * pv.fp8_stride;
  uint8_t* dst = pv.tq3 + int64_t(dp.dst_phys) * pv.tq3_stride;
  const uint4* c8 = reinterpret_cast<const uint4*>(src + fp8_codes_off(pv, h, kv) + int64_t(t) * d + 32 * g);
  const uint4 w0 = c8[0], w1 = c8[1];
  const float sigma = *reinterpret_cast<const float*>(src + fp8_scale_off(pv, h, kv));
  const uint32_t cw[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  float x[32];
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(cw[i], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(cw[i], true);
    x[4 * i + 0] = lo[0] * sigma;
    x[4 * i + 1] = lo[1] * sigma;
    x[4 * i + 2] = hi[0] * sigma;
    x[4 * i + 3] = hi[1] * sigma;
  }
#pragma unroll
  for (int j = 0; j < 32; ++j) a = fmaxf(a, fabsf(x[j]));
  const float q = fminf(a / 3.5f, 65504.0f);
  const _Float16 s16 = _Float16(q);            // round to nearest even
  const float s = float(s16);
  const float rs = __builtin_amdgcn_rcpf(s);    // s == 0 is settled below
  const float s4 = -4.0f * s;
  uint32_t w[3] = {0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    // code = floor(x / s) + 4 clamped to 0..7, without branches
    const float k = __builtin_rintf(__builtin_fmaf(x[j], rs, 4.0f));
    const float f = x[j] < __builtin_fmaf(k, s, s4) ? k - 1.0f : k;
    const uint32_t c = uint32_t(__builtin_amdgcn_fmed3f(f, 0.0f, 7.0f));
    const int bit = 3 * j;
    w[bit >> 5] |= c << (bit & 31);
    if ((bit & 31) > 29) w[(bit >> 5) + 1] |= c >> (32 - (bit & 31));
  }
  // all codes 4 when s == 0 (0b100 in every 3-bit field)
  constexpr uint32_t kFour[3] = {0x24924924u, 0x49249249u, 0x92492492u};
#pragma unroll
  for (int i = 0; i < 3; ++i) w[i] = s != 0.0f ? w[i] : kFour[i];
  uint32_t* out = reinterpret_cast<uint32_t*>(dst + tq3_codes_off(pv, h, kv) + int64_t(t) * row_bytes + 12 * g);
  out[0] = w[0];
  out[1] = w[1];
  out[2] = w[2];
  reinterpret_cast<uint16_t*>(dst + tq3_scale_off(pv, h, kv))[t * ng + g] = __builtin_bit_cast(uint16_t, s16);
}

// Grid (page, block of the page's groups).
template <int NG, int PP>
__global__ void __launch_bounds__(kThreads)
demote_tq3_kernel(PoolView pv, const DemotePage* __restrict__ plan) {
  const int rem = int(blockIdx.y) * kThreads + int(threadIdx.x);
  if (rem >= pv.Hkv * 2 * (PP ? PP : pv.P) * (NG ? NG : pv.d / 32)) return;
  demote_group<NG, PP>(pv, plan[blockIdx.x], rem);
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

// A decode step's cache writes (StepPlan): blocks [0, 2 Hkv n_append) append
// as append_inline_kernel, the blocks after them convert the n_conv pages as
// demote_tq3_kernel (one thread per group), the first thread of each
// converted page writing its page-table entry; block 0 applies the schedule
// patches.
template <bool kBf16>
__global__ void __launch_bounds__(kThreads)
step_kernel(PoolView pv, StepPlan plan, const float* __restrict__ k, const float* __restrict__ v) {
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < plan.n_patch; i += kThreads) plan.patch_base[plan.patch_off[i]] = plan.patch_val[i];
  const int n_app = plan.n_append * pv.Hkv * 2;
  if (int(blockIdx.x) < n_app) {
    const AppendPage ap = plan.pages[blockIdx.x / (pv.Hkv * 2)];
    if constexpr (kBf16)
      append_bf16_block(pv, ap, k, v);
    else
      append_fp8_block(pv, ap, k, v);
    return;
  }
  if constexpr (!kBf16) {
    const int per = demote_groups(pv);
    const int task = (int(blockIdx.x) - n_app) * kThreads + int(threadIdx.x);
    const int c = task / per, rem = task % per;
    if (c >= plan.n_conv) return;              // past the last page (or a patch-only launch)
    const DemotePage dp = plan.conv[c];
    if (rem == 0) const_cast<int32_t*>(pv.pt)[dp.pad0] = dp.pad1;
    demote_group(pv, dp, rem);
  }
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

hipError_t launch_step(const PoolView& pv, const StepPlan& plan, const float* k, const float* v,
                       hipStream_t s) {
  if (plan.n_append < 0 || plan.n_append > kInlinePages || plan.n_conv < 0 || plan.n_conv > kStepConv ||
      plan.n_patch < 0 || plan.n_patch > kStepPatches || (pv.kind == kKindBf16 && plan.n_conv > 0))
    return hipErrorInvalidValue;
  const int per = pv.Hkv * 2 * pv.P * (pv.d / 32);
  const int blocks = plan.n_append * pv.Hkv * 2 + (plan.n_conv * per + kThreads - 1) / kThreads;
  if (blocks == 0 && plan.n_patch == 0) return hipSuccess;
  const dim3 grid(unsigned(blocks > 0 ? blocks : 1));
  if (pv.kind == kKindBf16)
    hipLaunchKernelGGL(step_kernel<true>, grid, dim3(kThreads), 0, s, pv, plan, k, v);
  else
    hipLaunchKernelGGL(step_kernel<false>, grid, dim3(kThreads), 0, s, pv, plan, k, v);
  return hipGetLastError();
}

hipError_t launch_demote(const PoolView& pv, const DemotePage* plan, int32_t n_pages,
                         hipStream_t s) {
  if (n_pages <= 0) return hipSuccess;
  const int per = pv.Hkv * 2 * pv.P * (pv.d / 32);
  const dim3 grid(unsigned(n_pages), unsigned((per + kThreads - 1) / kThreads));
  const int ng = pv.d / 32;
  if (ng == 4 && pv.P == 16)
    hipLaunchKernelGGL((demote_tq3_kernel<4, 16>), grid, dim3(kThreads), 0, s, pv, plan);
  else if (ng == 8 && pv.P == 64)
    hipLaunchKernelGGL((demote_tq3_kernel<8, 64>), grid, dim3(kThreads), 0, s, pv, plan);
  else if (ng == 8 && pv.P == 16)
    hipLaunchKernelGGL((demote_tq3_kernel<8, 16>), grid, dim3(kThreads), 0, s, pv, plan);
  else if (ng == 4 && pv.P == 64)
    hipLaunchKernelGGL((demote_tq3_kernel<4, 64>), grid, dim3(kThreads), 0, s, pv, plan);
  else if (ng == 2 && pv.P == 16)
    hipLaunchKernelGGL((demote_tq3_kernel<2, 16>), grid, dim3(kThreads), 0, s, pv, plan);
  else
    hipLaunchKernelGGL((demote_tq3_kernel<0, 0>), grid, dim3(kThreads), 0, s, pv, plan);
  return hipGetLastError();
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Read-bandwidth calibration: every byte of src read once with 16-byte
// nontemporal loads, four in flight per lane, grid-strided; an XOR of the data
// is stored to sink only if it equals a value no caller arranges (so the loads
// cannot be dropped).  bytes must be a multiple of 16.
__global__ void __launch_bounds__(256) stream_read_kernel(const u32x4* __restrict__ p, int64_t n_vec,
                                                          uint32_t* __restrict__ sink) {
  const int64_t tid = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t stride = int64_t(gridDim.x) * 256;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = tid;
  for (; i + 3 * stride < n_vec; i += 4 * stride) {
    u32x4 v[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) v[k] = __builtin_nontemporal_load(p + i + k * stride);
#pragma unroll
    for (int k = 0; k < 4; ++k) acc ^= v[k];
  }
  for (; i < n_vec; i += stride) acc ^= p[i];
  const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x9E3779B9u) sink[tid & 255] = r;
}

hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s) {
  if (bytes <= 0 || bytes % 16) return hipErrorInvalidValue;
  // 8 workgroups of 256 lanes per CU of the largest part (256 CUs)
  hipLaunchKernelGGL(stream_read_kernel, dim3(2048), dim3(256), 0, s, static_cast<const u32x4*>(src),
                     bytes / 16, sink);
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
