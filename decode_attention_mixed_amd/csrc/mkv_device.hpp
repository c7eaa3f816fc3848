// Device helpers shared by the kernels: page addressing and scalar codecs.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mkv_kernels.hpp"

namespace mkv {

// Address of a page record from its page-table entry (bit 31 = TQ3).  The
// gather kernel and the partial kernels both use this function.
__device__ __forceinline__ const uint8_t* page_address(const PoolView& pv, int32_t entry) {
  const int64_t idx = int64_t(entry & 0x7FFFFFFF);
  return entry < 0 ? pv.tq3 + idx * pv.tq3_stride : pv.fp8 + idx * pv.fp8_stride;
}

// ---- record offsets ---------------------------------------------------------
// FP8 record: codes [Hkv][2][P][d] | scale [Hkv][2] f32 | amax [Hkv][2] f32
__device__ __forceinline__ int64_t fp8_codes_off(const PoolView& pv, int h, int kv) {
  return int64_t(h * 2 + kv) * pv.P * pv.d;
}
__device__ __forceinline__ int64_t fp8_scale_off(const PoolView& pv, int h, int kv) {
  return 2ll * pv.Hkv * pv.P * pv.d + 4ll * (h * 2 + kv);
}
__device__ __forceinline__ int64_t fp8_amax_off(const PoolView& pv, int h, int kv) {
  return 2ll * pv.Hkv * pv.P * pv.d + 8ll * pv.Hkv + 4ll * (h * 2 + kv);
}
// TQ3 record: per kv-head block of P*d*7/8 bytes:
//   K codes [P][3d/8] | V codes [P][3d/8] | K scale [P][d/32] f16 | V scale [P][d/32] f16
__device__ __forceinline__ int64_t tq3_block_off(const PoolView& pv, int h) {
  return int64_t(h) * pv.P * pv.d * 7 / 8;
}
__device__ __forceinline__ int64_t tq3_codes_off(const PoolView& pv, int h, int kv) {
  return tq3_block_off(pv, h) + int64_t(kv) * pv.P * (3 * pv.d / 8);
}
__device__ __forceinline__ int64_t tq3_scale_off(const PoolView& pv, int h, int kv) {
  return tq3_block_off(pv, h) + 2ll * pv.P * (3 * pv.d / 8) + int64_t(kv) * pv.P * (pv.d / 16);
}

// ---- OCP E4M3 ---------------------------------------------------------------
// Exact value of an E4M3 byte (finite codes; the cache never stores NaN).
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag;
  if (e == 0)
    mag = float(m) * 0x1p-9f;                                   // subnormal m/8 * 2^-6
  else
    mag = __uint_as_float(((e + 120u) << 23) | (m << 20));      // 2^(e-7) * (1 + m/8)
  return (c & 0x80u) ? -mag : mag;
}

// Round a finite fp32 value to E4M3: nearest, ties to even code, saturating at
// +-448.  Works on the fp32 bit pattern so the result does not depend on the
// hardware conversion's rounding or saturation mode.  Both ranges are formed
// and one is selected (no branches):
//  * |x| < 2^-6: the subnormal grid m * 2^-9; |x| * 512 is exact and rint
//    rounds half to even (a result of 8 is the smallest normal code);
//  * otherwise the top 3 mantissa bits rounded to nearest even on the bit
//    pattern (adding 0x7FFFF plus the kept part's lowest bit carries into it
//    exactly when the dropped 20 bits are above half, or at half with an odd
//    kept part, and a carry moves into the exponent), rebased from the fp32
//    exponent bias to E4M3's (120 << 3), then saturated at 0x7E (448).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  const uint32_t bits = __float_as_uint(x);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t a = bits & 0x7FFFFFFFu;
  const uint32_t sub = uint32_t(__builtin_rintf(__uint_as_float(a) * 512.0f));
  const uint32_t nrm = min(((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - 960u, 0x7Eu);
  return sign | (a < 0x3C800000u ? sub : nrm);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(uint32_t(b) << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t b) {
  return float(__builtin_bit_cast(_Float16, b));
}

}  // namespace mkv
