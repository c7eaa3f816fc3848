// Per-format split-K partial-attention kernels for gfx950 (MFMA, f16 operands,
// fp32 accumulation).
//
// Minima-KV summary (brainszone.ai), "Como os resultados parciais sao
// combinados": pages of each numeric format are reduced by a kernel of their
// own, working on the stored format, to a partial attention state that a
// globally normalised merge combines.  State of a query head over a set of
// tokens, in the base-2 domain with t2 = softmax_scale * log2(e):
//   s2 = t2 * <q, k>,  m = reference maximum,  l = sum 2^(s2 - m),
//   acc = sum 2^(s2 - m) * v.
//
// Work decomposition.  One workgroup (4 wave64) per (work item = chunk of
// pages of one format of one sequence, kv-head).  A page is cut into 16-token
// tiles; wave w takes tiles w, w+4, ... and keeps its own state; the four
// states are merged through LDS and one partial state per query head of the
// kv-head is written.
//
// Tile computation (16 tokens x one kv-head x up to 16 query heads):
//  * QK^T on MFMA 16x16x32 f16 with A = key tile (tokens x 32 dims), B = the
//    query heads (32 dims x 16 head columns): D[t][h].  TQ3 multiplies each
//    32-dim group's D by its per-token fp16 scale before summing groups; FP8
//    applies its per-page scale once.
//  * Softmax: a reference maximum m per head column, raised (with headroom)
//    only when a tile exceeds it, so exp2 arguments stay <= 0 and rescaling
//    the accumulator is rare.
//  * PV on MFMA 16x16x32 f16.  P' (probabilities times the value scale) is
//    split into an f16 high part and an f16 low part (about 22 significant
//    bits together); A holds both parts of the lane's 4 tokens, exactly in
//    the lane layout QK^T produced, and B holds the value tile (read from LDS
//    with ds_read_b64_tr_b16) twice, so one MFMA adds hi*V + lo*V.  A single
//    f16 rounding of P' costs up to 2^-12 * |v| per weight, too much for
//    values with outlier channels.
//
// Operand encodings (all exact, all in the f16 normal range: MFMA products
// with subnormal f16 operands are not accumulated to full fp32 precision):
//  * TQ3: a 3-bit code c is masked into mantissa bits k..k+2 of an f16 whose
//    exponent encodes 1.0 (one AND-OR per two elements), then 1.0 is
//    subtracted (one packed add): the operand is c * 2^(k-10), finite for any
//    bit pattern, including unwritten poisoned slots.  The offset 3.5 is
//    restored exactly: for keys through the MFMA accumulator input
//    (-3.5 * sum q per group), for values through Z = sum_t P'[h][t],
//    accumulated by an MFMA against ones.
//  * FP8 E4M3 codes are widened by the hardware conversion to fp32 and packed
//    to f16 (every E4M3 value is an f16 normal number).  Value rows past the
//    valid tokens are zeroed because a poisoned byte may decode to NaN.
//  * Queries are bf16; per head they are scaled by a power of two so the
//    largest magnitude is in [64, 128) and, for TQ3, by 2^(7-k) to cancel each
//    slot's mantissa position k.  The compensating factors are folded into
//    the score scale.
#include <hip/hip_runtime.h>

#include "mkv_device.hpp"

namespace mkv {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kHeadroom = 2.0f;   // log2 units added when the reference max is raised
constexpr float kLog2e = 1.4426950408889634f;

// ---- TQ3 unit unpack -------------------------------------------------------
// A unit is 8 consecutive codes (24 bits, code i at bit 3i; bits 24..31 are
// ignored).  It becomes four dwords of f16 pairs holding c * 2^(k-10):
//   slot:        0   1   2   3   4   5   6   7
//   code index:  6   3   7   2   4   0   5   1     (kSlotCode)
//   bit pos k:   0   7   3   4   0   4   3   7     (kSlotShift)
// built from the unit rotated right by 18 and by 12 (the rotations put two
// codes of each dword inside the two 10-bit mantissa fields).
__device__ constexpr int kSlotCode[8] = {6, 3, 7, 2, 4, 0, 5, 1};
__device__ constexpr int kSlotShift[8] = {0, 7, 3, 4, 0, 4, 3, 7};

__device__ __forceinline__ uint32_t one_minus(uint32_t biased) {
  const half2v h = __builtin_bit_cast(half2v, biased) - half2v{_Float16(1.0f), _Float16(1.0f)};
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ u32x4 tq3_unit_to_f16(uint32_t x) {
  const uint32_t r18 = __builtin_amdgcn_alignbit(x, x, 18);
  const uint32_t r12 = __builtin_amdgcn_alignbit(x, x, 12);
  u32x4 o;
  o[0] = one_minus((r18 & 0x03800007u) | 0x3C003C00u);   // c6 -> bits 0..2,   c3 -> bits 23..25
  o[1] = one_minus((r18 & 0x00700038u) | 0x3C003C00u);   // c7 -> bits 3..5,   c2 -> bits 20..22
  o[2] = one_minus((r12 & 0x00700007u) | 0x3C003C00u);   // c4 -> bits 0..2,   c0 -> bits 20..22
  o[3] = one_minus((r12 & 0x03800038u) | 0x3C003C00u);   // c5 -> bits 3..5,   c1 -> bits 23..25
  return o;
}

// The four 24-bit units of a 12-byte group held as three little-endian dwords.
__device__ __forceinline__ void tq3_split_units(uint32_t d0, uint32_t d1, uint32_t d2,
                                                uint32_t u[4]) {
  u[0] = d0;
  u[1] = __builtin_amdgcn_alignbit(d1, d0, 24);
  u[2] = __builtin_amdgcn_alignbit(d2, d1, 16);
  u[3] = d2 >> 8;
}

// ---- FP8 -> f16 -------------------------------------------------------------
// Two fp32 values -> an f16 pair, rounded toward zero.
__device__ __forceinline__ uint32_t pkrtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
__device__ __forceinline__ float f16lo(uint32_t u) { return float(__builtin_bit_cast(half2v, u)[0]); }
__device__ __forceinline__ float f16hi(uint32_t u) { return float(__builtin_bit_cast(half2v, u)[1]); }

// Four E4M3 bytes -> two dwords of f16 pairs (exact: the hardware widening to
// fp32 is exact and every finite E4M3 value is an f16 normal number).
__device__ __forceinline__ u32x2 fp8x4_to_f16(uint32_t w) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  u32x2 o;
  o[0] = pkrtz(lo[0], lo[1]);
  o[1] = pkrtz(hi[0], hi[1]);
  return o;
}

// P' of the lane's 4 tokens -> MFMA 16x16x32 A operand: slots 0..3 hold the
// f16 high parts (round toward zero), slots 4..7 the f16 low parts of the
// exact fp32 remainders.
__device__ __forceinline__ half8 split_hi_lo(const float w[4]) {
  const uint32_t h01 = pkrtz(w[0], w[1]);
  const uint32_t h23 = pkrtz(w[2], w[3]);
  const uint32_t l01 = pkrtz(w[0] - f16lo(h01), w[1] - f16hi(h01));
  const uint32_t l23 = pkrtz(w[2] - f16lo(h23), w[3] - f16hi(h23));
  const u32x4 u = {h01, h23, l01, l23};
  return __builtin_bit_cast(half8, u);
}

// B operand for the hi/lo PV MFMA: the 4 value entries twice.
__device__ __forceinline__ half8 dup4(short4v v) {
  const u32x2 u = __builtin_bit_cast(u32x2, v);
  const u32x4 d = {u[0], u[1], u[0], u[1]};
  return __builtin_bit_cast(half8, d);
}

__device__ __forceinline__ short4v read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
}

// ---- cross-lane helpers -----------------------------------------------------
// Reduce over the four lanes {c, c+16, c+32, c+48} (same column, four quads).
__device__ __forceinline__ float quad_max(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Power-of-two exponent E with max|q| * 2^E in [64, 128) (0 for a zero row).
__device__ __forceinline__ int q_shift(float amax) {
  return amax > 0.0f ? 6 - __builtin_amdgcn_frexp_expf(amax) + 1 : 0;
}

// Number of 16-token tiles in work item `it` and the page/tile of tile i.
struct TileRef {
  int page, sub, nvalid;
};
__device__ __forceinline__ int n_tiles(const WorkItem& it, int tpp) {
  return (it.npages - 1) * tpp + (it.last_ntok + 15) / 16;
}
__device__ __forceinline__ TileRef tile_ref(const WorkItem& it, int tpp, int i) {
  TileRef r;
  r.page = i / tpp;
  r.sub = i % tpp;
  const int ntok = (r.page == it.npages - 1) ? it.last_ntok : tpp * 16;
  r.nvalid = min(16, ntok - 16 * r.sub);
  return r;
}

// Per-wave softmax state of the 16 head columns (lane (col, quad) holds the
// state of column col for its 4 tokens of each tile).
struct SoftState {
  float m = -INFINITY;   // reference max of column col (same in the 4 quads)
  float l = 0.0f;        // this lane's share of the denominator
};

// LDS image used after the tile loop to merge the four waves' states of the
// 16 head columns before one partial state per query head is written.
template <int D>
struct MergeLds {
  float m[kWaves][16];
  float l[kWaves][16];
  float acc[kWaves][16][D + 1];
};

}  // namespace

// ---------------------------------------------------------------------------
// TQ3 partial kernel
// ---------------------------------------------------------------------------
template <int NG>
__global__ void __launch_bounds__(kThreads) partial_tq3_mfma(DecodeArgs a) {
  constexpr int D = 32 * NG;
  constexpr int GPL = NG > 4 ? NG / 4 : 1;      // groups each lane loads
  constexpr int NT = D / 16;                    // PV N-tiles
  constexpr int VROW = 2 * D + 16;              // LDS value-tile row stride (bytes)
  constexpr int KST = 4 * NG;                   // dwords per token in the key staging
  struct WaveLds {
    uint32_t kst[16 * KST];                     // key units, [token][unit][group]
    uint8_t vt[16 * VROW];                      // value tile, [token][D] f16
    float corr[16];
  };
  union Lds {
    WaveLds w[kWaves];
    MergeLds<D> mg;
  };
  __shared__ Lds lds;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;                    // token (loads) / head column (outputs)
  const int quad = lane >> 4;
  const WorkItem it = a.items[blockIdx.x];
  const int hk = blockIdx.y;
  const PoolView& pv = a.pv;
  const int G = a.Hq / pv.Hkv;
  const int tpp = pv.P / 16;
  WaveLds& W = lds.w[wave];

  // ---- query operand: column col = query head hk*G + col (zero if col >= G)
  half8 qop[NG];
  float F;                                      // score multiplier of this column
  {
    const bool live = col < G;
    const uint16_t* qrow = a.q + (int64_t(it.b) * a.Hq + int64_t(hk) * G + col) * D;
    float qv[NG][8];
    float amax = 0.0f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (live) raw = *reinterpret_cast<const u32x4*>(qrow + 32 * g + 8 * quad);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w = raw[i >> 1];
        qv[g][i] = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
        amax = fmaxf(amax, fabsf(qv[g][i]));
      }
    }
    amax = quad_max(amax);
    const int E = q_shift(amax);
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int s = 0; s < 8; ++s)
        qop[g][s] = _Float16(__builtin_amdgcn_ldexpf(qv[g][kSlotCode[s]], E + 7 - kSlotShift[s]));
    F = a.scale * kLog2e * __builtin_amdgcn_ldexpf(1.0f, 3 - E);
  }
  // bias_g = -3.5 * 2^(E-3) * sum_{j in g} q_j, from an MFMA against all-ones codes
  f32x4 bias[NG];
  {
    const half8 ones = __builtin_bit_cast(half8, tq3_unit_to_f16(0x00249249u));
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
      f32x4 s = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, qop[g], z, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[g][i] = -3.5f * s[i];
    }
  }

  f32x4 acc[NT];
  f32x4 zacc[NG];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int g = 0; g < NG; ++g) zacc[g] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  SoftState st;
  const half8 ones8 = {_Float16(1.0f), _Float16(1.0f), _Float16(1.0f), _Float16(1.0f),
                       _Float16(1.0f), _Float16(1.0f), _Float16(1.0f), _Float16(1.0f)};

  const int ntiles = n_tiles(it, tpp);
  const int32_t* pt_row = pv.pt + int64_t(it.seq) * pv.pt_stride;
  const int64_t kc_off = tq3_codes_off(pv, hk, 0), vc_off = tq3_codes_off(pv, hk, 1);
  const int64_t ks_off = tq3_scale_off(pv, hk, 0), vs_off = tq3_scale_off(pv, hk, 1);
  constexpr int ROWB = 3 * D / 8;

  for (int ti = wave; ti < ntiles; ti += kWaves) {
    const TileRef tr = tile_ref(it, tpp, ti);
    const uint8_t* page = page_address(pv, pt_row[a.pages[it.list_off + tr.page]]);
    const int t0 = 16 * tr.sub;
    // ---- loads: codes of group(s) quad(+4i) of token col; scales of tokens 4quad..+3
    uint32_t kc[GPL][3], vc[GPL][3];
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int g = quad + 4 * i;
      if (g < NG) {
        const uint32_t* kp = reinterpret_cast<const uint32_t*>(page + kc_off + (t0 + col) * ROWB + 12 * g);
        const uint32_t* vp = reinterpret_cast<const uint32_t*>(page + vc_off + (t0 + col) * ROWB + 12 * g);
        kc[i][0] = kp[0]; kc[i][1] = kp[1]; kc[i][2] = kp[2];
        vc[i][0] = vp[0]; vc[i][1] = vp[1]; vc[i][2] = vp[2];
      }
    }
    // scales of tokens 4quad..4quad+3, all groups: 8*NG contiguous bytes
    uint32_t skw[2 * NG], svw[2 * NG];
    {
      const uint32_t* ksp = reinterpret_cast<const uint32_t*>(page + ks_off + 2 * (t0 + 4 * quad) * NG);
      const uint32_t* vsp = reinterpret_cast<const uint32_t*>(page + vs_off + 2 * (t0 + 4 * quad) * NG);
#pragma unroll
      for (int i = 0; i < 2 * NG; ++i) {
        skw[i] = ksp[i];
        svw[i] = vsp[i];
      }
    }
    auto scale_of = [](const uint32_t* w, int i, int g) {
      const int e = i * NG + g;
      return f16_bits_to_f32(uint16_t(w[e >> 1] >> (16 * (e & 1))));
    };
    // ---- keys: stage units as [token][unit][group], read back [token][quad][*]
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int g = quad + 4 * i;
      if (g < NG) {
        uint32_t u[4];
        tq3_split_units(kc[i][0], kc[i][1], kc[i][2], u);
#pragma unroll
        for (int un = 0; un < 4; ++un) W.kst[col * KST + un * NG + g] = u[un];
      }
    }
    // ---- values: unpack to f16 rows of the LDS tile
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
      const int g = quad + 4 * i;
      if (g < NG) {
        uint32_t u[4];
        tq3_split_units(vc[i][0], vc[i][1], vc[i][2], u);
#pragma unroll
        for (int un = 0; un < 4; ++un)
          *reinterpret_cast<u32x4*>(W.vt + col * VROW + 2 * (32 * g + 8 * un)) = tq3_unit_to_f16(u[un]);
      }
    }
    __builtin_amdgcn_wave_barrier();
    // ---- QK^T per group, scaled by the per-token group scale
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const uint32_t unit = W.kst[col * KST + quad * NG + g];
      const half8 kop = __builtin_bit_cast(half8, tq3_unit_to_f16(unit));
      const f32x4 dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[g], bias[g], 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] += dg[i] * scale_of(skw, i, g);
    }
    // ---- softmax bookkeeping (column col, tokens 4quad..4quad+3)
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = (4 * quad + i < tr.nvalid) ? s[i] * F : -INFINITY;
      tmax = fmaxf(tmax, s[i]);
    }
    tmax = quad_max(tmax);
    if (__any(tmax > st.m)) {
      const float m_new = tmax > st.m ? tmax + kHeadroom : st.m;
      const float corr = exp2f(st.m - m_new);          // 0 on the first tile
      st.m = m_new;
      st.l *= corr;
      if (quad == 0) W.corr[col] = corr;
      __builtin_amdgcn_wave_barrier();
      // accumulator rows are heads 4quad..4quad+3
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = W.corr[4 * quad + i];
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j][i] *= c;
#pragma unroll
        for (int g = 0; g < NG; ++g) zacc[g][i] *= c;
      }
      __builtin_amdgcn_wave_barrier();
    }
    float p[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[i] = exp2f(s[i] - st.m);
      st.l += p[i];
    }
    // ---- P' = p * value scale (hi/lo f16), Z += P' * 1, acc += P' * V
    half8 pp[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        w[i] = (4 * quad + i < tr.nvalid) ? p[i] * scale_of(svw, i, g) : 0.0f;
      pp[g] = split_hi_lo(w);
      zacc[g] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pp[g], ones8, zacc[g], 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int row = 4 * quad + (col >> 2);
      const int colb = 2 * (16 * j + 4 * (col & 3));
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pp[j >> 1], dup4(read_tr(W.vt + row * VROW + colb)),
                                                       acc[j], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  // ---- per-wave finalisation: l per column, acc in true units
  const float lcol = quad_sum(st.l);
  __syncthreads();                               // tile buffers are reused below
  MergeLds<D>& M = lds.mg;
  if (quad == 0) {
    M.m[wave][col] = st.m;
    M.l[wave][col] = lcol;
  }
  // acc[j][i] holds head 4quad+i, value-tile column p = 16j+col
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int p = 16 * j + col;
    const int slot = p & 7;
    const int dim = (p & ~7) + kSlotCode[slot];
    const float up = __builtin_amdgcn_ldexpf(1.0f, 10 - kSlotShift[slot]);
#pragma unroll
    for (int i = 0; i < 4; ++i) M.acc[wave][4 * quad + i][dim] = acc[j][i] * up - 3.5f * zacc[j >> 1][i];
  }
  __syncthreads();
  // ---- merge the four waves and write the partial state
  const int64_t base = int64_t(it.chunk) * a.Hq + int64_t(hk) * G;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, dim = idx % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (M.l[w][h] > 0.0f) mx = fmaxf(mx, M.m[w][h]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if (!(M.l[w][h] > 0.0f)) continue;
      const float f = exp2f(M.m[w][h] - mx);
      lsum += M.l[w][h] * f;
      o += M.acc[w][h][dim] * f;
    }
    a.pacc[(base + h) * D + dim] = o;
    if (dim == 0) {
      a.pm[base + h] = mx;
      a.pl[base + h] = lsum;
    }
  }
}

// ---------------------------------------------------------------------------
// FP8 partial kernel
// ---------------------------------------------------------------------------
template <int NG>
__global__ void __launch_bounds__(kThreads) partial_fp8_mfma(DecodeArgs a) {
  constexpr int D = 32 * NG;
  constexpr int NT = D / 16;
  constexpr int VROW = 2 * D + 16;
  constexpr int LB = D / 4;                     // bytes of a row each lane loads
  struct WaveLds {
    uint8_t vt[16 * VROW];
    float corr[16];
  };
  union Lds {
    WaveLds w[kWaves];
    MergeLds<D> mg;
  };
  __shared__ Lds lds;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int quad = lane >> 4;
  const WorkItem it = a.items[blockIdx.x];
  const int hk = blockIdx.y;
  const PoolView& pv = a.pv;
  const int G = a.Hq / pv.Hkv;
  const int tpp = pv.P / 16;
  WaveLds& W = lds.w[wave];

  // ---- query operand: MFMA r, lane (col, quad), slot s <-> dim quad*LB + 8r + s
  half8 qop[NG];
  float F;
  {
    const bool live = col < G;
    const uint16_t* qrow = a.q + (int64_t(it.b) * a.Hq + int64_t(hk) * G + col) * D;
    float qv[NG][8];
    float amax = 0.0f;
#pragma unroll
    for (int r = 0; r < NG; ++r) {
      u32x4 raw = {0u, 0u, 0u, 0u};
      if (live) raw = *reinterpret_cast<const u32x4*>(qrow + quad * LB + 8 * r);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t w = raw[i >> 1];
        qv[r][i] = __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
        amax = fmaxf(amax, fabsf(qv[r][i]));
      }
    }
    amax = quad_max(amax);
    const int E = q_shift(amax);
#pragma unroll
    for (int r = 0; r < NG; ++r)
#pragma unroll
      for (int s = 0; s < 8; ++s) qop[r][s] = _Float16(__builtin_amdgcn_ldexpf(qv[r][s], E));
    F = a.scale * kLog2e * __builtin_amdgcn_ldexpf(1.0f, -E);
  }

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  SoftState st;

  const int ntiles = n_tiles(it, tpp);
  const int32_t* pt_row = pv.pt + int64_t(it.seq) * pv.pt_stride;
  const int64_t kc_off = fp8_codes_off(pv, hk, 0), vc_off = fp8_codes_off(pv, hk, 1);
  const int64_t ks_off = fp8_scale_off(pv, hk, 0), vs_off = fp8_scale_off(pv, hk, 1);

  for (int ti = wave; ti < ntiles; ti += kWaves) {
    const TileRef tr = tile_ref(it, tpp, ti);
    const uint8_t* page = page_address(pv, pt_row[a.pages[it.list_off + tr.page]]);
    const int t0 = 16 * tr.sub;
    const float sigk = *reinterpret_cast<const float*>(page + ks_off);
    const float sigv = *reinterpret_cast<const float*>(page + vs_off);
    uint32_t kw[LB / 4], vw[LB / 4];
    {
      const uint32_t* kp = reinterpret_cast<const uint32_t*>(page + kc_off + (t0 + col) * D + quad * LB);
      const uint32_t* vp = reinterpret_cast<const uint32_t*>(page + vc_off + (t0 + col) * D + quad * LB);
#pragma unroll
      for (int i = 0; i < LB / 4; ++i) {
        kw[i] = kp[i];
        vw[i] = vp[i];
      }
    }
    // ---- values: f16 rows of the LDS tile (rows past the valid tokens zeroed)
    const bool vrow_ok = col < tr.nvalid;
#pragma unroll
    for (int i = 0; i < LB / 4; i += 2) {
      const u32x2 a0 = fp8x4_to_f16(vw[i]);
      const u32x2 a1 = fp8x4_to_f16(vw[i + 1]);
      u32x4 o = {a0[0], a0[1], a1[0], a1[1]};
      if (!vrow_ok) o = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<u32x4*>(W.vt + col * VROW + 2 * (quad * LB + 4 * i)) = o;
    }
    __builtin_amdgcn_wave_barrier();
    // ---- QK^T over all dims
    f32x4 dsum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int r = 0; r < NG; ++r) {
      const u32x2 k0 = fp8x4_to_f16(kw[2 * r]);
      const u32x2 k1 = fp8x4_to_f16(kw[2 * r + 1]);
      const u32x4 ku = {k0[0], k0[1], k1[0], k1[1]};
      dsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ku), qop[r], dsum, 0, 0, 0);
    }
    const float fk = F * sigk;
    float s[4];
    float tmax = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      s[i] = (4 * quad + i < tr.nvalid) ? dsum[i] * fk : -INFINITY;
      tmax = fmaxf(tmax, s[i]);
    }
    tmax = quad_max(tmax);
    if (__any(tmax > st.m)) {
      const float m_new = tmax > st.m ? tmax + kHeadroom : st.m;
      const float corr = exp2f(st.m - m_new);
      st.m = m_new;
      st.l *= corr;
      if (quad == 0) W.corr[col] = corr;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float c = W.corr[4 * quad + i];
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j][i] *= c;
      }
      __builtin_amdgcn_wave_barrier();
    }
    float w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = exp2f(s[i] - st.m);
      st.l += p;
      w[i] = (4 * quad + i < tr.nvalid) ? p * sigv : 0.0f;
    }
    const half8 pp = split_hi_lo(w);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      const int row = 4 * quad + (col >> 2);
      const int colb = 2 * (16 * j + 4 * (col & 3));
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pp, dup4(read_tr(W.vt + row * VROW + colb)),
                                                       acc[j], 0, 0, 0);
    }
    __builtin_amdgcn_wave_barrier();
  }

  const float lcol = quad_sum(st.l);
  __syncthreads();
  MergeLds<D>& M = lds.mg;
  if (quad == 0) {
    M.m[wave][col] = st.m;
    M.l[wave][col] = lcol;
  }
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) M.acc[wave][4 * quad + i][16 * j + col] = acc[j][i];
  __syncthreads();
  const int64_t base = int64_t(it.chunk) * a.Hq + int64_t(hk) * G;
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, dim = idx % D;
    float mx = -INFINITY;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2)
      if (M.l[w2][h] > 0.0f) mx = fmaxf(mx, M.m[w2][h]);
    float lsum = 0.0f, o = 0.0f;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
      if (!(M.l[w2][h] > 0.0f)) continue;
      const float f = exp2f(M.m[w2][h] - mx);
      lsum += M.l[w2][h] * f;
      o += M.acc[w2][h][dim] * f;
    }
    a.pacc[(base + h) * D + dim] = o;
    if (dim == 0) {
      a.pm[base + h] = mx;
      a.pl[base + h] = lsum;
    }
  }
}

hipError_t launch_partial_tq3(const DecodeArgs& a, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid(unsigned(a.n_items), unsigned(a.pv.Hkv));
  switch (a.pv.d) {
    case 32: hipLaunchKernelGGL(partial_tq3_mfma<1>, grid, dim3(kThreads), 0, s, a); break;
    case 64: hipLaunchKernelGGL(partial_tq3_mfma<2>, grid, dim3(kThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL(partial_tq3_mfma<4>, grid, dim3(kThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL(partial_tq3_mfma<8>, grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_partial_fp8(const DecodeArgs& a, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  const dim3 grid(unsigned(a.n_items), unsigned(a.pv.Hkv));
  switch (a.pv.d) {
    case 32: hipLaunchKernelGGL(partial_fp8_mfma<1>, grid, dim3(kThreads), 0, s, a); break;
    case 64: hipLaunchKernelGGL(partial_fp8_mfma<2>, grid, dim3(kThreads), 0, s, a); break;
    case 128: hipLaunchKernelGGL(partial_fp8_mfma<4>, grid, dim3(kThreads), 0, s, a); break;
    case 256: hipLaunchKernelGGL(partial_fp8_mfma<8>, grid, dim3(kThreads), 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace mkv
