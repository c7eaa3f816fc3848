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
// Work decomposition.  One launch covers both formats: one workgroup (4
// wave64) per (work item = chunk of at most 240 pages of one format of one
// sequence, block of NH kv-heads).  Each wave walks its quarter of the
// chunk's 16-token tiles for the NH kv-heads (its pages' page-table entries
// held one per lane, or staged in LDS for the workgroup), with the next tiles'
// bytes in flight: copied by 16-byte loads straight into a ring of LDS
// half-slots in the mixed kernel, held in registers in the BF16 control
// kernel.  The four waves' softmax states are combined through LDS and one
// partial state per query head is written.
//
// Tile computation (16 tokens x up to 16 query-head columns; column c is
// query head hk*G + c of kv-head hk, columns c >= G are zero):
//  * QK^T on MFMA 16x16x32 f16: A = the key tile (tokens x 32 dims), B = the
//    query columns, D[t][c].  TQ3 scales each 32-dim group
//    by its per-token fp16 scale before summing the groups; FP8 applies its
//    per-page scale once.
//  * Softmax: a reference maximum per column, raised (with headroom) only when
//    a tile exceeds it, so exp2 arguments stay <= 0 and rescaling the
//    accumulator is rare.
//  * PV on MFMA 16x16x32 f16.  P' (probabilities times the value scale) is
//    split into an f16 high part and an f16 low part (about 22 significant
//    bits together); A holds both parts of the lane's 4 tokens, exactly in
//    the lane layout QK^T produced, and B holds the value tile (read from LDS
//    with ds_read_b64_tr_b16) twice, so one MFMA adds hi*V + lo*V.  A single
//    f16 rounding of P' costs up to 2^-12 * |v| per weight, too much for
//    values with outlier channels.
//
// Operand encodings (all exact):
//  * TQ3: a 3-bit code c is masked into bits k..k+2 of an f16 whose other
//    bits are zero, the number c * 2^(k-24) (see the TQ3 operand section
//    below); the centring (c - 3.5) is applied outside the MFMA.  Any bit
//    pattern, including unwritten poisoned slots, gives a finite operand.
//  * FP8 E4M3 codes are widened by the hardware conversion to fp32 and packed
//    to f16 (every E4M3 value is an f16 normal number).  Value rows past the
//    valid tokens are zeroed because a poisoned byte may decode to NaN.
//  * Queries are bf16; per head they are scaled by a power of two so the
//    largest magnitude is in [64, 128) and, for TQ3, by 2^(7-k) to cancel each
//    slot's mantissa position k.  The compensating factors are folded into
//    the score scale.
#include <hip/hip_runtime.h>

#include <cstdlib>

#include "mkv_device.hpp"

namespace mkv {

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWaves = kWavesPerWorkgroup;
constexpr int kThreads = 64 * kWaves;
constexpr float kHeadroom = 2.0f;   // log2 units added when the reference max is raised
constexpr float kLog2e = 1.4426950408889634f;

// ---- small ALU helpers -------------------------------------------------------
// (x & m) | b in one instruction; m lives in an SGPR and b in a VGPR (a VOP3
// encoding on this architecture takes neither literals nor two scalars).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t b) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(m), "v"(b));
  return r;
}

// A VGPR holding zero, opaque to the compiler.
__device__ __forceinline__ uint32_t vgpr_opaque_zero() {
  uint32_t r;
  asm volatile("v_mov_b32 %0, 0" : "=v"(r));
  return r;
}

// Per-half unsigned 16-bit maximum.
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
  uint32_t r;
  asm("v_pk_max_u16 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Half h (0 low, 1 high) of an f16 pair as fp32.
__device__ __forceinline__ float f16_half(uint32_t w, int h) {
  return float(__builtin_bit_cast(_Float16, uint16_t(w >> (16 * h))));
}

// ---- TQ3 codes as f16 MFMA operands -------------------------------------------
// A 3-bit code c placed at bits k .. k+2 (k <= 8) of an f16 half whose other
// bits are zero is the number c * 2^(k-24): for k <= 7 a subnormal, for
// k = 8 the code's top bit is the exponent's lowest bit, and the encodings
// with exponent field 1 continue the subnormal grid (value = bits * 2^-24).
// The MFMA multiplies such inputs exactly, so one AND of a 32-bit window of a
// code stream with a mask yields two codes as operands, each carrying a power
// of two that the other operand (or the result) takes back.  The centring
// (c - 3.5) is applied outside the MFMA: for keys through the accumulator's
// initial value, for values through the probability mass of the tile.
//
// Precision: the f16 MFMA sums its products in a fixed-width window placed
// by the operands' exponent fields, and these operands all read as exponent
// -14, whatever c and k.  A product c * 2^(k-24) * b thus counts as large as
// 2^-14 * b, and the sum's rounding grain follows the largest such nominal
// product: about 2^(10-k) / c times coarser than for normal operands of the
// same values.  (Measured on 16x16x32 tiles with C = 0 and slots down to
// k = 0: errors near 2^-24 absolute on sums near 2^-5.)  The codes are
// therefore placed as high in the half as the bit stream allows.
//
// Key operands.  Quad q of the MFMA's A operand takes codes 8q .. 8q+7 of the
// group (bits 24q .. 24q+23 of its 96-bit stream).  Window W starts at bit
// 24q - 8, so code e sits at bits 8 + 3e of W; dword j of the operand is
// (W >> 3j) & kKeyMask, which keeps code j at k = 8 in the low half and code
// j + 4 at k = 4 in the high half.  The 8 k-slots of the lane hold
//   slot:        0   1   2   3   4   5   6   7
//   code 8q + :  0   4   1   5   2   6   3   7     (kSlotCode)
//   bit pos k:   8   4   8   4   8   4   8   4     (kSlotShift)
// (No cover of the 8 codes by 4 dwords keeps every k above 4: a dword's two
// codes sit 16 + k_hi - k_lo bits apart, a multiple of 3, so with all k >= 3
// they are 4, 5 or 6 codes apart; codes 3 and 4 then pair only as (3, 7) and
// (0, 4), the rest as (1, 5) and (2, 6), and distance 4 means k_hi = k_lo - 4
// <= 4.)  W is the funnel shift by 24 - 8q of
// the dwords q - 1 and q of the group (for quad 0 the dword before the group:
// its bits land only where the mask clears them).
constexpr int kSlotCode[8] = {0, 4, 1, 5, 2, 6, 3, 7};
constexpr int kSlotShift[8] = {8, 4, 8, 4, 8, 4, 8, 4};
constexpr uint32_t kKeyMask = (7u << 8) | (7u << 20);    // codes at k = 8 (low), 4 (high)
// Checks the table against the windows: W starts 8 bits before the quad's
// first code; dword j is W shifted right by 3j.
constexpr bool key_slot_ok(int slot) {
  const int code = kSlotCode[slot], k = kSlotShift[slot];
  const int j = slot >> 1, half = slot & 1;
  const int pos = 3 * code + 8 - 3 * j;                    // code position in W >> 3j
  return pos == 16 * half + k && ((kKeyMask >> pos) & 7u) == 7u && pos + 2 <= 31 - 3 * j && k >= 0 &&
         k <= 8;
}
static_assert(key_slot_ok(0) && key_slot_ok(1) && key_slot_ok(2) && key_slot_ok(3) && key_slot_ok(4) &&
                  key_slot_ok(5) && key_slot_ok(6) && key_slot_ok(7),
              "key operand slots");

// Operand of one key unit from dwords q - 1 and q of the group (see above).
__device__ __forceinline__ u32x4 tq3_key_operand(uint32_t lo, uint32_t hi, uint32_t s1) {
  const uint32_t w = __builtin_amdgcn_alignbit(hi, lo, s1);
  return u32x4{w & kKeyMask, (w >> 3) & kKeyMask, (w >> 6) & kKeyMask, (w >> 9) & kKeyMask};
}

// ---- TQ3 value group unpack ------------------------------------------------
// A group is 32 codes held as three little-endian dwords, code i at bits
// 3i .. 3i+2.  Read as a ring of 96 bits, any 32-bit window starting at bit b
// is one funnel shift of two of the dwords (no shift for b = 0, 32, 64).  One
// AND of a window keeps two codes, code lo at bits k_lo .. k_lo+2 of the low
// half and code hi at bits 16+k_hi .. 18+k_hi, the numbers c * 2^(k-24)
// (k <= 8, see the operand section above).  The sixteen pairs below,
// (window start, lo, hi), put every code at k >= 4, which bounds the MFMA's
// rounding grain for these operands to 2^6 times that of normal operands
// (as for the keys).  They take eight shifted windows; an exact-cover search
// over all window starts finds none with fewer at k >= 4 (k >= 3 takes six,
// any k three).  The bit offsets follow from the table.  (Value tiles are
// unpacked once per tile by the lane that loads the group, so the whole group
// is at hand.)
struct Tq3Pair {
  int win, lo, hi;
};
constexpr Tq3Pair kValuePairs[16] = {
    {0, 2, 8},    {13, 6, 11},  {13, 7, 12},  {22, 9, 14},  {22, 10, 15}, {32, 13, 18},
    {43, 16, 21}, {43, 17, 22}, {51, 19, 25}, {54, 20, 26}, {64, 23, 28}, {64, 24, 29},
    {75, 27, 1},  {82, 30, 3},  {88, 0, 5},   {88, 31, 4}};
constexpr int kValueMinK = 4;
constexpr int kappa_lo(const Tq3Pair& p) { return (3 * p.lo - p.win + 96) % 96; }
constexpr int kappa_hi(const Tq3Pair& p) { return (3 * p.hi - p.win + 96) % 96 - 16; }
constexpr uint32_t pair_mask(const Tq3Pair& p) {
  return (7u << kappa_lo(p)) | (7u << (16 + kappa_hi(p)));
}
constexpr bool is_cover(const Tq3Pair (&t)[16]) {
  uint32_t seen = 0;
  for (const Tq3Pair& p : t) {
    const int a = kappa_lo(p), b = kappa_hi(p);
    if (a < kValueMinK || a > 8 || b < kValueMinK || b > 8 || p.win < 0 || p.win >= 96) return false;
    const uint32_t bits = (1u << p.lo) | (1u << p.hi);
    if ((seen & bits) != 0 || p.lo == p.hi) return false;
    seen |= bits;
  }
  return seen == 0xFFFFFFFFu;
}
static_assert(is_cover(kValuePairs), "TQ3 value pair cover");

// Value position 2p + h (half h of pair p) as a byte (dim-in-group |
// (8 - k) << 5), 8 per 64-bit word, for run-time lookups.
constexpr uint64_t value_pos_word(int w) {
  uint64_t r = 0;
  for (int i = 0; i < 8; ++i) {
    const int pos = 8 * w + i;
    const Tq3Pair& p = kValuePairs[pos / 2];
    const int e = (pos & 1) ? (p.hi | ((8 - kappa_hi(p)) << 5)) : (p.lo | ((8 - kappa_lo(p)) << 5));
    r |= uint64_t(e) << (8 * i);
  }
  return r;
}
constexpr uint64_t kValuePos[4] = {value_pos_word(0), value_pos_word(1), value_pos_word(2),
                                   value_pos_word(3)};

// 32-bit window of a group starting at ring bit b (a constant after unrolling).
__device__ __forceinline__ uint32_t group_window(const uint32_t (&w)[3], int b) {
  const uint32_t lo = w[b >> 5], hi = w[((b >> 5) + 1) % 3];
  return (b & 31) == 0 ? lo : __builtin_amdgcn_alignbit(hi, lo, b & 31);
}

// Value group -> 16 dwords of f16 pairs c * 2^(k-24), pair p in dword p.
__device__ __forceinline__ void tq3_value_group(const uint32_t (&w)[3], uint32_t (&o)[16]) {
#pragma unroll
  for (int p = 0; p < 16; ++p) o[p] = group_window(w, kValuePairs[p].win) & pair_mask(kValuePairs[p]);
}

// ---- FP8 -> f16 -------------------------------------------------------------
__device__ __forceinline__ uint32_t pkrtz(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}

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

// ---- P' hi/lo ----------------------------------------------------------------
// The PV MFMA 16x16x32 A operand of the lane's 4 tokens: k-slots 0..3 hold
// hi = f16(p*s), k-slots 4..7 lo = f16(p*s - hi), each one fused multiply-
// add of fp32 p and the scale rounded to f16 (the compiler emits
// v_fma_mix{lo,hi}_f16), so hi + lo carries p*s to about 22 bits.  The B
// operand holds the lane's 4 value entries in both halves, so one MFMA adds
// hi*V + lo*V (products exact in fp32).
__device__ __forceinline__ half8 pprime(const float p[4], const float sv[4]) {
  half8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const _Float16 h = _Float16(__builtin_fmaf(p[i], sv[i], 0.0f));
    r[i] = h;
    r[4 + i] = _Float16(__builtin_fmaf(p[i], sv[i], -float(h)));
  }
  return r;
}

// The same from f16 scales held in halves of dwords, written as explicit
// mixed-precision FMAs (the compiler widens the scales first otherwise):
// pair word of f16(p_a * s_a) | f16(p_b * s_b) << 16, s_a half HA of wa,
// s_b half HB of wb; and the pair word of the remainders f16(p * s - hi).
#define MKV_MIX_HI(HA, HB)                                                              \
  "v_fma_mixlo_f16 %0, %1, %2, 0 op_sel:[0," #HA ",0] op_sel_hi:[0,1,0]\n\t"            \
  "v_fma_mixhi_f16 %0, %3, %4, 0 op_sel:[0," #HB ",0] op_sel_hi:[0,1,0]"
#define MKV_MIX_LO(HA, HB)                                                              \
  "v_fma_mixlo_f16 %0, %1, %2, -%5 op_sel:[0," #HA ",0] op_sel_hi:[0,1,1]\n\t"                \
  "v_fma_mixhi_f16 %0, %3, %4, -%5 op_sel:[0," #HB ",1] op_sel_hi:[0,1,1]"
template <int HA, int HB>
__device__ __forceinline__ uint32_t mix_hi(float pa, uint32_t wa, float pb, uint32_t wb) {
  uint32_t d;
  if constexpr (HA == 0 && HB == 0) asm(MKV_MIX_HI(0, 0) : "=&v"(d) : "v"(pa), "v"(wa), "v"(pb), "v"(wb));
  else if constexpr (HA == 0 && HB == 1) asm(MKV_MIX_HI(0, 1) : "=&v"(d) : "v"(pa), "v"(wa), "v"(pb), "v"(wb));
  else if constexpr (HA == 1 && HB == 0) asm(MKV_MIX_HI(1, 0) : "=&v"(d) : "v"(pa), "v"(wa), "v"(pb), "v"(wb));
  else asm(MKV_MIX_HI(1, 1) : "=&v"(d) : "v"(pa), "v"(wa), "v"(pb), "v"(wb));
  return d;
}
template <int HA, int HB>
__device__ __forceinline__ uint32_t mix_lo(float pa, uint32_t wa, float pb, uint32_t wb, uint32_t hi) {
  uint32_t d;
  if constexpr (HA == 0 && HB == 0) asm(MKV_MIX_LO(0, 0) : "=&v"(d) : "v"(pa), "v"(wa), "v"(pb), "v"(wb), "v"(hi));
  else if constexpr (HA == 0 && HB == 1) asm(MKV_MIX_LO(0, 1) : "=&v"(d) : "v"(pa), "v"(wa), "v"(pb), "v"(wb), "v"(hi));
  else if constexpr (HA == 1 && HB == 0) asm(MKV_MIX_LO(1, 0) : "=&v"(d) : "v"(pa), "v"(wa), "v"(pb), "v"(wb), "v"(hi));
  else asm(MKV_MIX_LO(1, 1) : "=&v"(d) : "v"(pa), "v"(wa), "v"(pb), "v"(wb), "v"(hi));
  return d;
}
#undef MKV_MIX_HI
#undef MKV_MIX_LO
// p * (f16 half H of w) + c in fp32
template <int H>
__device__ __forceinline__ float fma_mix_f32(float p, uint32_t w, float c) {
  float r;
  if constexpr (H == 0) asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p), "v"(w), "v"(c));
  else asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[0,1,0] op_sel_hi:[0,1,0]" : "=v"(r) : "v"(p), "v"(w), "v"(c));
  return r;
}

// Value scales of pass ps for the lane's 4 tokens, from the slot's scale rows
// sp (token t: NG f16): NG >= 2: sw[i] = the scales of groups 2ps, 2ps + 1 of
// token i; NG = 1: sw[0], sw[1] = tokens (0, 1) and (2, 3).  (Rows past the
// valid tokens of a tile hold 0 by then: the tile loop clears them.)
template <int NG>
__device__ __forceinline__ void tq3_pass_scales(const uint32_t* sp, int ps, uint32_t (&sw)[4]) {
  if constexpr (NG >= 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sw[i] = sp[i * (NG / 2) + ps];
  } else {
    sw[0] = sp[0];
    sw[1] = sp[1];
    sw[2] = sw[3] = 0u;
  }
}

// P' of the lane's 4 tokens for group 2ps + H of a pass (scales as
// tq3_pass_scales gives them; NG = 1: H = 0).  hi = pair words of tokens
// (0, 1), (2, 3); lo = their remainders; mass += sum of p * s.
template <int NG, int H>
__device__ __forceinline__ void pprime_tq3(const float p[4], const uint32_t (&sw)[4], uint32_t (&hi)[2],
                                           uint32_t (&lo)[2], float& mass) {
  constexpr int HA = NG >= 2 ? H : 0, HB = NG >= 2 ? H : 1;
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t wa = NG >= 2 ? sw[2 * k] : sw[k], wb = NG >= 2 ? sw[2 * k + 1] : sw[k];
    hi[k] = mix_hi<HA, HB>(p[2 * k], wa, p[2 * k + 1], wb);
    lo[k] = mix_lo<HA, HB>(p[2 * k], wa, p[2 * k + 1], wb, hi[k]);
    mass = fma_mix_f32<HA>(p[2 * k], wa, mass);
    mass = fma_mix_f32<HB>(p[2 * k + 1], wb, mass);
  }
}

// FP8: one scale for all four tokens (page-head scale).
__device__ __forceinline__ half8 pprime_uniform(const float p[4], float s) {
  const float sv[4] = {s, s, s, s};
  return pprime(p, sv);
}

// acc += P' * V for one 16-dim N-tile.
__device__ __forceinline__ f32x4 pv_mfma(half8 pp, half8 v, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(pp, v, acc, 0, 0, 0);
}

__device__ __forceinline__ short4v read_tr(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4v*)(p));
}

// B operand of the PV MFMA: the value entries V[4quad + j][n] of the lane's
// column n, transposed out of the row-major LDS tile, in both halves (read
// twice, so the operand lands in place without register copies).  p2 is p
// plus a zero the compiler cannot see through, so the two reads are not
// merged and remain free to be scheduled early.
__device__ __forceinline__ half8 value_operand(const uint8_t* p, const uint8_t* p2) {
  const u32x2 a = __builtin_bit_cast(u32x2, read_tr(p));
  const u32x2 b = __builtin_bit_cast(u32x2, read_tr(p2));
  const u32x4 d = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(half8, d);
}

// Two kv-heads per wave: the PV MFMA's K dimension holds head 0's four tokens
// of the lane quad in k-slots 0..3 and head 1's in 4..7.  The B operand is
// V_0 | V_1 of the lane's column (one transposing read from each head's tile);
// the A operand carries the lane's P' (its column belongs to one head) in that
// head's slots and zeros in the other's, split into a hi and a lo MFMA.  Both
// heads then accumulate into one accumulator per N-tile, each output row
// receiving only its own head's values.
__device__ __forceinline__ void split_pprime(half8 pp, bool head1, half8& a_hi, half8& a_lo) {
  const u32x4 w = __builtin_bit_cast(u32x4, pp);     // hi 0-1, hi 2-3, lo 0-1, lo 2-3
  const u32x4 h = {head1 ? 0u : w[0], head1 ? 0u : w[1], head1 ? w[0] : 0u, head1 ? w[1] : 0u};
  const u32x4 l = {head1 ? 0u : w[2], head1 ? 0u : w[3], head1 ? w[2] : 0u, head1 ? w[3] : 0u};
  a_hi = __builtin_bit_cast(half8, h);
  a_lo = __builtin_bit_cast(half8, l);
}
__device__ __forceinline__ half8 value_operand_heads(const uint8_t* p0, const uint8_t* p1) {
  const u32x2 a = __builtin_bit_cast(u32x2, read_tr(p0));
  const u32x2 b = __builtin_bit_cast(u32x2, read_tr(p1));
  const u32x4 d = {a[0], a[1], b[0], b[1]};
  return __builtin_bit_cast(half8, d);
}

// ---- cross-lane helpers -----------------------------------------------------

// Orders one wave's LDS accesses around this point (writes before later reads
// of other lanes' data, reads before later overwrites).  The LDS executes one
// wave's operations in program order, so no hardware wait is needed: this is
// a compiler barrier only (a memory fence here would wait for every
// outstanding LDS operation).
__device__ __forceinline__ void wave_lds_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_wave_barrier();
}

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
  return amax > 0.0f ? 7 - __builtin_amdgcn_frexp_expf(amax) : 0;
}

// ---- tiles -------------------------------------------------------------------
// A work item's tiles: tile (page, sub) covers tokens 16*sub .. 16*sub+15 of
// the item's page `page` (pages hold P = 16 * tpp tokens); tiles are numbered
// page * tpp + sub.  The four waves of a workgroup take consecutive quarters
// of the item's tiles.  Cursors are wave-uniform and advance without division.
// (When the tiles do not divide by four the later quarters hold one more.
// Rotating which wave takes which quarter per workgroup measured about 1 us
// slower on the long-context launch.)
struct Cursor {
  int page = 0, sub = 0;
};
struct TileGeom {
  int tpp;          // tiles per page
  int item_last;    // the item's last page (npages - 1)
  int last_ntok;    // valid tokens of that page
  int stop_page;    // last tile of this wave's range
  int stop_sub;
  int ntiles;       // tiles in this wave's range (may be 0)
  Cursor first;     // first tile of the range
};
__device__ __forceinline__ TileGeom wave_tiles(const WorkItem& it, int tpp, int wave) {
  TileGeom g;
  g.tpp = tpp;
  g.item_last = it.npages - 1;
  g.last_ntok = it.last_ntok;
  const int total = g.item_last * tpp + (it.last_ntok + 15) / 16;
  const int t0 = (total * wave) / kWaves, t1 = (total * (wave + 1)) / kWaves;
  g.ntiles = t1 - t0;
  g.first.page = t0 / tpp;
  g.first.sub = t0 - g.first.page * tpp;
  const int tl = max(t1 - 1, t0);
  g.stop_page = tl / tpp;
  g.stop_sub = tl - g.stop_page * tpp;
  return g;
}
__device__ __forceinline__ void advance(Cursor& c, const TileGeom& g) {
  if (++c.sub == g.tpp) {
    c.sub = 0;
    ++c.page;
  }
}
// Prefetch cursor: stops on the range's last tile, so loads issued past the
// end re-read it (every wave issues the same number of loads per tile, which
// keeps the compiler's memory-counter waits exact).
__device__ __forceinline__ void advance_clamped(Cursor& c, const TileGeom& g) {
  if (c.page != g.stop_page || c.sub != g.stop_sub) advance(c, g);
}
__device__ __forceinline__ int valid_in_tile(const Cursor& c, const TileGeom& g) {
  return c.page == g.item_last ? min(16, g.last_ntok - 16 * c.sub) : 16;
}

// ---- record loads -------------------------------------------------------------
// A page record is read through a buffer resource: the record base sits in
// scalar registers, each lane adds a fixed 32-bit offset and the tile's
// position is a wave-uniform scalar offset, so a tile's loads need no per-lane
// address arithmetic.  Dword 3 selects 32-bit untyped data; the record size
// bounds the lane offsets (anything past it would read as zero).
constexpr int kRawBufferWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t record_rsrc(const uint8_t* rec, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(rec), 0, int(bytes), kRawBufferWord3);
}
__device__ __forceinline__ uint32_t rec_load1(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, int tile_off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, lane_off, tile_off, 0);
}
__device__ __forceinline__ u32x2 rec_load2(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, int tile_off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, lane_off, tile_off, 0);
}
__device__ __forceinline__ u32x3 rec_load3(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, int tile_off) {
  return __builtin_amdgcn_raw_buffer_load_b96(r, lane_off, tile_off, 0);
}
__device__ __forceinline__ u32x4 rec_load4(__amdgpu_buffer_rsrc_t r, uint32_t lane_off, int tile_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, lane_off, tile_off, 0);
}

// Page-table entries of a work item's pages (resolved by the host when it
// builds the schedule, which any page-table change invalidates), staged once
// per workgroup.
__device__ __forceinline__ void stage_entries(int32_t* ent, const DecodeArgs& a, const WorkItem& it) {
  for (int p = threadIdx.x; p < it.npages; p += kThreads) ent[p] = a.entries[it.list_off + p];
  __syncthreads();
}
__device__ __forceinline__ const uint8_t* entry_page(const PoolView& pv, const int32_t* ent, int page) {
  return page_address(pv, __builtin_amdgcn_readfirstlane(ent[page]));
}

// Issue priority from the share of the wave's tiles already done: 3 in the
// first quarter down to 0 in the last.  The two waves sharing a SIMD come from
// different workgroups, and among ready waves the hardware issues the older
// one first, so with equal priorities the workgroup dispatched first runs well
// ahead and the other one ends its range alone on the SIMD.  With these levels
// a wave that gets ahead yields to the one behind, and the pair ends closer
// together.  Only used when every workgroup of the launch is resident from the
// start (otherwise a newly started wave would hold back nearly finished ones).
__device__ __forceinline__ void pace_priority(int done, int total) {
  const int x = 4 * done;
  if (x < total) __builtin_amdgcn_s_setprio(3);
  else if (x < 2 * total) __builtin_amdgcn_s_setprio(2);
  else if (x < 3 * total) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// Runs the tile pipeline over the wave's range: R raw buffers in flight;
// prepare() runs once the first loads are issued; process(raw, cursor,
// refill) consumes one tile and calls refill(raw) to
// load a later one.  The steady-state loop issues the same loads on every
// path.  pace: set the wave's issue priority from its progress.
template <int R, typename Raw, typename Load, typename Prepare, typename Process>
__device__ __forceinline__ void run_tiles(const TileGeom& g, bool pace, Load load, Prepare prepare,
                                          Process process) {
  if (g.ntiles == 0) return;
  Raw ring[R];
  Cursor lc = g.first;
#pragma unroll
  for (int k = 0; k < R; ++k) {
    load(lc, ring[k]);
    advance_clamped(lc, g);
  }
  prepare();
  Cursor pc = g.first;
  int ti = 0;
  for (; ti + R <= g.ntiles; ti += R) {
    if (pace) pace_priority(ti, g.ntiles);
#pragma unroll
    for (int k = 0; k < R; ++k) {
      process(ring[k], pc, [&](Raw& r) {
        load(lc, r);
        advance_clamped(lc, g);
      });
      advance(pc, g);
    }
  }
  if (pace) __builtin_amdgcn_s_setprio(0);
#pragma unroll
  for (int k = 0; k < R - 1; ++k) {
    if (ti + k < g.ntiles) {
      process(ring[k], pc, [](Raw&) {});
      advance(pc, g);
    }
  }
}

// Per-wave softmax state of column col (lane (col, quad) holds the state of
// column col for its 4 tokens of each tile).
struct SoftState {
  float m = -INFINITY;   // reference max of column col (same in the 4 quads)
  float l = 0.0f;        // this lane's share of the denominator
};

// LDS image for combining the four waves' states of one work item: per wave
// the reference max and denominator of the 16 columns and the accumulator
// rows of the live columns in true units (row stride padded).
template <int D>
struct MergeLds {
  static constexpr int ROW = D + 4;
  float m[kWaves][16];
  float l[kWaves][16];
  float acc[kWaves][16 * ROW];
};

// Combine the waves' states in M and write the item's partial state of the
// ncol query heads starting at hq0 (all threads of the workgroup call this,
// with M.m, M.l and M.acc written and visible; nothing may follow it that
// needs every thread).  Thread (c, s) takes column c and the 16-byte slices
// of dims 4s + 64k: it forms the column's wave weights 2^(m_w - M) itself
// (the 16 threads of a column the same way), so the combine needs no further
// barrier, and its LDS reads and global stores are 16-byte vectors, eight
// consecutive lanes on consecutive slices.
template <int D>
__device__ __forceinline__ void merge_waves_and_store(MergeLds<D>& M, const DecodeArgs& a, int chunk,
                                                      int hq0, int ncol) {
  const int c = int(threadIdx.x) >> 4, s = int(threadIdx.x) & 15;
  if (c >= ncol) return;
  float mx = -INFINITY;
#pragma unroll
  for (int w = 0; w < kWaves; ++w)
    if (M.l[w][c] > 0.0f) mx = fmaxf(mx, M.m[w][c]);
  float f[kWaves];
  float lsum = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    f[w] = M.l[w][c] > 0.0f ? exp2f(M.m[w][c] - mx) : 0.0f;
    lsum += M.l[w][c] * f[w];
  }
  const int64_t row = int64_t(chunk) * a.Hq + hq0 + c;
  if (s == 0) {
    a.pm[row] = mx;
    a.pl[row] = lsum;
  }
  // (a wave without tiles has weight 0 and a zero accumulator, so every wave
  // enters the sum, in wave order)
  if constexpr (D >= 64) {
#pragma unroll
    for (int k = 0; k < D / 64; ++k) {
      const int dim = 4 * s + 64 * k;
      f32x4 o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&M.acc[w][c * MergeLds<D>::ROW + dim]);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = __builtin_fmaf(v[e], f[w], o[e]);
      }
      *reinterpret_cast<f32x4*>(a.pacc + row * D + dim) = o;
    }
  } else {
    const int dim = (D / 16) * s;
    f32x2 o = {0.0f, 0.0f};
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const f32x2 v = *reinterpret_cast<const f32x2*>(&M.acc[w][c * MergeLds<D>::ROW + dim]);
      o[0] = __builtin_fmaf(v[0], f[w], o[0]);
      o[1] = __builtin_fmaf(v[1], f[w], o[1]);
    }
    *reinterpret_cast<f32x2*>(a.pacc + row * D + dim) = o;
  }
}

template <int NACC>
__device__ __forceinline__ void softmax_step(SoftState& st, float s[4], float p[4],
                                             f32x4 (&acc)[NACC], float* corr_lds, int col, int quad) {
  float tmax = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
  tmax = quad_max(tmax);
  if (__any(tmax > st.m)) {
    const float m_new = tmax > st.m ? tmax + kHeadroom : st.m;
    const float corr = exp2f(st.m - m_new);   // 0 on the first tile
    st.m = m_new;
    st.l *= corr;
    if (quad == 0) corr_lds[col] = corr;
    wave_lds_sync();
    // accumulator rows are columns 4quad..4quad+3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float c = corr_lds[4 * quad + i];
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j][i] *= c;
    }
    wave_lds_sync();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = __builtin_amdgcn_exp2f(s[i] - st.m);
    st.l += p[i];
  }
}

// Query rows -> MFMA B operands, NH kv-heads per wave.  Column col is query
// head hq0 + col (live if col < NH * G) and belongs to kv-head jcol = col / G
// of the wave; qop[j] holds the column only for j == jcol (zero otherwise), so
// the MFMAs of the NH kv-heads accumulate into one D.  For MFMA g the lane's 8
// k-slots hold the head dims fetch(qrow, g, v) reads into v[0..7]; conv(x, E,
// s) turns value x of slot s into the operand, given the column's exponent E
// (max|q| * 2^E in [64, 128)).  qh[g] is the column's operand before the
// kv-head selection.  Returns E.
template <int NG, int NH, typename Fetch, typename Conv>
__device__ __forceinline__ int load_query(const DecodeArgs& a, int b, int hq0, int col, int ncol,
                                          int jcol, half8 (&qop)[NH][NG], half8 (&qh)[NG],
                                          Fetch fetch, Conv conv) {
  constexpr int D = 32 * NG;
  const bool live = col < ncol;
  const uint16_t* qrow = a.q + (int64_t(b) * a.Hq + hq0 + (live ? col : 0)) * D;
  float qv[NG][8];
  float amax = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    fetch(qrow, g, qv[g]);
#pragma unroll
    for (int s = 0; s < 8; ++s) {
      qv[g][s] = live ? qv[g][s] : 0.0f;
      amax = fmaxf(amax, fabsf(qv[g][s]));
    }
  }
  amax = quad_max(amax);
  const int E = q_shift(amax);
#pragma unroll
  for (int g = 0; g < NG; ++g) {
#pragma unroll
    for (int s = 0; s < 8; ++s) qh[g][s] = conv(qv[g][s], E, s);
    const u32x4 w = __builtin_bit_cast(u32x4, qh[g]);
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      u32x4 o;
#pragma unroll
      for (int x = 0; x < 4; ++x) o[x] = jcol == j ? w[x] : 0u;
      qop[j][g] = __builtin_bit_cast(half8, o);
    }
  }
  return E;
}

// Row stride (bytes) of an f16 value tile in LDS: the stride in dwords is
// 12 mod 64, so row r starts at bank 12r mod 64 and the 16 rows of a 16-byte
// row write hit distinct banks.
constexpr int value_row_bytes(int D) { return 2 * D + 4 * (((12 - D / 2) % 64 + 64) % 64); }
// LDS row of token t in a value tile: tokens 0..7 take the even rows and
// 8..15 the odd ones.  A transposing 8-byte read serves 32 lanes at a time,
// 8 rows (tokens 0..7 or 8..15) of 8 banks each; the even (odd) rows start
// 24 banks apart mod 64 and so cover all 64 banks once.
__device__ __forceinline__ int value_row(int t) { return t < 8 ? 2 * t : 2 * t - 15; }
static_assert(value_row_bytes(128) == 304 && value_row_bytes(64) % 16 == 0 &&
                  (value_row_bytes(32) / 4) % 64 == 12 && (value_row_bytes(256) / 4) % 64 == 12,
              "value row stride");

// The 2NG scale dwords of a lane's four tokens (16-byte reads; 8 bytes when
// NG = 1).
template <int NG>
__device__ __forceinline__ void load_scale_dwords(const uint32_t* p, uint32_t (&o)[2 * NG]) {
  if constexpr (NG == 1) {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    o[0] = w[0];
    o[1] = w[1];
  } else {
#pragma unroll
    for (int x = 0; x < NG / 2; ++x) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(p + 4 * x);
#pragma unroll
      for (int y = 0; y < 4; ++y) o[4 * x + y] = w[y];
    }
  }
}

// LDS images of the two work-item kinds (one of them per workgroup).
template <int NG, int NH>
struct Fp8Lds {
  static constexpr int D = 32 * NG;
  static constexpr int VROW = value_row_bytes(D);
  struct Wave {
    alignas(16) uint8_t vt[NH][16 * VROW];
    float corr[16];
  };
  int32_t ent[kMaxChunkPages];
  Wave w[kWaves];
};

// Accumulator of head j for output row i: acc[j * NT + jt][i]; rows of the
// other heads of the wave hold unused sums.
template <int NH, int NT>
__device__ __forceinline__ float pick_head(const f32x4 (&acc)[NH * NT], int jc, int jt, int i) {
  float v = acc[jt][i];
#pragma unroll
  for (int j = 1; j < NH; ++j) v = jc == j ? acc[j * NT + jt][i] : v;
  return v;
}

}  // namespace

namespace {

// ---------------------------------------------------------------------------
// Mixed FP8/TQ3 work items.
//
// One workgroup of four wave64 per (work item, block of NH kv-heads); each
// wave takes a contiguous quarter of the item's 16-token tiles.  A tile's
// bytes are copied from the page record into the wave's own LDS by 16-byte
// loads that write LDS directly (no register holds raw page bytes).  A tile
// travels as two halves, the key half (key codes and scales of its heads) and
// the value half, through a ring of three half-slots: while tile i is
// computed, the key half and then the value half of tile i + 1 are in flight
// (the key half of tile i + 1 is issued once tile i's values are consumed,
// its value half once tile i's keys are consumed).  An FP8 tile is processed
// as NH one-head tiles, whose key half fills one slot.
// ---------------------------------------------------------------------------
template <int NG, int NH>
struct Mix {
  static constexpr int D = 32 * NG;
  static constexpr int NT = D / 16;                     // PV N-tiles
  static constexpr int ROWB = 12 * NG;                  // TQ3 code bytes of a token row
  static constexpr int SCB = 2 * NG;                    // TQ3 scale bytes of a token
  static constexpr int THALF = 16 * (ROWB + SCB);       // TQ3 key (or value) half of one head
  static constexpr int FHALF = 16 * D;                  // FP8 key (or value) half of one head
  static constexpr int SLOT = NG == 8 ? 4096 : 2048;    // bytes of a half-slot
  static constexpr int NSLOT = 3;
  static constexpr int PASS = NG < 2 ? NG : 2;          // 32-dim groups per value pass
  static constexpr int NPASS = NG / PASS;
  static constexpr int VROWB = 64 * PASS;               // bytes of a value-tile row
  static constexpr int VBUF = NH * 16 * VROWB;          // value tile of the NH heads
  static constexpr int WAVE = NSLOT * SLOT + VBUF;      // LDS bytes of one wave
  static constexpr int CPH = (12 * NG + 63) / 64;      // code loads per head of a TQ3 half
  static constexpr int TNI = NH * (CPH + 1);            // load instructions of a TQ3 half
  static constexpr int SCOFF = NH * 16 * ROWB;          // scales of a TQ3 half-slot
  // TQ3 mode leaves the end of each half-slot unwritten: it holds the key
  // centring values of the wave's columns, 16 bytes (the value four times,
  // an MFMA accumulator's initial value as read) per column and group, KPS
  // groups per slot
  static constexpr int KIOFF = (NH * THALF + 15) / 16 * 16;
  static constexpr int KPS = (SLOT - KIOFF) / 256;
  static constexpr int kinit_off(int g) { return (g / KPS) * SLOT + KIOFF + (g % KPS) * 256; }
  // the workgroup's shared copies: centring values of group g in wave
  // g mod 4's half-slot tails; the query operands of (kv-head j, group g),
  // 1 KB each, in the value tiles (free until the tile loop)
  static __device__ uint8_t* kinit_addr(uint8_t* smem, int g) {
    return smem + (g % kWaves) * WAVE + VBUF + kinit_off(g / kWaves);
  }
  static constexpr int QPW = VBUF / 1024;               // operand blocks per value tile
  static __device__ uint8_t* qop_addr(uint8_t* smem, int j, int g) {
    const int k = j * NG + g;
    return smem + (k / QPW) * WAVE + (k % QPW) * 1024;
  }
  static_assert(2 * NG <= 64, "one scale load per head and half");
  static constexpr int FVEC = FHALF / 16;
  static constexpr int FNI = (FVEC + 63) / 64;
  static constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }
  static constexpr size_t SMEM = cmax(size_t(kWaves) * WAVE, sizeof(MergeLds<D>));
  static_assert(NH * THALF <= SLOT && FHALF <= SLOT, "a half-tile fits a slot");
  static_assert(KPS * NSLOT >= (NG + kWaves - 1) / kWaves, "key centring values fit the slots' tails");
  static_assert(QPW * kWaves >= NH * NG, "query operands fit the value tiles");
  static_assert(TNI <= 4 && FNI <= 4, "load instructions per half");
};

// Position of 32-byte segment `seg` of value-tile row r.  The transposing
// reads of a half-wave touch 8 rows at one segment; XOR-ing the segment index
// with bits of the row spreads those 8 reads over the banks.
template <int VROWB>
__device__ __forceinline__ int vseg(int r, int seg) {
  if constexpr (VROWB == 128) return seg ^ ((r >> 1) & 3);
  else return seg ^ ((r >> 2) & 1);
}
// Byte offset (0 or 16) of the first 16-byte half of a segment in value-tile
// row r.  16-byte writes are served 8 lanes at a time: with 128-byte rows the
// segment swizzle alone leaves pairs of rows on the same banks, and swapping
// the halves in odd rows separates them (the transposing reads, which only
// permute within a segment, are unaffected).
template <int VROWB>
__device__ __forceinline__ int vhalf(int r) {
  return VROWB == 128 ? 16 * (r & 1) : 0;
}

// p with address bit 4 flipped (an asm statement: the result is formed where
// it is used instead of being kept live; one instruction, no copy of p).
__device__ __forceinline__ uint8_t* flip16(uint8_t* p) {
  const uint32_t a = uint32_t(uintptr_t((__attribute__((address_space(3))) uint8_t*)(p)));
  uint32_t r;
  asm volatile("v_xor_b32 %0, 16, %1" : "=v"(r) : "v"(a));
  return (uint8_t*)(__attribute__((address_space(3))) uint8_t*)(uintptr_t(r));
}

// LDS byte address of a pointer into this workgroup's LDS.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(uintptr_t((const __attribute__((address_space(3))) uint8_t*)(p)));
}

// Value operands of the PV MFMAs of one group: for N-tiles n0 and n0 + 1 of
// the pass, the transposing reads from the value tiles of heads 0 and 1 (NH =
// 2) or twice from the one tile (NH = 1).  Written as one asm block that waits
// for its reads: the compiler would otherwise make such a read wait for every
// load into LDS still in flight (the next tiles' halves), since it cannot tell
// that they write other slots.
template <int NH, int HEAD1_OFF = 0>
__device__ __forceinline__ void value_operands2(uint32_t a0, uint32_t a1, half8& v0, half8& v1) {
  u32x2 x0, x1, y0, y1;
  if constexpr (NH == 2) {
    // the second kv-head's rows sit HEAD1_OFF bytes on
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %4 offset:%6\n\t"
        "ds_read_b64_tr_b16 %2, %5\n\t"
        "ds_read_b64_tr_b16 %3, %5 offset:%6\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(y0), "=&v"(y1)
        : "v"(a0), "v"(a1), "n"(HEAD1_OFF)
        : "memory");
  } else {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %4\n\t"
        "ds_read_b64_tr_b16 %1, %4\n\t"
        "ds_read_b64_tr_b16 %2, %5\n\t"
        "ds_read_b64_tr_b16 %3, %5\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(x0), "=&v"(x1), "=&v"(y0), "=&v"(y1)
        : "v"(a0), "v"(a1)
        : "memory");
  }
  v0 = __builtin_bit_cast(half8, u32x4{x0[0], x0[1], x1[0], x1[1]});
  v1 = __builtin_bit_cast(half8, u32x4{y0[0], y0[1], y1[0], y1[1]});
}

// max without the quieting the compiler adds to fmaxf (the values here are
// never signalling NaNs)
__device__ __forceinline__ float vmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float quad_max2(float x) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// 16 bytes from the record (voff: this lane's byte offset) into LDS at
// dst + 16 * lane (dst is the same for the whole wave).
__device__ __forceinline__ void lds_load16(__amdgpu_buffer_rsrc_t r, uint8_t* dst, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0, 0);
}

// Four E4M3 bytes -> two dwords of f16 pairs, each value times sc (a power
// of two 2^j, -5 <= j <= 7): exact, since every E4M3 value times such a power
// is an f16 normal number (the smallest, 2^-9, stays at or above 2^-14, the
// largest, 448, at or below 57344).
__device__ __forceinline__ u32x2 fp8x4_to_f16_s(uint32_t w, float sc = 1.0f) {
  u32x2 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, sc, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, sc, true));
  return o;
}

// Power-of-two split of an FP8 value scale sv between P' and the value codes:
// P' = p * sv * 2^k with codes times 2^-k leaves every product P' * code
// unchanged.  k is chosen so that sv * 2^k < 2^10 sits high in the f16 range:
// then P' and its f16 remainder stay normal for all but negligible p, where
// P' = p * sv alone (sv = amax / 448, often below 2^-6) would put the
// remainder on the subnormal grid, an absolute error that codes up to 448
// magnify.  (Wave-uniform; clamped to the exact range of fp8x4_to_f16_s.)
__device__ __forceinline__ int fp8_value_shift(float sv) {
  return min(5, max(-7, 10 - __builtin_amdgcn_frexp_expf(sv)));
}

// Softmax step of one tile for the lane's column (as softmax_step, with the
// accumulator rows' correction factors read from the lanes of their columns;
// `live` false: the column takes no token of this tile).
template <int NACC, typename OnRescale>
__device__ __forceinline__ void softmax_live(SoftState& st, float s[4], float p[4], f32x4 (&acc)[NACC],
                                             int quad, bool live, OnRescale on_rescale) {
  float tmax = vmax(vmax(s[0], s[1]), vmax(s[2], s[3]));
  tmax = quad_max2(tmax);
  if (__any(tmax > st.m)) {
    // a column whose maximum does not rise keeps a factor of exactly 1 (its
    // maximum may still be -inf: no live token of it seen yet)
    const bool rise = tmax > st.m;
    const float m_new = rise ? tmax + kHeadroom : st.m;
    const float corr = rise ? exp2f(st.m - m_new) : 1.0f;   // 0 on the column's first tile
    st.m = m_new;
    st.l *= corr;
    on_rescale(corr);
    // accumulator row i of this lane is column 4quad + i, whose factor lane
    // 4quad + i (column 4quad + i, quad 0) holds
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float c = __shfl(corr, 4 * quad + i, 64);
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j][i] *= c;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float e = __builtin_amdgcn_exp2f(s[i] - st.m);
    p[i] = live ? e : 0.0f;
    st.l += p[i];
  }
}

// The same for a live column whose scores still take a wave-uniform factor
// fs >= 0: the maximum is taken over the raw scores (a non-negative factor
// keeps their order, so max(s) * fs is the maximum of the products exactly)
// and each weight is 2^(fs * s - m) from one fma.  Scores of -inf need
// fs > 0.
template <int NACC, typename OnRescale>
__device__ __forceinline__ void softmax_scaled(SoftState& st, const float s[4], float fs, float p[4],
                                               f32x4 (&acc)[NACC], int quad, OnRescale on_rescale) {
  float tmax = vmax(vmax(s[0], s[1]), vmax(s[2], s[3]));
  tmax = quad_max2(tmax) * fs;
  if (__any(tmax > st.m)) {
    const bool rise = tmax > st.m;
    const float m_new = rise ? tmax + kHeadroom : st.m;
    const float corr = rise ? exp2f(st.m - m_new) : 1.0f;   // 0 on the column's first tile
    st.m = m_new;
    st.l *= corr;
    on_rescale(corr);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float c = __shfl(corr, 4 * quad + i, 64);
#pragma unroll
      for (int j = 0; j < NACC; ++j) acc[j][i] *= c;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], fs, -st.m));
    st.l += p[i];
  }
}

// Page-table entries of a wave's pages, one per lane (a wave's tiles span at
// most 64 pages), read per tile with readlane.
struct WavePages {
  int32_t ent;
  int first;
  __device__ __forceinline__ const uint8_t* page(const PoolView& pv, int pg) const {
    return page_address(pv, __builtin_amdgcn_readlane(ent, pg - first));
  }
};
__device__ __forceinline__ WavePages wave_pages(const DecodeArgs& a, const WorkItem& it, const TileGeom& g) {
  const int lane = threadIdx.x & 63;
  WavePages w;
  w.first = g.first.page;
  const int n = g.stop_page - g.first.page + 1;
  w.ent = lane < n ? a.entries[it.list_off + w.first + lane] : 0;
  return w;
}

// ---------------------------------------------------------------------------
// TQ3 work item
// ---------------------------------------------------------------------------
template <int NG, int NH>
__device__ __forceinline__ void tq3_item(const DecodeArgs& a, const WorkItem& it, uint8_t* smem) {
  using C = Mix<NG, NH>;
  constexpr int D = C::D, NT = C::NT, ROWB = C::ROWB, TNI = C::TNI;
  constexpr int VROWB = C::VROWB, PASS = C::PASS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;                    // token (keys) / head column (outputs)
  const int quad = lane >> 4;
  const PoolView& pv = a.pv;
  const int hk0 = blockIdx.y * NH;               // the workgroup's kv-heads
  const int G = a.Hq / pv.Hkv;
  const int ncol = NH * G;
  const int hq0 = hk0 * G;
  const int jcol = col < ncol ? col / G : 0;    // kv-head (within the workgroup) of column col
  uint8_t* vt = smem + wave * C::WAVE;          // this wave's value tile, then its slots
  uint8_t* wl = vt + C::VBUF;
  const TileGeom tg = wave_tiles(it, pv.P / 16, wave);

  f32x4 acc[NT];                                // one per N-tile, both kv-heads' rows
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  SoftState st;
  // probability mass of the lane's column times the value scale, per group
  // (this lane's tokens): the value codes enter the MFMA uncentred, so the
  // accumulator of group g misses -3.5 times this sum
  float vmass[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) vmass[g] = 0.0f;

  const WavePages wp = wave_pages(a, it, tg);
  // query rows of the lane's column: fetched now, converted once the first
  // tile's loads are in flight
  const bool qlive = col < ncol;
  const uint16_t* qrow = a.q + (int64_t(it.b) * a.Hq + hq0 + (qlive ? col : 0)) * D;
  u32x4 qraw[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) qraw[g] = *reinterpret_cast<const u32x4*>(qrow + 32 * g + 8 * quad);

  // A half-slot holds the key (value) codes of the NH heads, 16 token rows
  // each, then their scales.  Each code load copies up to 64 16-byte vectors
  // of one head's rows (lane l: bytes 16l..), each scale load the 2NG scale
  // vectors of one head; the tile and head positions are scalar offsets.
  const int BLK = pv.P * 28 * NG;                // TQ3 bytes of one kv-head of a page
  const uint32_t voff_c = 16u * uint32_t(lane);
  Cursor lc = tg.first;                          // next tile whose halves are loaded
  int ls = 0;                                    // next slot to fill
  auto issue = [&](bool value_half) {
    const auto rsrc = record_rsrc(wp.page(pv, lc.page), pv.tq3_stride);
    uint8_t* dst = wl + ls * C::SLOT;
    const int code0 = hk0 * BLK + (value_half ? pv.P * ROWB : 0) + lc.sub * 16 * ROWB;
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int x = 0; x < C::CPH; ++x)
        if (64 * x + lane < 12 * NG)
          lds_load16(rsrc, dst + j * 16 * ROWB + 1024 * x, voff_c, code0 + j * BLK + 1024 * x);
    if (lane < 2 * NG)
#pragma unroll
      for (int j = 0; j < NH; ++j)
        lds_load16(rsrc, dst + NH * 16 * ROWB + j * 16 * C::SCB, voff_c,
                   (hk0 + j) * BLK + 2 * pv.P * ROWB + (value_half ? pv.P * C::SCB : 0) +
                       lc.sub * 16 * C::SCB);
    ls = ls == C::NSLOT - 1 ? 0 : ls + 1;
    if (value_half) advance_clamped(lc, tg);     // past the end, the last tile is loaded again
  };
  if (tg.ntiles > 0) {
    issue(false);
    issue(true);
    issue(false);
  }

  // Query operands, shared by the workgroup's waves (same sequence and
  // kv-heads): slot s of MFMA g holds dim 32g + 8quad + kSlotCode[s], scaled
  // by 2^(E + 7 - kSlotShift[s]) against the key slot's 2^(k-24), so each
  // product is c * q * 2^(E-17); E is the column's exponent (max|q| * 2^E in
  // [64, 128)).  Wave w converts the groups g = w mod 4 and publishes their
  // operands for each kv-head of the wave (zero outside that head's columns)
  // through the value tiles, which no wave uses before its first tile's
  // values, and the key centring -3.5 * sum of q * 2^(E-17) over the group's
  // dims as (v, v, v, v) per column in a half-slot tail, where the tile
  // loop reads it as the groups' accumulator initial value.
  half8 qop[NH][NG];
  float F;
  {
    // max |q| of the column: the magnitude bits of bf16 values order like
    // unsigned integers (no NaN in a query), so packed 16-bit maxima do
    uint32_t mbits = 0u;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
      for (int x = 0; x < 4; ++x) mbits = pk_max_u16(mbits, qraw[g][x] & 0x7FFF7FFFu);
    float amax = __uint_as_float(max(mbits & 0xFFFFu, mbits >> 16) << 16);
    amax = qlive ? quad_max(amax) : 0.0f;
    const int E = q_shift(amax);
    // the sign of the softmax scale goes to the query operands (exact), so
    // the score factor F is never negative
    const float qsign = a.scale < 0.0f ? -1.0f : 1.0f;
    F = __builtin_fabsf(a.scale) * kLog2e * __builtin_amdgcn_ldexpf(1.0f, 17 - E);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      if (g % kWaves != wave) continue;
      half8 qh;
      float part = 0.0f;
#pragma unroll
      for (int sl = 0; sl < 8; ++sl) {
        const int e = kSlotCode[sl];
        const float x = qlive ? qsign * bf16_to_f32(uint16_t(qraw[g][e >> 1] >> (16 * (e & 1)))) : 0.0f;
        qh[sl] = _Float16(__builtin_amdgcn_ldexpf(x, E + 7 - kSlotShift[sl]));
        part = __builtin_fmaf(float(qh[sl]), __builtin_amdgcn_ldexpf(1.0f, kSlotShift[sl] - 24), part);
      }
      const float kinit = -3.5f * quad_sum(part);
      if (quad == 0) *reinterpret_cast<f32x4*>(C::kinit_addr(smem, g) + 16 * col) = f32x4{kinit, kinit, kinit, kinit};
      const u32x4 w = __builtin_bit_cast(u32x4, qh);
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const u32x4 o = {jcol == j ? w[0] : 0u, jcol == j ? w[1] : 0u, jcol == j ? w[2] : 0u, jcol == j ? w[3] : 0u};
        *reinterpret_cast<u32x4*>(C::qop_addr(smem, j, g) + 16 * lane) = o;
      }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int g = 0; g < NG; ++g)
        qop[j][g] = *reinterpret_cast<const half8*>(C::qop_addr(smem, j, g) + 16 * lane);
    __syncthreads();                             // the value tiles are free again
  }

  if (tg.ntiles > 0) {
    // lane constant: the funnel shift of the key window (dwords quad - 1 and
    // quad of the group; quad 0 reads the dword before the group, which the
    // value tile in front of the slots keeps inside this workgroup's LDS)
    const uint32_t ks1 = uint32_t(24 - 8 * quad);
    // byte offset of the lane's key dwords in a slot (kept opaque so that the
    // slot's constant part stays in the scalar base and the per-MFMA offsets
    // fit the LDS instructions' immediate fields)
    uint32_t klane = uint32_t(C::VBUF + col * ROWB + 4 * (quad - 1));
    asm volatile("" : "+v"(klane));
    // value-tile addresses of the transposing reads (row 4quad + col/4,
    // 8 bytes at column 4(col & 3) of N-tile n of the pass): segment n of a
    // row is segment 0 with n XOR-ed into bits 5.. of the address (the tile
    // sits at a multiple of 1 KB and a row's offset has those bits clear)
    const int vr = 4 * quad + (col >> 2);
    const uint32_t va0 = lds_addr(vt) + uint32_t(vr * VROWB + 32 * vseg<VROWB>(vr, 0) + ((8 * (col & 3)) ^ vhalf<VROWB>(vr)));
    const uint32_t va1 = va0 ^ 32u;
    // value unpack: lane -> (group ug of the pass, token ut, head uj), the
    // group fastest: a half-wave's raw reads (three dwords per lane at
    // 12 ut + 3 ug, one head) then spread over more banks than with the
    // token fastest, and eight consecutive lanes still write eight distinct
    // 16-byte bank groups of the swizzled value tile; spare lanes repeat a
    // real one's work
    const int ci = lane % (16 * NH * PASS);
    const int ug = ci % PASS, ut = (ci / PASS) & 15, uj = ci / (16 * PASS);

    Cursor pc = tg.first;
    int ks = 0;                                  // slot of this tile's key half
    for (int ti = 0; ti < tg.ntiles; ++ti) {
      if (a.pace) pace_priority(ti, tg.ntiles);
      const int vs = ks == C::NSLOT - 1 ? 0 : ks + 1;
      const int nvalid = valid_in_tile(pc, tg);
      const uint8_t* kb = wl + ks * C::SLOT;
      const uint8_t* vb = wl + vs * C::SLOT;
      const uint8_t* kq = vt + ks * C::SLOT + klane;    // = kb + lane's row and dword

      // ---- keys: QK^T per group, both kv-heads into one D, scaled per token
      wait_vm<2 * TNI>();                        // this tile's key half has landed
      uint32_t ksd[2 * NG];
      load_scale_dwords<NG>(reinterpret_cast<const uint32_t*>(kb + C::SCOFF + jcol * 16 * C::SCB + 8 * NG * quad), ksd);
      float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        f32x4 dg = *reinterpret_cast<const f32x4*>(C::kinit_addr(smem, g) + 16 * col);
#pragma unroll
        for (int j = 0; j < NH; ++j) {
          const uint32_t* u = reinterpret_cast<const uint32_t*>(kq + j * 16 * ROWB + 12 * g);
          dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(
              __builtin_bit_cast(half8, tq3_key_operand(u[0], u[1], ks1)), qop[j][g], dg, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[i] = __builtin_fmaf(dg[i], f16_half(ksd[(i * NG + g) >> 1], (i * NG + g) & 1), s[i]);
      }
      wait_lds();                                // the key half is consumed: its slot takes
      issue(true);                               // the next tile's value half
      // score factor F enters the softmax's exponent fma; a partial tile
      // scales its scores first and masks the rows past the valid tokens
      const bool partial = nvalid < 16;
      float fs = F;
      if (partial) {
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = 4 * quad + i >= nvalid ? -INFINITY : s[i] * F;
        fs = 1.0f;
      }
      float p[4];
      softmax_scaled(st, s, fs, p, acc, quad, [&](float c) {
#pragma unroll
        for (int g = 0; g < NG; ++g) vmass[g] *= c;
      });

      // ---- values: per pass of PASS groups, unpack into the value tile, then
      // P' = p * value scale (hi/lo f16) and acc += P' * V
      wait_vm<2 * TNI>();                        // this tile's value half has landed
      if (partial) {
        // rows past the valid tokens: their value scales (unwritten memory,
        // possibly NaN, and p = 0 times NaN is NaN) become 0; the scale rows
        // of the slot are [head][token][group] f16
        uint16_t* vsc = reinterpret_cast<uint16_t*>(wl + vs * C::SLOT + C::SCOFF);
        for (int x = lane; x < NH * 16 * NG; x += 64)
          if ((x / NG) % 16 >= nvalid) vsc[x] = 0;
        wave_lds_sync();
      }
      const uint32_t* vsp = reinterpret_cast<const uint32_t*>(vb + C::SCOFF + jcol * 16 * C::SCB + 8 * NG * quad);
#pragma unroll
      for (int ps = 0; ps < C::NPASS; ++ps) {
        // value scales of the pass for the lane's 4 tokens
        uint32_t sw[4];
        tq3_pass_scales<NG>(vsp, ps, sw);
        {
          const uint32_t* src = reinterpret_cast<const uint32_t*>(vb + uj * 16 * ROWB + ut * ROWB + 12 * (ps * PASS + ug));
          const uint32_t w[3] = {src[0], src[1], src[2]};
          uint32_t o[16];
          tq3_value_group(w, o);
          uint8_t* row = vt + (uj * 16 + ut) * VROWB + vhalf<VROWB>(ut);
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            uint8_t* c0 = row + 32 * vseg<VROWB>(ut, 2 * ug + h);
            *reinterpret_cast<u32x4*>(c0) = u32x4{o[8 * h], o[8 * h + 1], o[8 * h + 2], o[8 * h + 3]};
            *reinterpret_cast<u32x4*>(vhalf<VROWB>(1) ? flip16(c0) : c0 + 16) =
                u32x4{o[8 * h + 4], o[8 * h + 5], o[8 * h + 6], o[8 * h + 7]};
          }
        }
        wave_lds_sync();
#pragma unroll
        for (int gs = 0; gs < PASS; ++gs) {
          const int g = ps * PASS + gs;
          uint32_t phi[2], plo[2];
          if (gs == 0) pprime_tq3<NG, 0>(p, sw, phi, plo, vmass[g]);
          else pprime_tq3<NG, 1>(p, sw, phi, plo, vmass[g]);
          half8 bv[2];
          value_operands2<NH, 16 * VROWB>(va0 ^ uint32_t(64 * gs), va1 ^ uint32_t(64 * gs), bv[0], bv[1]);
          if constexpr (NH == 2) {
            half8 a_hi, a_lo;
            split_pprime(__builtin_bit_cast(half8, u32x4{phi[0], phi[1], plo[0], plo[1]}), jcol == 1, a_hi, a_lo);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              acc[2 * g + h] = pv_mfma(a_hi, bv[h], acc[2 * g + h]);
              acc[2 * g + h] = pv_mfma(a_lo, bv[h], acc[2 * g + h]);
            }
          } else {
#pragma unroll
            for (int h = 0; h < 2; ++h)
              acc[2 * g + h] = pv_mfma(__builtin_bit_cast(half8, u32x4{phi[0], phi[1], plo[0], plo[1]}), bv[h],
                                       acc[2 * g + h]);
          }
        }
        wave_lds_sync();
      }
      wait_lds();                                // the value half is consumed: its slot takes
      issue(false);                              // the tile after next's key half
      advance(pc, tg);
      ks = ks >= C::NSLOT - 2 ? ks - (C::NSLOT - 2) : ks + 2;
    }
    if (a.pace) __builtin_amdgcn_s_setprio(0);
    wait_vm<0>();                                // no load into LDS outlives the loop
  }

  // ---- combine the four waves' states through LDS (the slots are reused once
  // every wave is past its last tile) and write the item's state
  const float lcol = quad_sum(st.l);
  // centring term of each accumulator row (column 4quad + i) and group
  float cent[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float m = -3.5f * quad_sum(vmass[g]);
#pragma unroll
    for (int i = 0; i < 4; ++i) cent[g][i] = __shfl(m, 4 * quad + i, 64);
  }
  __syncthreads();
  auto& M = *reinterpret_cast<MergeLds<D>*>(smem);
  if (quad == 0) {
    M.m[wave][col] = st.m;
    M.l[wave][col] = lcol;
  }
  // accumulator column col of N-tile jt holds value position 16 (jt & 1) + col
  // of group jt / 2 (half pos & 1 of value pair pos / 2), scaled by 2^(k-24)
  const uint64_t we = (col & 8) ? kValuePos[1] : kValuePos[0];
  const uint64_t wo = (col & 8) ? kValuePos[3] : kValuePos[2];
  const int ee = int(we >> (8 * (col & 7))) & 255, eo = int(wo >> (8 * (col & 7))) & 255;
  const float up_e = __builtin_amdgcn_ldexpf(1.0f, 16 + (ee >> 5));      // 2^(24 - k)
  const float up_o = __builtin_amdgcn_ldexpf(1.0f, 16 + (eo >> 5));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * quad + i;
    if (c >= ncol) continue;
    float* dst = M.acc[wave] + c * MergeLds<D>::ROW;
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
      dst[32 * (jt >> 1) + ((jt & 1) ? (eo & 31) : (ee & 31))] =
          __builtin_fmaf(acc[jt][i], (jt & 1) ? up_o : up_e, cent[jt >> 1][i]);
  }
  __syncthreads();
  merge_waves_and_store<D>(M, a, it.chunk, hq0, ncol);
}

// ---------------------------------------------------------------------------
// FP8 work item: each 16-token tile is NH one-head tiles
// ---------------------------------------------------------------------------
template <int NG, int NH>
__device__ __forceinline__ void fp8_item(const DecodeArgs& a, const WorkItem& it, uint8_t* smem) {
  using C = Mix<NG, NH>;
  constexpr int D = C::D, NT = C::NT, FNI = C::FNI, VROWB = C::VROWB, PASS = C::PASS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int quad = lane >> 4;
  const PoolView& pv = a.pv;
  const int hk0 = blockIdx.y * NH;
  const int G = a.Hq / pv.Hkv;
  const int ncol = NH * G;
  const int hq0 = hk0 * G;
  const int jcol = col < ncol ? col / G : 0;
  uint8_t* vt = smem + wave * C::WAVE;
  uint8_t* wl = vt + C::VBUF;
  const TileGeom tg = wave_tiles(it, pv.P / 16, wave);

  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  SoftState st;

  if (tg.ntiles > 0) {
    const WavePages wp = wave_pages(a, it, tg);
    const bool qlive = col < ncol;
    const uint16_t* qrow = a.q + (int64_t(it.b) * a.Hq + hq0 + (qlive ? col : 0)) * D;
    u32x4 qraw[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) qraw[g] = *reinterpret_cast<const u32x4*>(qrow + 32 * g + 8 * quad);

    // a one-head half is 16 consecutive token rows of that head's key (or
    // value) block.  Rows are D bytes apart, a multiple of the LDS bank width,
    // so the 16 rows of a tile read at one column would share banks; at D >=
    // 128 the load therefore swizzles each row's 16-byte chunks: slot chunk
    // (t, c) holds record chunk (t, c ^ sw(t)) with sw(t) = t mod (rows per
    // load instruction), which keeps each lane's record offset constant
    const int PD = pv.P * D;
    constexpr int CPR = D / 16;                   // 16-byte chunks per row
    constexpr int RPI = 64 / CPR;                 // rows per load instruction
    constexpr bool SWZ = D >= 128;
    static_assert(!SWZ || RPI <= CPR, "the swizzle stays within a row");
    const uint32_t voff_c = SWZ ? 16u * uint32_t((lane / CPR) * CPR + ((lane % CPR) ^ (lane / CPR)))
                                : 16u * uint32_t(lane);
    Cursor lc = tg.first;
    int lj = 0;                                  // head of the next one-head tile to load
    int ls = 0;
    auto issue = [&](bool value_half) {
      const auto rsrc = record_rsrc(wp.page(pv, lc.page), pv.fp8_stride);
      uint8_t* dst = wl + ls * C::SLOT;
      const int so = ((hk0 + lj) * 2 + (value_half ? 1 : 0)) * PD + lc.sub * 16 * D;
#pragma unroll
      for (int x = 0; x < FNI; ++x)
        if (64 * x + lane < C::FVEC) lds_load16(rsrc, dst + 1024 * x, voff_c, so + 1024 * x);
      ls = ls == C::NSLOT - 1 ? 0 : ls + 1;
      if (value_half) {
        if (++lj == NH) {
          lj = 0;
          advance_clamped(lc, tg);
        }
      }
    };
    issue(false);
    issue(true);
    issue(false);

    half8 qop[NH][NG];
    float F;
    {
      half8 qh[NG];
      const int E = load_query<NG, NH>(
          a, it.b, hq0, col, ncol, jcol, qop, qh,
          [&](const uint16_t*, int r, float (&v)[8]) {
#pragma unroll
            for (int s = 0; s < 8; ++s) v[s] = bf16_to_f32(uint16_t(qraw[r][s >> 1] >> (16 * (s & 1))));
          },
          [](float x, int E, int) { return _Float16(__builtin_amdgcn_ldexpf(x, E)); });
      F = a.scale * kLog2e * __builtin_amdgcn_ldexpf(1.0f, -E);
    }
    const int vr = 4 * quad + (col >> 2);
    uint32_t vrd[2 * PASS];
#pragma unroll
    for (int n = 0; n < 2 * PASS; ++n) vrd[n] = uint32_t(vr * VROWB + 32 * vseg<VROWB>(vr, n) + 8 * (col & 3));
    const uint32_t vt_addr = lds_addr(vt);
    // value conversion: lane -> (token ut, quarter uq of the pass's 32 PASS dims)
    const int ut = lane & 15, uq = lane >> 4;

    Cursor pc = tg.first;
    int ks = 0;
    for (int ti = 0; ti < tg.ntiles; ++ti) {
      if (a.pace) pace_priority(ti, tg.ntiles);
      const int nvalid = valid_in_tile(pc, tg);
      const uint8_t* page = wp.page(pv, pc.page);
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const int vs = ks == C::NSLOT - 1 ? 0 : ks + 1;
        const uint8_t* kb = wl + ks * C::SLOT;
        const uint8_t* vb = wl + vs * C::SLOT;
        const bool live = jcol == j && col < ncol;
        // page-head scales of head hk0 + j (wave-uniform)
        const float sk = *reinterpret_cast<const float*>(page + fp8_scale_off(pv, hk0 + j, 0));
        const float sv0 = *reinterpret_cast<const float*>(page + fp8_scale_off(pv, hk0 + j, 1));
        const int kv = fp8_value_shift(sv0);
        const float sv = __builtin_amdgcn_ldexpf(sv0, kv);             // P' scale
        const float vsc = __builtin_amdgcn_ldexpf(1.0f, -kv);          // code scale

        wait_vm<2 * FNI>();
        f32x4 dsum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int r = 0; r < NG; ++r) {
          // logical bytes 32 r + 8 quad of row col: chunk 2 r + quad / 2
          const int chunk = SWZ ? (2 * r + (quad >> 1)) ^ (col % RPI) : 2 * r + (quad >> 1);
          const u32x2 w = *reinterpret_cast<const u32x2*>(kb + col * D + 16 * chunk + 8 * (quad & 1));
          const u32x2 k0 = fp8x4_to_f16_s(w[0]);
          const u32x2 k1 = fp8x4_to_f16_s(w[1]);
          const u32x4 ku = {k0[0], k0[1], k1[0], k1[1]};
          dsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ku), qop[j][r], dsum, 0, 0, 0);
        }
        wait_lds();
        issue(true);
        const float fk = F * sk;
        float s[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = live && 4 * quad + i < nvalid ? dsum[i] * fk : -INFINITY;
        float p[4];
        softmax_live(st, s, p, acc, quad, live, [](float) {});
        const half8 pp = pprime_uniform(p, sv);

        wait_vm<2 * FNI>();
#pragma unroll
        for (int ps = 0; ps < C::NPASS; ++ps) {
          {
            // token ut's dims 32 PASS ps + 8 PASS uq .. +8 PASS, widened to f16
            // (rows past the valid tokens are zeroed: an unwritten byte may be NaN)
            constexpr int NB = 8 * PASS;                     // bytes (dims) per lane
            const int vbyte = 32 * PASS * ps + NB * uq;      // logical bytes of row ut
            const uint8_t* src = vb + ut * D + (SWZ ? 16 * ((vbyte >> 4) ^ (ut % RPI)) + (vbyte & 15) : vbyte);
            uint32_t o[NB / 2];
            if constexpr (NB == 16) {
              const u32x4 w = *reinterpret_cast<const u32x4*>(src);
#pragma unroll
              for (int x = 0; x < 4; ++x) {
                const u32x2 h = fp8x4_to_f16_s(w[x], vsc);
                o[2 * x] = h[0];
                o[2 * x + 1] = h[1];
              }
            } else {
              const u32x2 w = *reinterpret_cast<const u32x2*>(src);
#pragma unroll
              for (int x = 0; x < 2; ++x) {
                const u32x2 h = fp8x4_to_f16_s(w[x], vsc);
                o[2 * x] = h[0];
                o[2 * x + 1] = h[1];
              }
            }
            if (ut >= nvalid) {
#pragma unroll
              for (int x = 0; x < NB / 2; ++x) o[x] = 0u;
            }
            uint8_t* row = vt + ut * VROWB;
#pragma unroll
            for (int k = 0; k < NB / 8; ++k) {
              const int byte = 2 * NB * uq + 16 * k;           // f16 bytes within the row
              *reinterpret_cast<u32x4*>(row + 32 * vseg<VROWB>(ut, byte >> 5) + (byte & 31)) =
                  u32x4{o[4 * k], o[4 * k + 1], o[4 * k + 2], o[4 * k + 3]};
            }
          }
          wave_lds_sync();
#pragma unroll
          for (int n = 0; n < 2 * PASS; n += 2) {
            half8 bv[2];
            value_operands2<1>(vt_addr + vrd[n], vt_addr + vrd[n + 1], bv[0], bv[1]);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int jt = 2 * PASS * ps + n + h;
              acc[jt] = pv_mfma(pp, bv[h], acc[jt]);
            }
          }
          wave_lds_sync();
        }
        wait_lds();
        issue(false);
        ks = ks >= C::NSLOT - 2 ? ks - (C::NSLOT - 2) : ks + 2;
      }
      advance(pc, tg);
    }
    if (a.pace) __builtin_amdgcn_s_setprio(0);
    wait_vm<0>();
  }

  const float lcol = quad_sum(st.l);
  __syncthreads();
  auto& M = *reinterpret_cast<MergeLds<D>*>(smem);
  if (quad == 0) {
    M.m[wave][col] = st.m;
    M.l[wave][col] = lcol;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * quad + i;
    if (c >= ncol) continue;
    float* dst = M.acc[wave] + c * MergeLds<D>::ROW;
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) dst[16 * jt + col] = acc[jt][i];
  }
  __syncthreads();
  merge_waves_and_store<D>(M, a, it.chunk, hq0, ncol);
}

}  // namespace

// ---------------------------------------------------------------------------
// BF16 work item (control pools): the dense single-format cache.  Structure
// of the FP8 item without scales or widening: a lane's quarter row of keys is
// the MFMA operand as loaded, value rows go to the LDS tile as loaded.
// ---------------------------------------------------------------------------
// P as a bf16 hi + lo pair in one A operand (about 16 significant bits).
__device__ __forceinline__ bf16x8 pprime_bf16(const float p[4]) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const __bf16 h = __bf16(p[i]);
    r[i] = h;
    r[4 + i] = __bf16(p[i] - float(h));
  }
  return r;
}

template <int NG, int NH, int R>
__device__ __forceinline__ void bf16_item(const DecodeArgs& a, const WorkItem& it, uint8_t* smem) {
  auto& lds = *reinterpret_cast<Fp8Lds<NG, NH>*>(smem);   // same LDS image as FP8 items
  constexpr int D = 32 * NG;
  constexpr int NT = D / 16;
  constexpr int VROW = Fp8Lds<NG, NH>::VROW;
  constexpr int LD = D / 4;                     // dims of a row each lane loads
  constexpr int LW = LD / 2;                    // their dwords

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;
  const int quad = lane >> 4;
  const PoolView& pv = a.pv;
  stage_entries(lds.ent, a, it);
  const int hk0 = blockIdx.y * NH;               // the workgroup's kv-heads
  if (hk0 >= pv.Hkv) return;
  const int G = a.Hq / pv.Hkv;
  const int ncol = NH * G;
  const int hq0 = hk0 * G;
  const int jcol = col < ncol ? col / G : 0;
  auto& W = lds.w[wave];
  const uint8_t* vbase = W.vt[0] + value_row(4 * quad + (col >> 2)) * VROW + 8 * (col & 3);
  const uint8_t* vbase2 = vbase + vgpr_opaque_zero();

  // ---- query operand: MFMA r, lane (col, quad), slot s <-> dim quad*LD + 8r + s,
  // taken as stored (bf16); zero outside the lane's column's kv-head
  bf16x8 qop[NH][NG];
  const float F = a.scale * kLog2e;
  auto prepare = [&]() {
    const bool live = col < ncol;
    const uint16_t* qrow = a.q + (int64_t(it.b) * a.Hq + hq0 + (live ? col : 0)) * D;
#pragma unroll
    for (int r = 0; r < NG; ++r) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + quad * LD + 8 * r);
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        u32x4 o;
#pragma unroll
        for (int x = 0; x < 4; ++x) o[x] = live && jcol == j ? w[x] : 0u;
        qop[j][r] = __builtin_bit_cast(bf16x8, o);
      }
    }
  };

  f32x4 acc[NH * NT];
#pragma unroll
  for (int j = 0; j < NH * NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  SoftState st;

  uint32_t row_off[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) row_off[j] = uint32_t((hk0 + j) * 2 * pv.P * D * 2 + col * D * 2 + quad * LD * 2);
  const int vrow_delta = pv.P * D * 2;                 // V rows follow the K rows
  struct Raw {
    uint32_t kw[NH][LW];
    uint32_t vw[NH][LW];
  };
  auto load = [&](const Cursor& c, Raw& r) {
    const auto rec = record_rsrc(entry_page(pv, lds.ent, c.page), pv.fp8_stride);
    const int kso = 16 * c.sub * D * 2;                  // the tile's first K row
    const int vso = kso + vrow_delta;                    // and its first V row
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int x = 0; x < LW / 4; ++x) {
        const u32x4 kw = rec_load4(rec, row_off[j] + 16 * x, kso);
        const u32x4 vw = rec_load4(rec, row_off[j] + 16 * x, vso);
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          r.kw[j][4 * x + y] = kw[y];
          r.vw[j][4 * x + y] = vw[y];
        }
      }
  };
  const TileGeom tg = wave_tiles(it, pv.P / 16, wave);

  auto process = [&](Raw& raw, const Cursor& c, auto refill) {
    const int nvalid = valid_in_tile(c, tg);
    // ---- value rows to the LDS tiles (rows past the valid tokens zeroed: an
    // unwritten slot may hold any bits, and p = 0 times NaN is NaN)
    const bool vrow_ok = col < nvalid;
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int x = 0; x < LW / 4; ++x) {
        u32x4 o = {raw.vw[j][4 * x], raw.vw[j][4 * x + 1], raw.vw[j][4 * x + 2], raw.vw[j][4 * x + 3]};
        if (!vrow_ok) o = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(W.vt[j] + value_row(col) * VROW + 2 * quad * LD + 16 * x) = o;
      }
    // ---- QK^T over all dims and both kv-heads into one accumulator (the
    // query operands are zero outside each lane's own kv-head)
    f32x4 dsum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int r = 0; r < NG; ++r) {
        const u32x4 ku = {raw.kw[j][4 * r], raw.kw[j][4 * r + 1], raw.kw[j][4 * r + 2], raw.kw[j][4 * r + 3]};
        dsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ku), qop[j][r], dsum, 0, 0, 0);
      }
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = dsum[i] * F;
    refill(raw);
    wave_lds_sync();
    if (nvalid < 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * quad + i >= nvalid) s[i] = -INFINITY;
    }
    float p[4];
    softmax_step(st, s, p, acc, W.corr, col, quad);

    const bf16x8 pp = pprime_bf16(p);
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        const half8 bv = value_operand(vbase + j * (16 * VROW) + 32 * jt, vbase2 + j * (16 * VROW) + 32 * jt);
        acc[j * NT + jt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pp, __builtin_bit_cast(bf16x8, bv),
                                                                 acc[j * NT + jt], 0, 0, 0);
      }
    wave_lds_sync();
  };
  run_tiles<R, Raw>(tg, a.pace != 0, load, prepare, process);

  const float lcol = quad_sum(st.l);
  __syncthreads();
  auto& M = *reinterpret_cast<MergeLds<D>*>(smem);
  if (quad == 0) {
    M.m[wave][col] = st.m;
    M.l[wave][col] = lcol;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * quad + i;
    if (c >= ncol) continue;
    const int jc = c / G;
    float* dst = M.acc[wave] + c * MergeLds<D>::ROW;
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) dst[16 * jt + col] = pick_head<NH, NT>(acc, jc, jt, i);
  }
  __syncthreads();
  merge_waves_and_store<D>(M, a, it.chunk, hq0, ncol);
}

// ---------------------------------------------------------------------------
// One launch for both formats: workgroup x takes work item x (FP8 or TQ3).
// Four waves per SIMD at head dim <= 128 (at most 128 VGPRs and 10 KB of LDS
// per wave); two at head dim 256.
// ---------------------------------------------------------------------------
//
// The work items' address comes first among the arguments, so the kernel can
// receive it preloaded in scalar registers (built with a kernel-argument
// preload count of 2): the item load then waits for no argument load.
template <int NG, int NH>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NG < 8 ? 4 : 2)))
partial_mixed(const WorkItem* __restrict__ items, DecodeArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t smem[Mix<NG, NH>::SMEM];
  const WorkItem it = items[blockIdx.x];
  if (it.fmt == 0)
    fp8_item<NG, NH>(a, it, smem);
  else
    tq3_item<NG, NH>(a, it, smem);
}

// Control pools: every work item is BF16.  Two waves per SIMD; one tile in
// flight (a BF16 tile row share is 4x the TQ3 one).
template <int NG, int NH>
__global__ void __launch_bounds__(kThreads, 2) partial_bf16(const WorkItem* __restrict__ items, DecodeArgs a) {
  constexpr size_t kSmem = Mix<NG, NH>::cmax(sizeof(Fp8Lds<NG, NH>), sizeof(MergeLds<32 * NG>));
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  const WorkItem it = items[blockIdx.x];
  bf16_item<NG, NH, 1>(a, it, smem);
}

namespace {

template <typename F>
hipError_t with_bf16_kernel(int d, int nh, F f) {
  if (nh == 2) {
    switch (d) {
      case 32: return f(partial_bf16<1, 2>);
      case 64: return f(partial_bf16<2, 2>);
      case 128: return f(partial_bf16<4, 2>);
      default: return hipErrorInvalidValue;
    }
  }
  switch (d) {
    case 32: return f(partial_bf16<1, 1>);
    case 64: return f(partial_bf16<2, 1>);
    case 128: return f(partial_bf16<4, 1>);
    case 256: return f(partial_bf16<8, 1>);
    default: return hipErrorInvalidValue;
  }
}

template <typename F>
hipError_t with_kernel(int d, int nh, F f) {
  if (nh == 2) {
    switch (d) {
      case 32: return f(partial_mixed<1, 2>);
      case 64: return f(partial_mixed<2, 2>);
      case 128: return f(partial_mixed<4, 2>);
      default: return hipErrorInvalidValue;
    }
  }
  switch (d) {
    case 32: return f(partial_mixed<1, 1>);
    case 64: return f(partial_mixed<2, 1>);
    case 128: return f(partial_mixed<4, 1>);
    case 256: return f(partial_mixed<8, 1>);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Grid: one workgroup per (work item, block of NH kv-heads); the workgroup's
// waves split the item's tiles (NH chosen by the schedule).
hipError_t launch_partial(const DecodeArgs& a, hipStream_t s) {
  if (a.n_items <= 0) return hipSuccess;
  const int nh = a.nh;
  const dim3 grid(unsigned(a.n_items), unsigned((a.pv.Hkv + nh - 1) / nh));
  auto launch = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, a.items, a);
    return hipGetLastError();
  };
  return a.pv.kind == kKindBf16 ? with_bf16_kernel(a.pv.d, nh, launch) : with_kernel(a.pv.d, nh, launch);
}

hipError_t partial_resident_waves(int d, int nh, int kind, int* waves) {
  int dev = 0, cus = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  auto query = [&](auto kernel) {
    int blocks = 0;
    const hipError_t r = hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, kernel, kThreads, 0);
    if (r == hipSuccess) *waves = cus * blocks * kWaves;
    return r;
  };
  return kind == kKindBf16 ? with_bf16_kernel(d, nh, query) : with_kernel(d, nh, query);
}

}  // namespace mkv
