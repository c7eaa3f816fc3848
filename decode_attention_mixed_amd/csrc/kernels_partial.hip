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
// wave64) per (work item = chunk of at most 256 pages of one format of one
// sequence, block of NH kv-heads).  The workgroup first copies the chunk's
// page-table entries to LDS; each wave then walks its quarter of the chunk's
// 16-token tiles for the NH kv-heads, with the raw bytes of the next R tiles
// in flight (a ring of register buffers).  The four waves' softmax states are
// combined through LDS and one partial state per query head is written.
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
// Operand encodings (all exact, all in the f16 normal range: MFMA products
// with subnormal f16 operands are not accumulated to full fp32 precision):
//  * TQ3: a 3-bit code c is masked into mantissa bits k..k+2 (1 <= k <= 7)
//    of an f16 whose exponent encodes 1.0 (one AND-OR per two elements), then
//    1 + 3.5 * 2^(k-10) is subtracted (one packed add): the operand is the
//    centred code (c - 3.5) * 2^(k-10), exact and finite for any bit pattern,
//    including unwritten poisoned slots.
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

// A VGPR holding the f16 pair (1.0, 1.0), opaque to constant folding.
__device__ __forceinline__ uint32_t vgpr_one_pair() {
  uint32_t r;
  asm volatile("v_mov_b32 %0, 0x3c003c00" : "=v"(r));
  return r;
}

// Half h (0 low, 1 high) of an f16 pair as fp32.
__device__ __forceinline__ float f16_half(uint32_t w, int h) {
  return float(__builtin_bit_cast(_Float16, uint16_t(w >> (16 * h))));
}

// f16 pair subtraction (x - c) with c given as the bits of two f16 values.
__device__ __forceinline__ uint32_t sub_f16x2(uint32_t x, uint32_t c) {
  const half2v h = __builtin_bit_cast(half2v, x) - __builtin_bit_cast(half2v, c);
  return __builtin_bit_cast(uint32_t, h);
}

// f16 bits of 1 + 3.5 * 2^(k-10) = 1 + 7 * 2^(k-11)
constexpr uint32_t center_bits(int k) { return 0x3C00u + (7u << (k - 1)); }

// ---- TQ3 key unit unpack ---------------------------------------------------
// A unit is 8 consecutive codes (24 bits, code i at bit 3i; bits 24..31 are
// ignored).  It becomes four dwords of f16 pairs holding (c - 3.5) * 2^(k-10):
//   slot:        0   1   2   3   4   5   6   7
//   code index:  2   6   3   7   4   0   5   1     (kSlotCode)
//   bit pos k:   6   2   7   3   3   7   3   7     (kSlotShift)
// Dword j takes the unit rotated right by 0, 2, 9 or 12 bits, which puts two
// codes inside the two 10-bit mantissa fields at positions k >= 1; the codes
// are AND-ed into the mantissas of (1.0, 1.0) and (1 + 3.5 * 2^(k-10)) is
// subtracted.  Both operands of the subtraction lie in [1, 2) and the
// constant has at most 10 fraction bits because k >= 1, so the result is
// exact and, as |c - 3.5| >= 1/2, an f16 normal number.
constexpr int kSlotCode[8] = {2, 6, 3, 7, 4, 0, 5, 1};
constexpr int kSlotShift[8] = {6, 2, 7, 3, 3, 7, 3, 7};
constexpr uint32_t center_pair(int slot) {
  return center_bits(kSlotShift[slot]) | (center_bits(kSlotShift[slot + 1]) << 16);
}
static_assert(center_pair(0) == 0x3C0E3CE0u && center_pair(2) == 0x3C1C3DC0u &&
                  center_pair(4) == 0x3DC03C1Cu && center_pair(6) == 0x3DC03C1Cu,
              "centering constants");

__device__ __forceinline__ u32x4 tq3_unit_to_f16(uint32_t x, uint32_t one) {
  const uint32_t r2 = __builtin_amdgcn_alignbit(x, x, 2);
  const uint32_t r9 = __builtin_amdgcn_alignbit(x, x, 9);
  const uint32_t r12 = __builtin_amdgcn_alignbit(x, x, 12);
  u32x4 o;
  o[0] = sub_f16x2(and_or(x, 0x001C01C0u, one), center_pair(0));     // c2 -> bits 6..8, c6 -> 18..20
  o[1] = sub_f16x2(and_or(r2, 0x00380380u, one), center_pair(2));    // c3 -> bits 7..9, c7 -> 19..21
  o[2] = sub_f16x2(and_or(r9, 0x03800038u, one), center_pair(4));    // c4 -> bits 3..5, c0 -> 23..25
  o[3] = sub_f16x2(and_or(r12, 0x03800038u, one), center_pair(6));   // c5 -> bits 3..5, c1 -> 23..25
  return o;
}

// The four 24-bit units of a 12-byte group held as three little-endian dwords.
__device__ __forceinline__ void tq3_split_units(const uint32_t d[3], uint32_t u[4]) {
  u[0] = d[0];
  u[1] = __builtin_amdgcn_alignbit(d[1], d[0], 24);
  u[2] = __builtin_amdgcn_alignbit(d[2], d[1], 16);
  u[3] = d[2] >> 8;
}

// ---- TQ3 value group unpack ------------------------------------------------
// A group is 32 codes held as three little-endian dwords, code i at bits
// 3i .. 3i+2.  Read as a ring of 96 bits, any 32-bit window starting at bit b
// is one funnel shift of two of the dwords (no shift for b = 0, 32, 64).  One
// AND-OR of a window keeps two codes, code lo at bits k_lo .. k_lo+2 of the
// low half and code hi at bits 16+k_hi .. 18+k_hi (1 <= k <= 7, inside the
// f16 mantissa field), on top of the exponent of 1.0; subtracting
// 1 + 3.5 * 2^(k-10) leaves (c - 3.5) * 2^(k-10).  Both operands lie in
// [1, 2) and the constant has at most 10 fraction bits because k >= 1, so the
// difference is exact and, as |c - 3.5| >= 1/2, an f16 normal number.  The
// sixteen pairs below, (window start, lo, hi), cover the group with six
// shifted windows; the bit offsets follow from them.  (Value tiles are
// unpacked once per tile by the lane that loads the group, so the whole group
// is at hand; key operands are unpacked per MFMA chunk from units instead.)
struct Tq3Pair {
  int win, lo, hi;
};
constexpr Tq3Pair kValuePairs[16] = {
    {0, 2, 7},    {6, 3, 8},    {6, 4, 9},    {13, 5, 10},  {13, 6, 12},  {32, 11, 17},
    {32, 13, 18}, {40, 14, 19}, {41, 15, 20}, {41, 16, 21}, {64, 22, 28}, {64, 23, 29},
    {70, 24, 30}, {70, 25, 31}, {77, 26, 0},  {77, 27, 1}};
constexpr int kappa_lo(const Tq3Pair& p) { return (3 * p.lo - p.win + 96) % 96; }
constexpr int kappa_hi(const Tq3Pair& p) { return (3 * p.hi - p.win + 96) % 96 - 16; }
constexpr uint32_t pair_mask(const Tq3Pair& p) {
  return (7u << kappa_lo(p)) | (7u << (16 + kappa_hi(p)));
}
constexpr bool is_cover(const Tq3Pair (&t)[16], int kmin) {
  uint32_t seen = 0;
  for (const Tq3Pair& p : t) {
    const int a = kappa_lo(p), b = kappa_hi(p);
    if (a < kmin || a > 7 || b < kmin || b > 7 || p.win < 0 || p.win >= 96) return false;
    const uint32_t bits = (1u << p.lo) | (1u << p.hi);
    if ((seen & bits) != 0 || p.lo == p.hi) return false;
    seen |= bits;
  }
  return seen == 0xFFFFFFFFu;
}
static_assert(is_cover(kValuePairs, 1), "TQ3 value pair cover");
constexpr uint32_t value_center(const Tq3Pair& p) {
  return center_bits(kappa_lo(p)) | (center_bits(kappa_hi(p)) << 16);
}

// Value position 2p + h (half h of pair p) as a byte (dim-in-group | k << 5),
// 8 per 64-bit word, for run-time lookups.
constexpr uint64_t value_pos_word(int w) {
  uint64_t r = 0;
  for (int i = 0; i < 8; ++i) {
    const int pos = 8 * w + i;
    const Tq3Pair& p = kValuePairs[pos / 2];
    const int e = (pos & 1) ? (p.hi | (kappa_hi(p) << 5)) : (p.lo | (kappa_lo(p) << 5));
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

// Value group -> 16 dwords of centred f16 pairs, pair p in dword p.
__device__ __forceinline__ void tq3_value_group(const uint32_t (&w)[3], uint32_t one,
                                                uint32_t (&o)[16]) {
#pragma unroll
  for (int p = 0; p < 16; ++p)
    o[p] = sub_f16x2(and_or(group_window(w, kValuePairs[p].win), pair_mask(kValuePairs[p]), one),
                     value_center(kValuePairs[p]));
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
// rows of the live columns in true units (row stride padded); then per wave
// and column the weight 2^(m_w - M) of that wave's state.
template <int D>
struct MergeLds {
  static constexpr int ROW = D + 4;
  float m[kWaves][16];
  float l[kWaves][16];
  float f[kWaves][16];
  float acc[kWaves][16 * ROW];
};

// Combine the waves' states in M and write the item's partial state of the
// ncol query heads starting at hq0 (all threads of the workgroup call this,
// with M.m, M.l and M.acc written and visible).
template <int D>
__device__ __forceinline__ void merge_waves_and_store(MergeLds<D>& M, const DecodeArgs& a, int chunk,
                                                      int hq0, int ncol) {
  const int64_t base = int64_t(chunk) * a.Hq + hq0;
  float mx = -INFINITY, lsum = 0.0f;
  if (threadIdx.x < 16) {
    // per column: the common reference max and the waves' weights
    const int c = threadIdx.x;
#pragma unroll
    for (int w = 0; w < kWaves; ++w)
      if (M.l[w][c] > 0.0f) mx = fmaxf(mx, M.m[w][c]);
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float f = M.l[w][c] > 0.0f ? exp2f(M.m[w][c] - mx) : 0.0f;
      M.f[w][c] = f;
      lsum += M.l[w][c] * f;
    }
  }
  // (the global stores come after the barrier: a barrier's release fence
  // would otherwise wait for them to reach memory)
  __syncthreads();
  if (int(threadIdx.x) < ncol) {
    a.pm[base + threadIdx.x] = mx;
    a.pl[base + threadIdx.x] = lsum;
  }
  // (a wave without tiles has weight 0 and a zero accumulator, so every wave
  // enters the sum; the loop has its maximum trip count so that all LDS
  // reads can be issued together)
  constexpr int kIter = (16 * D + kThreads - 1) / kThreads;
#pragma unroll
  for (int k = 0; k < kIter; ++k) {
    const int idx = threadIdx.x + kThreads * k;
    const int c = idx / D, dim = idx % D;
    if (c < ncol) {
      float o = 0.0f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) o = __builtin_fmaf(M.acc[w][c * MergeLds<D>::ROW + dim], M.f[w][c], o);
      a.pacc[(base + c) * D + dim] = o;
    }
  }
}

// Softmax step of one tile for the lane's column: scores s (fp32, already
// multiplied by the column's score factor and masked) -> probabilities p;
// rescales the accumulators when the reference max must rise.
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
struct Tq3Lds {
  static constexpr int D = 32 * NG;
  static constexpr int VROW = value_row_bytes(D);
  // key units as [group][token][unit]: a lane stores its group's four units
  // with one 16-byte write, and the 64 lanes reading one unit each for a
  // group hit the 64 banks once
  static constexpr int SD = 16 * NG;            // scale dwords of a tile (K then V)
  struct Wave {
    alignas(16) uint32_t kst[NH][64 * NG];      // key units, [group][token][unit]
    alignas(16) uint8_t vt[NH][16 * VROW];      // value tiles, [token][D] f16
    alignas(16) uint32_t sc[NH][SD + 4];        // tile scales as f16 [K, V][token][group] (padded)
    float corr[16];
  };
  int32_t ent[kMaxChunkPages];                  // page-table entries of the work item
  Wave w[kWaves];
};

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

// ---------------------------------------------------------------------------
// TQ3 work item: the workgroup owns NH kv-heads; each wave a quarter of the tiles
// ---------------------------------------------------------------------------
template <int NG, int NH, int R>
__device__ __forceinline__ void tq3_item(const DecodeArgs& a, const WorkItem& it, uint8_t* smem) {
  auto& lds = *reinterpret_cast<Tq3Lds<NG, NH>*>(smem);
  constexpr int D = 32 * NG;
  constexpr int GPL = NG > 4 ? NG / 4 : 1;      // groups each lane loads per head
  constexpr int NT = D / 16;                    // PV N-tiles per head
  constexpr int VROW = Tq3Lds<NG, NH>::VROW;
  constexpr int ROWB = 3 * D / 8;               // code bytes per token row
  constexpr int SD = Tq3Lds<NG, NH>::SD;
  constexpr int SPL = (SD + 63) / 64;           // scale dwords each lane loads per head

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;                    // token (loads) / head column (outputs)
  const int quad = lane >> 4;
  const PoolView& pv = a.pv;
  stage_entries(lds.ent, a, it);
  const int hk0 = blockIdx.y * NH;               // the workgroup's kv-heads
  if (hk0 >= pv.Hkv) return;
  const int G = a.Hq / pv.Hkv;
  const int ncol = NH * G;
  const int hq0 = hk0 * G;
  const int jcol = col < ncol ? col / G : 0;    // kv-head (within the wave) of column col
  auto& W = lds.w[wave];
  const uint32_t one = vgpr_one_pair();
  // the lane's value-tile reads (head 0, N-tile 0): row 4quad + col/4, dims
  // 4(col & 3) .. +3; a second base for the duplicate read
  const uint8_t* vbase = W.vt[0] + value_row(4 * quad + (col >> 2)) * VROW + 8 * (col & 3);
  const uint8_t* vbase2 = vbase + vgpr_opaque_zero();

  // ---- query operands: slot s of MFMA g holds dim 32g + 8quad + kSlotCode[s],
  // scaled by 2^(E + 7 - kSlotShift[s]) against the key slot's 2^(k-10)
  // (prepared once the first tiles' loads are in flight)
  half8 qop[NH][NG];
  float F;
  auto prepare = [&]() {
    half8 qh[NG];
    const int E = load_query<NG, NH>(
        a, it.b, hq0, col, ncol, jcol, qop, qh,
        [&](const uint16_t* qrow, int g, float (&v)[8]) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + 32 * g + 8 * quad);
#pragma unroll
          for (int s = 0; s < 8; ++s) {
            const int e = kSlotCode[s];
            v[s] = bf16_to_f32(uint16_t(w[e >> 1] >> (16 * (e & 1))));
          }
        },
        [](float x, int E, int s) { return _Float16(__builtin_amdgcn_ldexpf(x, E + 7 - kSlotShift[s])); });
    F = a.scale * kLog2e * __builtin_amdgcn_ldexpf(1.0f, 3 - E);
  };

  f32x4 acc[NT];                                // one per N-tile, both kv-heads' rows
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  SoftState st;

  // Per-lane byte offsets inside a record (the tile's first token is added per
  // tile).  Lane (token col, quad) loads group quad (+4i) of that token; with
  // fewer than 4 groups the spare quads repeat a real group's load, and spare
  // lanes of the scale load repeat a real scale dword (results unused).
  // (unsigned 32-bit lane offsets added to a wave-uniform base address map
  // to loads with a scalar base and a vector offset)
  uint32_t code_off[NH][GPL], sc_off[NH][SPL];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    const uint32_t cb = uint32_t(tq3_codes_off(pv, hk0 + j, 0));
    const uint32_t kb = uint32_t(tq3_scale_off(pv, hk0 + j, 0));
    const uint32_t vb = uint32_t(tq3_scale_off(pv, hk0 + j, 1));
#pragma unroll
    for (int i = 0; i < GPL; ++i) code_off[j][i] = cb + col * ROWB + 12 * ((quad + 4 * i) % NG);
#pragma unroll
    for (int i = 0; i < SPL; ++i) {
      const int e = (lane + 64 * i) & (SD - 1);
      sc_off[j][i] = e < 8 * NG ? kb + 4 * e : vb + 4 * (e - 8 * NG);
    }
  }
  const int vcode_delta = pv.P * ROWB;                  // V codes follow the K codes

  struct Raw {
    uint32_t kc[NH][GPL][3];                    // K codes: one 12-byte group of token col
    uint32_t vc[NH][GPL][3];                    // V codes, same group and token
    uint32_t sc[NH][SPL];                       // the lane's share of the tile's scales
  };
  auto load = [&](const Cursor& c, Raw& r) {
    const auto rec = record_rsrc(entry_page(pv, lds.ent, c.page), pv.tq3_stride);
    const int kso = 16 * c.sub * ROWB;                   // the tile's first K row
    const int vso = kso + vcode_delta;                   // and its first V row
    const int sso = 32 * c.sub * NG;                     // and its scales
#pragma unroll
    for (int j = 0; j < NH; ++j) {
#pragma unroll
      for (int i = 0; i < GPL; ++i) {
        const u32x3 kw = rec_load3(rec, code_off[j][i], kso);
        const u32x3 vw = rec_load3(rec, code_off[j][i], vso);
#pragma unroll
        for (int x = 0; x < 3; ++x) {
          r.kc[j][i][x] = kw[x];
          r.vc[j][i][x] = vw[x];
        }
      }
#pragma unroll
      for (int i = 0; i < SPL; ++i) r.sc[j][i] = rec_load1(rec, sc_off[j][i], sso);
    }
  };
  const TileGeom tg = wave_tiles(it, pv.P / 16, wave);

  // Tile body: the raw buffer is consumed into LDS, refilled with a later
  // tile, and the tile is computed from LDS.
  auto process = [&](Raw& raw, const Cursor& c, auto refill) {
    const int nvalid = valid_in_tile(c, tg);
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      // scales: the lane's dword holds f16 k0 = 2e' and k0 + 1 of the tile's
      // K (e < 8NG) or V block, f16 k being (token k / NG, group k % NG), and
      // is stored in place ([K, V][token][group]).  Value scales of masked
      // tokens become 0 (an unwritten slot may hold NaN, and p = 0 times NaN
      // is NaN).
#pragma unroll
      for (int i = 0; i < SPL; ++i) {
        const int e = lane + 64 * i;
        if (e < SD) {
          const bool is_v = e >= 8 * NG;
          const int k0 = 2 * (is_v ? e - 8 * NG : e);
          const int t0 = k0 / NG, t1 = (k0 + 1) / NG;
          uint32_t w = raw.sc[j][i];
          if (is_v && t0 >= nvalid) w &= 0xFFFF0000u;
          if (is_v && t1 >= nvalid) w &= 0x0000FFFFu;
          W.sc[j][e] = w;
        }
      }
#pragma unroll
      for (int i = 0; i < GPL; ++i) {
        const int g = quad + 4 * i;
        if (g < NG) {
          uint32_t u[4];
          tq3_split_units(raw.kc[j][i], u);
          *reinterpret_cast<u32x4*>(&W.kst[j][64 * g + 4 * col]) = u32x4{u[0], u[1], u[2], u[3]};
          uint32_t o[16];
          tq3_value_group(raw.vc[j][i], one, o);
          uint8_t* vd = W.vt[j] + value_row(col) * VROW + 64 * g;
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4)
            *reinterpret_cast<u32x4*>(vd + 16 * c4) = u32x4{o[4 * c4], o[4 * c4 + 1], o[4 * c4 + 2], o[4 * c4 + 3]};
        }
      }
    }
    refill(raw);
    wave_lds_sync();

    // ---- QK^T per group (the NH kv-heads into one D), scaled per token by
    // the group's key scale of the lane's column's kv-head
    // the lane's tokens 4quad .. 4quad+3 hold 2NG consecutive scale dwords of
    // each block: token 4quad+i, group g is half (i NG + g) & 1 of dword
    // (i NG + g) >> 1
    const uint32_t* scl = W.sc[jcol] + 2 * NG * quad;   // + 8NG: V scales
    uint32_t ksd[2 * NG];
    load_scale_dwords<NG>(scl, ksd);
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      f32x4 dg = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int j = 0; j < NH; ++j) {
        const half8 kop =
            __builtin_bit_cast(half8, tq3_unit_to_f16(W.kst[j][64 * g + 4 * col + quad], one));
        dg = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[j][g], dg, 0, 0, 0);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[i] = __builtin_fmaf(dg[i], f16_half(ksd[(i * NG + g) >> 1], (i * NG + g) & 1), s[i]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] *= F;
    if (nvalid < 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * quad + i >= nvalid) s[i] = -INFINITY;
    }
    float p[4];
    softmax_step(st, s, p, acc, W.corr, col, quad);

    // ---- per group: P' = p * value scale (hi/lo f16), acc_j += P' * V_j
    uint32_t vsd[2 * NG];
    load_scale_dwords<NG>(scl + 8 * NG, vsd);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float sv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) sv[i] = f16_half(vsd[(i * NG + g) >> 1], (i * NG + g) & 1);
      const half8 pp = pprime(p, sv);
      if constexpr (NH == 2) {
        half8 a_hi, a_lo;
        split_pprime(pp, jcol == 1, a_hi, a_lo);
#pragma unroll
        for (int jt = 2 * g; jt < 2 * g + 2; ++jt) {
          const half8 bv = value_operand_heads(vbase + 32 * jt, vbase + 16 * VROW + 32 * jt);
          acc[jt] = pv_mfma(a_hi, bv, acc[jt]);
          acc[jt] = pv_mfma(a_lo, bv, acc[jt]);
        }
      } else {
#pragma unroll
        for (int jt = 2 * g; jt < 2 * g + 2; ++jt)
          acc[jt] = pv_mfma(pp, value_operand(vbase + 32 * jt, vbase2 + 32 * jt), acc[jt]);
      }
    }
    wave_lds_sync();
  };
  run_tiles<R, Raw>(tg, a.pace != 0, load, prepare, process);

  // ---- combine the four waves' states through LDS (the tile staging is
  // reused once every wave is past its last tile) and write the item's state
  const float lcol = quad_sum(st.l);
  __syncthreads();
  auto& M = *reinterpret_cast<MergeLds<D>*>(smem);
  if (quad == 0) {
    M.m[wave][col] = st.m;
    M.l[wave][col] = lcol;
  }
  // accumulator column col of N-tile jt holds value position 16 (jt & 1) + col
  // of group jt / 2 (half pos & 1 of value pair pos / 2), scaled by 2^(k-10)
  const uint64_t we = (col & 8) ? kValuePos[1] : kValuePos[0];
  const uint64_t wo = (col & 8) ? kValuePos[3] : kValuePos[2];
  const int ee = int(we >> (8 * (col & 7))) & 255, eo = int(wo >> (8 * (col & 7))) & 255;
  const float up_e = __builtin_amdgcn_ldexpf(1.0f, 10 - (ee >> 5));
  const float up_o = __builtin_amdgcn_ldexpf(1.0f, 10 - (eo >> 5));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = 4 * quad + i;
    if (c >= ncol) continue;
    float* dst = M.acc[wave] + c * MergeLds<D>::ROW;
#pragma unroll
    for (int jt = 0; jt < NT; ++jt)
      dst[32 * (jt >> 1) + ((jt & 1) ? (eo & 31) : (ee & 31))] = acc[jt][i] * ((jt & 1) ? up_o : up_e);
  }
  __syncthreads();
  merge_waves_and_store<D>(M, a, it.chunk, hq0, ncol);
}

// ---------------------------------------------------------------------------
// FP8 work item: the workgroup owns NH kv-heads; each wave a quarter of the tiles
// ---------------------------------------------------------------------------
template <int NG, int NH, int R>
__device__ __forceinline__ void fp8_item(const DecodeArgs& a, const WorkItem& it, uint8_t* smem) {
  auto& lds = *reinterpret_cast<Fp8Lds<NG, NH>*>(smem);
  constexpr int D = 32 * NG;
  constexpr int NT = D / 16;
  constexpr int VROW = Fp8Lds<NG, NH>::VROW;
  constexpr int LB = D / 4;                     // bytes of a row each lane loads

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

  // ---- query operand: MFMA r, lane (col, quad), slot s <-> dim quad*LB + 8r + s
  // (prepared once the first tiles' loads are in flight)
  half8 qop[NH][NG];
  float F;
  auto prepare = [&]() {
    half8 qh[NG];
    const int E = load_query<NG, NH>(
        a, it.b, hq0, col, ncol, jcol, qop, qh,
        [&](const uint16_t* qrow, int r, float (&v)[8]) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(qrow + quad * LB + 8 * r);
#pragma unroll
          for (int s = 0; s < 8; ++s) v[s] = bf16_to_f32(uint16_t(w[s >> 1] >> (16 * (s & 1))));
        },
        [](float x, int E, int) { return _Float16(__builtin_amdgcn_ldexpf(x, E)); });
    F = a.scale * kLog2e * __builtin_amdgcn_ldexpf(1.0f, -E);
  };

  f32x4 acc[NT];                                // one per N-tile, both kv-heads' rows
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  SoftState st;

  uint32_t code_off[NH], ks_off[NH], vs_off[NH];
#pragma unroll
  for (int j = 0; j < NH; ++j) {
    code_off[j] = uint32_t(fp8_codes_off(pv, hk0 + j, 0)) + col * D + quad * LB;
    ks_off[j] = uint32_t(fp8_scale_off(pv, hk0 + j, 0));
    vs_off[j] = uint32_t(fp8_scale_off(pv, hk0 + j, 1));
  }
  const int vcode_delta = pv.P * D;
  struct Raw {
    uint32_t kw[NH][LB / 4];
    uint32_t vw[NH][LB / 4];
    float sigk[NH], sigv[NH];
  };
  auto load = [&](const Cursor& c, Raw& r) {
    const auto rec = record_rsrc(entry_page(pv, lds.ent, c.page), pv.fp8_stride);
    const int kso = 16 * c.sub * D;                      // the tile's first K row
    const int vso = kso + vcode_delta;                   // and its first V row
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      if constexpr (LB % 16 == 0) {
#pragma unroll
        for (int x = 0; x < LB / 16; ++x) {
          const u32x4 kw = rec_load4(rec, code_off[j] + 16 * x, kso);
          const u32x4 vw = rec_load4(rec, code_off[j] + 16 * x, vso);
#pragma unroll
          for (int y = 0; y < 4; ++y) {
            r.kw[j][4 * x + y] = kw[y];
            r.vw[j][4 * x + y] = vw[y];
          }
        }
      } else {
        static_assert(LB == 8, "an FP8 lane row share is 8 or a multiple of 16 bytes");
        const u32x2 kw = rec_load2(rec, code_off[j], kso);
        const u32x2 vw = rec_load2(rec, code_off[j], vso);
        r.kw[j][0] = kw[0];
        r.kw[j][1] = kw[1];
        r.vw[j][0] = vw[0];
        r.vw[j][1] = vw[1];
      }
      r.sigk[j] = __builtin_bit_cast(float, rec_load1(rec, 0, ks_off[j]));
      r.sigv[j] = __builtin_bit_cast(float, rec_load1(rec, 0, vs_off[j]));
    }
  };
  const TileGeom tg = wave_tiles(it, pv.P / 16, wave);

  auto process = [&](Raw& raw, const Cursor& c, auto refill) {
    const int nvalid = valid_in_tile(c, tg);
    // ---- values: f16 rows of the LDS tiles (rows past the valid tokens zeroed)
    const bool vrow_ok = col < nvalid;
#pragma unroll
    for (int j = 0; j < NH; ++j)
#pragma unroll
      for (int i = 0; i < LB / 4; i += 2) {
        const u32x2 a0 = fp8x4_to_f16(raw.vw[j][i]);
        const u32x2 a1 = fp8x4_to_f16(raw.vw[j][i + 1]);
        u32x4 o = {a0[0], a0[1], a1[0], a1[1]};
        if (!vrow_ok) o = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(W.vt[j] + value_row(col) * VROW + 2 * (quad * LB + 4 * i)) = o;
      }
    // ---- QK^T over all dims, per kv-head, keys widened to f16 operands from
    // the raw words (page-head scale applied per column)
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float sv = raw.sigv[0];
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      f32x4 dsum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int r = 0; r < NG; ++r) {
        const u32x2 k0 = fp8x4_to_f16(raw.kw[j][2 * r]);
        const u32x2 k1 = fp8x4_to_f16(raw.kw[j][2 * r + 1]);
        const u32x4 ku = {k0[0], k0[1], k1[0], k1[1]};
        dsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8, ku), qop[j][r], dsum, 0, 0, 0);
      }
      const float fk = jcol == j ? F * raw.sigk[j] : 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) s[i] = __builtin_fmaf(dsum[i], fk, s[i]);
      if (j > 0) sv = jcol == j ? raw.sigv[j] : sv;
    }
    refill(raw);
    wave_lds_sync();
    if (nvalid < 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (4 * quad + i >= nvalid) s[i] = -INFINITY;
    }
    float p[4];
    softmax_step(st, s, p, acc, W.corr, col, quad);

    const half8 pp = pprime_uniform(p, sv);
    if constexpr (NH == 2) {
      half8 a_hi, a_lo;
      split_pprime(pp, jcol == 1, a_hi, a_lo);
#pragma unroll
      for (int jt = 0; jt < NT; ++jt) {
        const half8 bv = value_operand_heads(vbase + 32 * jt, vbase + 16 * VROW + 32 * jt);
        acc[jt] = pv_mfma(a_hi, bv, acc[jt]);
        acc[jt] = pv_mfma(a_lo, bv, acc[jt]);
      }
    } else {
#pragma unroll
      for (int jt = 0; jt < NT; ++jt)
        acc[jt] = pv_mfma(pp, value_operand(vbase + 32 * jt, vbase2 + 32 * jt), acc[jt]);
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
    float* dst = M.acc[wave] + c * MergeLds<D>::ROW;
#pragma unroll
    for (int jt = 0; jt < NT; ++jt) dst[16 * jt + col] = acc[jt][i];
  }
  __syncthreads();
  merge_waves_and_store<D>(M, a, it.chunk, hq0, ncol);
}

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
// ---------------------------------------------------------------------------
template <int NG, int NH>
struct PartialCfg {
  static constexpr int kRingTq3 = 2;                 // TQ3 tiles in flight per wave
  // FP8 rows are 4x the TQ3 bytes: one tile in flight with two kv-heads or
  // head dim 256, within the register budget of the waves per SIMD
  static constexpr int kRingFp8 = NH == 1 && NG < 8 ? 2 : 1;
  static constexpr size_t cmax(size_t x, size_t y) { return x > y ? x : y; }
  static constexpr size_t kSmem =
      cmax(cmax(sizeof(Tq3Lds<NG, NH>), sizeof(Fp8Lds<NG, NH>)), sizeof(MergeLds<32 * NG>));
};

// Three waves per SIMD (168 VGPRs) at head dim <= 128 -- two kv-heads per
// wave fit because they share one accumulator per N-tile; two waves at 256.
template <int NG, int NH>
__global__ void __launch_bounds__(kThreads, NG < 8 ? 3 : 2) partial_mixed(DecodeArgs a) {
  using Cfg = PartialCfg<NG, NH>;
  __shared__ __attribute__((aligned(16))) uint8_t smem[Cfg::kSmem];
  const WorkItem it = a.items[blockIdx.x];
  if (it.fmt == 0)
    fp8_item<NG, NH, Cfg::kRingFp8>(a, it, smem);
  else
    tq3_item<NG, NH, Cfg::kRingTq3>(a, it, smem);
}

// Control pools: every work item is BF16.  Two waves per SIMD; one tile in
// flight (a BF16 tile row share is 4x the TQ3 one).
template <int NG, int NH>
__global__ void __launch_bounds__(kThreads, 2) partial_bf16(DecodeArgs a) {
  constexpr size_t kSmem = PartialCfg<NG, NH>::cmax(sizeof(Fp8Lds<NG, NH>), sizeof(MergeLds<32 * NG>));
  __shared__ __attribute__((aligned(16))) uint8_t smem[kSmem];
  const WorkItem it = a.items[blockIdx.x];
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
    hipLaunchKernelGGL(kernel, grid, dim3(kThreads), 0, s, a);
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
