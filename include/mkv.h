/*
 * mkv.h — C-ABI of libmkv: decode attention run directly over a paged KV cache
 * whose pages are held in mixed numeric formats (FP8 anchors, packed TQ3
 * archive), for AMD Instinct MI355X (gfx950).
 *
 * What the library implements (Minima-KV summaries, brainszone.ai, pt and fr):
 *  - "O que os autores propoem": the KV cache is a hierarchy of pages and each
 *    page is stored in its own numeric format.
 *  - "Ancoras em FP8, arquivo em TQ3": recent and anchor pages stay FP8, older
 *    non-anchor pages are converted to packed TQ3, and every page of a live
 *    request stays directly addressable.
 *  - "Como os resultados parciais sao combinados": per-format kernels produce
 *    partial attention states that a globally normalised online-softmax merge
 *    combines, so decode runs on the heterogeneous cache with no dense
 *    single-format copy.
 *
 * Formats (the pages name them but fix no layout; this library fixes):
 *  - FP8 = OCP E4M3 with one fp32 scale per (page, kv-head, K or V):
 *    sigma = amax / 448 (1.0 when amax == 0), codes rounded to nearest-even,
 *    saturating at +-448.
 *  - TQ3 = per 32-element group of head_dim an fp16 scale s = absmax / 3.5 and
 *    32 three-bit codes c decoding to (c - 3.5) * s, packed as a little-endian
 *    bit stream of 12 bytes (code j of a token row at stream bit 3j).
 *  - Page records, with Hkv kv-heads, head dim d and P tokens per page:
 *      FP8: codes [Hkv][2 (K,V)][P][d] u8 | scale [Hkv][2] f32 | amax [Hkv][2] f32
 *      TQ3: per kv-head h a block of P*d*7/8 bytes:
 *           K codes [P][3d/8] | V codes [P][3d/8] | K scale [P][d/32] f16 | V scale [P][d/32] f16
 *  - Page-table entry: int32, bit 31 = format (0 FP8, 1 TQ3), bits 0..30 =
 *    physical page index in that format's slab.
 *
 * Control pools (kv_kind = MKV_KIND_BF16): the dense single-format cache the
 * summaries measure the mixed cache against (section "O que as medicoes
 * mostram", subsection "Memoria e compressao": compression relative to BF16
 * and to FP8; section "Verificacao canario": the canary's throughput relative
 * to its control).  Every row is stored as bf16, rounded to nearest even;
 * record [Hkv][2 (K,V)][P][d] bf16, in the slab that holds FP8 pages in a
 * mixed pool (fp8_pages is its capacity, tq3_pages must be 0); page-table
 * entries have bit 31 clear.  mkv_append stores bf16 rows, mkv_demote
 * returns MKV_ESTATE, mkv_decode runs a BF16 partial kernel and the same
 * merge.  The all-FP8 comparison needs no special pool: a mixed pool whose
 * pages are never demoted.
 *
 * Conventions shared by every call:
 *  - All functions are extern "C"; no C++ exception crosses the boundary.
 *  - Device pointers are plain HIP device addresses (e.g. from a torch tensor).
 *    Host pointers are marked "host".
 *  - Every device effect is enqueued on the caller's stream and the call
 *    returns without waiting, except mkv_pool_create, mkv_pool_destroy and the
 *    calls documented as synchronous.  All calls on one pool must be issued
 *    from one host thread, on one stream (or the caller orders the streams).
 *  - A call validates all of its arguments and capacity before it enqueues any
 *    work or changes any metadata: a non-OK status leaves the pool's metadata
 *    (lengths, page tables, free pages) unchanged.  When a HIP call fails after
 *    the metadata was changed (MKV_EHIP from mkv_append, mkv_append_step,
 *    mkv_demote or mkv_materialize), the change is rolled back; work already
 *    enqueued before the failing HIP call may still run, but it only writes
 *    pages and page-table slots the restored metadata does not reference, and
 *    the cached decode schedule is rebuilt by the next mkv_decode.
 *  - Errors: MKV_EINVAL bad argument, MKV_ENOMEM a slab has too few free
 *    pages, MKV_ESTATE an operation the sequence's state forbids, MKV_ERANGE a
 *    capacity of the pool descriptor is exceeded, MKV_EHIP a HIP runtime
 *    error (text in mkv_last_error()).
 */
#ifndef MKV_H
#define MKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MKV_OK = 0,
  MKV_EINVAL = -1,
  MKV_ENOMEM = -2,
  MKV_ESTATE = -3,
  MKV_ERANGE = -4,
  MKV_EHIP = -5
} mkv_status;

enum { MKV_FMT_FP8 = 0, MKV_FMT_TQ3 = 1, MKV_FMT_BF16 = 2 };
enum { MKV_KIND_MIXED = 0, MKV_KIND_BF16 = 1 };

typedef struct mkv_pool mkv_pool; /* opaque; owned by the library */

/* Pool geometry and capacities.  Limits: 1 <= num_kv_heads <= 64;
 * head_dim in {32, 64, 128, 256}; page_size a multiple of 16, at most 256. */
typedef struct {
  int32_t num_kv_heads;      /* Hkv */
  int32_t head_dim;          /* d */
  int32_t page_size;         /* P tokens per page */
  int32_t max_seqs;          /* sequence ids are 0 .. max_seqs-1 */
  int32_t max_pages_per_seq; /* page-table row length */
  int32_t max_batch;         /* largest B accepted by mkv_decode */
  int32_t max_q_heads;       /* largest Hq accepted by mkv_decode */
  int32_t max_chunks;        /* partial-state slots per decode; 0 = library default,
                                max(4096 + 2 * max_batch, floor below); a nonzero value
                                must be >= max_batch * (2 + ceil(max_pages_per_seq / 256)),
                                since a split-K chunk spans at most 256 pages */
  int64_t fp8_pages;         /* FP8 slab capacity in pages */
  int64_t tq3_pages;         /* TQ3 slab capacity in pages */
  uint64_t placement_seed;   /* 0: pages handed out in index order; else a seeded shuffle */
  int32_t kv_kind;           /* MKV_KIND_MIXED (0): FP8/TQ3 cache; MKV_KIND_BF16: control pool */
} mkv_pool_desc;

typedef struct {
  int64_t live_tokens;
  int64_t fp8_pages_live, tq3_pages_live;
  int64_t fp8_pages_free, tq3_pages_free;
  int64_t kv_bytes;            /* algorithmic bytes one decode of all live tokens reads:
                                  codes + TQ3 group scales + FP8 page-head scales */
  double bytes_per_token;      /* kv_bytes / live_tokens (one layer) */
  double ratio_vs_bf16;        /* (2 * Hkv * d * 2 bytes) / bytes_per_token */
  double ratio_vs_fp8;         /* (2 * Hkv * d * 1 byte) / bytes_per_token */
  int64_t dense_shadow_bytes;  /* always 0: no dense single-format copy exists */
  int64_t dense_fallbacks;     /* always 0: decode never leaves the mixed path */
} mkv_stats;

/* Per-kernel device time accumulated while profiling is on (milliseconds):
 * the partial kernel (both formats, one launch per decode), the merge, the
 * cache-write launches that append (mkv_append, mkv_append_step, and the one
 * launch of an mkv_decode_step, which may convert pages too) and the
 * conversion launches (mkv_demote, and mkv_decode_step's separate ones). */
typedef struct {
  double ms_partial, ms_merge;
  int64_t n_partial, n_merge;
  double ms_append, ms_demote;
  int64_t n_append, n_demote;
} mkv_profile;

/* Device bytes a pool with this descriptor needs (slabs, page tables,
 * schedule and partial-state workspace).  Returns 0 for an invalid descriptor. */
size_t mkv_pool_bytes(const mkv_pool_desc* desc);

/* Bytes of one page record of the given format (layout above): MKV_FMT_FP8
 * or MKV_FMT_TQ3 for a mixed pool, MKV_FMT_BF16 for a control pool; 0 if the
 * format does not belong to the descriptor's kind or the descriptor is invalid. */
size_t mkv_record_bytes(const mkv_pool_desc* desc, int32_t fmt);

/* Create a pool on the current HIP device.  device_mem: NULL to let the
 * library hipMalloc mkv_pool_bytes(desc) bytes (freed by mkv_pool_destroy), or
 * a caller-owned device buffer of at least that many bytes that must outlive
 * the pool.  Synchronous.  *out receives the pool on MKV_OK. */
mkv_status mkv_pool_create(const mkv_pool_desc* desc, void* device_mem, size_t bytes,
                           mkv_pool** out);

/* Destroy a pool: waits for the device, frees library-owned memory. */
mkv_status mkv_pool_destroy(mkv_pool* pool);

/* Free every page of sequence `seq` and set its length to 0 (host metadata
 * immediately; freed pages are reused in stream order). */
mkv_status mkv_seq_reset(mkv_pool* pool, int32_t seq, hipStream_t stream);

/* Append n tokens to sequence `seq` as FP8 ("Ancoras em FP8": new pages start
 * FP8; in a control pool, as bf16 rows rounded to nearest even, with none of
 * the scale handling below).  k, v: device fp32 [n][Hkv][d], row-major,
 * finite values, 16-byte aligned (MKV_EINVAL otherwise).  New pages
 * come from the FP8 free list.  The FP8 scale of a page-head is recomputed when
 * new rows raise its running amax and the page's earlier rows are re-encoded
 * against it, so a page filled by one call equals one-shot quantisation.
 * MKV_ESTATE if the sequence's last page is TQ3 and partially filled;
 * MKV_ENOMEM if the FP8 slab lacks pages; MKV_ERANGE past max_pages_per_seq. */
mkv_status mkv_append(mkv_pool* pool, int32_t seq, int32_t n, const float* k, const float* v,
                      hipStream_t stream);

/* One decode step's new rows: append one token to each of B distinct
 * sequences, row b of k and v (device fp32 [B][Hkv][d], 16-byte aligned) to
 * seq_ids[b] (host int32 [B]), with one kernel launch; otherwise as mkv_append (FP8 rows with
 * rescale-on-grow, or bf16 rows in a control pool).  A sequence whose last
 * page is full gets a new FP8 page.  All sequences are validated before any
 * changes (MKV_EINVAL for a repeated or bad id, MKV_ESTATE for a frozen TQ3
 * tail, MKV_ENOMEM, MKV_ERANGE for B > max_batch or a full page table).  The
 * caller decides which pages leave the recent window and calls mkv_demote
 * ("Ancoras em FP8, arquivo em TQ3": recent and protected pages stay FP8).
 * With B <= 32 the step copies nothing to the device: the plan goes in the
 * kernel arguments, and when no page opens the same launch refreshes the
 * token counts of the pool's cached decode schedule, so the next mkv_decode
 * of that batch (on the same stream) uploads nothing either. */
mkv_status mkv_append_step(mkv_pool* pool, const int32_t* seq_ids, int32_t B, const float* k,
                           const float* v, hipStream_t stream);

/* Convert the listed logical pages of `seq` from FP8 to packed TQ3
 * ("Ancoras em FP8, arquivo em TQ3": older non-anchor pages are converted).
 * logical_pages: host int32 [n], distinct, each an FP8 page of the sequence.
 * Each page gets a TQ3 page, its page-table entry is rewritten and the FP8
 * page returns to the free list.  Codes: x = fp32(e4m3(c) * sigma) per element,
 * then per 32-group s = fp16(fp32(absmax / 3.5)) (clamped to 65504) and
 * c = #{b in -3..3 : x >= b*s} (c = 4 when s == 0).  Demoting a partially
 * filled last page is allowed; the sequence then accepts no more appends.
 * The pool's cached decode schedule moves the converted pages from FP8 to
 * TQ3 work items where it can (else the next decode rebuilds it).
 * MKV_ESTATE in a control pool (n > 0). */
mkv_status mkv_demote(mkv_pool* pool, int32_t seq, const int32_t* logical_pages, int32_t n,
                      hipStream_t stream);

/* Anchor policy of mkv_decode_step ("Ancoras em FP8, arquivo em TQ3": recent
 * and protected pages stay FP8, older ones are converted).  window_tokens >= 0
 * turns it on: after each step's append, every FP8 page of a stepped sequence
 * whose tokens all lie before the sequence's last window_tokens tokens, that
 * is not protected and that the policy has not passed before, is converted to
 * TQ3 (as mkv_demote).  Each sequence keeps a cursor: pages below it were
 * passed, and a page passed while protected keeps its format for good.
 * window_tokens < 0 turns the policy off (the default).  MKV_ESTATE for a
 * control pool with window_tokens >= 0. */
mkv_status mkv_set_anchor_window(mkv_pool* pool, int32_t window_tokens);

/* Marks (protect != 0) or clears the listed logical pages of `seq` as
 * protected from the anchor policy (attention sinks, pages the caller pins).
 * lps: host int32 [n], each in [0, max_pages_per_seq) (pages may lie past the
 * sequence's current end).  mkv_seq_reset clears a sequence's marks and its
 * policy cursor.  MKV_EINVAL for a bad id or page. */
mkv_status mkv_protect_pages(mkv_pool* pool, int32_t seq, const int32_t* lps, int32_t n, int32_t protect);

/* One step of a decode loop: mkv_append_step(seq_ids, B, k, v), then the
 * anchor policy's conversions for the stepped sequences (mkv_set_anchor_window),
 * then mkv_decode(seq_ids, B, q, Hq, softmax_scale, out, lse), all on
 * `stream` in that order, from one call.  k, v: device fp32 [B][Hkv][d]
 * (row b to seq_ids[b]); q, out, lse as in mkv_decode.  Arguments, the
 * append's metadata and the TQ3 capacity for the conversions are checked
 * before anything is enqueued: any error there (MKV_EINVAL, MKV_ERANGE,
 * MKV_ESTATE, MKV_ENOMEM as in the three calls) leaves the pool unchanged.
 * Past that point only device-side failures remain: MKV_EHIP from the
 * append leaves the pool unchanged; MKV_EHIP from the conversions keeps the
 * append and takes every conversion back (the policy's cursors do not move,
 * so the next step retries them); MKV_EHIP, or MKV_ERANGE for a batch over
 * max_chunks chunks, from the decode keeps the append and the conversions.
 * A step that opens no page and converts nothing (with B <= 32) uploads
 * nothing; otherwise its metadata goes up in batched upload launches and the
 * conversions in one launch. */
mkv_status mkv_decode_step(mkv_pool* pool, const int32_t* seq_ids, int32_t B, const float* k,
                           const float* v, const void* q, int32_t Hq, float softmax_scale, float* out,
                           float* lse, hipStream_t stream);

/* Decode attention for one query token per sequence ("Como os resultados
 * parciais sao combinados").  seq_ids: host int32 [B] of non-empty sequences.
 * q: device bf16 [B][Hq][d], 16-byte aligned; query head h reads kv-head
 * h / (Hq / Hkv).
 * softmax_scale: fp32 factor on <q, k>.  out: device fp32 [B][Hq][d];
 * lse: device fp32 [B][Hq], natural-log log-sum-exp of the scaled scores.
 * One partial-kernel launch reduces split-K page chunks of each sequence,
 * each chunk in its own format (FP8 and TQ3 code paths), and a merge kernel
 * combines their (max, denominator, unnormalised accumulator) states (a
 * per-lane merge when no sequence has more than 16 chunks, else a
 * wave-reduced one).  The split-K schedule is cached per pool and rebuilt
 * only when the batch or Hq changed, or pages changed in a way the pool could
 * not fold into it (mkv_append_step and mkv_demote edit the cached schedule
 * for the pages they open or convert where they can; token counts are
 * patched); the result of a given schedule is bit-reproducible.
 * MKV_EINVAL for B < 1, an id outside [0, max_seqs), an empty sequence, Hq
 * not a multiple of Hkv, Hq / Hkv > 16, or a misaligned q;
 * MKV_ERANGE for B > max_batch or Hq > max_q_heads. */
mkv_status mkv_decode(mkv_pool* pool, const int32_t* seq_ids, int32_t B, const void* q,
                      int32_t Hq, float softmax_scale, float* out, float* lse,
                      hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): mkv_decode
 * with the same arguments, kernels, results and errors, except that the
 * partial states live in a fixed workspace of 16 MiB that the library holds on
 * every GPU it runs on (from module load until the process ends) instead of in
 * the pool.  No call allocates or frees device memory, and nothing is
 * cleared: every state the merge reads is written by the same call first.
 * Capacity: n_chunks * Hq * (d + 2) * 4 bytes (plus alignment) of partial
 * states, where n_chunks is the split-K chunk count of the batch; a batch over
 * that limit returns MKV_ERANGE before any work is enqueued.  All calls on one
 * GPU share its workspace, which keeps the last call's contents: calls that
 * overlap on one GPU (concurrent streams, or pools of one device used from
 * several threads) race and must be ordered by the caller. */
mkv_status mkv_decode_static(mkv_pool* pool, const int32_t* seq_ids, int32_t B, const void* q,
                             int32_t Hq, float softmax_scale, float* out, float* lse,
                             hipStream_t stream);

/* Materialising profile (Minima-KV summary, "Qualidade em contexto longo":
 * the hybrid pages expanded into dense tensors, a diagnostic the decode path
 * never uses).  Appends every token of sequence src_seq of the mixed pool src
 * to the empty sequence dst_seq of the control pool dst (kv_kind
 * MKV_KIND_BF16, same num_kv_heads, head_dim and page_size, same device), one
 * destination page per source page.  Each element is the fp32 value the
 * decode kernels use -- fp32(e4m3(c) * sigma) for an FP8 page, (c - 3.5) * s
 * for a TQ3 page -- rounded to bf16 (nearest even).  mkv_decode on dst then
 * runs dense attention over the materialised rows.  Both pools must be used
 * on `stream` (or ordered by the caller).
 * MKV_EINVAL for pools of the wrong kinds or geometries, an empty source, or
 * bad ids; MKV_ESTATE if dst_seq is not empty; MKV_ENOMEM / MKV_ERANGE if dst
 * lacks pages. */
mkv_status mkv_materialize(mkv_pool* src, int32_t src_seq, mkv_pool* dst, int32_t dst_seq,
                           hipStream_t stream);

/* Introspection (host metadata; no device work). */
mkv_status mkv_seq_info(mkv_pool* pool, int32_t seq, int32_t* len, int32_t* n_pages);
/* entries: host int32 [cap] receives the sequence's page-table entries. */
mkv_status mkv_page_table(mkv_pool* pool, int32_t seq, int32_t* entries, int32_t cap);
mkv_status mkv_pool_stats(mkv_pool* pool, mkv_stats* out);

/* Copy the records of logical pages first .. first+n-1 of `seq`, read through
 * the device page table with the same address function the partial kernels
 * use, into dst (device), one slot of max(record bytes) per page in logical
 * order.  For checking placement and packing. */
mkv_status mkv_debug_gather(mkv_pool* pool, int32_t seq, int32_t first, int32_t n, void* dst,
                            hipStream_t stream);

/* Read-bandwidth calibration (not part of the decode path): one kernel reads
 * every byte of src (device, `bytes` a multiple of 16, 16-byte aligned) once
 * with 16-byte loads, the access the partial kernel's record loads use.  A
 * lane writes to sink (device, 256 uint32, caller-owned) only when the XOR of
 * the data it read equals one fixed constant, which keeps the loads live;
 * timing the call gives the device's read ceiling for the roofline.
 * MKV_EINVAL for a null pointer, a misaligned src or a size not a multiple of
 * 16. */
mkv_status mkv_debug_read_bandwidth(const void* src, size_t bytes, uint32_t* sink, hipStream_t stream);

/* The decode schedule the device holds: the one the pool's last mkv_decode
 * used, with the edits later mkv_append_step and mkv_demote calls made to it.
 * Synchronous (waits for the device, then copies).  `info` receives the
 * counts.  items_host (8 int32 per work item, FP8 items first: batch entry,
 * sequence, page-list offset, pages, valid tokens of the last page, partial-
 * state slot, format 0 FP8 / 1 TQ3, last logical page), entries_host (the
 * page-table entries of the items' page lists, in list order) and
 * chunk_base_host (B + 1 partial-slot offsets by batch entry) may be NULL; a
 * non-NULL buffer smaller than its part gives MKV_ERANGE.  MKV_ESTATE when the
 * pool holds no current schedule (no decode since the last change that the
 * cached schedule could not absorb). */
typedef struct {
  int32_t batch;           /* B of the decoded batch */
  int32_t n_items;         /* work items */
  int32_t n_list;          /* page-list entries in use */
  int32_t n_chunks;        /* partial-state slots */
  int32_t max_seq_chunks;  /* most slots of one batch entry */
  int32_t heads_per_wave;  /* kv-heads per partial-kernel workgroup */
  int32_t resident_waves;  /* partial-kernel waves the device holds at once (a schedule below the
                              split-K floor fills three quarters of them where four fit a SIMD,
                              all of them otherwise) */
  int32_t pad0;
} mkv_schedule_info;
mkv_status mkv_debug_schedule(mkv_pool* pool, mkv_schedule_info* info, int32_t* items_host,
                              int32_t items_cap, int32_t* entries_host, int32_t entries_cap,
                              int32_t* chunk_base_host, int32_t base_cap);

/* Profiling: when enabled, the calls bracket each kernel with HIP events;
 * mkv_profile_read waits for the device and returns the accumulated times
 * (then clears them). */
mkv_status mkv_profile_enable(mkv_pool* pool, int32_t on);
mkv_status mkv_profile_read(mkv_pool* pool, mkv_profile* out);

const char* mkv_status_string(mkv_status s);
const char* mkv_last_error(void); /* thread-local detail of the last error */

#ifdef __cplusplus
}
#endif

#endif /* MKV_H */
