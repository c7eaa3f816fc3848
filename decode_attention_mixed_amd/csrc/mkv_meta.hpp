// Host-side metadata of a mixed-format page pool: geometry, slab free lists,
// page tables, sequence lengths and the split-K decode schedule.
//
// Pure C++17 with no HIP dependency, so it is unit-tested on the CPU.  The
// device mirrors (page table, schedule) are uploaded by the ABI layer.
//
// Page-table entries: bit 31 = format (0 FP8, 1 TQ3), bits 0..30 = physical
// page index in that format's slab.  Every live page of a sequence keeps an
// entry for as long as the sequence holds it (Minima-KV summary, brainszone.ai,
// section "Ancoras em FP8, arquivo em TQ3": pages stay addressable; conversion
// re-encodes a page, it never drops one).
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "mkv_status.h"

namespace mkv {

constexpr int32_t kPtTq3Bit = int32_t(0x80000000u);
constexpr int32_t kPtIndexMask = 0x7FFFFFFF;
constexpr int kSlabAlign = 256;

inline bool pt_is_tq3(int32_t e) { return e < 0; }
inline int32_t pt_index(int32_t e) { return e & kPtIndexMask; }
inline int32_t pt_make(int fmt, int32_t idx) { return fmt ? (idx | kPtTq3Bit) : idx; }

// Pool kinds: the mixed FP8/TQ3 cache, or the dense BF16 control cache (one
// slab of BF16 pages, held in the FP8 slab's place; no TQ3 slab, no demotion).
constexpr int32_t kKindMixed = 0;
constexpr int32_t kKindBf16 = 1;

struct Desc {  // mirror of mkv_pool_desc (kept free of the C header's HIP include)
  int32_t Hkv, d, P, max_seqs, max_pages_per_seq, max_batch, max_q_heads, max_chunks;
  int64_t fp8_pages, tq3_pages;
  uint64_t placement_seed;
  int32_t kind;
};

struct Geom {
  int32_t Hkv = 0, d = 0, P = 0;
  int32_t kind = kKindMixed;
  int64_t fp8_rec = 0, tq3_rec = 0;       // record bytes (fp8_rec: BF16 record in a control pool)
  int64_t fp8_stride = 0, tq3_stride = 0; // slab strides (records rounded up to 256 B)
  int32_t max_chunks = 0;                 // resolved partial-state capacity
};

// Validates a descriptor and derives the geometry.  Returns MKV_OK or MKV_EINVAL.
int validate_desc(const Desc& d, Geom* g, std::string* err);

// Free list of physical page indices.  With seed 0 pages are handed out in
// index order; otherwise the order is a seeded Fisher-Yates shuffle.
class FreeList {
 public:
  void init(int64_t n, uint64_t seed);
  int64_t size() const { return int64_t(stack_.size()); }
  int32_t pop() { int32_t v = stack_.back(); stack_.pop_back(); return v; }
  void push(int32_t v) { stack_.push_back(v); }
 private:
  std::vector<int32_t> stack_;
};

struct Seq {
  int32_t len = 0;
  std::vector<int32_t> pt;  // one entry per logical page
};

// One page an append touches: rows row0 .. row0+nrows-1 of page `phys`
// receive source rows src_row .. src_row+nrows-1.  pt_slot >= 0: the append
// also writes page-table entry pt_entry at that index of the device page
// table (a decode step's batched append opens pages this way).
struct AppendPage {
  int32_t lp, phys, row0, nrows, src_row, pt_slot, pt_entry, pad0;
};
// One page a demote converts.
struct DemotePage {
  int32_t lp, src_phys, dst_phys, ntok, pad0, pad1, pad2, pad3;
};
// One page the materialising copy expands: the source page-table entry (either
// format) and the destination page of a BF16 control pool.
struct MaterialisePage {
  int32_t lp, src_entry, dst_phys, ntok, pad0, pad1, pad2, pad3;
};

// One unit of split-K work: `npages` logical pages of one format of one
// sequence, listed at pages[list_off ..]; the last listed page (logical page
// last_lp) holds last_ntok valid tokens.  `chunk` is the partial-state slot.
struct WorkItem {
  int32_t b, seq, list_off, npages, last_ntok, chunk, fmt, last_lp;
};

// Upper bound on WorkItem::npages: the partial kernel stages a work item's
// page-table entries in a fixed LDS array of this length.
constexpr int32_t kMaxChunkPages = 256;
// Waves per partial-kernel workgroup; a workgroup takes one work item and
// heads_per_wave kv-heads of it, its waves splitting the item's tiles.
constexpr int32_t kWavesPerWorkgroup = 4;

// kv-heads per partial-kernel wave (and workgroup): two when the query
// columns of two kv-heads fit the 16 MFMA columns (G <= 8), the kv-head count
// is even and d <= 128 (register budget); else one.  The work that does not
// depend on the kv-head (softmax, probability scaling) is then shared by two
// heads.
inline int32_t heads_per_wave(int32_t d, int32_t Hkv, int32_t G) {
  return (d <= 128 && 2 * G <= 16 && Hkv % 2 == 0) ? 2 : 1;
}

// Split-K policy.  By default the page list of each (sequence, format) is cut
// into near-equal chunks so that all items of a batch cost about the same and
// together they fill the partial kernel's resident waves once (an item takes
// ceil(Hkv / kWavesPerWorkgroup) workgroups); an FP8 page counts
// fp8_page_cost TQ3 pages.  A
// nonzero fixed_chunk_pages cuts every list into chunks of exactly that many
// pages instead (the last one shorter).  Chunks grow when a batch would need
// more than max_chunks of them; no chunk exceeds kMaxChunkPages.
struct SchedPolicy {
  int32_t target_waves = 2048;   // resident partial-kernel waves on the device
  int32_t min_chunk_pages = 4;   // smallest balanced chunk (shorter lists stay whole)
  int32_t fixed_chunk_pages = 0; // 0: balanced chunks
  int32_t heads_per_wave = 0;    // kv-heads per partial-kernel workgroup; 0: heads_per_wave()
  float fp8_page_cost = 1.0f;    // cost of an FP8 page relative to a TQ3 page (measured: about equal)
};

struct Schedule {
  std::vector<WorkItem> items[2];   // per format (FP8, TQ3)
  std::vector<int32_t> pages;       // logical page ids referenced by the items
  std::vector<int32_t> entries;     // their page-table entries (what the device reads)
  std::vector<int32_t> chunk_base;  // [B + 1] prefix sums of chunks per batch entry
  int32_t heads_per_wave = 1;       // kv-heads per partial-kernel workgroup
  int32_t n_chunks = 0;
  int32_t chunk_pages = 0;          // largest chunk of the schedule
  int32_t max_seq_chunks = 0;       // most chunks of one batch entry
};

class Meta {
 public:
  int init(const Desc& d, std::string* err);

  const Geom& geom() const { return g_; }
  const Desc& desc() const { return d_; }
  uint64_t version() const { return version_; }
  // Changes only when pages are added, converted or freed (not when tokens
  // land in an existing page): a schedule built at one layout version stays
  // valid up to the items' last_ntok.
  uint64_t layout_version() const { return layout_version_; }
  const Seq& seq(int32_t s) const { return seqs_[size_t(s)]; }
  int64_t fp8_free() const { return free_[0].size(); }
  int64_t tq3_free() const { return free_[1].size(); }

  // Each call validates everything first; on failure nothing changes.
  int append(int32_t seq, int32_t n, std::vector<AppendPage>* plan, std::string* err);
  // One token to each of B distinct sequences (row b to seq_ids[b]), all or
  // nothing; plan entries take src_row = b, and a page opened by the step
  // carries its page-table slot (seq * pt_stride + lp) and entry.
  int append_step(const int32_t* seq_ids, int32_t B, int32_t pt_stride,
                  std::vector<AppendPage>* plan, std::string* err);
  int demote(int32_t seq, const int32_t* lps, int32_t n, std::vector<DemotePage>* plan,
             std::string* err);
  int reset(int32_t seq, std::string* err);

  int build_schedule(const int32_t* seq_ids, int32_t B, int32_t Hq, const SchedPolicy& pol,
                     Schedule* out, std::string* err) const;

  // Algorithmic bytes a decode of the given sequences reads (codes, TQ3 group
  // scales, FP8 page-head scales).
  int64_t kv_bytes(const int32_t* seq_ids, int32_t B) const;
  int64_t seq_kv_bytes(int32_t s) const;
  int64_t live_tokens() const;
  int64_t live_pages(int fmt) const;

 private:
  int check_seq(int32_t s, std::string* err) const;
  Desc d_{};
  Geom g_{};
  FreeList free_[2];
  std::vector<Seq> seqs_;
  uint64_t version_ = 1;
  uint64_t layout_version_ = 1;
};

// Number of tokens held by logical page lp of a sequence of length len.
inline int32_t page_tokens(int32_t len, int32_t P, int32_t lp) {
  int32_t rest = len - lp * P;
  return rest < P ? rest : P;
}

}  // namespace mkv
