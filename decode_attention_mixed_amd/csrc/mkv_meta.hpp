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
  // The page pop() would return k calls from now (k < size()).
  int32_t peek(int64_t k) const { return stack_[stack_.size() - 1 - size_t(k)]; }
  void truncate(int64_t n) { stack_.resize(size_t(n)); }
 private:
  std::vector<int32_t> stack_;
};

struct Seq {
  int32_t len = 0;
  std::vector<int32_t> pt;      // one entry per logical page
  std::vector<uint8_t> prot;    // nonzero: logical page protected from the anchor policy
  int32_t policy_next = 0;      // pages below this were passed by the anchor policy
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
constexpr int32_t kMaxChunkPages = 240;
// Pages per chunk below which the split-K floor does not apply (shorter
// batches are cut for one round of the resident waves instead).
constexpr int32_t kFloorChunkPages = 16;
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
// fp8_page_cost TQ3 pages (by default the cost that gave the shortest partial
// kernels in a measured sweep: 0.6 with one kv-head per wave, 1.2 with two,
// since FP8 tiles hold one kv-head and TQ3 tiles that many).  min_items raises that count (a split-K floor:
// more, shorter chunks) for batches of at least min_items * kFloorChunkPages
// pages, as far as min_chunk_pages allows.  A
// nonzero fixed_chunk_pages cuts every list into chunks of exactly that many
// pages instead (the last one shorter).  Chunks grow when a batch would need
// more than max_chunks of them; no chunk exceeds kMaxChunkPages.
struct SchedPolicy {
  int32_t target_waves = 2048;   // partial-kernel waves a schedule fills (the library passes the
                                 // resident waves, or three quarters of them where four fit a SIMD)
  int32_t min_items = 256;       // split-K floor: at least this many items for batches of
                                 // min_items * kFloorChunkPages pages or more
  int32_t min_chunk_pages = 4;   // smallest balanced chunk (shorter lists stay whole)
  int32_t fixed_chunk_pages = 0; // 0: balanced chunks
  int32_t heads_per_wave = 0;    // kv-heads per partial-kernel workgroup; 0: heads_per_wave()
  float fp8_page_cost = 0.0f;    // cost of an FP8 page relative to a TQ3 page; 0: 0.6 or 1.2
};

struct Schedule {
  std::vector<WorkItem> items[2];   // per format (FP8, TQ3)
  std::vector<int32_t> cap[2];      // list capacity of each item (room to grow in place)
  std::vector<int32_t> pages;       // logical page ids referenced by the items (-1: spare room)
  std::vector<int32_t> entries;     // their page-table entries (what the device reads)
  std::vector<int32_t> chunk_base;  // [B + 1] prefix sums of chunks per batch entry
  int32_t heads_per_wave = 1;       // kv-heads per partial-kernel workgroup
  int32_t n_chunks = 0;
  int32_t chunk_pages = 0;          // largest chunk of the schedule
  int32_t max_seq_chunks = 0;       // most chunks of one batch entry
};

// What a mutating Meta call changed, recorded so that the caller can take the
// call back when the device work that goes with it cannot be enqueued (the
// C-ABI promises that a failed call leaves the pool unchanged).  Within one
// call a free list is either only popped or only pushed.
struct Undo {
  struct SeqLen {
    int32_t seq, len, npages;
  };
  struct Entry {
    int32_t seq, lp, entry;
  };
  uint64_t version = 0, layout_version = 0;
  int64_t free_size[2] = {0, 0};
  std::vector<int32_t> popped[2];   // pages taken from each free list, in pop order
  std::vector<SeqLen> lens;         // first recorded state of each touched sequence
  std::vector<Entry> entries;       // page-table entries overwritten, in order
  bool armed = false;
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
  const FreeList& free_list(int fmt) const { return free_[fmt ? 1 : 0]; }
  int64_t fp8_free() const { return free_[0].size(); }
  int64_t tq3_free() const { return free_[1].size(); }

  // Each call validates everything first; on failure nothing changes.  With
  // an Undo record, a successful call also records what it changed, and
  // rollback() restores the state before the call (valid only while no other
  // mutating call has run since).
  int append(int32_t seq, int32_t n, std::vector<AppendPage>* plan, std::string* err,
             Undo* undo = nullptr);
  // One token to each of B distinct sequences (row b to seq_ids[b]), all or
  // nothing; plan entries take src_row = b, and a page opened by the step
  // carries its page-table slot (seq * pt_stride + lp) and entry.
  int append_step(const int32_t* seq_ids, int32_t B, int32_t pt_stride,
                  std::vector<AppendPage>* plan, std::string* err, Undo* undo = nullptr);
  int demote(int32_t seq, const int32_t* lps, int32_t n, std::vector<DemotePage>* plan,
             std::string* err, Undo* undo = nullptr);
  int reset(int32_t seq, std::string* err);
  void rollback(const Undo& u);

  // Anchor policy (recent and protected pages stay FP8, older ones are
  // converted).  protect() marks (on) or clears logical pages of seq, which
  // may lie past its current end (below max_pages_per_seq); the policy never
  // demotes a marked page.  policy_pages() lists, without changing anything,
  // the pages the policy converts at seq's current length: the FP8 pages,
  // not marked, whose tokens all lie before the last `window` tokens and that
  // the policy has not passed yet, in logical order; *next receives the new
  // cursor, which set_policy_next() stores once the conversion is done (a
  // page passed while marked keeps its format from then on).  reset() clears
  // a sequence's marks and cursor.
  int protect(int32_t seq, const int32_t* lps, int32_t n, bool on, std::string* err);
  void policy_pages(int32_t seq, int32_t window, std::vector<int32_t>* lps, int32_t* next) const;
  void set_policy_next(int32_t seq, int32_t next) { seqs_[size_t(seq)].policy_next = next; }

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
  void arm(Undo* u) const;
  int32_t take(int f, Undo* u);
  static void note_seq(Undo* u, int32_t s, const Seq& q);
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

// ---- edits of a cached decode schedule ------------------------------------
// A schedule built for batch `ids` stays usable across calls that change the
// cache, when it is brought up to date instead of rebuilt.  Each function
// edits *sc in place and returns true, or returns false and leaves *sc as it
// was when the edit does not apply (the caller then rebuilds).  list_cap is
// the room of the device copy's page-list array (entries).

// Every item's last-page token count from the sequences' current lengths.
void schedule_refresh_tokens(const Meta& m, Schedule* sc);

// Spare list room the schedule builder leaves after the last item of each
// (batch entry, format) list, the items that decode steps grow: pages opened
// by appends join the last FP8 item, converted pages the last TQ3 item.
constexpr int32_t kGrowSlack = 32;

// The page-list ranges [first, last) an in-place schedule edit rewrote (for
// the upload of the changed words only).
struct ListEdits {
  std::vector<std::pair<size_t, size_t>> ranges;
  void add(size_t a, size_t b) { if (b > a) ranges.emplace_back(a, b); }
};

// Both edits below change *sc in place and record the list words they
// rewrote in *edits (if given).  An item grows in its list's spare room, or,
// without room, its list moves to the end of the list arrays with
// kGrowSlack spare pages.  They return false when the edit does not apply;
// *sc is then left partly edited and must be rebuilt.
//
// Pages were opened by an append step (plan rows src_row -> ids_of_rows):
// for each batch entry of a sequence that got a page, its last FP8 item (the
// one ending at the highest logical page) takes the page.  Does not apply to
// an entry with no FP8 item, a full chunk, or no room left.
bool schedule_extend(const Meta& m, const std::vector<int32_t>& ids, const int32_t* ids_of_rows,
                     const std::vector<AppendPage>& plan, size_t list_cap, Schedule* sc,
                     ListEdits* edits = nullptr);

// Pages of sequence seq were demoted: in each batch entry of the sequence the
// FP8 item listing a page drops it in place (its first page by starting its
// list one word later), and the entry's last TQ3 item
// (highest last page) takes it.  That TQ3 item's previous last page must be
// full (only an item's last page may hold fewer tokens).  Does not apply when
// an FP8 item would become empty, an entry has no TQ3 item, a chunk is full
// or there is no room.
bool schedule_demote(const Meta& m, const std::vector<int32_t>& ids, int32_t seq,
                     const std::vector<DemotePage>& plan, size_t list_cap, Schedule* sc,
                     ListEdits* edits = nullptr);

// Checks that sc is a valid decode schedule of batch ids for the current
// metadata: chunk_base partitions the partial-state slots by batch entry;
// every item lists 1..kMaxChunkPages pages of its sequence in its format, with
// their current page-table entries, ends at last_lp with last_ntok tokens and
// has full pages before that; every live page of each batch entry appears in
// exactly one of the entry's items.  Returns MKV_OK or MKV_EINVAL with the
// first violation in *why.
int check_schedule(const Meta& m, const int32_t* ids, int32_t B, const Schedule& sc,
                   std::string* why);

}  // namespace mkv
