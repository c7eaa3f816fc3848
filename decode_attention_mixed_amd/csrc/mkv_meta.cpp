// Host metadata of the mixed-format page pool (see mkv_meta.hpp).
#include "mkv_meta.hpp"

#include <algorithm>
#include <queue>
#include <utility>

namespace mkv {

namespace {

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// splitmix64: a small, well-mixed 64-bit generator for the placement shuffle.
struct SplitMix64 {
  uint64_t s;
  uint64_t next() {
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
  }
};

int fail(std::string* err, int code, const char* msg) {
  if (err) *err = msg;
  return code;
}

}  // namespace

int validate_desc(const Desc& d, Geom* g, std::string* err) {
  if (d.Hkv < 1 || d.Hkv > 64) return fail(err, MKV_S_EINVAL, "num_kv_heads must be in 1..64");
  if (d.d != 32 && d.d != 64 && d.d != 128 && d.d != 256)
    return fail(err, MKV_S_EINVAL, "head_dim must be 32, 64, 128 or 256");
  if (d.P < 16 || d.P > 256 || d.P % 16)
    return fail(err, MKV_S_EINVAL, "page_size must be a multiple of 16 in 16..256");
  if (d.max_seqs < 1 || d.max_pages_per_seq < 1 || d.max_batch < 1)
    return fail(err, MKV_S_EINVAL, "max_seqs, max_pages_per_seq and max_batch must be >= 1");
  if (int64_t(d.max_pages_per_seq) * d.P > int64_t(INT32_MAX))
    return fail(err, MKV_S_EINVAL, "max_pages_per_seq * page_size overflows int32");
  if (d.max_q_heads < d.Hkv || d.max_q_heads > 16 * d.Hkv)
    return fail(err, MKV_S_EINVAL, "max_q_heads must be in Hkv..16*Hkv");
  if (d.fp8_pages < 1 || d.fp8_pages > int64_t(kPtIndexMask) || d.tq3_pages < 0 ||
      d.tq3_pages > int64_t(kPtIndexMask))
    return fail(err, MKV_S_EINVAL, "slab page counts must be in 1..2^31-1 (FP8) and 0..2^31-1 (TQ3)");
  if (d.max_chunks < 0) return fail(err, MKV_S_EINVAL, "max_chunks must be >= 0");
  if (d.kind != kKindMixed && d.kind != kKindBf16)
    return fail(err, MKV_S_EINVAL, "kv_kind must be MKV_KIND_MIXED or MKV_KIND_BF16");
  if (d.kind == kKindBf16 && d.tq3_pages != 0)
    return fail(err, MKV_S_EINVAL, "a BF16 control pool has no TQ3 slab (tq3_pages must be 0)");
  Geom r;
  r.Hkv = d.Hkv;
  r.d = d.d;
  r.P = d.P;
  r.kind = d.kind;
  // BF16 control record: K and V rows [Hkv][2][P][d] bf16, nothing else
  r.fp8_rec = d.kind == kKindBf16 ? 4ll * d.Hkv * d.P * d.d : 2ll * d.Hkv * d.P * d.d + 16ll * d.Hkv;
  r.tq3_rec = int64_t(d.Hkv) * d.P * d.d * 7 / 8;
  r.fp8_stride = round_up(r.fp8_rec, kSlabAlign);
  r.tq3_stride = round_up(r.tq3_rec, kSlabAlign);
  // A batch entry needs at most ceil(n8 / C) + ceil(n3 / C) chunks at the
  // largest chunk C = kMaxChunkPages, which is below 2 + ceil(pages / C).
  const int64_t need =
      int64_t(d.max_batch) * (2 + (int64_t(d.max_pages_per_seq) + kMaxChunkPages - 1) / kMaxChunkPages);
  const int64_t mc = d.max_chunks ? int64_t(d.max_chunks) : std::max<int64_t>(4096 + 2 * int64_t(d.max_batch), need);
  if (mc < need || mc > (int64_t(1) << 30))
    return fail(err, MKV_S_EINVAL,
                "max_chunks must be at least max_batch * (2 + ceil(max_pages_per_seq / 240))");
  r.max_chunks = int32_t(mc);
  if (g) *g = r;
  return MKV_S_OK;
}

void FreeList::init(int64_t n, uint64_t seed) {
  stack_.resize(size_t(n));
  for (int64_t i = 0; i < n; ++i) stack_[size_t(i)] = int32_t(n - 1 - i);  // pop() yields 0, 1, ...
  if (seed && n > 1) {
    SplitMix64 rng{seed};
    for (int64_t i = n - 1; i > 0; --i) {
      int64_t j = int64_t(rng.next() % uint64_t(i + 1));
      std::swap(stack_[size_t(i)], stack_[size_t(j)]);
    }
  }
}

int Meta::init(const Desc& d, std::string* err) {
  int st = validate_desc(d, &g_, err);
  if (st != MKV_S_OK) return st;
  d_ = d;
  free_[0].init(d.fp8_pages, d.placement_seed);
  // A different stream of the same seed for the TQ3 slab.
  free_[1].init(d.tq3_pages, d.placement_seed ? d.placement_seed ^ 0xA5A5A5A5DEADBEEFull : 0);
  seqs_.assign(size_t(d.max_seqs), Seq{});
  version_ = 1;
  layout_version_ = 1;
  return MKV_S_OK;
}

int Meta::check_seq(int32_t s, std::string* err) const {
  if (s < 0 || s >= d_.max_seqs) return fail(err, MKV_S_EINVAL, "sequence id out of range");
  return MKV_S_OK;
}

void Meta::arm(Undo* u) const {
  if (!u) return;
  u->version = version_;
  u->layout_version = layout_version_;
  for (int f = 0; f < 2; ++f) {
    u->free_size[f] = free_[f].size();
    u->popped[f].clear();
  }
  u->lens.clear();
  u->entries.clear();
  u->armed = true;
}

int32_t Meta::take(int f, Undo* u) {
  const int32_t v = free_[f].pop();
  if (u) u->popped[f].push_back(v);
  return v;
}

void Meta::note_seq(Undo* u, int32_t s, const Seq& q) {
  if (!u) return;
  for (const Undo::SeqLen& x : u->lens)
    if (x.seq == s) return;
  u->lens.push_back(Undo::SeqLen{s, q.len, int32_t(q.pt.size())});
}

void Meta::rollback(const Undo& u) {
  if (!u.armed) return;
  for (size_t i = u.entries.size(); i-- > 0;) {
    const Undo::Entry& e = u.entries[i];
    seqs_[size_t(e.seq)].pt[size_t(e.lp)] = e.entry;
  }
  for (const Undo::SeqLen& x : u.lens) {
    Seq& q = seqs_[size_t(x.seq)];
    q.len = x.len;
    q.pt.resize(size_t(x.npages));
  }
  for (int f = 0; f < 2; ++f) {
    // the untouched bottom of the stack, then the taken pages in reverse pop order
    free_[f].truncate(u.free_size[f] - int64_t(u.popped[f].size()));
    for (size_t i = u.popped[f].size(); i-- > 0;) free_[f].push(u.popped[f][i]);
  }
  version_ = u.version;
  layout_version_ = u.layout_version;
}

int Meta::append(int32_t s, int32_t n, std::vector<AppendPage>* plan, std::string* err,
                 Undo* undo) {
  plan->clear();
  int st = check_seq(s, err);
  if (st) return st;
  if (n < 0) return fail(err, MKV_S_EINVAL, "token count must be >= 0");
  if (n == 0) return MKV_S_OK;
  Seq& q = seqs_[size_t(s)];
  const int32_t P = g_.P;
  if (q.len % P != 0 && pt_is_tq3(q.pt.back()))
    return fail(err, MKV_S_ESTATE, "last page is TQ3 and partially filled; the sequence is frozen");
  int64_t new_len = int64_t(q.len) + n;
  int64_t need = (new_len + P - 1) / P;
  if (need > d_.max_pages_per_seq)
    return fail(err, MKV_S_ERANGE, "sequence would exceed max_pages_per_seq");
  int64_t fresh = need - int64_t(q.pt.size());
  if (fresh > free_[0].size()) return fail(err, MKV_S_ENOMEM, "FP8 slab has too few free pages");
  // Commit.
  arm(undo);
  note_seq(undo, s, q);
  for (int64_t i = 0; i < fresh; ++i) q.pt.push_back(pt_make(0, take(0, undo)));
  int32_t pos = q.len;
  int32_t src = 0;
  while (src < n) {
    int32_t lp = pos / P;
    int32_t row0 = pos % P;
    int32_t take = std::min(P - row0, n - src);
    plan->push_back(AppendPage{lp, pt_index(q.pt[size_t(lp)]), row0, take, src, -1, 0, 0});
    pos += take;
    src += take;
  }
  q.len = int32_t(new_len);
  ++version_;
  if (fresh > 0) ++layout_version_;
  return MKV_S_OK;
}

int Meta::append_step(const int32_t* ids, int32_t B, int32_t pt_stride,
                      std::vector<AppendPage>* plan, std::string* err, Undo* undo) {
  plan->clear();
  if (B < 0 || (B > 0 && !ids)) return fail(err, MKV_S_EINVAL, "bad sequence list");
  // validate everything first
  int64_t fresh = 0;
  std::vector<int32_t> sorted(ids, ids + B);
  std::sort(sorted.begin(), sorted.end());
  for (int32_t i = 1; i < B; ++i)
    if (sorted[size_t(i)] == sorted[size_t(i) - 1]) return fail(err, MKV_S_EINVAL, "sequence listed twice");
  for (int32_t b = 0; b < B; ++b) {
    int st = check_seq(ids[b], err);
    if (st) return st;
    const Seq& q = seqs_[size_t(ids[b])];
    if (q.len % g_.P != 0 && pt_is_tq3(q.pt.back()))
      return fail(err, MKV_S_ESTATE, "last page is TQ3 and partially filled; the sequence is frozen");
    if (q.len % g_.P == 0) {
      if (int64_t(q.pt.size()) + 1 > d_.max_pages_per_seq)
        return fail(err, MKV_S_ERANGE, "sequence would exceed max_pages_per_seq");
      ++fresh;
    }
  }
  if (fresh > free_[0].size()) return fail(err, MKV_S_ENOMEM, "FP8 slab has too few free pages");
  // commit
  arm(undo);
  for (int32_t b = 0; b < B; ++b) {
    Seq& q = seqs_[size_t(ids[b])];
    note_seq(undo, ids[b], q);
    const int32_t row0 = q.len % g_.P;
    int32_t slot = -1, entry = 0;
    if (row0 == 0) {
      q.pt.push_back(pt_make(0, take(0, undo)));
      slot = ids[b] * pt_stride + int32_t(q.pt.size()) - 1;
      entry = q.pt.back();
    }
    const int32_t lp = int32_t(q.pt.size()) - 1;
    plan->push_back(AppendPage{lp, pt_index(q.pt.back()), row0, 1, b, slot, entry, 0});
    ++q.len;
  }
  if (B) ++version_;
  if (fresh > 0) ++layout_version_;
  return MKV_S_OK;
}

int Meta::demote(int32_t s, const int32_t* lps, int32_t n, std::vector<DemotePage>* plan,
                 std::string* err, Undo* undo) {
  plan->clear();
  int st = check_seq(s, err);
  if (st) return st;
  if (n < 0 || (n > 0 && !lps)) return fail(err, MKV_S_EINVAL, "bad page list");
  if (g_.kind == kKindBf16 && n > 0)
    return fail(err, MKV_S_ESTATE, "a BF16 control pool holds one format; pages are never converted");
  Seq& q = seqs_[size_t(s)];
  std::vector<char> seen(q.pt.size(), 0);
  for (int32_t i = 0; i < n; ++i) {
    int32_t lp = lps[i];
    if (lp < 0 || size_t(lp) >= q.pt.size())
      return fail(err, MKV_S_EINVAL, "logical page out of range");
    if (seen[size_t(lp)]) return fail(err, MKV_S_EINVAL, "logical page listed twice");
    seen[size_t(lp)] = 1;
    if (pt_is_tq3(q.pt[size_t(lp)])) return fail(err, MKV_S_ESTATE, "page is already TQ3");
  }
  if (n > free_[1].size()) return fail(err, MKV_S_ENOMEM, "TQ3 slab has too few free pages");
  arm(undo);
  for (int32_t i = 0; i < n; ++i) {
    int32_t lp = lps[i];
    int32_t src = pt_index(q.pt[size_t(lp)]);
    int32_t dst = take(1, undo);
    if (undo) undo->entries.push_back(Undo::Entry{s, lp, q.pt[size_t(lp)]});
    q.pt[size_t(lp)] = pt_make(1, dst);
    free_[0].push(src);
    plan->push_back(DemotePage{lp, src, dst, page_tokens(q.len, g_.P, lp), 0, 0, 0, 0});
  }
  if (n) {
    ++version_;
    ++layout_version_;
  }
  return MKV_S_OK;
}

int Meta::reset(int32_t s, std::string* err) {
  int st = check_seq(s, err);
  if (st) return st;
  Seq& q = seqs_[size_t(s)];
  for (int32_t e : q.pt) free_[pt_is_tq3(e) ? 1 : 0].push(pt_index(e));
  q.pt.clear();
  q.len = 0;
  q.prot.clear();
  q.policy_next = 0;
  ++version_;
  ++layout_version_;
  return MKV_S_OK;
}

int Meta::protect(int32_t s, const int32_t* lps, int32_t n, bool on, std::string* err) {
  int st = check_seq(s, err);
  if (st) return st;
  if (n < 0 || (n > 0 && !lps)) return fail(err, MKV_S_EINVAL, "bad page list");
  for (int32_t i = 0; i < n; ++i)
    if (lps[i] < 0 || lps[i] >= d_.max_pages_per_seq)
      return fail(err, MKV_S_EINVAL, "logical page out of range");
  Seq& q = seqs_[size_t(s)];
  for (int32_t i = 0; i < n; ++i) {
    const size_t lp = size_t(lps[i]);
    if (lp >= q.prot.size()) {
      if (!on) continue;
      q.prot.resize(lp + 1, 0);
    }
    q.prot[lp] = on ? 1 : 0;
  }
  return MKV_S_OK;
}

void Meta::policy_pages(int32_t s, int32_t window, std::vector<int32_t>* lps, int32_t* next) const {
  lps->clear();
  const Seq& q = seqs_[size_t(s)];
  *next = q.policy_next;
  if (window < 0) return;
  // pages wholly before the window: tokens [lp P, (lp + 1) P) all below len - window
  const int32_t full = std::max(0, (q.len - window) / g_.P);
  for (int32_t lp = q.policy_next; lp < full; ++lp) {
    const bool marked = size_t(lp) < q.prot.size() && q.prot[size_t(lp)];
    if (!marked && !pt_is_tq3(q.pt[size_t(lp)])) lps->push_back(lp);
  }
  *next = std::max(q.policy_next, full);
}

int Meta::build_schedule(const int32_t* ids, int32_t B, int32_t Hq, const SchedPolicy& pol,
                         Schedule* out, std::string* err) const {
  if (B < 1 || !ids) return fail(err, MKV_S_EINVAL, "batch must hold at least one sequence");
  if (B > d_.max_batch) return fail(err, MKV_S_ERANGE, "batch exceeds max_batch");
  if (Hq < 1 || Hq % g_.Hkv) return fail(err, MKV_S_EINVAL, "Hq must be a positive multiple of Hkv");
  if (Hq > d_.max_q_heads) return fail(err, MKV_S_ERANGE, "Hq exceeds max_q_heads");
  if (Hq / g_.Hkv > 16) return fail(err, MKV_S_EINVAL, "Hq / Hkv must be at most 16");
  for (int32_t b = 0; b < B; ++b) {
    if (check_seq(ids[b], err)) return MKV_S_EINVAL;
    if (seqs_[size_t(ids[b])].len == 0) return fail(err, MKV_S_EINVAL, "empty sequence in batch");
  }
  const int32_t heads_per_block =
      pol.heads_per_wave > 0 ? pol.heads_per_wave : heads_per_wave(g_.d, g_.Hkv, Hq / g_.Hkv);
  if (heads_per_block != 1 && (heads_per_block != 2 || g_.Hkv % 2 || 2 * (Hq / g_.Hkv) > 16 || g_.d > 128))
    return fail(err, MKV_S_EINVAL, "unsupported kv-heads per wave");
  // Per-format page counts of each batch entry.  A wave walks an FP8 page one
  // kv-head at a time and a TQ3 page heads_per_block kv-heads at a time; the
  // default cost of an FP8 page in TQ3 pages is the one that gave the
  // shortest partial kernels in a sweep of the cost (0.6 with one kv-head per
  // workgroup, 1.2 with two).
  std::vector<int32_t> n8(size_t(B), 0), n3(size_t(B), 0);
  int64_t total_pages = 0;
  double total_cost = 0.0;
  const double c8 = pol.fp8_page_cost > 0.0f ? double(pol.fp8_page_cost) : (heads_per_block == 2 ? 1.2 : 0.6);
  for (int32_t b = 0; b < B; ++b) {
    for (int32_t e : seqs_[size_t(ids[b])].pt) (pt_is_tq3(e) ? n3 : n8)[size_t(b)]++;
    total_pages += int64_t(seqs_[size_t(ids[b])].pt.size());
    total_cost += c8 * n8[size_t(b)] + n3[size_t(b)];
  }
  // Chunk count of each (entry, format) list: chunks of `fixed` pages, or
  // near-equal chunks of about `budget` cost.
  int64_t fixed = pol.fixed_chunk_pages;
  auto chunks_of = [&](int32_t n, double page_cost, double budget) -> int64_t {
    if (n == 0) return 0;
    int64_t per;
    if (fixed > 0) {
      per = fixed;
    } else {
      const int64_t k = std::max<int64_t>(1, int64_t(n * page_cost / budget));
      per = std::max<int64_t>((n + k - 1) / k, std::min<int32_t>(n, std::max(1, pol.min_chunk_pages)));
    }
    per = std::min<int64_t>(per, kMaxChunkPages);
    return (n + per - 1) / per;
  };
  const int64_t waves_per_item =
      int64_t(kWavesPerWorkgroup) * ((g_.Hkv + heads_per_block - 1) / heads_per_block);
  // the split-K floor holds for batches long enough to give each of its chunks
  // kFloorChunkPages pages; shorter ones fill the resident waves once
  const int64_t floor_items =
      total_pages >= int64_t(pol.min_items) * kFloorChunkPages ? int64_t(pol.min_items) : int64_t(0);
  const int64_t target_items =
      std::max<int64_t>({int64_t(1), pol.target_waves / waves_per_item, floor_items});
  double budget = std::max(1.0, total_cost / double(target_items));
  std::vector<int64_t> k8(static_cast<size_t>(B)), k3(static_cast<size_t>(B));
  int64_t count = 0;
  for (int attempt = 0;; ++attempt) {
    count = 0;
    for (int32_t b = 0; b < B; ++b) {
      k8[size_t(b)] = chunks_of(n8[size_t(b)], c8, budget);
      k3[size_t(b)] = chunks_of(n3[size_t(b)], 1.0, budget);
      count += k8[size_t(b)] + k3[size_t(b)];
    }
    // Balanced chunks are counted down (floor); hand the spare slots up to the
    // target, one at a time, to the lists whose chunks cost the most.
    // (A heap ordered by chunk cost, ties to the lowest list index 2b + f.)
    if (fixed == 0 && attempt == 0) {
      const int64_t cap = std::min<int64_t>(target_items, g_.max_chunks);
      auto cost_of = [&](int32_t list, double* per) {
        const int32_t b = list >> 1, f = list & 1;
        const int32_t n = f ? n3[size_t(b)] : n8[size_t(b)];
        const int64_t k = f ? k3[size_t(b)] : k8[size_t(b)];
        if (n == 0 || k >= n || (n + k) / (k + 1) < pol.min_chunk_pages) return false;
        *per = double(n) * (f ? 1.0 : c8) / double(k);
        return *per > 0.0;
      };
      using Entry = std::pair<double, int32_t>;   // (cost per chunk, list)
      auto lower = [](const Entry& x, const Entry& y) {
        return x.first < y.first || (x.first == y.first && x.second > y.second);
      };
      std::priority_queue<Entry, std::vector<Entry>, decltype(lower)> heap(lower);
      if (count < cap)
        for (int32_t list = 0; list < 2 * B; ++list) {
          double per;
          if (cost_of(list, &per)) heap.emplace(per, list);
        }
      while (count < cap && !heap.empty()) {
        const int32_t list = heap.top().second;
        heap.pop();
        ++((list & 1) ? k3 : k8)[size_t(list >> 1)];
        ++count;
        double per;
        if (cost_of(list, &per)) heap.emplace(per, list);
      }
    }
    if (count <= g_.max_chunks) break;
    // Too many chunks: coarser chunks (fixed chunks double, balanced budgets grow).
    bool at_cap = true;
    for (int32_t b = 0; b < B; ++b)
      at_cap = at_cap && k8[size_t(b)] == (n8[size_t(b)] + kMaxChunkPages - 1) / kMaxChunkPages &&
               k3[size_t(b)] == (n3[size_t(b)] + kMaxChunkPages - 1) / kMaxChunkPages;
    if (at_cap || attempt > 64) return fail(err, MKV_S_ERANGE, "batch needs more than max_chunks chunks");
    budget *= 1.5;
    fixed *= 2;
  }
  out->items[0].clear();
  out->items[1].clear();
  out->cap[0].clear();
  out->cap[1].clear();
  out->pages.clear();
  out->pages.reserve(size_t(total_pages));
  out->entries.clear();
  out->entries.reserve(size_t(total_pages));
  out->chunk_base.assign(size_t(B) + 1, 0);
  // spare room after each entry's last FP8 and TQ3 item, as far as the list
  // capacity allows
  const int64_t list_cap = int64_t(d_.max_batch) * int64_t(d_.max_pages_per_seq);
  const int32_t slack = int32_t(std::max<int64_t>(
      0, std::min<int64_t>(kGrowSlack, (list_cap - total_pages) / std::max<int64_t>(1, 2 * int64_t(B)))));
  int32_t nc = 0, largest = 0;
  for (int32_t b = 0; b < B; ++b) {
    out->chunk_base[size_t(b)] = nc;
    const Seq& q = seqs_[size_t(ids[b])];
    for (int fmt = 0; fmt < 2; ++fmt) {
      const int32_t n = fmt ? n3[size_t(b)] : n8[size_t(b)];
      const int64_t k = fmt ? k3[size_t(b)] : k8[size_t(b)];
      if (n == 0) continue;
      // chunk i holds n / k pages, the first n % k chunks one more
      const int32_t small = int32_t(n / k), extra = int32_t(n % k);
      std::vector<WorkItem>& items = out->items[fmt];
      int32_t chunk_idx = -1, left = 0;
      for (int32_t lp = 0; lp < int32_t(q.pt.size()); ++lp) {
        if (int(pt_is_tq3(q.pt[size_t(lp)])) != fmt) continue;
        if (left == 0) {
          ++chunk_idx;
          left = small + (chunk_idx < extra ? 1 : 0);
          items.push_back(WorkItem{b, ids[b], int32_t(out->pages.size()), 0, 0, nc++, fmt, 0});
          out->cap[fmt].push_back(left);
        }
        out->pages.push_back(lp);
        out->entries.push_back(q.pt[size_t(lp)]);
        items.back().npages++;
        items.back().last_ntok = page_tokens(q.len, g_.P, lp);
        items.back().last_lp = lp;
        largest = std::max(largest, items.back().npages);
        --left;
      }
      // the list's last item (its pages end the arrays) gets the spare room
      const int32_t room = std::min(slack, kMaxChunkPages - items.back().npages);
      if (room > 0) {
        out->pages.insert(out->pages.end(), size_t(room), -1);
        out->entries.insert(out->entries.end(), size_t(room), 0);
        out->cap[fmt].back() += room;
      }
    }
  }
  out->chunk_base[size_t(B)] = nc;
  out->n_chunks = nc;
  out->max_seq_chunks = 0;
  for (int32_t b = 0; b < B; ++b)
    out->max_seq_chunks =
        std::max(out->max_seq_chunks, out->chunk_base[size_t(b) + 1] - out->chunk_base[size_t(b)]);
  out->chunk_pages = largest;
  out->heads_per_wave = heads_per_block;
  return MKV_S_OK;
}

int64_t Meta::seq_kv_bytes(int32_t s) const {
  const Seq& q = seqs_[size_t(s)];
  int64_t t = 0;
  for (int32_t lp = 0; lp < int32_t(q.pt.size()); ++lp) {
    int64_t n = page_tokens(q.len, g_.P, lp);
    if (g_.kind == kKindBf16)
      t += n * 4 * g_.Hkv * g_.d;                  // K and V bf16 rows
    else if (pt_is_tq3(q.pt[size_t(lp)]))
      t += n * g_.Hkv * g_.d * 7 / 8;
    else
      t += n * 2 * g_.Hkv * g_.d + 8ll * g_.Hkv;
  }
  return t;
}

int64_t Meta::kv_bytes(const int32_t* ids, int32_t B) const {
  int64_t t = 0;
  for (int32_t b = 0; b < B; ++b) t += seq_kv_bytes(ids[b]);
  return t;
}

int64_t Meta::live_tokens() const {
  int64_t t = 0;
  for (const Seq& q : seqs_) t += q.len;
  return t;
}

int64_t Meta::live_pages(int fmt) const {
  int64_t t = 0;
  for (const Seq& q : seqs_)
    for (int32_t e : q.pt) t += (int(pt_is_tq3(e)) == fmt);
  return t;
}


// ---- edits of a cached decode schedule ----------------------------------------

void schedule_refresh_tokens(const Meta& m, Schedule* sc) {
  const int32_t P = m.geom().P;
  for (auto& list : sc->items)
    for (WorkItem& it : list) it.last_ntok = page_tokens(m.seq(it.seq).len, P, it.last_lp);
}

namespace {

// Item idx of list f takes (lp, entry) as its new last page: in its spare
// room, or with its list copied to the end of the list arrays with up to
// kGrowSlack spare pages (false when the arrays would exceed list_cap).
bool grow_item(Schedule& sc, int f, size_t idx, int32_t lp, int32_t entry, size_t list_cap,
               ListEdits* edits) {
  WorkItem& it = sc.items[f][idx];
  int32_t& cap = sc.cap[f][idx];
  if (it.npages >= cap) {
    const int32_t room = std::max(0, std::min(kGrowSlack, kMaxChunkPages - it.npages - 1));
    const size_t off = sc.entries.size();
    if (off + size_t(it.npages) + 1 + size_t(room) > list_cap) return false;
    for (int32_t i = 0; i < it.npages; ++i) {
      const int32_t e = sc.entries[size_t(it.list_off + i)], p = sc.pages[size_t(it.list_off + i)];
      sc.entries.push_back(e);
      sc.pages.push_back(p);
    }
    sc.entries.insert(sc.entries.end(), size_t(1 + room), 0);
    sc.pages.insert(sc.pages.end(), size_t(1 + room), -1);
    if (edits) edits->add(off, off + size_t(it.npages));
    it.list_off = int32_t(off);
    cap = it.npages + 1 + room;
  }
  const size_t at = size_t(it.list_off + it.npages);
  sc.entries[at] = entry;
  sc.pages[at] = lp;
  if (edits) edits->add(at, at + 1);
  it.npages += 1;
  it.last_lp = lp;
  sc.chunk_pages = std::max(sc.chunk_pages, it.npages);
  return true;
}

// Index of entry b's last item of list f (highest last page), or -1.
int64_t last_item(const Schedule& sc, int f, int32_t b) {
  int64_t best = -1;
  for (size_t i = 0; i < sc.items[f].size(); ++i) {
    const WorkItem& it = sc.items[f][i];
    if (it.b == b && (best < 0 || it.last_lp > sc.items[f][size_t(best)].last_lp)) best = int64_t(i);
  }
  return best;
}

}  // namespace

bool schedule_extend(const Meta& m, const std::vector<int32_t>& ids, const int32_t* ids_of_rows,
                     const std::vector<AppendPage>& plan, size_t list_cap, Schedule* sc,
                     ListEdits* edits) {
  for (const AppendPage& ap : plan) {
    if (ap.pt_slot < 0) continue;
    const int32_t seq = ids_of_rows[ap.src_row];
    for (size_t b = 0; b < ids.size(); ++b) {
      if (ids[b] != seq) continue;
      const int64_t last = last_item(*sc, 0, int32_t(b));
      if (last < 0 || sc->items[0][size_t(last)].npages >= kMaxChunkPages) return false;
      if (!grow_item(*sc, 0, size_t(last), ap.lp, ap.pt_entry, list_cap, edits)) return false;
    }
  }
  schedule_refresh_tokens(m, sc);
  return true;
}

bool schedule_demote(const Meta& m, const std::vector<int32_t>& ids, int32_t seq,
                     const std::vector<DemotePage>& plan, size_t list_cap, Schedule* sc,
                     ListEdits* edits) {
  const Seq& q = m.seq(seq);
  const int32_t P = m.geom().P;
  for (size_t b = 0; b < ids.size(); ++b) {
    if (ids[b] != seq) continue;
    for (const DemotePage& dp : plan) {
      WorkItem* src = nullptr;
      int32_t at = -1;
      for (WorkItem& it : sc->items[0]) {
        if (it.b != int32_t(b)) continue;
        for (int32_t i = 0; i < it.npages && at < 0; ++i)
          if (sc->pages[size_t(it.list_off + i)] == dp.lp) at = i;
        if (at >= 0) {
          src = &it;
          break;
        }
      }
      if (!src || src->npages < 2) return false;
      if (at == 0) {
        // the item's first page (the oldest page of a recency window): the
        // list starts one word later, no word moves
        src->list_off += 1;
        sc->cap[0][size_t(src - sc->items[0].data())] -= 1;
      } else {
        for (int32_t i = at; i + 1 < src->npages; ++i) {
          sc->entries[size_t(src->list_off + i)] = sc->entries[size_t(src->list_off + i + 1)];
          sc->pages[size_t(src->list_off + i)] = sc->pages[size_t(src->list_off + i + 1)];
        }
        if (edits) edits->add(size_t(src->list_off + at), size_t(src->list_off + src->npages - 1));
      }
      --src->npages;
      src->last_lp = sc->pages[size_t(src->list_off + src->npages - 1)];
      const int64_t dst = last_item(*sc, 1, int32_t(b));
      if (dst < 0 || sc->items[1][size_t(dst)].npages >= kMaxChunkPages ||
          page_tokens(q.len, P, sc->items[1][size_t(dst)].last_lp) != P)
        return false;
      if (!grow_item(*sc, 1, size_t(dst), dp.lp, q.pt[size_t(dp.lp)], list_cap, edits)) return false;
    }
  }
  schedule_refresh_tokens(m, sc);
  return true;
}

int check_schedule(const Meta& m, const int32_t* ids, int32_t B, const Schedule& sc,
                   std::string* why) {
  auto bad = [&](const std::string& msg) { return fail(why, MKV_S_EINVAL, msg.c_str()); };
  if (B < 1 || int32_t(sc.chunk_base.size()) != B + 1 || sc.chunk_base[0] != 0)
    return bad("chunk_base must hold B + 1 offsets starting at 0");
  for (int32_t b = 0; b < B; ++b)
    if (sc.chunk_base[size_t(b) + 1] < sc.chunk_base[size_t(b)]) return bad("chunk_base decreases");
  if (sc.chunk_base[size_t(B)] != sc.n_chunks) return bad("chunk_base does not end at n_chunks");
  if (sc.entries.size() != sc.pages.size()) return bad("entries and pages differ in length");
  const int32_t P = m.geom().P;
  std::vector<char> slot_seen(size_t(std::max(0, sc.n_chunks)), 0);
  std::vector<std::vector<int32_t>> seen(static_cast<size_t>(B));   // per entry: times each page is listed
  std::vector<int32_t> items_of(size_t(B), 0);
  for (int32_t b = 0; b < B; ++b) seen[size_t(b)].assign(m.seq(ids[b]).pt.size(), 0);
  int32_t largest = 0;
  for (int f = 0; f < 2; ++f) {
    for (const WorkItem& it : sc.items[f]) {
      const std::string at = "item of entry " + std::to_string(it.b) + " chunk " + std::to_string(it.chunk);
      if (it.b < 0 || it.b >= B || it.seq != ids[it.b]) return bad(at + ": wrong batch entry or sequence");
      if (it.fmt != f) return bad(at + ": format differs from its list");
      if (it.npages < 1 || it.npages > kMaxChunkPages) return bad(at + ": page count out of range");
      if (it.list_off < 0 || size_t(it.list_off) + size_t(it.npages) > sc.pages.size())
        return bad(at + ": page list outside the arrays");
      if (it.chunk < sc.chunk_base[size_t(it.b)] || it.chunk >= sc.chunk_base[size_t(it.b) + 1])
        return bad(at + ": partial-state slot outside its entry's range");
      if (slot_seen[size_t(it.chunk)]++) return bad(at + ": partial-state slot used twice");
      items_of[size_t(it.b)]++;
      largest = std::max(largest, it.npages);
      const Seq& q = m.seq(it.seq);
      for (int32_t i = 0; i < it.npages; ++i) {
        const int32_t lp = sc.pages[size_t(it.list_off + i)];
        if (lp < 0 || size_t(lp) >= q.pt.size()) return bad(at + ": logical page out of range");
        if (sc.entries[size_t(it.list_off + i)] != q.pt[size_t(lp)])
          return bad(at + ": entry differs from the page table at page " + std::to_string(lp));
        if (int(pt_is_tq3(q.pt[size_t(lp)])) != f) return bad(at + ": page of the other format");
        if (i + 1 < it.npages && page_tokens(q.len, P, lp) != P)
          return bad(at + ": a page before the item's last is not full");
        seen[size_t(it.b)][size_t(lp)]++;
      }
      const int32_t last = sc.pages[size_t(it.list_off + it.npages - 1)];
      if (last != it.last_lp) return bad(at + ": last_lp is not the last listed page");
      if (it.last_ntok != page_tokens(q.len, P, last)) return bad(at + ": last_ntok is stale");
    }
  }
  int32_t most = 0;
  for (int32_t b = 0; b < B; ++b) {
    for (size_t lp = 0; lp < seen[size_t(b)].size(); ++lp)
      if (seen[size_t(b)][lp] != 1)
        return bad("entry " + std::to_string(b) + " lists page " + std::to_string(lp) + " " +
                   std::to_string(seen[size_t(b)][lp]) + " times");
    const int32_t n = sc.chunk_base[size_t(b) + 1] - sc.chunk_base[size_t(b)];
    if (n != items_of[size_t(b)]) return bad("entry " + std::to_string(b) + " has slots without items");
    most = std::max(most, n);
  }
  if (sc.max_seq_chunks != most) return bad("max_seq_chunks is wrong");
  if (sc.chunk_pages < largest) return bad("chunk_pages is below the largest item");
  return MKV_S_OK;
}

}  // namespace mkv
