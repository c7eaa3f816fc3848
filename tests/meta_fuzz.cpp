// Randomised exercise of the host metadata layer, built with ASan/UBSan by
// tests/test_host_meta.py.  After every operation it checks that every
// physical page is either free or owned by exactly one live logical page.
// It also checks schedules:
//  * every schedule the builder returns passes check_schedule: each live page
//    of each batch entry is listed once, with its current page-table entry;
//  * a cached schedule kept current by the edit functions passes as well,
//    after append steps that open pages and after demotions;
//  * a copy of the page-list words updated only where the edits say they
//    wrote (what the device receives) agrees with the schedule on every
//    listed word.
// It also takes random calls back with their undo record and compares the
// whole state with a copy taken before the call.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <string>
#include <vector>

#include "mkv_meta.hpp"

using namespace mkv;

static void die(const char* m, const std::string& why = "") {
  std::printf("FAIL: %s %s\n", m, why.c_str());
  std::exit(1);
}

static bool same_state(const Meta& a, const Meta& b, int max_seqs) {
  if (a.version() != b.version() || a.layout_version() != b.layout_version()) return false;
  for (int f = 0; f < 2; ++f) {
    const FreeList& x = a.free_list(f);
    const FreeList& y = b.free_list(f);
    if (x.size() != y.size()) return false;
    for (int64_t k = 0; k < x.size(); ++k)
      if (x.peek(k) != y.peek(k)) return false;
  }
  for (int s = 0; s < max_seqs; ++s)
    if (a.seq(s).len != b.seq(s).len || a.seq(s).pt != b.seq(s).pt) return false;
  return true;
}

int main() {
  std::mt19937_64 rng(12345);
  Desc d{4, 64, 16, 6, 40, 6, 16, 0, 60, 50, 99, 0};
  Meta m;
  std::string err;
  if (m.init(d, &err)) die(err.c_str());
  const size_t list_cap = size_t(d.max_batch) * size_t(d.max_pages_per_seq);
  // a cached schedule for a batch, kept current by the edit functions
  std::vector<int32_t> cached_ids;
  Schedule cached;
  bool cached_ok = false;
  std::vector<int32_t> dev(list_cap, -7);   // the device's copy of the list words
  ListEdits edits;
  int edits_applied = 0, rollbacks = 0;
  for (int step = 0; step < 100000; ++step) {
    const int op = int(rng() % 12);
    const int s = int(rng() % 7) - (rng() % 20 == 0 ? 1 : 0);  // occasionally invalid ids
    const bool take_back = rng() % 4 == 0;
    Meta before = take_back ? m : Meta();
    Undo undo;
    int st = -1;
    if (op < 4) {
      std::vector<AppendPage> plan;
      st = m.append(s, int(rng() % 70) - 2, &plan, &err, &undo);
      if (st == 0 && !undo.popped[0].empty()) cached_ok = false;   // pages opened: rebuild
      if (cached_ok) schedule_refresh_tokens(m, &cached);
    } else if (op < 6) {
      // one token to each of a few distinct sequences
      std::vector<int32_t> ids;
      for (int q = 0; q < d.max_seqs; ++q)
        if (rng() % 2) ids.push_back(q);
      if (ids.empty()) continue;
      const uint64_t lay0 = m.layout_version();
      std::vector<AppendPage> plan;
      st = m.append_step(ids.data(), int32_t(ids.size()), d.max_pages_per_seq, &plan, &err, &undo);
      if (st == 0 && cached_ok && m.layout_version() != lay0) {
        edits.ranges.clear();
        cached_ok = schedule_extend(m, cached_ids, ids.data(), plan, list_cap, &cached, &edits);
        edits_applied += cached_ok;
      } else if (st == 0 && cached_ok) {
        schedule_refresh_tokens(m, &cached);
      }
    } else if (op < 9) {
      if (s < 0 || s >= d.max_seqs) continue;
      const int np = int(m.seq(s).pt.size());
      std::vector<int32_t> lps;
      for (int i = 0; i < np; ++i)
        if (rng() % 3 == 0) lps.push_back(i);
      if (rng() % 10 == 0) lps.push_back(np + 1);
      std::vector<DemotePage> plan;
      st = m.demote(s, lps.data(), int32_t(lps.size()), &plan, &err, &undo);
      if (st == 0 && cached_ok && !plan.empty()) {
        edits.ranges.clear();
        cached_ok = schedule_demote(m, cached_ids, s, plan, list_cap, &cached, &edits);
        edits_applied += cached_ok;
      }
    } else if (op == 9) {
      m.reset(s, &err);
      cached_ok = false;
      continue;
    } else {
      std::vector<int32_t> ids;
      for (int i = 0; i < 1 + int(rng() % 6); ++i) ids.push_back(int32_t(rng() % 6));
      Schedule sc;
      SchedPolicy pol;
      pol.fixed_chunk_pages = int(rng() % 9);          // 0: balanced chunks
      pol.target_waves = 1 + int(rng() % 4096);
      pol.min_items = int(rng() % 300);
      pol.fp8_page_cost = 0.25f + float(rng() % 8);
      if (m.build_schedule(ids.data(), int32_t(ids.size()), 16, pol, &sc, &err) == 0) {
        if (check_schedule(m, ids.data(), int32_t(ids.size()), sc, &err)) die("built schedule", err);
        cached_ids = ids;
        cached = sc;
        cached_ok = true;
        if (cached.entries.size() > list_cap) die("schedule exceeds the list capacity");
        std::copy(cached.entries.begin(), cached.entries.end(), dev.begin());   // full upload
        edits.ranges.clear();
      }
      continue;
    }
    if (take_back && st == 0) {
      m.rollback(undo);
      ++rollbacks;
      if (!same_state(m, before, d.max_seqs)) die("rollback did not restore the state");
      cached_ok = false;
    }
    if (cached_ok &&
        check_schedule(m, cached_ids.data(), int32_t(cached_ids.size()), cached, &err))
      die("edited schedule", err);
    if (cached_ok) {
      if (cached.entries.size() > list_cap || cached.pages.size() != cached.entries.size())
        die("edited schedule exceeds the list capacity");
      for (const auto& r : edits.ranges) {
        if (r.second > cached.entries.size()) die("edit range past the list");
        std::copy(cached.entries.begin() + std::ptrdiff_t(r.first), cached.entries.begin() + std::ptrdiff_t(r.second),
                  dev.begin() + std::ptrdiff_t(r.first));
      }
      edits.ranges.clear();
      for (int f = 0; f < 2; ++f)
        for (const WorkItem& it : cached.items[f])
          for (int32_t i = 0; i < it.npages; ++i)
            if (dev[size_t(it.list_off + i)] != cached.entries[size_t(it.list_off + i)])
              die("an edit changed a listed word outside its recorded ranges");
    }
    // ownership invariant
    std::vector<int> own8(size_t(d.fp8_pages), 0), own3(size_t(d.tq3_pages), 0);
    for (int q = 0; q < d.max_seqs; ++q)
      for (int32_t e : m.seq(q).pt) (pt_is_tq3(e) ? own3 : own8)[size_t(pt_index(e))]++;
    int64_t used8 = 0, used3 = 0;
    for (int v : own8) {
      if (v > 1) die("fp8 page owned twice");
      used8 += v;
    }
    for (int v : own3) {
      if (v > 1) die("tq3 page owned twice");
      used3 += v;
    }
    if (used8 + m.fp8_free() != d.fp8_pages) die("fp8 page leak");
    if (used3 + m.tq3_free() != d.tq3_pages) die("tq3 page leak");
  }
  if (edits_applied < 50 || rollbacks < 100) die("too few schedule edits or rollbacks exercised");
  std::printf("ok (%d schedule edits, %d rollbacks)\n", edits_applied, rollbacks);
  return 0;
}
