// Randomised exercise of the host metadata layer, built with ASan/UBSan by
// tests/test_host_meta.py.  Checks invariants after every operation: every
// physical page is either free or owned by exactly one live logical page, and
// every schedule covers every live page exactly once.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "mkv_meta.hpp"

using namespace mkv;

static void die(const char* m) {
  std::printf("FAIL: %s\n", m);
  std::exit(1);
}

int main() {
  std::mt19937_64 rng(12345);
  Desc d{4, 64, 16, 6, 40, 6, 16, 0, 60, 50, 99};
  Meta m;
  std::string err;
  if (m.init(d, &err)) die(err.c_str());
  for (int step = 0; step < 20000; ++step) {
    int op = int(rng() % 10);
    int s = int(rng() % 7) - (rng() % 20 == 0 ? 1 : 0);  // occasionally invalid ids
    if (op < 5) {
      std::vector<AppendPage> plan;
      int n = int(rng() % 70) - 2;
      m.append(s, n, &plan, &err);
    } else if (op < 8) {
      if (s < 0 || s >= d.max_seqs) continue;
      int np = int(m.seq(s).pt.size());
      std::vector<int32_t> lps;
      for (int i = 0; i < np; ++i)
        if (rng() % 3 == 0) lps.push_back(i);
      if (rng() % 10 == 0) lps.push_back(np + 1);
      std::vector<DemotePage> plan;
      m.demote(s, lps.data(), int32_t(lps.size()), &plan, &err);
    } else if (op == 8) {
      m.reset(s, &err);
    } else {
      std::vector<int32_t> ids;
      for (int i = 0; i < 1 + int(rng() % 6); ++i) ids.push_back(int32_t(rng() % 6));
      Schedule sc;
      SchedPolicy pol;
      pol.fixed_chunk_pages = int(rng() % 9);          // 0: balanced chunks
      pol.target_waves = 1 + int(rng() % 4096);
      pol.fp8_page_cost = 0.25f + float(rng() % 8);
      if (m.build_schedule(ids.data(), int32_t(ids.size()), 16, pol, &sc, &err) == 0) {
        size_t total = 0;
        for (int32_t id : ids) total += m.seq(id).pt.size();
        size_t covered = 0;
        for (int f = 0; f < 2; ++f)
          for (const WorkItem& it : sc.items[f]) covered += size_t(it.npages);
        if (covered != total) die("schedule coverage");
      }
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
  std::printf("ok\n");
  return 0;
}
