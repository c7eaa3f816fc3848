// CPU-only entry points over the host metadata layer (pool geometry, free
// lists, page tables, split-K scheduler), so its logic can be tested without a
// GPU.  Built into libmkv_hosttest.so with the host compiler; never part of
// libmkv.so.
#include <cstring>
#include <string>
#include <vector>

#include "mkv.h"
#include "mkv_meta.hpp"

namespace {
thread_local std::string g_herr;
mkv::Desc to_desc(const mkv_pool_desc& d) {
  return mkv::Desc{d.num_kv_heads, d.head_dim, d.page_size, d.max_seqs, d.max_pages_per_seq,
                   d.max_batch,    d.max_q_heads, d.max_chunks, d.fp8_pages, d.tq3_pages,
                   d.placement_seed, d.kv_kind};
}
}  // namespace

struct mkvh {
  mkv::Meta meta;
};

extern "C" {

int mkvh_create(const mkv_pool_desc* desc, mkvh** out) {
  *out = nullptr;
  mkvh* h = new mkvh();
  int st = h->meta.init(to_desc(*desc), &g_herr);
  if (st) {
    delete h;
    return st;
  }
  *out = h;
  return 0;
}

void mkvh_destroy(mkvh* h) { delete h; }

// plan_out receives 8 int32 per touched page: lp, phys, row0, nrows, src_row,
// pt_slot, pt_entry, 0 (pt_slot -1 for mkvh_append).
int mkvh_append_step(mkvh* h, const int32_t* ids, int32_t B, int32_t pt_stride, int32_t* plan_out,
                     int32_t cap, int32_t* n_plan) {
  std::vector<mkv::AppendPage> plan;
  int st = h->meta.append_step(ids, B, pt_stride, &plan, &g_herr);
  *n_plan = int32_t(plan.size());
  if (!st && int32_t(plan.size()) <= cap) std::memcpy(plan_out, plan.data(), plan.size() * 32);
  return st;
}

int mkvh_append(mkvh* h, int32_t seq, int32_t n, int32_t* plan_out, int32_t cap, int32_t* n_plan) {
  std::vector<mkv::AppendPage> plan;
  int st = h->meta.append(seq, n, &plan, &g_herr);
  *n_plan = int32_t(plan.size());
  if (!st && int32_t(plan.size()) <= cap) std::memcpy(plan_out, plan.data(), plan.size() * 32);
  return st;
}

// plan_out receives 8 int32 per page: lp, src_phys, dst_phys, ntok, 0, 0, 0, 0.
int mkvh_demote(mkvh* h, int32_t seq, const int32_t* lps, int32_t n, int32_t* plan_out,
                int32_t cap, int32_t* n_plan) {
  std::vector<mkv::DemotePage> plan;
  int st = h->meta.demote(seq, lps, n, &plan, &g_herr);
  *n_plan = int32_t(plan.size());
  if (!st && int32_t(plan.size()) <= cap) std::memcpy(plan_out, plan.data(), plan.size() * 32);
  return st;
}

int mkvh_reset(mkvh* h, int32_t seq) { return h->meta.reset(seq, &g_herr); }

int mkvh_protect(mkvh* h, int32_t seq, const int32_t* lps, int32_t n, int32_t on) {
  return h->meta.protect(seq, lps, n, on != 0, &g_herr);
}

// Anchor policy query of seq at its current length: the pages it converts
// (up to cap into lps_out, the count into *n) and the cursor it would store.
void mkvh_policy_pages(mkvh* h, int32_t seq, int32_t window, int32_t* lps_out, int32_t cap, int32_t* n,
                       int32_t* next) {
  std::vector<int32_t> lps;
  h->meta.policy_pages(seq, window, &lps, next);
  *n = int32_t(lps.size());
  if (int32_t(lps.size()) <= cap) std::memcpy(lps_out, lps.data(), lps.size() * 4);
}

void mkvh_set_policy_next(mkvh* h, int32_t seq, int32_t next) { h->meta.set_policy_next(seq, next); }

int32_t mkvh_seq_len(mkvh* h, int32_t seq) { return h->meta.seq(seq).len; }

int32_t mkvh_page_table(mkvh* h, int32_t seq, int32_t* out, int32_t cap) {
  const std::vector<int32_t>& pt = h->meta.seq(seq).pt;
  if (int32_t(pt.size()) <= cap) std::memcpy(out, pt.data(), pt.size() * 4);
  return int32_t(pt.size());
}

int64_t mkvh_free(mkvh* h, int32_t fmt) { return fmt ? h->meta.tq3_free() : h->meta.fp8_free(); }

int64_t mkvh_kv_bytes(mkvh* h, const int32_t* ids, int32_t B) { return h->meta.kv_bytes(ids, B); }

uint64_t mkvh_version(mkvh* h) { return h->meta.version(); }

uint64_t mkvh_layout_version(mkvh* h) { return h->meta.layout_version(); }

// items_out: 8 int32 per item (b, seq, list_off, npages, last_ntok, chunk, fmt, 0), FP8 items
// first.  counts_out: n_fp8_items, n_tq3_items, n_pages, n_chunks, chunk_pages.
int mkvh_schedule(mkvh* h, const int32_t* ids, int32_t B, int32_t Hq, int32_t chunk_pages,
                  int32_t target_waves, int32_t* items_out, int32_t items_cap, int32_t* pages_out,
                  int32_t pages_cap, int32_t* base_out, int32_t* counts_out) {
  mkv::SchedPolicy pol;
  pol.fixed_chunk_pages = chunk_pages > 0 ? chunk_pages : 0;
  if (target_waves > 0) pol.target_waves = target_waves;
  mkv::Schedule sc;
  int st = h->meta.build_schedule(ids, B, Hq, pol, &sc, &g_herr);
  if (st) return st;
  const int32_t n8 = int32_t(sc.items[0].size()), n3 = int32_t(sc.items[1].size());
  counts_out[0] = n8;
  counts_out[1] = n3;
  counts_out[2] = int32_t(sc.pages.size());
  counts_out[3] = sc.n_chunks;
  counts_out[4] = sc.chunk_pages;
  if (n8 + n3 <= items_cap) {
    std::memcpy(items_out, sc.items[0].data(), size_t(n8) * 32);
    std::memcpy(items_out + 8 * n8, sc.items[1].data(), size_t(n3) * 32);
  }
  if (int32_t(sc.pages.size()) <= pages_cap)
    std::memcpy(pages_out, sc.pages.data(), sc.pages.size() * 4);
  std::memcpy(base_out, sc.chunk_base.data(), sc.chunk_base.size() * 4);
  return 0;
}

// Builds a schedule (as mkvh_schedule) and checks it with check_schedule.
int mkvh_check_schedule(mkvh* h, const int32_t* ids, int32_t B, int32_t Hq, int32_t chunk_pages,
                        int32_t target_waves, int32_t min_items, int32_t* n_chunks) {
  mkv::SchedPolicy pol;
  pol.fixed_chunk_pages = chunk_pages > 0 ? chunk_pages : 0;
  if (target_waves > 0) pol.target_waves = target_waves;
  pol.min_items = min_items;
  mkv::Schedule sc;
  int st = h->meta.build_schedule(ids, B, Hq, pol, &sc, &g_herr);
  if (st) return st;
  *n_chunks = sc.n_chunks;
  return mkv::check_schedule(h->meta, ids, B, sc, &g_herr);
}

// An append (or demote) that is taken back with its undo record, as the
// C-ABI does when the device work of the call cannot be enqueued.
int mkvh_append_rollback(mkvh* h, int32_t seq, int32_t n) {
  std::vector<mkv::AppendPage> plan;
  mkv::Undo undo;
  int st = h->meta.append(seq, n, &plan, &g_herr, &undo);
  if (!st) h->meta.rollback(undo);
  return st;
}

int mkvh_demote_rollback(mkvh* h, int32_t seq, const int32_t* lps, int32_t n) {
  std::vector<mkv::DemotePage> plan;
  mkv::Undo undo;
  int st = h->meta.demote(seq, lps, n, &plan, &g_herr, &undo);
  if (!st) h->meta.rollback(undo);
  return st;
}

int mkvh_append_step_rollback(mkvh* h, const int32_t* ids, int32_t B, int32_t pt_stride) {
  std::vector<mkv::AppendPage> plan;
  mkv::Undo undo;
  int st = h->meta.append_step(ids, B, pt_stride, &plan, &g_herr, &undo);
  if (!st) h->meta.rollback(undo);
  return st;
}

const char* mkvh_last_error(void) { return g_herr.c_str(); }

}  // extern "C"
