// C-ABI of libmkv (declared in include/mkv.h): argument validation, device
// memory layout, stream-ordered metadata uploads and kernel launches.
#include "mkv.h"

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "mkv_kernels.hpp"
#include "mkv_meta.hpp"

static_assert(MKV_OK == MKV_S_OK && MKV_EINVAL == MKV_S_EINVAL && MKV_ENOMEM == MKV_S_ENOMEM &&
                  MKV_ESTATE == MKV_S_ESTATE && MKV_ERANGE == MKV_S_ERANGE &&
                  MKV_EHIP == MKV_S_EHIP,
              "status codes must agree");
static_assert(sizeof(mkv::WorkItem) == 32 && sizeof(mkv::AppendPage) == 32 &&
                  sizeof(mkv::DemotePage) == 32 && sizeof(mkv::MaterialisePage) == 32,
              "device plan records are 32 bytes");

namespace {

thread_local std::string g_err;

mkv_status set_err(mkv_status s, const std::string& msg) {
  g_err = msg;
  return s;
}

#define MKV_HIP(call)                                                                  \
  do {                                                                                 \
    hipError_t e_ = (call);                                                            \
    if (e_ != hipSuccess)                                                              \
      return set_err(MKV_EHIP, std::string(#call) + ": " + hipGetErrorString(e_));     \
  } while (0)

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

mkv::Desc to_desc(const mkv_pool_desc& d) {
  return mkv::Desc{d.num_kv_heads, d.head_dim, d.page_size, d.max_seqs, d.max_pages_per_seq,
                   d.max_batch,    d.max_q_heads, d.max_chunks, d.fp8_pages, d.tq3_pages,
                   d.placement_seed, d.kv_kind};
}

// Device memory layout of a pool (offsets from the base of its block).
struct Layout {
  size_t fp8, tq3, pt, sched, sched_bytes, plan, plan_bytes, pm, pl, pacc, total;
  // The schedule region holds chunk_base, then the work items, then (at the
  // next 256-byte boundary after the items) the page-list entries, so a
  // rebuilt schedule is one contiguous upload.
  size_t items_cap;  // work items that fit the schedule region
  size_t items_off;  // offset of the items inside the region (chunk_base is at 0)
};

// Offset of the page-list entries of a schedule with n_items items.
inline size_t entries_off(const Layout& L, size_t n_items) {
  return L.items_off + align256(n_items * sizeof(mkv::WorkItem));
}

Layout make_layout(const mkv::Desc& d, const mkv::Geom& g) {
  Layout L{};
  size_t o = 0;
  L.fp8 = o;
  o = align256(o + size_t(d.fp8_pages) * size_t(g.fp8_stride));
  L.tq3 = o;
  o = align256(o + size_t(d.tq3_pages) * size_t(g.tq3_stride));
  L.pt = o;
  o = align256(o + size_t(d.max_seqs) * size_t(d.max_pages_per_seq) * 4);
  L.items_cap = size_t(g.max_chunks);
  L.items_off = align256((size_t(d.max_batch) + 1) * 4);
  L.sched_bytes = align256(entries_off(L, L.items_cap) +
                           size_t(d.max_batch) * size_t(d.max_pages_per_seq) * 4);
  L.sched = o;
  o += L.sched_bytes;
  L.plan_bytes = align256(size_t(std::max(d.max_pages_per_seq, d.max_batch)) * 32);
  L.plan = o;
  o += L.plan_bytes;
  const size_t slots = size_t(g.max_chunks) * size_t(d.max_q_heads);
  L.pm = o;
  o = align256(o + slots * 4);
  L.pl = o;
  o = align256(o + slots * 4);
  L.pacc = o;
  o = align256(o + slots * size_t(d.d) * 4);
  L.total = o;
  return L;
}

struct ProfEvent {
  int kind;
  hipEvent_t a, b;
};

// Keeps the caller's current device and switches to the pool's for the call.
struct DeviceGuard {
  int prev = -1;
  bool switched = false;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev)
      switched = hipSetDevice(dev) == hipSuccess;
  }
  ~DeviceGuard() {
    if (switched) (void)hipSetDevice(prev);
  }
};

}  // namespace

struct mkv_pool {
  mkv::Meta meta;
  mkv_pool_desc desc{};
  Layout lay{};
  int device = 0;
  uint8_t* mem = nullptr;
  bool owns_mem = false;
  // pinned staging ring for host -> device metadata uploads: an upload takes
  // the next slot, waiting only for that slot's previous copy, so the host can
  // run several calls ahead of the device (the copies themselves are stream-
  // ordered behind the kernels that read the previous contents)
  static constexpr int kStagingSlots = 4;
  uint8_t* staging_mem = nullptr;        // coherent pinned host memory
  const uint32_t* staging_dev = nullptr; // the same memory as the device reads it
  uint8_t* staging = nullptr;            // the slot being filled
  size_t staging_bytes = 0;              // bytes per slot
  hipEvent_t staging_ev[kStagingSlots] = {};
  bool staging_pending[kStagingSlots] = {};
  int staging_slot = 0;
  // cached decode schedule
  bool sched_valid = false;
  uint64_t sched_version = 0;
  uint64_t sched_layout = 0;   // page-layout version the schedule was built at
  int32_t sched_Hq = 0;
  std::vector<int32_t> sched_ids;
  mkv::Schedule sched;
  int32_t target_waves[2] = {2048, 1024};   // resident partial-kernel waves, 1 or 2 heads per wave
  int32_t merge_narrow_max = 16;            // per-lane merge up to this many chunks per entry
  bool pace = true;                         // progress-paced wave priorities (one-round launches)
  // profiling
  bool prof = false;
  std::vector<ProfEvent> prof_events;
  std::vector<ProfEvent> prof_free;
  double prof_ms[2] = {0, 0};    // partial, merge
  int64_t prof_n[2] = {0, 0};

  mkv::PoolView view() const {
    const mkv::Geom& g = meta.geom();
    return mkv::PoolView{mem + lay.fp8, mem + lay.tq3,
                         reinterpret_cast<const int32_t*>(mem + lay.pt), g.fp8_stride,
                         g.tq3_stride, g.Hkv, g.d, g.P, desc.max_pages_per_seq, g.kind};
  }

  // Selects the next staging slot, once its previous upload has completed.
  mkv_status wait_staging() {
    staging_slot = (staging_slot + 1) % kStagingSlots;
    if (staging_pending[staging_slot]) {
      MKV_HIP(hipEventSynchronize(staging_ev[staging_slot]));
      staging_pending[staging_slot] = false;
    }
    staging = staging_mem + size_t(staging_slot) * staging_bytes;
    return MKV_OK;
  }
};

namespace {

struct Upload {
  size_t dst_off;  // offset in the pool's device block
  size_t bytes;
};

// Copy the staged bytes (laid out back to back, whole 32-bit words) to their
// device offsets: one upload-kernel launch reading the staging slot.
mkv_status flush_uploads(mkv_pool* p, const std::vector<Upload>& ups, hipStream_t s) {
  if (ups.size() > size_t(mkv::kUploadSegs)) return set_err(MKV_EINVAL, "too many upload segments");
  mkv::UploadSet u{};
  u.src = p->staging_dev + (p->staging - p->staging_mem) / 4;
  size_t src = 0;
  for (const Upload& up : ups) {
    if (up.bytes % 4 || up.dst_off % 4) return set_err(MKV_EINVAL, "upload not in whole words");
    if (up.bytes) {
      u.dst[u.nseg] = reinterpret_cast<uint32_t*>(p->mem + up.dst_off);
      u.src_word[u.nseg] = uint32_t(src / 4);
      u.words[u.nseg] = uint32_t(up.bytes / 4);
      ++u.nseg;
    }
    src += up.bytes;
  }
  MKV_HIP(mkv::launch_upload(u, s));
  MKV_HIP(hipEventRecord(p->staging_ev[p->staging_slot], s));
  p->staging_pending[p->staging_slot] = true;
  return MKV_OK;
}

mkv_status upload_pt_row_and_plan(mkv_pool* p, int32_t seq, const void* plan, size_t plan_bytes,
                                  hipStream_t s) {
  mkv_status st = p->wait_staging();
  if (st) return st;
  const std::vector<int32_t>& pt = p->meta.seq(seq).pt;
  const size_t pt_bytes = pt.size() * 4;
  std::memcpy(p->staging, plan, plan_bytes);
  if (pt_bytes) std::memcpy(p->staging + plan_bytes, pt.data(), pt_bytes);
  std::vector<Upload> ups{{p->lay.plan, plan_bytes},
                          {p->lay.pt + size_t(seq) * size_t(p->desc.max_pages_per_seq) * 4,
                           pt_bytes}};
  return flush_uploads(p, ups, s);
}

ProfEvent* prof_begin(mkv_pool* p, int kind, hipStream_t s) {
  if (!p->prof) return nullptr;
  ProfEvent e{kind, nullptr, nullptr};
  if (!p->prof_free.empty()) {
    e = p->prof_free.back();
    p->prof_free.pop_back();
    e.kind = kind;
  } else if (hipEventCreate(&e.a) != hipSuccess || hipEventCreate(&e.b) != hipSuccess) {
    return nullptr;
  }
  if (hipEventRecord(e.a, s) != hipSuccess) return nullptr;
  p->prof_events.push_back(e);
  return &p->prof_events.back();
}

void prof_end(mkv_pool*, ProfEvent* e, hipStream_t s) {
  if (e) (void)hipEventRecord(e->b, s);
}

mkv_status prof_collect(mkv_pool* p) {
  for (ProfEvent& e : p->prof_events) {
    MKV_HIP(hipEventSynchronize(e.b));
    float ms = 0.0f;
    MKV_HIP(hipEventElapsedTime(&ms, e.a, e.b));
    p->prof_ms[e.kind] += ms;
    p->prof_n[e.kind] += 1;
    p->prof_free.push_back(e);
  }
  p->prof_events.clear();
  return MKV_OK;
}

// Split-K policy of a pool: balanced chunks for the device's resident
// partial-kernel waves.  Environment overrides (for tuning): MKV_CHUNK_PAGES
// (fixed chunk length), MKV_TARGET_WAVES, MKV_FP8_PAGE_COST,
// MKV_HEADS_PER_WAVE; MKV_MERGE_NARROW_MAX (read at pool creation) sets the
// largest per-entry chunk count merged by the per-lane merge kernel, and
// MKV_PACE=0 (read at pool creation) turns off the progress-paced wave
// priorities of one-round partial launches.
mkv::SchedPolicy pool_policy(const mkv_pool* p, int32_t Hq) {
  mkv::SchedPolicy pol;
  const mkv::Geom& g = p->meta.geom();
  pol.heads_per_wave = mkv::heads_per_wave(g.d, g.Hkv, Hq / g.Hkv);
  if (const char* e = std::getenv("MKV_HEADS_PER_WAVE")) {
    const int nh = std::atoi(e);
    if (nh == 1 || (nh == 2 && g.d <= 128 && g.Hkv % 2 == 0 && 2 * (Hq / g.Hkv) <= 16)) pol.heads_per_wave = nh;
  }
  pol.target_waves = p->target_waves[pol.heads_per_wave - 1];
  if (const char* e = std::getenv("MKV_CHUNK_PAGES")) pol.fixed_chunk_pages = std::max(0, std::atoi(e));
  if (const char* e = std::getenv("MKV_TARGET_WAVES")) pol.target_waves = std::max(1, std::atoi(e));
  if (const char* e = std::getenv("MKV_FP8_PAGE_COST")) pol.fp8_page_cost = float(std::atof(e));
  return pol;
}

}  // namespace

extern "C" {

size_t mkv_pool_bytes(const mkv_pool_desc* desc) {
  if (!desc) return 0;
  mkv::Geom g;
  if (mkv::validate_desc(to_desc(*desc), &g, nullptr) != MKV_S_OK) return 0;
  return make_layout(to_desc(*desc), g).total;
}

size_t mkv_record_bytes(const mkv_pool_desc* desc, int32_t fmt) {
  if (!desc) return 0;
  mkv::Geom g;
  if (mkv::validate_desc(to_desc(*desc), &g, nullptr) != MKV_S_OK) return 0;
  if (g.kind == mkv::kKindBf16) return fmt == MKV_FMT_BF16 ? size_t(g.fp8_rec) : 0;
  if (fmt == MKV_FMT_FP8) return size_t(g.fp8_rec);
  if (fmt == MKV_FMT_TQ3) return size_t(g.tq3_rec);
  return 0;
}

mkv_status mkv_pool_create(const mkv_pool_desc* desc, void* device_mem, size_t bytes,
                           mkv_pool** out) {
  if (!desc || !out) return set_err(MKV_EINVAL, "null argument");
  *out = nullptr;
  mkv_pool* p = new (std::nothrow) mkv_pool();
  if (!p) return set_err(MKV_ENOMEM, "host allocation failed");
  std::string err;
  int st = p->meta.init(to_desc(*desc), &err);
  if (st != MKV_S_OK) {
    delete p;
    return set_err(mkv_status(st), err);
  }
  p->desc = *desc;
  p->lay = make_layout(to_desc(*desc), p->meta.geom());
  auto cleanup = [&](mkv_status s, const std::string& msg) {
    if (p->staging_mem) (void)hipHostFree(p->staging_mem);
    for (hipEvent_t ev : p->staging_ev)
      if (ev) (void)hipEventDestroy(ev);
    if (p->owns_mem && p->mem) (void)hipFree(p->mem);
    delete p;
    return set_err(s, msg);
  };
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) return cleanup(MKV_EHIP, hipGetErrorString(e));
  for (int nh = 1; nh <= 2; ++nh) {
    if (nh == 2 && desc->head_dim > 128) break;
    int waves = 0;
    e = mkv::partial_resident_waves(desc->head_dim, nh, desc->kv_kind, &waves);
    if (e != hipSuccess) return cleanup(MKV_EHIP, std::string("occupancy query: ") + hipGetErrorString(e));
    if (waves > 0) p->target_waves[nh - 1] = waves;
  }
  if (const char* ev = std::getenv("MKV_MERGE_NARROW_MAX")) p->merge_narrow_max = std::max(0, std::atoi(ev));
  if (const char* ev = std::getenv("MKV_PACE")) p->pace = std::atoi(ev) != 0;
  if (device_mem) {
    if (bytes < p->lay.total) return cleanup(MKV_ERANGE, "device buffer smaller than mkv_pool_bytes");
    if (reinterpret_cast<uintptr_t>(device_mem) % 256)
      return cleanup(MKV_EINVAL, "device buffer must be 256-byte aligned");
    p->mem = static_cast<uint8_t*>(device_mem);
  } else {
    void* m = nullptr;
    e = hipMalloc(&m, p->lay.total);
    if (e != hipSuccess) return cleanup(MKV_EHIP, std::string("hipMalloc: ") + hipGetErrorString(e));
    p->mem = static_cast<uint8_t*>(m);
    p->owns_mem = true;
  }
  p->staging_bytes = std::max(p->lay.sched_bytes, p->lay.plan_bytes +
                                                      size_t(desc->max_pages_per_seq) * 4);
  p->staging_bytes = align256(p->staging_bytes);
  void* h = nullptr;
  // coherent: the upload kernel reads it directly, so no GPU cache may keep
  // an older copy of a slot
  e = hipHostMalloc(&h, p->staging_bytes * mkv_pool::kStagingSlots,
                    hipHostMallocMapped | hipHostMallocCoherent);
  if (e != hipSuccess) return cleanup(MKV_EHIP, std::string("hipHostMalloc: ") + hipGetErrorString(e));
  p->staging_mem = static_cast<uint8_t*>(h);
  void* hd = nullptr;
  e = hipHostGetDevicePointer(&hd, h, 0);
  if (e != hipSuccess)
    return cleanup(MKV_EHIP, std::string("hipHostGetDevicePointer: ") + hipGetErrorString(e));
  p->staging_dev = static_cast<const uint32_t*>(hd);
  p->staging = p->staging_mem;
  for (hipEvent_t& ev : p->staging_ev) {
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return cleanup(MKV_EHIP, hipGetErrorString(e));
  }
  *out = p;
  return MKV_OK;
}

mkv_status mkv_pool_destroy(mkv_pool* p) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  DeviceGuard guard(p->device);
  hipError_t e = hipDeviceSynchronize();
  for (ProfEvent& ev : p->prof_events) {
    (void)hipEventDestroy(ev.a);
    (void)hipEventDestroy(ev.b);
  }
  for (ProfEvent& ev : p->prof_free) {
    (void)hipEventDestroy(ev.a);
    (void)hipEventDestroy(ev.b);
  }
  for (hipEvent_t ev : p->staging_ev)
    if (ev) (void)hipEventDestroy(ev);
  if (p->staging_mem) (void)hipHostFree(p->staging_mem);
  if (p->owns_mem && p->mem) (void)hipFree(p->mem);
  delete p;
  if (e != hipSuccess) return set_err(MKV_EHIP, hipGetErrorString(e));
  return MKV_OK;
}

mkv_status mkv_seq_reset(mkv_pool* p, int32_t seq, hipStream_t) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  std::string err;
  int st = p->meta.reset(seq, &err);
  if (st) return set_err(mkv_status(st), err);
  return MKV_OK;
}

mkv_status mkv_append(mkv_pool* p, int32_t seq, int32_t n, const float* k, const float* v,
                      hipStream_t s) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  if (n > 0 && (!k || !v)) return set_err(MKV_EINVAL, "null K or V");
  DeviceGuard guard(p->device);
  std::vector<mkv::AppendPage> plan;
  std::string err;
  int st = p->meta.append(seq, n, &plan, &err);
  if (st) return set_err(mkv_status(st), err);
  if (plan.empty()) return MKV_OK;
  mkv_status r = upload_pt_row_and_plan(p, seq, plan.data(), plan.size() * sizeof(plan[0]), s);
  if (r) return r;
  const auto* dplan = reinterpret_cast<const mkv::AppendPage*>(p->mem + p->lay.plan);
  if (p->meta.geom().kind == mkv::kKindBf16)
    MKV_HIP(mkv::launch_append_bf16(p->view(), dplan, int32_t(plan.size()), k, v, s));
  else
    MKV_HIP(mkv::launch_append(p->view(), dplan, int32_t(plan.size()), k, v, s));
  return MKV_OK;
}

namespace {

mkv_status commit_schedule(mkv_pool* p, std::vector<mkv::WorkItem>&& fp8,
                           std::vector<mkv::WorkItem>&& tq3, std::vector<int32_t>&& entries,
                           std::vector<int32_t>&& pages, int32_t chunk_pages, size_t from,
                           hipStream_t s);

// A decode step opened pages: extend the cached schedule instead of leaving a
// rebuild to the next decode.  For each batch entry of a sequence that got a
// new page, that entry's last FP8 item (the one ending at the highest logical
// page) takes the page: its page list is copied, one longer, to the end of
// the list array, and the items plus the new tail go up in one upload.
// Returns false, changing nothing, where that does not apply (an entry with
// no FP8 item, a full chunk, no room left in the list array).
bool extend_schedule(mkv_pool* p, const int32_t* seq_ids, const std::vector<mkv::AppendPage>& plan,
                     hipStream_t s, mkv_status* err) {
  const mkv::Schedule& sc = p->sched;
  const size_t cap = size_t(p->desc.max_batch) * size_t(p->desc.max_pages_per_seq);
  std::vector<mkv::WorkItem> fp8 = sc.items[0];
  std::vector<int32_t> entries = sc.entries, pages = sc.pages;
  const size_t old_size = entries.size();
  int32_t chunk_pages = sc.chunk_pages;
  for (const mkv::AppendPage& ap : plan) {
    if (ap.pt_slot < 0) continue;
    const int32_t seq = seq_ids[ap.src_row];
    for (size_t b = 0; b < p->sched_ids.size(); ++b) {
      if (p->sched_ids[b] != seq) continue;
      mkv::WorkItem* last = nullptr;
      for (mkv::WorkItem& it : fp8)
        if (it.b == int32_t(b) && (!last || it.last_lp > last->last_lp)) last = &it;
      if (!last || last->npages >= mkv::kMaxChunkPages || entries.size() + last->npages + 1 > cap)
        return false;
      const int32_t off = int32_t(entries.size());
      for (int32_t i = 0; i < last->npages; ++i) {
        const int32_t e = entries[size_t(last->list_off + i)], lp = pages[size_t(last->list_off + i)];
        entries.push_back(e);
        pages.push_back(lp);
      }
      entries.push_back(ap.pt_entry);
      pages.push_back(ap.lp);
      last->list_off = off;
      last->npages += 1;
      last->last_lp = ap.lp;
      chunk_pages = std::max(chunk_pages, last->npages);
    }
  }
  std::vector<mkv::WorkItem> tq3 = sc.items[1];
  *err = commit_schedule(p, std::move(fp8), std::move(tq3), std::move(entries), std::move(pages),
                         chunk_pages, old_size, s);
  return *err == MKV_OK;
}

// Commits an edited copy of the cached schedule: token counts of every item,
// then one upload of the items and of the page list from word `from` on.
mkv_status commit_schedule(mkv_pool* p, std::vector<mkv::WorkItem>&& fp8,
                           std::vector<mkv::WorkItem>&& tq3, std::vector<int32_t>&& entries,
                           std::vector<int32_t>&& pages, int32_t chunk_pages, size_t from,
                           hipStream_t s) {
  mkv_status err = p->wait_staging();
  if (err) return err;
  mkv::Schedule& sc = p->sched;
  sc.items[0] = std::move(fp8);
  sc.items[1] = std::move(tq3);
  sc.entries = std::move(entries);
  sc.pages = std::move(pages);
  sc.chunk_pages = chunk_pages;
  const int32_t P = p->meta.geom().P;
  size_t off = 0;
  for (auto& list : sc.items)
    for (mkv::WorkItem& it : list) {
      it.last_ntok = mkv::page_tokens(p->meta.seq(it.seq).len, P, it.last_lp);
      std::memcpy(p->staging + off, &it, sizeof(it));
      off += sizeof(it);
    }
  const size_t n_items = sc.items[0].size() + sc.items[1].size();
  const size_t tail = (sc.entries.size() - from) * 4;
  std::memcpy(p->staging + off, sc.entries.data() + from, tail);
  p->sched_valid = false;
  err = flush_uploads(p, {{p->lay.sched + p->lay.items_off, off},
                          {p->lay.sched + entries_off(p->lay, n_items) + from * 4, tail}}, s);
  if (err) return err;
  p->sched_version = p->meta.version();
  p->sched_layout = p->meta.layout_version();
  p->sched_valid = true;
  return MKV_OK;
}

// Pages of sequence `seq` were demoted: in the cached schedule, each batch
// entry of the sequence drops every such page from the FP8 item listing it
// (in place) and its last TQ3 item (highest last page) takes it, its list
// copied one longer to the end of the list array.  The TQ3 item's previous
// last page must be full, since only an item's last page may hold fewer
// tokens.  Returns false, changing nothing, where that does not apply (an FP8
// item would become empty, an entry with no TQ3 item, a full chunk, no room).
bool demote_in_schedule(mkv_pool* p, int32_t seq, const std::vector<mkv::DemotePage>& plan,
                        hipStream_t s, mkv_status* err) {
  const mkv::Schedule& sc = p->sched;
  const size_t cap = size_t(p->desc.max_batch) * size_t(p->desc.max_pages_per_seq);
  std::vector<mkv::WorkItem> fp8 = sc.items[0], tq3 = sc.items[1];
  std::vector<int32_t> entries = sc.entries, pages = sc.pages;
  int32_t chunk_pages = sc.chunk_pages;
  const mkv::Seq& q = p->meta.seq(seq);
  const int32_t P = p->meta.geom().P;
  for (size_t b = 0; b < p->sched_ids.size(); ++b) {
    if (p->sched_ids[b] != seq) continue;
    for (const mkv::DemotePage& dp : plan) {
      mkv::WorkItem* src = nullptr;
      int32_t at = -1;
      for (mkv::WorkItem& it : fp8) {
        if (it.b != int32_t(b)) continue;
        for (int32_t i = 0; i < it.npages && at < 0; ++i)
          if (pages[size_t(it.list_off + i)] == dp.lp) at = i;
        if (at >= 0) {
          src = &it;
          break;
        }
      }
      if (!src || src->npages < 2) return false;
      for (int32_t i = at; i + 1 < src->npages; ++i) {
        entries[size_t(src->list_off + i)] = entries[size_t(src->list_off + i + 1)];
        pages[size_t(src->list_off + i)] = pages[size_t(src->list_off + i + 1)];
      }
      --src->npages;
      src->last_lp = pages[size_t(src->list_off + src->npages - 1)];
      mkv::WorkItem* dst = nullptr;
      for (mkv::WorkItem& it : tq3)
        if (it.b == int32_t(b) && (!dst || it.last_lp > dst->last_lp)) dst = &it;
      if (!dst || dst->npages >= mkv::kMaxChunkPages ||
          mkv::page_tokens(q.len, P, dst->last_lp) != P || entries.size() + dst->npages + 1 > cap)
        return false;
      const int32_t off = int32_t(entries.size());
      for (int32_t i = 0; i < dst->npages; ++i) {
        const int32_t e = entries[size_t(dst->list_off + i)], lp = pages[size_t(dst->list_off + i)];
        entries.push_back(e);
        pages.push_back(lp);
      }
      entries.push_back(q.pt[size_t(dp.lp)]);
      pages.push_back(dp.lp);
      dst->list_off = off;
      dst->npages += 1;
      dst->last_lp = dp.lp;
      chunk_pages = std::max(chunk_pages, dst->npages);
    }
  }
  *err = commit_schedule(p, std::move(fp8), std::move(tq3), std::move(entries), std::move(pages),
                         chunk_pages, 0, s);
  return *err == MKV_OK;
}

}  // namespace

mkv_status mkv_append_step(mkv_pool* p, const int32_t* seq_ids, int32_t B, const float* k,
                           const float* v, hipStream_t s) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  if (B < 0 || (B > 0 && (!seq_ids || !k || !v))) return set_err(MKV_EINVAL, "null argument");
  if (B > p->desc.max_batch) return set_err(MKV_ERANGE, "B exceeds max_batch");
  if (B == 0) return MKV_OK;
  DeviceGuard guard(p->device);
  std::vector<mkv::AppendPage> plan;
  std::string err;
  const bool lists_current = p->sched_valid && p->sched_layout == p->meta.layout_version();
  int st = p->meta.append_step(seq_ids, B, p->desc.max_pages_per_seq, &plan, &err);
  if (st) return set_err(mkv_status(st), err);
  if (lists_current && p->meta.layout_version() != p->sched_layout) {
    mkv_status e = MKV_OK;
    if (!extend_schedule(p, seq_ids, plan, s, &e) && e) return e;
  }
  if (plan.size() <= size_t(mkv::kInlinePages)) {
    // Small step: the plan travels in the kernel arguments.  When the step
    // opened no page and the cached decode schedule predates it only in token
    // counts, the same launch brings the device items' last-page counts up to
    // date, so the next decode of that batch uploads nothing.
    mkv::InlinePlan ip{};
    std::memcpy(ip.pages, plan.data(), plan.size() * sizeof(plan[0]));
    std::vector<std::pair<mkv::WorkItem*, int32_t>> fixes;
    bool patch = p->sched_valid && p->sched_layout == p->meta.layout_version();
    if (patch) {
      const int32_t P = p->meta.geom().P;
      int32_t idx = 0;
      for (auto& list : p->sched.items)
        for (mkv::WorkItem& it : list) {
          const int32_t n = mkv::page_tokens(p->meta.seq(it.seq).len, P, it.last_lp);
          if (n != it.last_ntok) {
            if (ip.n_patch == mkv::kInlinePages) patch = false;
            if (!patch) break;
            ip.patch_off[ip.n_patch] = idx * int32_t(sizeof(mkv::WorkItem) / 4) +
                                       int32_t(offsetof(mkv::WorkItem, last_ntok) / 4);
            ip.patch_val[ip.n_patch++] = n;
            fixes.emplace_back(&it, n);
          }
          ++idx;
        }
    }
    if (!patch) ip.n_patch = 0;
    ip.patch_base = reinterpret_cast<int32_t*>(p->mem + p->lay.sched + p->lay.items_off);
    MKV_HIP(mkv::launch_append_inline(p->view(), ip, int32_t(plan.size()), k, v, s));
    if (patch) {
      for (auto& f : fixes) f.first->last_ntok = f.second;
      p->sched_version = p->meta.version();
    }
    return MKV_OK;
  }
  mkv_status r = p->wait_staging();
  if (r) return r;
  const size_t bytes = plan.size() * sizeof(plan[0]);
  std::memcpy(p->staging, plan.data(), bytes);
  r = flush_uploads(p, {{p->lay.plan, bytes}}, s);
  if (r) return r;
  const auto* dplan = reinterpret_cast<const mkv::AppendPage*>(p->mem + p->lay.plan);
  if (p->meta.geom().kind == mkv::kKindBf16)
    MKV_HIP(mkv::launch_append_bf16(p->view(), dplan, B, k, v, s));
  else
    MKV_HIP(mkv::launch_append(p->view(), dplan, B, k, v, s));
  return MKV_OK;
}

mkv_status mkv_demote(mkv_pool* p, int32_t seq, const int32_t* lps, int32_t n, hipStream_t s) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  DeviceGuard guard(p->device);
  std::vector<mkv::DemotePage> plan;
  std::string err;
  const bool lists_current = p->sched_valid && p->sched_layout == p->meta.layout_version();
  int st = p->meta.demote(seq, lps, n, &plan, &err);
  if (st) return set_err(mkv_status(st), err);
  if (plan.empty()) return MKV_OK;
  mkv_status r = upload_pt_row_and_plan(p, seq, plan.data(), plan.size() * sizeof(plan[0]), s);
  if (r) return r;
  MKV_HIP(mkv::launch_demote(p->view(),
                             reinterpret_cast<const mkv::DemotePage*>(p->mem + p->lay.plan),
                             int32_t(plan.size()), s));
  // keep the cached schedule current where the moved pages fit it
  if (lists_current && !demote_in_schedule(p, seq, plan, s, &r) && r) return r;
  return MKV_OK;
}

mkv_status mkv_decode(mkv_pool* p, const int32_t* seq_ids, int32_t B, const void* q, int32_t Hq,
                      float softmax_scale, float* out, float* lse, hipStream_t s) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  if (!q || !out || !lse || !seq_ids) return set_err(MKV_EINVAL, "null argument");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return set_err(MKV_EINVAL, "q must be 16-byte aligned");
  DeviceGuard guard(p->device);
  const bool same_batch = p->sched_valid && p->sched_Hq == Hq && int32_t(p->sched_ids.size()) == B &&
                          std::memcmp(p->sched_ids.data(), seq_ids, size_t(B) * 4) == 0;
  if (same_batch && p->sched_version != p->meta.version() &&
      p->sched_layout == p->meta.layout_version()) {
    // Only token counts changed (appends inside existing pages): the page lists
    // stand; refresh each item's last-page token count and upload the items.
    mkv_status r = p->wait_staging();
    if (r) return r;
    const int32_t P = p->meta.geom().P;
    size_t off = 0;
    for (auto& list : p->sched.items)
      for (mkv::WorkItem& it : list) {
        it.last_ntok = mkv::page_tokens(p->meta.seq(it.seq).len, P, it.last_lp);
        std::memcpy(p->staging + off, &it, sizeof(it));
        off += sizeof(it);
      }
    p->sched_valid = false;
    r = flush_uploads(p, {{p->lay.sched + p->lay.items_off, off}}, s);
    if (r) return r;
    p->sched_version = p->meta.version();
    p->sched_valid = true;
  }
  const bool same = same_batch && p->sched_version == p->meta.version();
  if (!same) {
    std::string err;
    mkv::Schedule sc;
    int st = p->meta.build_schedule(seq_ids, B, Hq, pool_policy(p, Hq), &sc, &err);
    if (st) return set_err(mkv_status(st), err);
    mkv_status r = p->wait_staging();
    if (r) return r;
    // the staging slot mirrors the schedule region: one copy
    const size_t n8 = sc.items[0].size(), n3 = sc.items[1].size();
    const size_t eoff = entries_off(p->lay, n8 + n3);
    uint8_t* st8 = p->staging;
    std::memcpy(st8, sc.chunk_base.data(), sc.chunk_base.size() * 4);
    std::memcpy(st8 + p->lay.items_off, sc.items[0].data(), n8 * 32);
    std::memcpy(st8 + p->lay.items_off + n8 * 32, sc.items[1].data(), n3 * 32);
    std::memcpy(st8 + eoff, sc.entries.data(), sc.entries.size() * 4);
    p->sched_valid = false;
    r = flush_uploads(p, {{p->lay.sched, eoff + sc.entries.size() * 4}}, s);
    if (r) return r;
    p->sched = std::move(sc);
    p->sched_ids.assign(seq_ids, seq_ids + B);
    p->sched_Hq = Hq;
    p->sched_version = p->meta.version();
    p->sched_layout = p->meta.layout_version();
    p->sched_valid = true;
  }
  const mkv::Schedule& sc = p->sched;
  uint8_t* region = p->mem + p->lay.sched;
  const mkv::WorkItem* items = reinterpret_cast<const mkv::WorkItem*>(region + p->lay.items_off);
  mkv::DecodeArgs a{};
  a.pv = p->view();
  a.entries = reinterpret_cast<const int32_t*>(
      region + entries_off(p->lay, sc.items[0].size() + sc.items[1].size()));
  a.chunk_base = reinterpret_cast<const int32_t*>(region);
  a.q = static_cast<const uint16_t*>(q);
  a.B = B;
  a.Hq = Hq;
  a.scale = softmax_scale;
  a.pm = reinterpret_cast<float*>(p->mem + p->lay.pm);
  a.pl = reinterpret_cast<float*>(p->mem + p->lay.pl);
  a.pacc = reinterpret_cast<float*>(p->mem + p->lay.pacc);
  a.out = out;
  a.lse = lse;
  a.nh = sc.heads_per_wave;
  a.max_seq_chunks = sc.max_seq_chunks;
  a.items = items;
  a.n_items = int32_t(sc.items[0].size() + sc.items[1].size());
  {
    const int64_t waves = int64_t(a.n_items) * ((a.pv.Hkv + a.nh - 1) / a.nh) * mkv::kWavesPerWorkgroup;
    a.pace = p->pace && waves <= p->target_waves[a.nh - 1] ? 1 : 0;
  }
  {
    ProfEvent* e = prof_begin(p, 0, s);
    MKV_HIP(mkv::launch_partial(a, s));
    prof_end(p, e, s);
  }
  ProfEvent* e = prof_begin(p, 1, s);
  MKV_HIP(mkv::launch_merge(a, p->merge_narrow_max, s));
  prof_end(p, e, s);
  return MKV_OK;
}

mkv_status mkv_materialize(mkv_pool* src, int32_t src_seq, mkv_pool* dst, int32_t dst_seq,
                           hipStream_t s) {
  if (!src || !dst || src == dst) return set_err(MKV_EINVAL, "two distinct pools are required");
  const mkv::Geom& gs = src->meta.geom();
  const mkv::Geom& gd = dst->meta.geom();
  if (gs.kind != mkv::kKindMixed || gd.kind != mkv::kKindBf16)
    return set_err(MKV_EINVAL, "source must be a mixed pool and destination a BF16 control pool");
  if (gs.Hkv != gd.Hkv || gs.d != gd.d || gs.P != gd.P)
    return set_err(MKV_EINVAL, "pools differ in num_kv_heads, head_dim or page_size");
  if (src->device != dst->device) return set_err(MKV_EINVAL, "pools live on different devices");
  if (src_seq < 0 || src_seq >= src->desc.max_seqs || dst_seq < 0 || dst_seq >= dst->desc.max_seqs)
    return set_err(MKV_EINVAL, "sequence id out of range");
  const mkv::Seq& sq = src->meta.seq(src_seq);
  if (sq.len == 0) return set_err(MKV_EINVAL, "empty source sequence");
  if (dst->meta.seq(dst_seq).len != 0) return set_err(MKV_ESTATE, "destination sequence is not empty");
  DeviceGuard guard(dst->device);
  std::vector<mkv::AppendPage> ap;
  std::string err;
  int st = dst->meta.append(dst_seq, sq.len, &ap, &err);
  if (st) return set_err(mkv_status(st), err);
  std::vector<mkv::MaterialisePage> plan;
  plan.reserve(ap.size());
  for (const mkv::AppendPage& a : ap)   // fresh pages: row0 == 0, one per source page
    plan.push_back(mkv::MaterialisePage{a.lp, sq.pt[size_t(a.lp)], a.phys, a.nrows, 0, 0, 0, 0});
  mkv_status r = upload_pt_row_and_plan(dst, dst_seq, plan.data(), plan.size() * sizeof(plan[0]), s);
  if (r) return r;
  MKV_HIP(mkv::launch_materialise(src->view(), dst->view(),
                                  reinterpret_cast<const mkv::MaterialisePage*>(dst->mem + dst->lay.plan),
                                  int32_t(plan.size()), s));
  return MKV_OK;
}

mkv_status mkv_seq_info(mkv_pool* p, int32_t seq, int32_t* len, int32_t* n_pages) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  if (seq < 0 || seq >= p->desc.max_seqs) return set_err(MKV_EINVAL, "sequence id out of range");
  const mkv::Seq& q = p->meta.seq(seq);
  if (len) *len = q.len;
  if (n_pages) *n_pages = int32_t(q.pt.size());
  return MKV_OK;
}

mkv_status mkv_page_table(mkv_pool* p, int32_t seq, int32_t* entries, int32_t cap) {
  if (!p || !entries) return set_err(MKV_EINVAL, "null argument");
  if (seq < 0 || seq >= p->desc.max_seqs) return set_err(MKV_EINVAL, "sequence id out of range");
  const mkv::Seq& q = p->meta.seq(seq);
  if (cap < int32_t(q.pt.size())) return set_err(MKV_ERANGE, "entries buffer too small");
  std::memcpy(entries, q.pt.data(), q.pt.size() * 4);
  return MKV_OK;
}

mkv_status mkv_pool_stats(mkv_pool* p, mkv_stats* o) {
  if (!p || !o) return set_err(MKV_EINVAL, "null argument");
  const mkv::Geom& g = p->meta.geom();
  std::memset(o, 0, sizeof(*o));
  o->live_tokens = p->meta.live_tokens();
  o->fp8_pages_live = p->meta.live_pages(0);
  o->tq3_pages_live = p->meta.live_pages(1);
  o->fp8_pages_free = p->meta.fp8_free();
  o->tq3_pages_free = p->meta.tq3_free();
  int64_t kvb = 0;
  for (int32_t sq = 0; sq < p->desc.max_seqs; ++sq) kvb += p->meta.seq_kv_bytes(sq);
  o->kv_bytes = kvb;
  if (o->live_tokens > 0) {
    o->bytes_per_token = double(kvb) / double(o->live_tokens);
    o->ratio_vs_bf16 = double(4ll * g.Hkv * g.d) / o->bytes_per_token;
    o->ratio_vs_fp8 = double(2ll * g.Hkv * g.d) / o->bytes_per_token;
  }
  o->dense_shadow_bytes = 0;
  o->dense_fallbacks = 0;
  return MKV_OK;
}

mkv_status mkv_debug_gather(mkv_pool* p, int32_t seq, int32_t first, int32_t n, void* dst,
                            hipStream_t s) {
  if (!p || !dst) return set_err(MKV_EINVAL, "null argument");
  if (seq < 0 || seq >= p->desc.max_seqs) return set_err(MKV_EINVAL, "sequence id out of range");
  const mkv::Seq& q = p->meta.seq(seq);
  if (first < 0 || n < 0 || int64_t(first) + n > int64_t(q.pt.size()))
    return set_err(MKV_EINVAL, "page range outside the sequence");
  DeviceGuard guard(p->device);
  const mkv::Geom& g = p->meta.geom();
  const int64_t slot = std::max(g.fp8_rec, g.tq3_rec);
  MKV_HIP(mkv::launch_gather(p->view(), seq, first, n, static_cast<uint8_t*>(dst), slot, s));
  return MKV_OK;
}

mkv_status mkv_profile_enable(mkv_pool* p, int32_t on) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  p->prof = on != 0;
  return MKV_OK;
}

mkv_status mkv_profile_read(mkv_pool* p, mkv_profile* o) {
  if (!p || !o) return set_err(MKV_EINVAL, "null argument");
  DeviceGuard guard(p->device);
  mkv_status r = prof_collect(p);
  if (r) return r;
  o->ms_partial = p->prof_ms[0];
  o->ms_merge = p->prof_ms[1];
  o->n_partial = p->prof_n[0];
  o->n_merge = p->prof_n[1];
  for (int i = 0; i < 2; ++i) {
    p->prof_ms[i] = 0;
    p->prof_n[i] = 0;
  }
  return MKV_OK;
}

const char* mkv_status_string(mkv_status s) {
  switch (s) {
    case MKV_OK: return "ok";
    case MKV_EINVAL: return "invalid argument";
    case MKV_ENOMEM: return "slab has too few free pages";
    case MKV_ESTATE: return "operation not allowed in the sequence's state";
    case MKV_ERANGE: return "capacity exceeded";
    case MKV_EHIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* mkv_last_error(void) { return g_err.c_str(); }

}  // extern "C"
