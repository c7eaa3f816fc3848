// C-ABI of libmkv (declared in include/mkv.h): argument validation, device
// memory layout, stream-ordered metadata uploads and kernel launches.
#include "mkv.h"

#include <hip/hip_runtime.h>

#include <algorithm>
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
  int32_t sched_waves[2] = {2048, 1024};    // waves a schedule below the split-K floor fills
  int32_t merge_narrow_max = 16;            // per-lane merge up to this many chunks per entry
  bool pace = true;                         // progress-paced wave priorities (one-round launches)
  int32_t anchor_window = -1;               // mkv_decode_step's anchor policy window (-1: off)
  void* static_ws = nullptr;                // the device's fixed workspace (mkv_decode_static)
  // profiling
  bool prof = false;
  std::vector<ProfEvent> prof_events;
  std::vector<ProfEvent> prof_free;
  double prof_ms[4] = {0, 0, 0, 0};    // partial, merge, append, demote
  int64_t prof_n[4] = {0, 0, 0, 0};

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

// K/V rows are read as 16-byte vectors.
bool rows_aligned(const float* k, const float* v) {
  return reinterpret_cast<uintptr_t>(k) % 16 == 0 && reinterpret_cast<uintptr_t>(v) % 16 == 0;
}

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

// Host bytes bound for a device offset of the pool (whole 32-bit words).
struct Piece {
  size_t dst_off;
  const void* src;
  size_t bytes;
};

// Uploads the pieces in order with as few upload launches as the segment
// count and the staging slot size allow.
mkv_status upload_pieces(mkv_pool* p, const std::vector<Piece>& pieces, hipStream_t s) {
  size_t i = 0;
  while (i < pieces.size()) {
    mkv_status r = p->wait_staging();
    if (r) return r;
    std::vector<Upload> ups;
    size_t off = 0;
    while (i < pieces.size() && ups.size() < size_t(mkv::kUploadSegs) &&
           off + pieces[i].bytes <= p->staging_bytes) {
      if (pieces[i].bytes) std::memcpy(p->staging + off, pieces[i].src, pieces[i].bytes);
      ups.push_back(Upload{pieces[i].dst_off, pieces[i].bytes});
      off += pieces[i].bytes;
      ++i;
    }
    if (ups.empty()) return set_err(MKV_EINVAL, "upload larger than a staging slot");
    r = flush_uploads(p, ups, s);
    if (r) return r;
  }
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

// Brackets the launches of its scope with a pair of profiling events of one
// kind (0 partial, 1 merge, 2 append, 3 demote) while profiling is on.
struct ProfScope {
  mkv_pool* p;
  hipStream_t s;
  size_t idx = SIZE_MAX;
  ProfScope(mkv_pool* pool, int kind, hipStream_t stream, bool on = true) : p(pool), s(stream) {
    if (!on || !p->prof) return;
    ProfEvent e{kind, nullptr, nullptr};
    if (!p->prof_free.empty()) {
      e = p->prof_free.back();
      p->prof_free.pop_back();
      e.kind = kind;
    } else if (hipEventCreate(&e.a) != hipSuccess || hipEventCreate(&e.b) != hipSuccess) {
      return;
    }
    if (hipEventRecord(e.a, s) != hipSuccess) {
      p->prof_free.push_back(e);
      return;
    }
    idx = p->prof_events.size();
    p->prof_events.push_back(e);
  }
  ~ProfScope() {
    if (idx != SIZE_MAX) (void)hipEventRecord(p->prof_events[idx].b, s);
  }
};

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
  pol.target_waves = p->sched_waves[pol.heads_per_wave - 1];
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
  e = mkv::static_workspace(p->device, &p->static_ws);
  if (e != hipSuccess) return cleanup(MKV_EHIP, std::string("static workspace: ") + hipGetErrorString(e));
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device);
  if (e != hipSuccess) return cleanup(MKV_EHIP, std::string("device attribute: ") + hipGetErrorString(e));
  for (int nh = 1; nh <= 2; ++nh) {
    if (nh == 2 && desc->head_dim > 128) break;
    int waves = 0;
    e = mkv::partial_resident_waves(desc->head_dim, nh, desc->kv_kind, &waves);
    if (e != hipSuccess) return cleanup(MKV_EHIP, std::string("occupancy query: ") + hipGetErrorString(e));
    if (waves > 0) {
      p->target_waves[nh - 1] = waves;
      // Where four waves fit a SIMD, schedules below the split-K floor fill
      // three of them: fewer, longer items pay the per-workgroup set-up and
      // combine less often, and three waves still hide the tile loop's
      // latencies (measured on the ragged batch: 25.4 against 26.7 us per
      // step); with two waves per SIMD every slot is needed.
      p->sched_waves[nh - 1] = cus > 0 && waves >= 16 * cus ? waves / 4 * 3 : waves;
    }
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
  if (n > 0 && !rows_aligned(k, v)) return set_err(MKV_EINVAL, "K and V must be 16-byte aligned");
  DeviceGuard guard(p->device);
  std::vector<mkv::AppendPage> plan;
  std::string err;
  mkv::Undo undo;
  int st = p->meta.append(seq, n, &plan, &err, &undo);
  if (st) return set_err(mkv_status(st), err);
  if (plan.empty()) return MKV_OK;
  mkv_status r = upload_pt_row_and_plan(p, seq, plan.data(), plan.size() * sizeof(plan[0]), s);
  if (r == MKV_OK) {
    const auto* dplan = reinterpret_cast<const mkv::AppendPage*>(p->mem + p->lay.plan);
    ProfScope ps(p, 2, s);
    const hipError_t e = p->meta.geom().kind == mkv::kKindBf16
                             ? mkv::launch_append_bf16(p->view(), dplan, int32_t(plan.size()), k, v, s)
                             : mkv::launch_append(p->view(), dplan, int32_t(plan.size()), k, v, s);
    if (e != hipSuccess) r = set_err(MKV_EHIP, std::string("append launch: ") + hipGetErrorString(e));
  }
  if (r) p->meta.rollback(undo);   // nothing of the append stays in the metadata
  return r;
}

namespace {

size_t list_cap(const mkv_pool* p) {
  return size_t(p->desc.max_batch) * size_t(p->desc.max_pages_per_seq);
}

// Pieces that bring the device copy of the cached schedule up to date after
// in-place edits: all item records and the list words the edits rewrote
// (sorted, runs closer than 64 words merged).
void schedule_pieces(const mkv_pool* p, mkv::ListEdits& ed, std::vector<Piece>* out) {
  const mkv::Schedule& sc = p->sched;
  const size_t n8 = sc.items[0].size(), n3 = sc.items[1].size();
  const size_t base = p->lay.sched + p->lay.items_off;
  out->push_back(Piece{base, sc.items[0].data(), n8 * sizeof(mkv::WorkItem)});
  out->push_back(Piece{base + n8 * sizeof(mkv::WorkItem), sc.items[1].data(), n3 * sizeof(mkv::WorkItem)});
  auto& r = ed.ranges;
  std::sort(r.begin(), r.end());
  std::vector<std::pair<size_t, size_t>> runs;
  for (const auto& x : r) {
    if (!runs.empty() && x.first <= runs.back().second + 64)
      runs.back().second = std::max(runs.back().second, x.second);
    else
      runs.push_back(x);
  }
  const size_t eoff = p->lay.sched + entries_off(p->lay, n8 + n3);
  for (const auto& x : runs)
    out->push_back(Piece{eoff + x.first * 4, sc.entries.data() + x.first, (x.second - x.first) * 4});
}

// Uploads what in-place edits changed and marks the cached schedule current;
// on failure it is dropped (the next decode rebuilds it).
mkv_status commit_edits(mkv_pool* p, mkv::ListEdits& ed, hipStream_t s) {
  p->sched_valid = false;
  std::vector<Piece> pieces;
  schedule_pieces(p, ed, &pieces);
  mkv_status r = upload_pieces(p, pieces, s);
  if (r) return r;
  p->sched_version = p->meta.version();
  p->sched_layout = p->meta.layout_version();
  p->sched_valid = true;
  return MKV_OK;
}

}  // namespace

namespace {

// The device side of an append step whose metadata is already committed: the
// append kernel (with the plan in its arguments for small steps, else an
// uploaded plan).  A small step that opened no page also brings the cached
// schedule's last-page token counts up to date in the same launch.
mkv_status append_step_device(mkv_pool* p, const int32_t*, int32_t B,
                              const std::vector<mkv::AppendPage>& plan, const float* k,
                              const float* v, hipStream_t s) {
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
    {
      ProfScope ps(p, 2, s);
      MKV_HIP(mkv::launch_append_inline(p->view(), ip, int32_t(plan.size()), k, v, s));
    }
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
  ProfScope ps(p, 2, s);
  if (p->meta.geom().kind == mkv::kKindBf16)
    MKV_HIP(mkv::launch_append_bf16(p->view(), dplan, B, k, v, s));
  else
    MKV_HIP(mkv::launch_append(p->view(), dplan, B, k, v, s));
  return MKV_OK;
}

}  // namespace

mkv_status mkv_append_step(mkv_pool* p, const int32_t* seq_ids, int32_t B, const float* k,
                           const float* v, hipStream_t s) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  if (B < 0 || (B > 0 && (!seq_ids || !k || !v))) return set_err(MKV_EINVAL, "null argument");
  if (B > 0 && !rows_aligned(k, v)) return set_err(MKV_EINVAL, "K and V must be 16-byte aligned");
  if (B > p->desc.max_batch) return set_err(MKV_ERANGE, "B exceeds max_batch");
  if (B == 0) return MKV_OK;
  DeviceGuard guard(p->device);
  std::vector<mkv::AppendPage> plan;
  std::string err;
  const bool lists_current = p->sched_valid && p->sched_layout == p->meta.layout_version();
  mkv::Undo undo;
  int st = p->meta.append_step(seq_ids, B, p->desc.max_pages_per_seq, &plan, &err, &undo);
  if (st) return set_err(mkv_status(st), err);
  mkv_status r = append_step_device(p, seq_ids, B, plan, k, v, s);
  if (r) {
    p->meta.rollback(undo);
    return r;
  }
  if (lists_current && p->meta.layout_version() != p->sched_layout) {
    // pages opened: extend the cached schedule where it applies; otherwise
    // (or if its upload fails) the next decode rebuilds it
    mkv::ListEdits ed;
    if (mkv::schedule_extend(p->meta, p->sched_ids, seq_ids, plan, list_cap(p), &p->sched, &ed))
      (void)commit_edits(p, ed, s);
    else
      p->sched_valid = false;
  }
  return MKV_OK;
}


namespace {

// mkv_demote on a pool whose device is current.
mkv_status demote_impl(mkv_pool* p, int32_t seq, const int32_t* lps, int32_t n, hipStream_t s) {
  std::vector<mkv::DemotePage> plan;
  std::string err;
  const bool lists_current = p->sched_valid && p->sched_layout == p->meta.layout_version();
  mkv::Undo undo;
  int st = p->meta.demote(seq, lps, n, &plan, &err, &undo);
  if (st) return set_err(mkv_status(st), err);
  if (plan.empty()) return MKV_OK;
  mkv_status r = upload_pt_row_and_plan(p, seq, plan.data(), plan.size() * sizeof(plan[0]), s);
  if (r == MKV_OK) {
    ProfScope ps(p, 3, s);
    const hipError_t e = mkv::launch_demote(
        p->view(), reinterpret_cast<const mkv::DemotePage*>(p->mem + p->lay.plan), int32_t(plan.size()), s);
    if (e != hipSuccess) r = set_err(MKV_EHIP, std::string("demote launch: ") + hipGetErrorString(e));
  }
  if (r) {
    p->meta.rollback(undo);
    return r;
  }
  // keep the cached schedule current where the moved pages fit it; otherwise
  // (or if its upload fails) the next decode rebuilds it
  if (lists_current) {
    mkv::ListEdits ed;
    if (mkv::schedule_demote(p->meta, p->sched_ids, seq, plan, list_cap(p), &p->sched, &ed))
      (void)commit_edits(p, ed, s);
    else
      p->sched_valid = false;
  }
  return MKV_OK;
}

}  // namespace

mkv_status mkv_demote(mkv_pool* p, int32_t seq, const int32_t* lps, int32_t n, hipStream_t s) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  DeviceGuard guard(p->device);
  return demote_impl(p, seq, lps, n, s);
}

mkv_status mkv_set_anchor_window(mkv_pool* p, int32_t window_tokens) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  if (window_tokens >= 0 && p->meta.geom().kind == mkv::kKindBf16)
    return set_err(MKV_ESTATE, "a BF16 control pool holds one format; pages are never converted");
  p->anchor_window = window_tokens < 0 ? -1 : window_tokens;
  return MKV_OK;
}

mkv_status mkv_protect_pages(mkv_pool* p, int32_t seq, const int32_t* lps, int32_t n, int32_t protect) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  std::string err;
  const int st = p->meta.protect(seq, lps, n, protect != 0, &err);
  return st ? set_err(mkv_status(st), err) : MKV_OK;
}

namespace {

// Where a decode keeps its partial states: the pool's workspace, or the
// device's fixed one (mkv_decode_static), which bounds the chunk count.
enum class StateHome { kPool, kStatic };

// Bytes of the partial states of n_chunks chunks of Hq heads (m, l, acc).
size_t state_bytes(int64_t n_chunks, int32_t Hq, int32_t d) {
  const size_t slots = size_t(n_chunks) * size_t(Hq);
  return 2 * align256(slots * 4) + slots * size_t(d) * 4;
}

mkv_status decode_impl(mkv_pool* p, const int32_t* seq_ids, int32_t B, const void* q, int32_t Hq,
                       float softmax_scale, float* out, float* lse, hipStream_t s, StateHome home) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  if (!q || !out || !lse || !seq_ids) return set_err(MKV_EINVAL, "null argument");
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return set_err(MKV_EINVAL, "q must be 16-byte aligned");
  const int32_t d = p->meta.geom().d;
  auto fits = [&](int64_t n_chunks) {
    if (home != StateHome::kStatic || state_bytes(n_chunks, Hq, d) <= mkv::kStaticWorkspaceBytes)
      return MKV_OK;
    return set_err(MKV_ERANGE, "partial states of " + std::to_string(n_chunks) + " chunks x " +
                                   std::to_string(Hq) + " heads need " +
                                   std::to_string(state_bytes(n_chunks, Hq, d)) +
                                   " bytes; the static workspace holds " +
                                   std::to_string(mkv::kStaticWorkspaceBytes));
  };
  if (home == StateHome::kStatic && !p->static_ws) return set_err(MKV_EHIP, "no static workspace");
  DeviceGuard guard(p->device);
  const bool same_batch = p->sched_valid && p->sched_Hq == Hq && int32_t(p->sched_ids.size()) == B &&
                          std::memcmp(p->sched_ids.data(), seq_ids, size_t(B) * 4) == 0;
  if (same_batch) {
    mkv_status r = fits(p->sched.n_chunks);
    if (r) return r;
  }
  if (same_batch && p->sched_version != p->meta.version() &&
      p->sched_layout == p->meta.layout_version()) {
    // Only token counts changed (appends inside existing pages): the page lists
    // stand; refresh each item's last-page token count and upload the items.
    mkv_status r = p->wait_staging();
    if (r) return r;
    mkv::schedule_refresh_tokens(p->meta, &p->sched);
    size_t off = 0;
    for (const auto& list : p->sched.items)
      for (const mkv::WorkItem& it : list) {
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
    mkv_status r = fits(sc.n_chunks);
    if (r) return r;
    r = p->wait_staging();
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
  if (home == StateHome::kStatic) {
    const size_t slots = size_t(sc.n_chunks) * size_t(Hq);
    uint8_t* ws = static_cast<uint8_t*>(p->static_ws);
    a.pm = reinterpret_cast<float*>(ws);
    a.pl = reinterpret_cast<float*>(ws + align256(slots * 4));
    a.pacc = reinterpret_cast<float*>(ws + 2 * align256(slots * 4));
  } else {
    a.pm = reinterpret_cast<float*>(p->mem + p->lay.pm);
    a.pl = reinterpret_cast<float*>(p->mem + p->lay.pl);
    a.pacc = reinterpret_cast<float*>(p->mem + p->lay.pacc);
  }
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
  // (profiling events are taken only on the pool-workspace path)
  const bool prof = home == StateHome::kPool;
  {
    ProfScope ps(p, 0, s, prof);
    MKV_HIP(mkv::launch_partial(a, s));
  }
  {
    ProfScope ps(p, 1, s, prof);
    MKV_HIP(mkv::launch_merge(a, p->merge_narrow_max, s));
  }
  return MKV_OK;
}

}  // namespace

mkv_status mkv_decode(mkv_pool* p, const int32_t* seq_ids, int32_t B, const void* q, int32_t Hq,
                      float softmax_scale, float* out, float* lse, hipStream_t s) {
  return decode_impl(p, seq_ids, B, q, Hq, softmax_scale, out, lse, s, StateHome::kPool);
}

mkv_status mkv_decode_step(mkv_pool* p, const int32_t* seq_ids, int32_t B, const float* k, const float* v,
                           const void* q, int32_t Hq, float softmax_scale, float* out, float* lse,
                           hipStream_t s) {
  if (!p) return set_err(MKV_EINVAL, "null pool");
  if (B < 1 || !seq_ids || !k || !v || !q || !out || !lse) return set_err(MKV_EINVAL, "null argument");
  if (!rows_aligned(k, v)) return set_err(MKV_EINVAL, "K and V must be 16-byte aligned");
  if (B > p->desc.max_batch) return set_err(MKV_ERANGE, "B exceeds max_batch");
  // the decode's argument checks come first: once the append is enqueued the
  // step can only fail on the device side
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0) return set_err(MKV_EINVAL, "q must be 16-byte aligned");
  const int32_t Hkv = p->meta.geom().Hkv;
  if (Hq < 1 || Hq % Hkv) return set_err(MKV_EINVAL, "Hq must be a positive multiple of Hkv");
  if (Hq > p->desc.max_q_heads) return set_err(MKV_ERANGE, "Hq exceeds max_q_heads");
  if (Hq / Hkv > 16) return set_err(MKV_EINVAL, "Hq / Hkv must be at most 16");
  DeviceGuard guard(p->device);
  std::vector<mkv::AppendPage> plan;
  std::string err;
  const bool lists_current = p->sched_valid && p->sched_layout == p->meta.layout_version();
  mkv::Undo undo;
  int st = p->meta.append_step(seq_ids, B, p->desc.max_pages_per_seq, &plan, &err, &undo);
  if (st) return set_err(mkv_status(st), err);

  // The anchor policy's conversions at the new lengths, checked against the
  // TQ3 slab, then applied to the metadata (each with its undo record).
  struct Conv {
    int32_t seq, next;
    std::vector<mkv::DemotePage> plan;
    mkv::Undo undo;
  };
  std::vector<Conv> conv;
  auto take_back = [&]() {
    for (size_t i = conv.size(); i-- > 0;) p->meta.rollback(conv[i].undo);
    p->meta.rollback(undo);
  };
  size_t n_conv = 0;
  if (p->anchor_window >= 0) {
    std::vector<int32_t> lps;
    std::vector<std::vector<int32_t>> todo(static_cast<size_t>(B));
    std::vector<int32_t> nexts(static_cast<size_t>(B));
    for (int32_t b = 0; b < B; ++b) {
      p->meta.policy_pages(seq_ids[b], p->anchor_window, &todo[size_t(b)], &nexts[size_t(b)]);
      n_conv += todo[size_t(b)].size();
    }
    if (int64_t(n_conv) > p->meta.tq3_free()) {
      p->meta.rollback(undo);
      return set_err(MKV_ENOMEM, "TQ3 slab has too few free pages for the anchor policy's conversions");
    }
    for (int32_t b = 0; b < B; ++b) {
      conv.push_back(Conv{seq_ids[b], nexts[size_t(b)], {}, {}});
      const auto& t = todo[size_t(b)];
      if (t.empty()) continue;
      st = p->meta.demote(seq_ids[b], t.data(), int32_t(t.size()), &conv.back().plan, &err, &conv.back().undo);
      if (st) {
        conv.pop_back();
        take_back();
        return set_err(mkv_status(st), err);
      }
    }
  }
  auto finish = [&]() {
    for (const Conv& c : conv) p->meta.set_policy_next(c.seq, c.next);
    return decode_impl(p, seq_ids, B, q, Hq, softmax_scale, out, lse, s, StateHome::kPool);
  };

  // One launch when it fits the kernel arguments: the appended pages, the
  // conversions (each writing its page-table entry) and the cached
  // schedule's edits as word patches.  The appended and converted FP8 pages
  // must differ (a window of 0 can convert the page this step filled).
  bool fused = plan.size() <= size_t(mkv::kInlinePages) && n_conv <= size_t(mkv::kStepConv);
  for (const Conv& c : conv)
    for (const mkv::DemotePage& dp : c.plan)
      for (const mkv::AppendPage& ap : plan) fused = fused && ap.phys != dp.src_phys;
  if (fused) {
    mkv::StepPlan sp{};
    sp.patch_base = reinterpret_cast<int32_t*>(p->mem + p->lay.sched + p->lay.items_off);
    sp.n_append = int32_t(plan.size());
    std::memcpy(sp.pages, plan.data(), plan.size() * sizeof(plan[0]));
    for (const Conv& c : conv)
      for (const mkv::DemotePage& dp : c.plan) {
        mkv::DemotePage x = dp;
        x.pad0 = c.seq * p->desc.max_pages_per_seq + dp.lp;
        x.pad1 = p->meta.seq(c.seq).pt[size_t(dp.lp)];
        sp.conv[sp.n_conv++] = x;
      }
    // schedule edits in place; their changed words become patches (or, past
    // the patch capacity, an upload before the launch)
    bool edited = false;
    mkv::ListEdits ed;
    if (lists_current) {
      const std::vector<mkv::WorkItem> before[2] = {p->sched.items[0], p->sched.items[1]};
      edited = mkv::schedule_extend(p->meta, p->sched_ids, seq_ids, plan, list_cap(p), &p->sched, &ed);
      for (const Conv& c : conv)
        if (edited && !c.plan.empty())
          edited = mkv::schedule_demote(p->meta, p->sched_ids, c.seq, c.plan, list_cap(p), &p->sched, &ed);
      if (edited) {
        const size_t words = sizeof(mkv::WorkItem) / 4;
        const size_t n8 = p->sched.items[0].size();
        const int32_t eword = int32_t((entries_off(p->lay, n8 + p->sched.items[1].size()) - p->lay.items_off) / 4);
        bool fits = true;
        auto patch = [&](int32_t off, int32_t val) {
          if (sp.n_patch == mkv::kStepPatches) {
            fits = false;
            return;
          }
          sp.patch_off[sp.n_patch] = off;
          sp.patch_val[sp.n_patch++] = val;
        };
        for (int f = 0; f < 2 && fits; ++f)
          for (size_t i = 0; i < before[f].size() && fits; ++i) {
            const int32_t* a = reinterpret_cast<const int32_t*>(&before[f][i]);
            const int32_t* b = reinterpret_cast<const int32_t*>(&p->sched.items[f][i]);
            for (size_t w = 0; w < words; ++w)
              if (a[w] != b[w]) patch(int32_t(((f ? n8 : 0) + i) * words + w), b[w]);
          }
        for (const auto& x : ed.ranges)
          for (size_t w = x.first; w < x.second && fits; ++w) patch(eword + int32_t(w), p->sched.entries[w]);
        if (!fits) {
          sp.n_patch = 0;
          p->sched_valid = false;
          std::vector<Piece> pieces;
          schedule_pieces(p, ed, &pieces);
          mkv_status r = upload_pieces(p, pieces, s);
          if (r) {
            take_back();
            return r;
          }
        }
      }
    }
    p->sched_valid = false;
    ProfScope ps(p, 2, s);
    const hipError_t e = mkv::launch_step(p->view(), sp, k, v, s);
    if (e != hipSuccess) {
      take_back();
      return set_err(MKV_EHIP, std::string("step launch: ") + hipGetErrorString(e));
    }
    if (edited) {
      p->sched_version = p->meta.version();
      p->sched_layout = p->meta.layout_version();
      p->sched_valid = true;
    }
    return finish();
  }

  // Otherwise batched uploads: the append plan (unless it travels in the
  // kernel arguments), the conversions' plan and the cached schedule's edits,
  // then the append; the converted sequences' page-table rows, then one
  // conversion launch (so that a failed append leaves the device page table
  // as the metadata it rolls back to).
  const bool inline_plan = plan.size() <= size_t(mkv::kInlinePages);
  const size_t a_bytes = inline_plan ? 0 : plan.size() * sizeof(plan[0]);
  std::vector<mkv::DemotePage> dplan;
  for (const Conv& c : conv) dplan.insert(dplan.end(), c.plan.begin(), c.plan.end());
  const size_t d_bytes = dplan.size() * sizeof(mkv::DemotePage);
  if (a_bytes + d_bytes > p->lay.plan_bytes) {
    // too large for one plan region: the calls one after another
    mkv_status r = append_step_device(p, seq_ids, B, plan, k, v, s);
    if (r) {
      take_back();
      return r;
    }
    p->sched_valid = false;
    for (const Conv& c : conv) {
      if (c.plan.empty()) continue;
      r = upload_pt_row_and_plan(p, c.seq, c.plan.data(), c.plan.size() * sizeof(c.plan[0]), s);
      if (r == MKV_OK) {
        ProfScope ps(p, 3, s);
        const hipError_t e = mkv::launch_demote(
            p->view(), reinterpret_cast<const mkv::DemotePage*>(p->mem + p->lay.plan), int32_t(c.plan.size()), s);
        if (e != hipSuccess) r = set_err(MKV_EHIP, std::string("demote launch: ") + hipGetErrorString(e));
      }
      if (r) return r;
    }
    return finish();
  }
  std::vector<Piece> pieces, rows;
  if (a_bytes) pieces.push_back(Piece{p->lay.plan, plan.data(), a_bytes});
  if (d_bytes) pieces.push_back(Piece{p->lay.plan + a_bytes, dplan.data(), d_bytes});
  for (const Conv& c : conv) {
    if (c.plan.empty()) continue;
    const std::vector<int32_t>& pt = p->meta.seq(c.seq).pt;
    rows.push_back(Piece{p->lay.pt + size_t(c.seq) * size_t(p->desc.max_pages_per_seq) * 4, pt.data(),
                         pt.size() * 4});
  }
  mkv::ListEdits ed;
  bool edited = false;
  if (lists_current) {
    edited = mkv::schedule_extend(p->meta, p->sched_ids, seq_ids, plan, list_cap(p), &p->sched, &ed);
    for (const Conv& c : conv)
      if (edited && !c.plan.empty())
        edited = mkv::schedule_demote(p->meta, p->sched_ids, c.seq, c.plan, list_cap(p), &p->sched, &ed);
    if (edited) schedule_pieces(p, ed, &pieces);
  }
  p->sched_valid = false;
  mkv_status r = upload_pieces(p, pieces, s);
  if (r == MKV_OK) {
    if (inline_plan) {
      mkv::InlinePlan ip{};
      std::memcpy(ip.pages, plan.data(), plan.size() * sizeof(plan[0]));
      ip.patch_base = reinterpret_cast<int32_t*>(p->mem + p->lay.sched + p->lay.items_off);
      ProfScope ps(p, 2, s);
      const hipError_t e = mkv::launch_append_inline(p->view(), ip, int32_t(plan.size()), k, v, s);
      if (e != hipSuccess) r = set_err(MKV_EHIP, std::string("append launch: ") + hipGetErrorString(e));
    } else {
      const auto* ap = reinterpret_cast<const mkv::AppendPage*>(p->mem + p->lay.plan);
      ProfScope ps(p, 2, s);
      const hipError_t e = p->meta.geom().kind == mkv::kKindBf16
                               ? mkv::launch_append_bf16(p->view(), ap, int32_t(plan.size()), k, v, s)
                               : mkv::launch_append(p->view(), ap, int32_t(plan.size()), k, v, s);
      if (e != hipSuccess) r = set_err(MKV_EHIP, std::string("append launch: ") + hipGetErrorString(e));
    }
  }
  if (r) {
    take_back();
    return r;
  }
  if (!dplan.empty()) {
    r = upload_pieces(p, rows, s);
    if (r == MKV_OK) {
      ProfScope ps(p, 3, s);
      const hipError_t e = mkv::launch_demote(
          p->view(), reinterpret_cast<const mkv::DemotePage*>(p->mem + p->lay.plan + a_bytes),
          int32_t(dplan.size()), s);
      if (e != hipSuccess) r = set_err(MKV_EHIP, std::string("demote launch: ") + hipGetErrorString(e));
    }
    if (r) {
      // the append stays; the conversions are taken back (their cursors do
      // not move, so the next step retries them)
      for (size_t i = conv.size(); i-- > 0;) p->meta.rollback(conv[i].undo);
      return r;
    }
  }
  if (edited) {
    p->sched_version = p->meta.version();
    p->sched_layout = p->meta.layout_version();
    p->sched_valid = true;
  }
  return finish();
}

mkv_status mkv_decode_static(mkv_pool* p, const int32_t* seq_ids, int32_t B, const void* q, int32_t Hq,
                             float softmax_scale, float* out, float* lse, hipStream_t s) {
  return decode_impl(p, seq_ids, B, q, Hq, softmax_scale, out, lse, s, StateHome::kStatic);
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
  mkv::Undo undo;
  int st = dst->meta.append(dst_seq, sq.len, &ap, &err, &undo);
  if (st) return set_err(mkv_status(st), err);
  std::vector<mkv::MaterialisePage> plan;
  plan.reserve(ap.size());
  for (const mkv::AppendPage& a : ap)   // fresh pages: row0 == 0, one per source page
    plan.push_back(mkv::MaterialisePage{a.lp, sq.pt[size_t(a.lp)], a.phys, a.nrows, 0, 0, 0, 0});
  mkv_status r = upload_pt_row_and_plan(dst, dst_seq, plan.data(), plan.size() * sizeof(plan[0]), s);
  if (r == MKV_OK) {
    const hipError_t e = mkv::launch_materialise(
        src->view(), dst->view(), reinterpret_cast<const mkv::MaterialisePage*>(dst->mem + dst->lay.plan),
        int32_t(plan.size()), s);
    if (e != hipSuccess) r = set_err(MKV_EHIP, std::string("materialise launch: ") + hipGetErrorString(e));
  }
  if (r) dst->meta.rollback(undo);
  return r;
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

mkv_status mkv_debug_read_bandwidth(const void* src, size_t bytes, uint32_t* sink, hipStream_t s) {
  if (!src || !sink) return set_err(MKV_EINVAL, "null argument");
  if (bytes == 0 || bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16)
    return set_err(MKV_EINVAL, "src must be 16-byte aligned and bytes a nonzero multiple of 16");
  MKV_HIP(mkv::launch_stream_read(src, int64_t(bytes), sink, s));
  return MKV_OK;
}

mkv_status mkv_debug_schedule(mkv_pool* p, mkv_schedule_info* info, int32_t* items_host,
                              int32_t items_cap, int32_t* entries_host, int32_t entries_cap,
                              int32_t* chunk_base_host, int32_t base_cap) {
  if (!p || !info) return set_err(MKV_EINVAL, "null argument");
  if (!p->sched_valid) return set_err(MKV_ESTATE, "no current decode schedule");
  const mkv::Schedule& sc = p->sched;
  const int32_t n_items = int32_t(sc.items[0].size() + sc.items[1].size());
  const int32_t n_list = int32_t(sc.entries.size());
  const int32_t B = int32_t(p->sched_ids.size());
  if ((items_host && items_cap < n_items) || (entries_host && entries_cap < n_list) ||
      (chunk_base_host && base_cap < B + 1))
    return set_err(MKV_ERANGE, "output buffer smaller than the schedule");
  DeviceGuard guard(p->device);
  MKV_HIP(hipDeviceSynchronize());
  const uint8_t* region = p->mem + p->lay.sched;
  if (items_host && n_items)
    MKV_HIP(hipMemcpy(items_host, region + p->lay.items_off, size_t(n_items) * sizeof(mkv::WorkItem),
                      hipMemcpyDeviceToHost));
  if (entries_host && n_list)
    MKV_HIP(hipMemcpy(entries_host, region + entries_off(p->lay, size_t(n_items)), size_t(n_list) * 4,
                      hipMemcpyDeviceToHost));
  if (chunk_base_host) MKV_HIP(hipMemcpy(chunk_base_host, region, size_t(B + 1) * 4, hipMemcpyDeviceToHost));
  info->batch = B;
  info->n_items = n_items;
  info->n_list = n_list;
  info->n_chunks = sc.n_chunks;
  info->max_seq_chunks = sc.max_seq_chunks;
  info->heads_per_wave = sc.heads_per_wave;
  info->resident_waves = p->target_waves[sc.heads_per_wave - 1];
  info->pad0 = 0;
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
  o->ms_append = p->prof_ms[2];
  o->ms_demote = p->prof_ms[3];
  o->n_append = p->prof_n[2];
  o->n_demote = p->prof_n[3];
  for (int i = 0; i < 4; ++i) {
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
