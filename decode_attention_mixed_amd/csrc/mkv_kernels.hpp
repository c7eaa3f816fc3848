// Launch interface between the C-ABI layer and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "mkv_meta.hpp"

namespace mkv {

// Device view of a pool: slab bases, page table and geometry.
struct PoolView {
  uint8_t* fp8;        // FP8 slab
  uint8_t* tq3;        // TQ3 slab
  const int32_t* pt;   // page table [max_seqs][pt_stride]
  int64_t fp8_stride;  // bytes between FP8 records (BF16 records in a control pool)
  int64_t tq3_stride;  // bytes between TQ3 records
  int32_t Hkv, d, P, pt_stride;
  int32_t kind;        // kKindMixed or kKindBf16 (control pool: BF16 pages in the FP8 slab)
};

struct DecodeArgs {
  PoolView pv;
  const WorkItem* items;    // work items (each of one format)
  int32_t n_items;
  const int32_t* entries;   // page-table entries of the items' pages (schedule order)
  const int32_t* chunk_base;// [B + 1]
  const uint16_t* q;        // bf16 [B][Hq][d]
  int32_t B, Hq;
  float scale;              // softmax scale on <q, k>
  float* pm;                // partial max      [chunks][Hq]
  float* pl;                // partial denom    [chunks][Hq]
  float* pacc;              // partial acc      [chunks][Hq][d]
  float* out;               // [B][Hq][d]
  float* lse;               // [B][Hq]
  int32_t nh;               // kv-heads per partial-kernel workgroup (1 or 2)
  int32_t max_seq_chunks;   // most partial states of one batch entry
  int32_t pace;             // 1: all partial-kernel workgroups are resident at once
};

hipError_t launch_append(const PoolView& pv, const AppendPage* plan, int32_t n_pages,
                         const float* k, const float* v, hipStream_t s);
hipError_t launch_demote(const PoolView& pv, const DemotePage* plan, int32_t n_pages,
                         hipStream_t s);
// Materialising profile: expand pages of a mixed pool (src) into bf16 rows of
// a control pool (dst).
hipError_t launch_materialise(const PoolView& src, const PoolView& dst, const MaterialisePage* plan,
                              int32_t n_pages, hipStream_t s);
// Control pools: store rows as bf16 (round to nearest even).
hipError_t launch_append_bf16(const PoolView& pv, const AppendPage* plan, int32_t n_pages,
                              const float* k, const float* v, hipStream_t s);
// A small append plan carried in the kernel arguments, so a decode step's
// append needs no upload: up to kInlinePages pages, and up to kInlinePages
// 32-bit stores into device memory (patch_base[patch_off[i]] = patch_val[i],
// done by the first block; a step uses them to bring a cached decode
// schedule's last-page token counts up to date).
constexpr int kInlinePages = 32;
struct InlinePlan {
  int32_t* patch_base;
  int32_t n_patch, pad0;
  AppendPage pages[kInlinePages];
  int32_t patch_off[kInlinePages];
  int32_t patch_val[kInlinePages];
};
// One decode step's cache writes in one launch, everything in the kernel
// arguments: the appended pages (as InlinePlan), the pages the anchor policy
// converts (DemotePage with pad0 = page-table slot, pad1 = its new entry,
// written by the kernel), and word patches of the cached schedule region
// (offsets in 32-bit words from patch_base).  The appended and the converted
// FP8 pages must be distinct.
constexpr int kStepConv = 16;
constexpr int kStepPatches = 128;
struct StepPlan {
  int32_t* patch_base;
  int32_t n_append, n_conv, n_patch, pad0;
  AppendPage pages[kInlinePages];
  DemotePage conv[kStepConv];
  int32_t patch_off[kStepPatches];
  int32_t patch_val[kStepPatches];
};
static_assert(sizeof(StepPlan) + sizeof(PoolView) + 2 * sizeof(void*) <= 4096,
              "the step kernel's arguments fit the 4 KB kernel-argument limit");
hipError_t launch_step(const PoolView& pv, const StepPlan& plan, const float* k, const float* v,
                       hipStream_t s);

// Metadata upload: up to kUploadSegs runs of 32-bit words copied from a
// device-mapped, coherent pinned host buffer (src, word offsets src_word) to
// device memory, in one launch (a copy-engine transfer of the same bytes adds
// more latency to the stream than this kernel takes).
constexpr int kUploadSegs = 16;
struct UploadSet {
  const uint32_t* src;
  int32_t nseg, pad0;
  uint32_t* dst[kUploadSegs];
  uint32_t src_word[kUploadSegs];
  uint32_t words[kUploadSegs];
};
hipError_t launch_upload(const UploadSet& u, hipStream_t s);
// The pool's kind picks the FP8 or the BF16 append.
hipError_t launch_append_inline(const PoolView& pv, const InlinePlan& plan, int32_t n_pages,
                                const float* k, const float* v, hipStream_t s);
hipError_t launch_gather(const PoolView& pv, int32_t seq, int32_t first, int32_t n,
                         uint8_t* dst, int64_t slot_bytes, hipStream_t s);
// Read-bandwidth calibration: reads bytes (a multiple of 16) of src once.
hipError_t launch_stream_read(const void* src, int64_t bytes, uint32_t* sink, hipStream_t s);
// Partial kernel of the pool's kind (mixed FP8/TQ3 or BF16 control).
hipError_t launch_partial(const DecodeArgs& a, hipStream_t s);
// Waves of the partial kernel (head dim d, nh kv-heads per wave, pool kind)
// resident on the current device at once.
hipError_t partial_resident_waves(int d, int nh, int kind, int* waves);
// Merge of the partial states; batches with at most narrow_max chunks per
// entry use the per-lane variant (no cross-lane reduction).
hipError_t launch_merge(const DecodeArgs& a, int narrow_max, hipStream_t s);

// Fixed per-device workspace for the partial states of an allocation-free
// decode (m, l and acc regions of chunks x Hq slots, each 256-byte aligned).
constexpr size_t kStaticWorkspaceBytes = size_t(16) << 20;
// Device address of that workspace on `device`, which must be the current
// device; looked up on the first call per device and cached.
hipError_t static_workspace(int device, void** out);

}  // namespace mkv
