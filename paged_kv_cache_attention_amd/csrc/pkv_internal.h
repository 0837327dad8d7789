// Internal types shared by the host runtime and the gfx950 kernels of libpkv.
#pragma once

#include <cstdint>

#include <hip/hip_runtime.h>

namespace pkv {

// Rows per block: the unit of the split-K work list.  A 16-row block of one
// head is one contiguous 16 x d_h slab when page_size is a multiple of 16.
constexpr int kBlockRows = 16;

// K/V element types (the values of pkv_dtype).
constexpr int kDtypeF32 = 0;
constexpr int kDtypeBF16 = 1;

// One request of a plan.  pt_row selects the request's row of the page-table
// array the launch receives; seq_len is the attended length t (newest row
// included).  nsplit > 1 means the request's chunks write partials starting at
// slot partial_base, and a merge produces the output.
struct ReqEntry {
  int32_t pt_row;
  int32_t seq_len;
  int32_t nsplit;
  int32_t partial_base;
};

// One split-K chunk: blocks [blk_begin, blk_end) of request req, split index
// split, with a copy of the request's entry so a workgroup starts from one
// 32-byte scalar load.
struct WorkItem {
  int32_t req;
  int32_t blk_begin;
  int32_t blk_end;
  int32_t split;
  ReqEntry rq;
};

// Plans of at most this many requests and work items are passed inline in
// the kernel arguments (2.75 KiB of the argument block).
constexpr int kInlineReqs = 48;
constexpr int kInlineItems = 64;

struct AttnArgs {
  const void* q;          // [n][H][D] pool dtype
  const void* k_new;      // [n][H_kv][D] rows to append at t-1 (fused append), or null
  const void* v_new;
  float* out;             // [n][H][D]
  char* k_layer;          // K pool of this layer: [P][H][S][D]
  char* v_layer;
  const int32_t* page_table;
  int64_t pt_stride;      // entries per page-table row
  const ReqEntry* reqs;
  const WorkItem* items;
  float* partials;        // [slots][H][D + 2]: (m, l, acc[D]); m in log2 units
  int32_t* merge_count;   // [n][H] arrival counters of split requests (self-resetting)
  const int32_t* merge_reqs;  // requests with nsplit > 1 (separate merge kernel)
  int32_t num_heads;      // query heads H
  int32_t num_kv_heads;   // K/V heads; H is a multiple of it
  int32_t page_size;
  int32_t head_width;
  int32_t fuse_append;    // 1: write k_new/v_new at row t-1 and attend with them
  int32_t merge_mode;     // MergeMode
  int32_t waves;          // waves per workgroup of the fast paths (4 or 8; 0: per kernel)
  int32_t head_tiles;     // workgroups per (item, K/V head), each serving an
                          // equal, consecutive share of its query heads
  int64_t page_bytes;     // H_kv * S * D * elt
  int64_t head_bytes;     // S * D * elt
  float scale_log2e;      // log2(e) / sqrt(D)
  // Small plans travel in the arguments themselves (no upload before the
  // launch): num_inline > 0 replaces reqs and items.
  int32_t num_inline;
  ReqEntry inline_reqs[kInlineReqs];
  WorkItem inline_items[kInlineItems];
};

// One prefill work tile: up to kPrefillTileRows consecutive rows of one
// request's chunk.
struct PrefillTile {
  int32_t pt_row;   // page-table row of the request
  int32_t start;    // position of the chunk's first row
  int32_t off;      // packed index of the chunk's first row in q, k, v and out
  int32_t i0;       // first chunk row of the tile
  int32_t nq;       // rows in the tile, 1..kPrefillTileRows
  int32_t key_end;  // the tile reads rows 0..key_end-1 (start + i0 + nq)
};

struct PrefillArgs {
  const void* q;          // [T][H][D] pool dtype, packed request after request
  const void* k_new;      // [T][H_kv][D] rows to write at start + i
  const void* v_new;
  float* out;             // [T][H][D]
  char* k_layer;          // K pool of this layer
  char* v_layer;
  const int32_t* page_table;
  int64_t pt_stride;
  const PrefillTile* tiles;
  int32_t num_tiles;
  int32_t num_heads;
  int32_t num_kv_heads;
  int32_t page_size;
  int64_t page_bytes;
  int64_t head_bytes;
  float scale_log2e;
  int32_t dtype;          // kDtypeF32 or kDtypeBF16
};

struct PatchBatch {
  static constexpr int kMax = 248;
  int32_t count;
  int32_t pad;
  int32_t offset[kMax];
  int32_t value[kMax];
};

// Copy-on-write page copies carried in kernel arguments: every layer's K and
// V of page src[i] are copied to page dst[i].
struct CopyBatch {
  static constexpr int kMax = 120;
  int32_t count;
  int32_t pad;
  int32_t src[kMax];
  int32_t dst[kMax];
};

enum class KernelPath { kFast, kGeneric };

// How split requests are merged.
//  kSeparate: chunks store partials; a second kernel merges (the kernel
//             boundary orders the partial stores before the merge reads).
//  kLastArriver: the chunk that arrives last at a (request, head) counter
//             merges.  Partials are stored with agent-scope atomic stores,
//             which write through to the device-coherent level; the writer
//             waits for them to complete before its relaxed counter
//             increment, and the last arriver reads them with agent-scope
//             atomic loads.  No L2 write-back or invalidate is needed.
//  kAuto:     a pool setting only -- each plan takes one of the two by the
//             bytes its launches read (plan_merge_mode); kernels never see it.
enum MergeMode : int32_t { kMergeSeparate = 0, kMergeAuto = 1, kMergeLastArriver = 2 };

// Launchers (kernels.hip).  Each returns the hipError_t of the launch.
hipError_t launch_attention(const AttnArgs& a, int dtype, int num_items, hipStream_t stream,
                            KernelPath* path_out);
hipError_t launch_merge(const AttnArgs& a, int num_split_reqs, hipStream_t stream);
hipError_t launch_kv_append(const AttnArgs& a, int dtype, int num_reqs, hipStream_t stream);
hipError_t launch_patches(int32_t* arena, const PatchBatch& b, hipStream_t stream);
hipError_t launch_page_copies(char* k_storage, char* v_storage, int64_t layer_bytes,
                              int64_t page_bytes, int32_t num_layers, const CopyBatch& b,
                              hipStream_t stream);
bool fast_path_supported(int dtype, int head_width, int page_size, int group);
// Whether the head width has a vector fast-path shape of its own (rows of
// 128, 256 or 512 bytes), as opposed to running a wider shape padded.
bool fast_width_native(int dtype, int head_width);
// Writes zero to count int32 values on the stream (a kernel, so that the
// clear is ordered with the launches that follow on any stream kind).
hipError_t launch_zero_i32(int32_t* p, int64_t count, hipStream_t stream);

// Device scratch of the allocation-free decode call (scratch.hip): one
// file-scope array per device, laid out as the plan (requests, work items,
// split requests), the merge arrival counters and the split-K partials.
constexpr size_t kScratchBytes = size_t(32) << 20;
constexpr size_t kScratchMetaOffset = 0;
constexpr size_t kScratchMetaBytes = size_t(2) << 20;
constexpr size_t kScratchCountersOffset = kScratchMetaBytes;
constexpr size_t kScratchCountersBytes = size_t(1) << 20;
constexpr size_t kScratchPartialsOffset = kScratchCountersOffset + kScratchCountersBytes;
constexpr size_t kScratchPartialsBytes = kScratchBytes - kScratchPartialsOffset;
constexpr int kScratchMaxReqs = 4096;
constexpr int kScratchMaxItems = 32768;
static_assert(kScratchMaxReqs * sizeof(ReqEntry) + kScratchMaxItems * sizeof(WorkItem) +
                      kScratchMaxReqs * sizeof(int32_t) <= kScratchMetaBytes,
              "the largest plan fits the scratch's plan region");
// The scratch's device address on `device`, which must be the current
// device: looked up once per device, then cached.
hipError_t scratch_address(int device, void** out);

// Prefill on matrix cores (bf16 head width 64, 128 or 256; float32 32, 64 or
// 128; pages of a multiple of 16 rows): an append launch writes the chunk's
// rows, then an attention launch runs the causal attention of every (tile,
// query head).
bool prefill_fast_supported(int dtype, int head_width, int page_size);
hipError_t launch_prefill_append(const PrefillArgs& a, int num_tiles, hipStream_t stream);
hipError_t launch_prefill_attention(const PrefillArgs& a, int num_tiles, hipStream_t stream);
constexpr int kPrefillTileRows = 128;

}  // namespace pkv
