// Host runtime and C ABI of libpkv: page pool and free list with reference
// counts, request caches (forks share pages, copy on write), their per-token
// or per-chunk transaction, split-K plans and prefill tiles, device
// page-table mirror.
//
// Sources (by page and section):
//  - riftco-transformer "Incremental Serving", "Paged KV-cache layout": shared
//    pool of per-layer key/value pages, request-local logical page tables, one
//    page ID valid in every layer, lazy lease, return on reset/destroy, 16-token
//    default pages, block count 0 = one maximum context.
//  - same page, "Request flow": begin / append_and_attend per layer / commit,
//    abort leaves the visible length unchanged.
//  - same page, "Stable C and Python sessions": options init with defaults,
//    capacity exhaustion reported to the caller, external synchronisation.
//  - learn_llm ch.38 "cached generation": every layer prepares before any
//    commit; rejected operations leave committed state unchanged; reset keeps
//    the allocation; work counters (appends, score values).
//  - "Incremental Serving", "Current scope": page sharing between requests and
//    copy-on-write prefixes, and a batched prefill, lie beyond paged storage
//    alone; both are built here on the same pool.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <new>
#include <string>
#include <unordered_map>
#include <vector>

#include <hip/hip_runtime.h>

#include "../../include/pkv.h"
#include "pkv_internal.h"

using pkv::AttnArgs;
using pkv::PatchBatch;
using pkv::PrefillArgs;
using pkv::PrefillTile;
using pkv::ReqEntry;
using pkv::WorkItem;

namespace {

thread_local std::string g_last_error;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pkv_status ok() {
  g_last_error.clear();
  return PKV_OK;
}

#define PKV_HIP_TRY(expr)                                                                  \
  do {                                                                                     \
    hipError_t e_ = (expr);                                                                \
    if (e_ != hipSuccess)                                                                  \
      return fail(PKV_ERR_DEVICE, "%s failed: %s", #expr, hipGetErrorString(e_));          \
  } while (0)

// SplitMix64, used only to shuffle the initial free list.
uint64_t splitmix_next(uint64_t& s) {
  s += 0x9E3779B97F4A7C15ull;
  uint64_t z = s;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

size_t elt_bytes(int32_t dtype) { return dtype == PKV_DTYPE_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

}  // namespace

enum PageOwner : uint8_t { kFree = 0, kCache = 1, kRaw = 2 };

struct pkv_plan {
  pkv_pool* pool = nullptr;
  bool internal = false;
  bool built = false;
  int32_t n = 0;
  int32_t pt_stride = 0;
  int32_t num_items = 0;
  int32_t total_splits = 0;
  int32_t num_split_reqs = 0;
  int32_t waves = 0;
  int32_t merge_mode = pkv::kMergeLastArriver;  // as launched (never kMergeAuto)
  bool any_split = false;
  bool inline_plan = false;    // reqs/items go in the kernel arguments
  bool meta_uploaded = false;  // reqs/items/merge list are in d_meta
  uint64_t rows_attended = 0;  // sum of t_r
  std::vector<ReqEntry> reqs;
  std::vector<WorkItem> items;
  std::vector<int32_t> merge_list;  // requests with nsplit > 1
  std::vector<int64_t> key;  // (pt_row, seq_len) pairs of the last build
  char* d_meta = nullptr;
  size_t d_meta_cap = 0;
  float* d_partials = nullptr;
  size_t partials_cap = 0;  // floats
  int32_t* d_counters = nullptr;  // [n][H] merge arrival counters, zero between launches
  size_t counters_cap = 0;
  char* h_stage = nullptr;
  size_t h_stage_cap = 0;
  hipEvent_t ev = nullptr;
  bool ev_pending = false;
  // Buffers replaced by a larger one.  Work already enqueued may still read
  // them, and freeing device or pinned memory waits for the whole device, so
  // they stay allocated until the plan is released (capacities double, so
  // together they stay below the final buffers' size).
  std::vector<void*> retired_dev;
  std::vector<void*> retired_host;
};

struct pkv_cache {
  pkv_pool* pool = nullptr;
  int32_t max_context = 0;
  int32_t slot = -1;
  int32_t len = 0;
  std::vector<int32_t> pages;
  bool pending = false;
  int32_t pending_pos = 0;        // first reserved position
  int32_t pending_count = 0;      // positions reserved by this begin
  int32_t pending_new_pages = 0;  // pages leased by this begin
  int32_t cow_logical = -1;       // logical page this begin copied on write, or -1
  int32_t cow_old = -1;           // the shared page that copy replaced
  std::vector<uint8_t> appended;
  int32_t appended_count = 0;
};

struct pkv_pool {
  pkv_pool_desc desc{};
  size_t elt = 4;
  int64_t head_bytes = 0, page_bytes = 0, layer_bytes = 0;
  std::vector<int32_t> free_stack;  // lease pops from the back
  std::vector<uint8_t> owner;
  std::vector<int32_t> refs;  // holders per page: caches, a raw lease, and a pending
                              // transaction's hold on the shared page it copied
  struct PageCopy {
    int32_t src, dst;
  };
  std::vector<PageCopy> copies;  // copy-on-write copies not yet enqueued
  int32_t raw_leased = 0;
  int32_t live_caches = 0;
  int32_t live_plans = 0;
  std::vector<int32_t> free_slots;
  int32_t arena_stride = 0;  // page-table entries per cache slot
  // device side (created lazily)
  bool host_only = false;
  int device = -1;
  int32_t* d_arena = nullptr;
  std::vector<std::pair<int32_t, int32_t>> patches;  // (arena offset, page)
  pkv_plan txn_plan;      // transactional steps
  pkv_plan call_plan;     // one-call batched forms
  pkv_plan prefill_plan;  // chunks of several rows per request
  pkv_counters counters{};
  int32_t merge_mode = pkv::kMergeAuto;  // the option; plans take plan_merge_mode()
  int32_t waves_option = 0;
  uint64_t opt_gen = 0;  // bumped by every option that changes a plan's shape
  bool profiling = false;
  bool validate = false;  // debug: check caller page-table entries before use
  enum TimedKind { kTimedAttention, kTimedMerge, kTimedPrefill };
  struct Timed {
    hipEvent_t start, end;
    TimedKind kind;
  };
  std::vector<Timed> timed;         // recorded, not yet summed
  std::vector<hipEvent_t> spare;    // reusable events
  pkv_profile profile{};
};

namespace {

int32_t lease_page(pkv_pool* p, uint8_t who) {
  const int32_t page = p->free_stack.back();
  p->free_stack.pop_back();
  p->owner[page] = who;
  p->refs[page] = 1;
  return page;
}

// Drops one holder of the page; the last one returns it to the free list.
// A page that becomes free cancels any copy still queued into it (its
// destination no longer belongs to anyone).
void release_page(pkv_pool* p, int32_t page) {
  if (--p->refs[page] > 0) return;
  p->owner[page] = kFree;
  p->free_stack.push_back(page);
  for (size_t i = 0; i < p->copies.size();) {
    if (p->copies[i].dst == page)
      p->copies.erase(p->copies.begin() + (std::ptrdiff_t)i);
    else
      ++i;
  }
}

void record_patch(pkv_cache* c, int32_t logical, int32_t page) {
  pkv_pool* p = c->pool;
  p->patches.emplace_back(c->slot * p->arena_stride + logical, page);
}

pkv_status ensure_device(pkv_pool* p, hipStream_t stream) {
  if (p->host_only) return PKV_OK;
  int dev = 0;
  PKV_HIP_TRY(hipGetDevice(&dev));
  if (p->device >= 0) {
    if (dev != p->device)
      return fail(PKV_ERR_INVALID_ARGUMENT, "pool lives on device %d, current device is %d",
                  p->device, dev);
    return PKV_OK;
  }
  const size_t bytes = (size_t)p->desc.max_caches * (size_t)p->arena_stride * sizeof(int32_t);
  void* arena = nullptr;
  if (hipMalloc(&arena, bytes) != hipSuccess)
    return fail(PKV_ERR_ALLOC, "device page-table arena of %zu bytes", bytes);
  // Cleared on the caller's stream, ahead of the patches that fill it.
  if (pkv::launch_zero_i32(static_cast<int32_t*>(arena), (int64_t)(bytes / sizeof(int32_t)),
                           stream) != hipSuccess) {
    (void)hipFree(arena);
    return fail(PKV_ERR_DEVICE, "clearing the page-table arena failed");
  }
  p->d_arena = static_cast<int32_t*>(arena);
  p->device = dev;
  return PKV_OK;
}

// Enqueues the copy-on-write page copies.  A queued copy's source is held by
// the pending transaction that made it (or by pkv_cache_grow until the copy
// is complete), so it stays allocated until the copy has run.
pkv_status flush_copies(pkv_pool* p, hipStream_t stream) {
  if (p->copies.empty()) return PKV_OK;
  if (!p->host_only) {
    for (size_t i = 0; i < p->copies.size();) {
      pkv::CopyBatch b{};
      b.count = 0;
      for (; i < p->copies.size() && b.count < pkv::CopyBatch::kMax; ++i, ++b.count) {
        b.src[b.count] = p->copies[i].src;
        b.dst[b.count] = p->copies[i].dst;
      }
      PKV_HIP_TRY(pkv::launch_page_copies(static_cast<char*>(p->desc.k_storage),
                                          static_cast<char*>(p->desc.v_storage), p->layer_bytes,
                                          p->page_bytes, p->desc.num_layers, b, stream));
    }
  }
  p->copies.clear();
  return PKV_OK;
}

pkv_status flush_patches(pkv_pool* p, hipStream_t stream) {
  pkv_status st = flush_copies(p, stream);
  if (st != PKV_OK) return st;
  if (p->host_only) {
    p->patches.clear();
    return PKV_OK;
  }
  // One patch per arena entry, the last one recorded: the patch kernel
  // writes a batch's entries in parallel, so two values for one entry (a
  // fork's shared page, then its copy on write) would race.
  if (p->patches.size() > 1) {
    std::unordered_map<int32_t, size_t> last;
    last.reserve(p->patches.size());
    for (size_t j = 0; j < p->patches.size(); ++j) last[p->patches[j].first] = j;
    if (last.size() < p->patches.size()) {
      std::vector<std::pair<int32_t, int32_t>> kept;
      kept.reserve(last.size());
      for (size_t j = 0; j < p->patches.size(); ++j)
        if (last[p->patches[j].first] == j) kept.push_back(p->patches[j]);
      p->patches.swap(kept);
    }
  }
  size_t i = 0;
  while (i < p->patches.size()) {
    PatchBatch b{};
    b.count = 0;
    for (; i < p->patches.size() && b.count < PatchBatch::kMax; ++i, ++b.count) {
      b.offset[b.count] = p->patches[i].first;
      b.value[b.count] = p->patches[i].second;
    }
    PKV_HIP_TRY(pkv::launch_patches(p->d_arena, b, stream));
  }
  p->patches.clear();
  return PKV_OK;
}

// The merge a plan's split requests use.  Automatic (the default): launches
// that read at least kSeparateMergeBytes of K/V merge in a separate kernel,
// smaller ones in place.  In place, each split chunk's last wave waits for its
// partial stores and then for the counter's reply before it can leave, and
// the last arrivers merge at the end of the launch; on long launches that
// costs more than a second launch (32-layer bf16 step, 4.3 GB per launch:
// 22.2 ms per step against 22.4-22.8 ms), while on short ones the second
// launch dominates (12-layer float32 step, 88 MB per launch: a separate merge
// adds ~4 us to each 21 us launch).
constexpr uint64_t kSeparateMergeBytes = 1ull << 30;

int32_t plan_merge_mode(const pkv_pool* p, uint64_t rows_attended) {
  if (p->merge_mode != pkv::kMergeAuto) return p->merge_mode;
  const uint64_t bytes = rows_attended * (uint64_t)p->desc.num_kv_heads * 2ull *
                         (uint64_t)p->desc.head_width * p->elt;
  return bytes >= kSeparateMergeBytes ? pkv::kMergeSeparate : pkv::kMergeLastArriver;
}

// Workgroup shape and split-K chunk size (in 16-row blocks) of a plan.
//
// Waves per workgroup: PKV_OPT_WAVES, or 0 to let the launcher choose per
// kernel (four for the vector kernels, eight or sixteen for a small
// multi-head batch and eight for a balanced batch kept whole, as below; eight
// for the matrix-core kernel when a workgroup serves 8 or 16 query heads,
// whose requests then finish in half the block steps per wave).
// Requests split into chunks sized for about kTargetChunks (chunk, query
// head) units -- four resident rounds of 256 CUs x 4 workgroups -- so a batch
// with few (request, head) pairs still fills the GPU and one long context
// does not serialise on one workgroup; a balanced batch of two or more
// resident rounds stays whole (below).
//
// A split launch of more than four rounds runs its workgroups longest chunk
// first and ends as the last ones drain.  Its requests split into whole
// chunks of `chunk` blocks with the remainder last (remainder_last), so the
// chunks dispatched at the end are short: on the 32-layer bf16 step split at
// 128 blocks (requests of 97-161 blocks) that measured 695.7-697.0 us per
// launch in six runs against 698-712 us with even chunks, whose runs often
// ended slower (that step now runs unsplit, below).  The other choices keep
// even chunks (the first blocks % nsplit take one block more): a one-round
// launch ends with its longest workgroup, which even chunks keep shortest.
struct SplitChoice {
  int32_t chunk;
  int32_t waves;
  bool remainder_last;
};

// Block range end of chunk s of a request of `blocks` blocks split nsplit ways
// from b0 (the end of chunk s - 1).
int32_t chunk_end(const SplitChoice& c, int32_t blocks, int32_t nsplit, int32_t s, int32_t b0) {
  if (c.remainder_last) return std::min(b0 + c.chunk, blocks);
  return b0 + blocks / nsplit + (s < blocks % nsplit ? 1 : 0);
}

SplitChoice choose_split(const pkv_pool* p, int32_t n, int64_t total_blocks, int32_t max_blocks) {
  // Work is counted in (block, query head) units: a workgroup serving a K/V
  // head does the work of its whole group, so grouped heads split like the
  // multi-head case (measured: splitting them further only adds partial
  // publishes).
  const int64_t H = p->desc.num_heads;
  const int32_t waves = p->waves_option;
  if (p->desc.split_blocks > 0) return {p->desc.split_blocks, waves, false};
  if (p->desc.split_blocks < 0) return {std::numeric_limits<int32_t>::max(), waves, false};
  constexpr int64_t kTargetChunks = 4096;
  const int64_t work = total_blocks * H;  // (block, head) units
  int64_t c = 8;
  while (c < 512 && c * kTargetChunks < work) c *= 2;
  // A batch of at least two resident rounds of (request, head) pairs whose
  // longest request is at most twice the average keeps every request whole:
  // no request can end the launch alone.  The 32-layer bf16 step (requests of
  // 97-161 blocks) then runs unsplit, with or without its aborted requests,
  // on eight-wave workgroups (multi-head; grouped kernels choose their own):
  // 695-697 us per launch in all 21 runs on the boxes measured, where four
  // waves landed there in 4 of 17 runs and at 704-710 us in the rest (two
  // modes of the same pool, by physical placement), and 128-block chunks at
  // 690-712.  The 256-request batch moved by 0.2%.
  if ((int64_t)n * H >= kTargetChunks / 2 && (int64_t)max_blocks * n <= 2 * total_blocks)
    return {std::numeric_limits<int32_t>::max(), waves ? waves : 8, false};
  // A small multi-head batch with enough (request, head) pairs for an
  // eight-wave workgroup on every CU: 32-block chunks over eight waves (four
  // blocks per wave) instead of 8-block chunks over four, so fewer requests
  // split and fewer partials are published and merged for the same loads in
  // flight (measured on the 12-layer float32 step: 24.5 -> 23.7 us per
  // launch; 16-, 24-, 48- and 64-block chunks over eight waves were slower).
  // For d_h <= 64 the same test at 64-block chunks picks sixteen-wave
  // workgroups instead: still four blocks per wave, but half the chunks, so
  // requests of up to 64 blocks stay whole and publish no partials (measured
  // on the same step: 24.2 -> 22.6 us per launch, where 32- and 48-block
  // chunks over sixteen waves and whole requests over eight were slower).
  // Sixteen waves are built for d_h <= 64 only, whose kernels fit the 128
  // registers a 1024-lane workgroup leaves per lane (bf16 d_h = 128 would
  // spill).
  // A batch with fewer pairs keeps the finer split, which is shorter per wave;
  // the one-wave generic kernel keeps it too.
  const bool small_mha = c == 8 && waves == 0 && p->desc.num_kv_heads == H &&
      pkv::fast_path_supported(p->desc.kv_dtype, p->desc.head_width, p->desc.page_size, 1);
  // Sixteen waves exist for the native row widths only (a padded width runs
  // a wider shape, which has no sixteen-wave form), so padded widths take
  // the eight-wave choice below.
  if (small_mha && p->desc.head_width <= 64 &&
      pkv::fast_width_native(p->desc.kv_dtype, p->desc.head_width) &&
      (total_blocks / 64 + n / 2) * H >= 256)
    return {64, 16, false};
  if (small_mha && (total_blocks / 32 + n / 2) * H >= 256) return {32, 8, false};
  // Chunks above the minimum mean more (chunk, head) units than four rounds.
  return {(int32_t)c, waves, c > 8};
}

// Frees the plan's buffers (at destroy: these frees wait for the device).
void plan_release(pkv_plan* pl) {
  for (void* d : pl->retired_dev) (void)hipFree(d);
  for (void* h : pl->retired_host) (void)hipHostFree(h);
  pl->retired_dev.clear();
  pl->retired_host.clear();
  if (pl->ev) {
    (void)hipEventSynchronize(pl->ev);
    (void)hipEventDestroy(pl->ev);
  }
  if (pl->d_meta) (void)hipFree(pl->d_meta);
  if (pl->d_partials) (void)hipFree(pl->d_partials);
  if (pl->d_counters) (void)hipFree(pl->d_counters);
  if (pl->h_stage) (void)hipHostFree(pl->h_stage);
  pl->ev = nullptr;
  pl->d_counters = nullptr;
  pl->counters_cap = 0;
  pl->d_meta = nullptr;
  pl->d_partials = nullptr;
  pl->h_stage = nullptr;
  pl->d_meta_cap = pl->partials_cap = pl->h_stage_cap = 0;
  pl->built = false;
}

struct MetaPart {
  const void* data;
  size_t bytes;
};

// Copies the parts, back to back, into the plan's device metadata buffer on
// the stream, through pinned host staging.  The staging buffer is reused only
// after the previous upload's copy has completed (an event on the stream);
// a grown device buffer replaces the old one, which is kept (see retired_dev).
pkv_status upload_meta(pkv_plan* pl, const MetaPart* parts, int nparts, hipStream_t stream) {
  size_t bytes = 0;
  for (int i = 0; i < nparts; ++i) bytes += parts[i].bytes;
  if (pl->ev_pending) {
    PKV_HIP_TRY(hipEventSynchronize(pl->ev));
    pl->ev_pending = false;
  }
  if (!pl->ev) PKV_HIP_TRY(hipEventCreateWithFlags(&pl->ev, hipEventDisableTiming));
  if (bytes > pl->d_meta_cap) {
    const size_t cap = std::max(bytes, pl->d_meta_cap * 2);
    void* d = nullptr;
    if (hipMalloc(&d, cap) != hipSuccess) return fail(PKV_ERR_ALLOC, "plan buffer %zu bytes", cap);
    if (pl->d_meta) pl->retired_dev.push_back(pl->d_meta);
    pl->d_meta = static_cast<char*>(d);
    pl->d_meta_cap = cap;
  }
  if (bytes > pl->h_stage_cap) {
    const size_t cap = std::max(bytes, pl->h_stage_cap * 2);
    void* h = nullptr;
    if (hipHostMalloc(&h, cap, hipHostMallocDefault) != hipSuccess)
      return fail(PKV_ERR_ALLOC, "pinned staging %zu bytes", cap);
    if (pl->h_stage) pl->retired_host.push_back(pl->h_stage);
    pl->h_stage = static_cast<char*>(h);
    pl->h_stage_cap = cap;
  }
  size_t off = 0;
  for (int i = 0; i < nparts; ++i) {
    if (parts[i].bytes) std::memcpy(pl->h_stage + off, parts[i].data, parts[i].bytes);
    off += parts[i].bytes;
  }
  PKV_HIP_TRY(hipMemcpyAsync(pl->d_meta, pl->h_stage, bytes, hipMemcpyHostToDevice, stream));
  PKV_HIP_TRY(hipEventRecord(pl->ev, stream));
  pl->ev_pending = true;
  return PKV_OK;
}

// Copies the plan's requests, work items and merge list to the device.
pkv_status upload_plan_meta(pkv_plan* pl, hipStream_t stream) {
  const MetaPart parts[3] = {{pl->reqs.data(), pl->reqs.size() * sizeof(ReqEntry)},
                             {pl->items.data(), pl->items.size() * sizeof(WorkItem)},
                             {pl->merge_list.data(), pl->merge_list.size() * sizeof(int32_t)}};
  pkv_status st = upload_meta(pl, parts, 3, stream);
  if (st == PKV_OK) pl->meta_uploaded = true;
  return st;
}

// Builds the split plan for n requests (rows[r] selects the page-table row,
// lens[r] the attended length) and uploads it on the stream.
pkv_status plan_build(pkv_plan* pl, int32_t n, const int32_t* rows, const int32_t* lens,
                      int32_t pt_stride, hipStream_t stream) {
  pkv_pool* p = pl->pool;
  const int64_t max_len = (int64_t)pt_stride * p->desc.page_size;
  int64_t total_blocks = 0;
  int32_t max_blocks = 0;
  for (int32_t r = 0; r < n; ++r) {
    if (lens[r] < 1 || lens[r] > max_len)
      return fail(PKV_ERR_INVALID_ARGUMENT, "seq_lens[%d]=%d outside [1, %lld]", r, lens[r],
                  (long long)max_len);
    const int32_t b = (lens[r] + pkv::kBlockRows - 1) / pkv::kBlockRows;
    total_blocks += b;
    max_blocks = std::max(max_blocks, b);
  }
  // The key holds the options generation too: a plan built before an option
  // changed its chunking or workgroup shape is rebuilt.
  std::vector<int64_t> key(2 * (size_t)n + 2);
  key[0] = pt_stride;
  key[1] = (int64_t)p->opt_gen;
  for (int32_t r = 0; r < n; ++r) {
    key[2 + 2 * r] = rows[r];
    key[3 + 2 * r] = lens[r];
  }
  if (pl->built && key == pl->key) return PKV_OK;  // identical plan already on the device
  pkv_status st = ensure_device(p, stream);
  if (st != PKV_OK) return st;

  const SplitChoice choice = choose_split(p, n, total_blocks, max_blocks);
  const int32_t chunk = choice.chunk;
  const bool upload = !p->host_only;
  std::vector<ReqEntry> reqs(n);
  std::vector<WorkItem> items;
  items.reserve((size_t)n * 2);
  int32_t slots = 0;
  uint64_t rows_attended = 0;
  for (int32_t r = 0; r < n; ++r) {
    const int32_t blocks = (lens[r] + pkv::kBlockRows - 1) / pkv::kBlockRows;
    const int32_t nsplit = (int32_t)(((int64_t)blocks + chunk - 1) / chunk);
    reqs[r] = ReqEntry{rows[r], lens[r], nsplit, nsplit > 1 ? slots : -1};
    if (nsplit > 1) slots += nsplit;
    int32_t b0 = 0;
    for (int32_t s = 0; s < nsplit; ++s) {
      const int32_t b1 = chunk_end(choice, blocks, nsplit, s, b0);
      items.push_back(WorkItem{r, b0, b1, s, reqs[r]});
      b0 = b1;
    }
    rows_attended += (uint64_t)lens[r];
  }
  std::vector<int32_t> merge_list;
  for (int32_t r = 0; r < n; ++r)
    if (reqs[r].nsplit > 1) merge_list.push_back(r);
  // Longest chunks first, so the short tail chunks fill in at the end.
  std::stable_sort(items.begin(), items.end(), [](const WorkItem& a, const WorkItem& b) {
    return (a.blk_end - a.blk_begin) > (b.blk_end - b.blk_begin);
  });

  // One launch holds a workgroup per (chunk, head) at most.
  if ((int64_t)items.size() * p->desc.num_heads > std::numeric_limits<int32_t>::max())
    return fail(PKV_ERR_INVALID_ARGUMENT, "%zu chunks x %d heads exceed one launch", items.size(),
                p->desc.num_heads);
  // Small plans are passed inline in the kernel arguments, so the launch
  // needs no upload; the device copy is made only if a separate merge
  // kernel needs it (upload_plan_meta).
  const bool inline_plan = n <= pkv::kInlineReqs && (int64_t)items.size() <= pkv::kInlineItems;
  if (upload) {
    const size_t part_floats = (size_t)slots * p->desc.num_heads * (p->desc.head_width + 2);
    if (part_floats > pl->partials_cap) {
      const size_t cap = std::max(part_floats, pl->partials_cap * 2);
      void* d = nullptr;
      if (hipMalloc(&d, cap * sizeof(float)) != hipSuccess)
        return fail(PKV_ERR_ALLOC, "partials %zu floats", cap);
      if (pl->d_partials) pl->retired_dev.push_back(pl->d_partials);
      pl->d_partials = static_cast<float*>(d);
      pl->partials_cap = cap;
    }
    const size_t counters = (size_t)n * p->desc.num_heads;
    if (counters > pl->counters_cap) {
      const size_t cap = std::max(counters, pl->counters_cap * 2);
      void* d = nullptr;
      if (hipMalloc(&d, cap * sizeof(int32_t)) != hipSuccess)
        return fail(PKV_ERR_ALLOC, "merge counters %zu", cap);
      // Zeroed on the stream of the launches that will use them.
      if (pkv::launch_zero_i32(static_cast<int32_t*>(d), (int64_t)cap, stream) != hipSuccess) {
        (void)hipFree(d);
        return fail(PKV_ERR_DEVICE, "clearing the merge counters failed");
      }
      if (pl->d_counters) pl->retired_dev.push_back(pl->d_counters);
      pl->d_counters = static_cast<int32_t*>(d);
      pl->counters_cap = cap;
    }
  }

  // From here the plan holds the new work; it counts as built again only
  // once the upload below has succeeded.
  pl->built = false;
  pl->reqs = std::move(reqs);
  pl->items = std::move(items);
  pl->merge_list = std::move(merge_list);
  pl->meta_uploaded = false;
  // The device copy is also made now when this pool's separate merge kernel
  // will need it, so a launch captured into a graph finds it there.
  const int32_t merge_mode = plan_merge_mode(p, rows_attended);
  const bool need_meta = !inline_plan || (slots > 0 && merge_mode == pkv::kMergeSeparate);
  if (upload && need_meta && (st = upload_plan_meta(pl, stream)) != PKV_OK) return st;
  pl->key = std::move(key);
  pl->n = n;
  pl->pt_stride = pt_stride;
  pl->num_items = (int32_t)pl->items.size();
  pl->total_splits = slots;
  pl->num_split_reqs = (int32_t)pl->merge_list.size();
  pl->waves = choice.waves;
  pl->merge_mode = merge_mode;
  pl->any_split = slots > 0;
  pl->inline_plan = inline_plan;
  pl->rows_attended = rows_attended;
  pl->built = true;
  return PKV_OK;
}

// A built plan as the kernels see it: its host copy (for inline plans),
// where its device copy and buffers are, and its launch shape.
struct PlanView {
  const ReqEntry* reqs;
  int32_t n;
  const WorkItem* items;
  int32_t num_items;
  int32_t pt_stride;
  int32_t waves;
  int32_t merge_mode;  // kMergeSeparate or kMergeLastArriver
  bool inline_plan;
  const char* d_meta;  // requests, then work items, then split requests
  float* d_partials;
  int32_t* d_counters;
};

AttnArgs make_args_view(const pkv_pool* p, const PlanView& v, int32_t layer,
                        const int32_t* page_table, const void* q, const void* k,
                        const void* vv, float* out, bool fuse) {
  AttnArgs a{};
  a.q = q;
  a.k_new = k;
  a.v_new = vv;
  a.out = out;
  a.k_layer = static_cast<char*>(p->desc.k_storage) + (int64_t)layer * p->layer_bytes;
  a.v_layer = static_cast<char*>(p->desc.v_storage) + (int64_t)layer * p->layer_bytes;
  a.page_table = page_table;
  a.pt_stride = v.pt_stride;
  a.reqs = reinterpret_cast<const ReqEntry*>(v.d_meta);
  a.items = reinterpret_cast<const WorkItem*>(v.d_meta + (size_t)v.n * sizeof(ReqEntry));
  a.partials = v.d_partials;
  a.merge_count = v.d_counters;
  a.merge_reqs = reinterpret_cast<const int32_t*>(v.d_meta + (size_t)v.n * sizeof(ReqEntry) +
                                                  (size_t)v.num_items * sizeof(WorkItem));
  a.merge_mode = v.merge_mode;
  a.waves = v.waves;
  a.num_heads = p->desc.num_heads;
  a.num_kv_heads = p->desc.num_kv_heads;
  a.page_size = p->desc.page_size;
  a.head_width = p->desc.head_width;
  a.fuse_append = fuse ? 1 : 0;
  a.page_bytes = p->page_bytes;
  a.head_bytes = p->head_bytes;
  a.scale_log2e = (float)(1.4426950408889634 / std::sqrt((double)p->desc.head_width));
  a.num_inline = 0;
  if (v.inline_plan) {
    a.num_inline = v.num_items;
    std::memcpy(a.inline_reqs, v.reqs, (size_t)v.n * sizeof(ReqEntry));
    std::memcpy(a.inline_items, v.items, (size_t)v.num_items * sizeof(WorkItem));
  }
  return a;
}

AttnArgs make_args(const pkv_plan* pl, int32_t layer, const int32_t* page_table,
                   const void* q, const void* k, const void* v, float* out, bool fuse) {
  const PlanView view{pl->reqs.data(), (int32_t)pl->reqs.size(), pl->items.data(),
                      (int32_t)pl->items.size(), pl->pt_stride, pl->waves, pl->merge_mode,
                      pl->inline_plan, pl->d_meta, pl->d_partials, pl->d_counters};
  return make_args_view(pl->pool, view, layer, page_table, q, k, v, out, fuse);
}

pkv_status check_ptr(const void* ptr, const char* name) {
  if (!ptr) return fail(PKV_ERR_INVALID_ARGUMENT, "%s is null", name);
  if (!aligned16(ptr)) return fail(PKV_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return PKV_OK;
}

// Debug validation of a caller's device page table: entries [0, used[i]) of
// row rows[i] are read back (waiting for the stream, so earlier writes to the
// table on it are seen) and must name pages of the pool.
pkv_status validate_table(const pkv_pool* p, const int32_t* page_table, int32_t pt_stride,
                          int32_t n, const int32_t* rows, const int32_t* used,
                          hipStream_t stream) {
  if (!p->validate || p->host_only) return PKV_OK;
  int32_t max_row = 0;
  for (int32_t i = 0; i < n; ++i) max_row = std::max(max_row, rows[i]);
  std::vector<int32_t> host((size_t)(max_row + 1) * pt_stride);
  PKV_HIP_TRY(hipMemcpyAsync(host.data(), page_table, host.size() * sizeof(int32_t),
                             hipMemcpyDeviceToHost, stream));
  PKV_HIP_TRY(hipStreamSynchronize(stream));
  for (int32_t i = 0; i < n; ++i) {
    const int32_t* row = host.data() + (size_t)rows[i] * pt_stride;
    for (int32_t j = 0; j < used[i]; ++j)
      if (row[j] < 0 || row[j] >= p->desc.num_pages)
        return fail(PKV_ERR_INVALID_ARGUMENT,
                    "page_table[%d][%d] = %d is not a page of the pool (0..%d); request %d",
                    rows[i], j, row[j], p->desc.num_pages - 1, i);
  }
  return PKV_OK;
}

// validate_table for a built decode plan: each request reads the pages of
// its t rows.
pkv_status validate_plan_table(const pkv_plan* pl, const int32_t* page_table,
                               hipStream_t stream) {
  const pkv_pool* p = pl->pool;
  if (!p->validate || p->host_only) return PKV_OK;
  std::vector<int32_t> rows(pl->reqs.size()), used(pl->reqs.size());
  for (size_t i = 0; i < pl->reqs.size(); ++i) {
    rows[i] = pl->reqs[i].pt_row;
    used[i] = (pl->reqs[i].seq_len + p->desc.page_size - 1) / p->desc.page_size;
  }
  return validate_table(p, page_table, pl->pt_stride, (int32_t)rows.size(), rows.data(),
                        used.data(), stream);
}

hipEvent_t take_event(pkv_pool* p) {
  if (!p->spare.empty()) {
    hipEvent_t e = p->spare.back();
    p->spare.pop_back();
    return e;
  }
  // Timing events without the system-scope cache write-back/invalidate, so
  // recording them costs little next to the kernels they bracket.
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) == hipSuccess) return e;
  (void)hipGetLastError();
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Algorithmic bytes of one attention launch: pool rows read, q, the appended
// rows (read from the inputs and written to the pool) and the context.
uint64_t launch_bytes(const pkv_plan* pl, bool fuse) {
  const pkv_pool* p = pl->pool;
  const uint64_t qrow = (uint64_t)p->desc.num_heads * p->desc.head_width;      // per request
  const uint64_t kvrow = (uint64_t)p->desc.num_kv_heads * p->desc.head_width;  // per request
  const uint64_t kv_rows = pl->rows_attended - (fuse ? (uint64_t)pl->n : 0);
  uint64_t b = kv_rows * kvrow * 2 * p->elt;         // K and V rows from the pool
  b += (uint64_t)pl->n * qrow * (p->elt + 4);        // q in, context out
  if (fuse) b += (uint64_t)pl->n * kvrow * 2 * p->elt * 2;  // new K/V rows in and out
  return b;
}

pkv_status run_attention(pkv_plan* pl, int32_t layer, const int32_t* page_table, const void* q,
                         const void* k, const void* v, float* out, bool fuse, hipStream_t stream) {
  pkv_pool* p = pl->pool;
  p->counters.kv_bytes_read += pl->rows_attended * (uint64_t)p->desc.num_kv_heads * 2ull *
                               (uint64_t)p->desc.head_width * p->elt;
  if (p->host_only) return PKV_OK;
  AttnArgs a = make_args(pl, layer, page_table, q, k, v, out, fuse);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (p->profiling) {
    e0 = take_event(p);
    e1 = take_event(p);
    if (!e0 || !e1) return fail(PKV_ERR_DEVICE, "hipEventCreate failed");
    PKV_HIP_TRY(hipEventRecord(e0, stream));
  }
  PKV_HIP_TRY(pkv::launch_attention(a, p->desc.kv_dtype, pl->num_items, stream, nullptr));
  if (p->profiling) {
    PKV_HIP_TRY(hipEventRecord(e1, stream));
    p->timed.push_back({e0, e1, pkv_pool::kTimedAttention});
    p->profile.algorithmic_bytes += launch_bytes(pl, fuse);
  }
  if (pl->any_split && pl->merge_mode == pkv::kMergeSeparate) {
    // The merge kernel reads the plan from the device: an inline plan built
    // before the pool switched to this mode is copied there once, on the
    // stream ahead of the merge.
    if (!pl->meta_uploaded) {
      pkv_status st = upload_plan_meta(pl, stream);
      if (st != PKV_OK) return st;
      a = make_args(pl, layer, page_table, q, k, v, out, fuse);
    }
    if (p->profiling) {
      e0 = take_event(p);
      e1 = take_event(p);
      if (!e0 || !e1) return fail(PKV_ERR_DEVICE, "hipEventCreate failed");
      PKV_HIP_TRY(hipEventRecord(e0, stream));
    }
    PKV_HIP_TRY(pkv::launch_merge(a, pl->num_split_reqs, stream));
    if (p->profiling) {
      PKV_HIP_TRY(hipEventRecord(e1, stream));
      p->timed.push_back({e0, e1, pkv_pool::kTimedMerge});
    }
  }
  return PKV_OK;
}

pkv_status check_layer(const pkv_pool* p, int32_t layer) {
  if (layer < 0 || layer >= p->desc.num_layers)
    return fail(PKV_ERR_INVALID_ARGUMENT, "layer %d outside [0, %d)", layer, p->desc.num_layers);
  return PKV_OK;
}

// Matrix-core prefill: the chunks cut into tiles of up to kPrefillTileRows
// rows, longest visible prefix first; an append launch writes every new row,
// then one attention launch covers all (tile, query head) pairs.  The tile
// list is uploaded once and reused by later layers of the same chunks.
pkv_status run_prefill_tiles(pkv_pool* p, int32_t n, const int32_t* rows, const int32_t* starts,
                             const int32_t* counts, int32_t pt_stride, int32_t layer,
                             const int32_t* page_table, const void* q, const void* k,
                             const void* v, float* out, uint64_t score_rows,
                             hipStream_t stream) {
  pkv_plan* pl = &p->prefill_plan;
  std::vector<int64_t> key(3 * (size_t)n + 3);
  key[0] = -1;  // never equal to a decode-plan key (those start with pt_stride)
  key[1] = pt_stride;
  key[2] = (int64_t)p->opt_gen;
  for (int32_t r = 0; r < n; ++r) {
    key[3 + 3 * r] = rows[r];
    key[4 + 3 * r] = starts[r];
    key[5 + 3 * r] = counts[r];
  }
  if (!(pl->built && key == pl->key)) {
    // Tiles grouped by request (they re-read the request's K/V), requests
    // with the longest visible prefix first, each request's longest tile
    // first.
    std::vector<int32_t> order(n), offs(n);
    int32_t off = 0;
    for (int32_t r = 0; r < n; ++r) {
      order[r] = r;
      offs[r] = off;
      off += counts[r];
    }
    std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
      return starts[x] + counts[x] > starts[y] + counts[y];
    });
    std::vector<PrefillTile> tiles;
    for (int32_t r : order) {
      const int32_t last = (counts[r] - 1) / pkv::kPrefillTileRows * pkv::kPrefillTileRows;
      for (int32_t i0 = last; i0 >= 0; i0 -= pkv::kPrefillTileRows) {
        const int32_t nq = std::min(pkv::kPrefillTileRows, counts[r] - i0);
        tiles.push_back(PrefillTile{rows[r], starts[r], offs[r], i0, nq, starts[r] + i0 + nq});
      }
    }
    pkv_status st = ensure_device(p, stream);
    if (st != PKV_OK) return st;
    pl->built = false;  // the device copy is replaced below
    const MetaPart part{tiles.data(), tiles.size() * sizeof(PrefillTile)};
    if ((st = upload_meta(pl, &part, 1, stream)) != PKV_OK) return st;
    pl->key = std::move(key);
    pl->built = true;
    pl->num_items = (int32_t)tiles.size();
    pl->reqs.clear();
    pl->items.clear();
  }
  PrefillArgs a{};
  a.q = q;
  a.k_new = k;
  a.v_new = v;
  a.out = out;
  a.k_layer = static_cast<char*>(p->desc.k_storage) + (int64_t)layer * p->layer_bytes;
  a.v_layer = static_cast<char*>(p->desc.v_storage) + (int64_t)layer * p->layer_bytes;
  a.page_table = page_table;
  a.pt_stride = pt_stride;
  a.tiles = reinterpret_cast<const PrefillTile*>(pl->d_meta);
  a.num_tiles = pl->num_items;
  a.num_heads = p->desc.num_heads;
  a.num_kv_heads = p->desc.num_kv_heads;
  a.page_size = p->desc.page_size;
  a.page_bytes = p->page_bytes;
  a.head_bytes = p->head_bytes;
  a.scale_log2e = (float)(1.4426950408889634 / std::sqrt((double)p->desc.head_width));
  a.dtype = p->desc.kv_dtype;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  if (p->profiling) {
    e0 = take_event(p);
    e1 = take_event(p);
    if (!e0 || !e1) return fail(PKV_ERR_DEVICE, "hipEventCreate failed");
  }
  PKV_HIP_TRY(pkv::launch_prefill_append(a, pl->num_items, stream));
  if (p->profiling) PKV_HIP_TRY(hipEventRecord(e0, stream));
  PKV_HIP_TRY(pkv::launch_prefill_attention(a, pl->num_items, stream));
  if (p->profiling) {
    PKV_HIP_TRY(hipEventRecord(e1, stream));
    p->timed.push_back({e0, e1, pkv_pool::kTimedPrefill});
    p->profile.prefill_flops +=
        score_rows * (uint64_t)p->desc.num_heads * 4ull * (uint64_t)p->desc.head_width;
  }
  return PKV_OK;
}

// A chunk of counts[r] new rows per request r at positions starts[r]...,
// packed request after request in q, k, v and out: every row is written to
// the pool, then each attends causally (row i of request r over rows
// 0..starts[r]+i).  Each new row is run as its own decode query of attended
// length starts[r]+i+1 on the request's page-table row, after all rows of
// the chunk are written (a fused append would race with the rows of the
// same chunk that other workgroups read).
pkv_status run_prefill(pkv_pool* p, int32_t n, const int32_t* rows, const int32_t* starts,
                       const int32_t* counts, int32_t pt_stride, int32_t layer,
                       const int32_t* page_table, const void* q, const void* k, const void* v,
                       float* out, hipStream_t stream) {
  const int64_t max_len = (int64_t)pt_stride * p->desc.page_size;
  int64_t total = 0;
  for (int32_t r = 0; r < n; ++r) {
    if (counts[r] < 1 || starts[r] < 0 || (int64_t)starts[r] + counts[r] > max_len)
      return fail(PKV_ERR_INVALID_ARGUMENT, "request %d: rows [%d, %d + %d) outside [0, %lld)", r,
                  starts[r], starts[r], counts[r], (long long)max_len);
    total += counts[r];
  }
  if (total > std::numeric_limits<int32_t>::max() / 2)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%lld rows in one prefill call", (long long)total);
  const int64_t D = p->desc.head_width;
  uint64_t score_rows = 0;  // sum over new rows of their attended lengths
  for (int32_t r = 0; r < n; ++r)
    score_rows += (uint64_t)counts[r] * starts[r] + (uint64_t)counts[r] * (counts[r] + 1) / 2;
  p->counters.kv_bytes_read += score_rows * (uint64_t)p->desc.num_kv_heads * 2ull * D * p->elt;
  if (!p->host_only &&
      pkv::prefill_fast_supported(p->desc.kv_dtype, p->desc.head_width, p->desc.page_size))
    return run_prefill_tiles(p, n, rows, starts, counts, pt_stride, layer, page_table, q, k, v,
                             out, score_rows, stream);
  std::vector<int32_t> vrows((size_t)total), vlens((size_t)total);
  size_t j = 0;
  for (int32_t r = 0; r < n; ++r)
    for (int32_t i = 0; i < counts[r]; ++i, ++j) {
      vrows[j] = rows[r];
      vlens[j] = starts[r] + i + 1;
    }
  pkv_plan* pl = &p->prefill_plan;
  pkv_status st = plan_build(pl, (int32_t)total, vrows.data(), vlens.data(), pt_stride, stream);
  if (st != PKV_OK) return st;
  if (!p->host_only) {
    AttnArgs a = make_args(pl, layer, page_table, q, k, v, out, false);
    PKV_HIP_TRY(pkv::launch_kv_append(a, p->desc.kv_dtype, (int32_t)total, stream));
  }
  // run_attention counts the decode-form K/V reads; this call counted its own
  const uint64_t before = p->counters.kv_bytes_read;
  st = run_attention(pl, layer, page_table, q, nullptr, nullptr, out, false, stream);
  p->counters.kv_bytes_read = before;
  return st;
}

// Shared body of the single and batched transactional layer step.
pkv_status txn_step(pkv_cache* const* caches, int32_t n, int32_t layer, const void* q,
                    const void* k, const void* v, float* out, void* stream) {
  if (!caches || n < 1) return fail(PKV_ERR_INVALID_ARGUMENT, "need at least one cache");
  for (int32_t i = 0; i < n; ++i)
    if (!caches[i]) return fail(PKV_ERR_INVALID_ARGUMENT, "caches[%d] is null", i);
  pkv_pool* p = caches[0]->pool;
  pkv_status st;
  if ((st = check_layer(p, layer)) != PKV_OK) return st;
  if ((st = check_ptr(q, "q")) != PKV_OK || (st = check_ptr(k, "k")) != PKV_OK ||
      (st = check_ptr(v, "v")) != PKV_OK || (st = check_ptr(out, "out")) != PKV_OK)
    return st;
  std::vector<int32_t> rows(n), lens(n), starts(n), counts(n);
  bool chunked = false;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_cache* c = caches[i];
    if (c->pool != p) return fail(PKV_ERR_INVALID_ARGUMENT, "caches[%d] belongs to another pool", i);
    if (!c->pending) return fail(PKV_ERR_BAD_STATE, "caches[%d] has no pending token", i);
    if (c->appended[layer])
      return fail(PKV_ERR_BAD_STATE, "caches[%d] already appended layer %d", i, layer);
    rows[i] = c->slot;
    lens[i] = c->pending_pos + 1;
    starts[i] = c->pending_pos;
    counts[i] = c->pending_count;
    chunked |= c->pending_count > 1;
  }
  if (n > 1) {
    std::vector<int32_t> sorted(rows);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
      return fail(PKV_ERR_INVALID_ARGUMENT, "a cache appears twice in the batch");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = ensure_device(p, s)) != PKV_OK) return st;
  if ((st = flush_patches(p, s)) != PKV_OK) return st;
  if (chunked) {
    st = run_prefill(p, n, rows.data(), starts.data(), counts.data(), p->arena_stride, layer,
                     p->d_arena, q, k, v, out, s);
    if (st != PKV_OK) return st;
  } else {
    if ((st = plan_build(&p->txn_plan, n, rows.data(), lens.data(), p->arena_stride, s)) !=
        PKV_OK)
      return st;
    if ((st = run_attention(&p->txn_plan, layer, p->d_arena, q, k, v, out, true, s)) != PKV_OK)
      return st;
  }
  for (int32_t i = 0; i < n; ++i) {
    caches[i]->appended[layer] = 1;
    caches[i]->appended_count += 1;
  }
  return ok();
}

// ---- the allocation-free decode call's plan --------------------------------
// Fixed host arrays (no heap): the plan is built here, then copied into the
// device scratch's plan region in one copy from na_stage.  Shared by every
// call, like the device scratch itself.
ReqEntry na_reqs[pkv::kScratchMaxReqs];
WorkItem na_items[pkv::kScratchMaxItems];
WorkItem na_tmp[pkv::kScratchMaxItems];
int32_t na_merge[pkv::kScratchMaxReqs];
char na_stage[pkv::kScratchMetaBytes];

// Stable sort of items[0..m) by decreasing chunk length, bottom-up merge
// sort through tmp (no allocation): the order plan_build's stable_sort
// gives, so both calls launch identical plans.
void sort_longest_first(WorkItem* items, WorkItem* tmp, int32_t m) {
  auto len = [](const WorkItem& w) { return w.blk_end - w.blk_begin; };
  WorkItem* src = items;
  WorkItem* dst = tmp;
  for (int32_t width = 1; width < m; width *= 2) {
    for (int32_t lo = 0; lo < m; lo += 2 * width) {
      const int32_t mid = std::min(lo + width, m), hi = std::min(lo + 2 * width, m);
      int32_t i = lo, j = mid, k = lo;
      while (i < mid && j < hi) dst[k++] = len(src[j]) > len(src[i]) ? src[j++] : src[i++];
      while (i < mid) dst[k++] = src[i++];
      while (j < hi) dst[k++] = src[j++];
    }
    std::swap(src, dst);
  }
  if (src != items) std::memcpy(items, src, (size_t)m * sizeof(WorkItem));
}

}  // namespace

extern "C" {

const char* pkv_version(void) { return "0.1.0"; }

const char* pkv_last_error(void) { return g_last_error.c_str(); }

void pkv_pool_desc_init(pkv_pool_desc* d) {
  if (!d) return;
  std::memset(d, 0, sizeof *d);
  d->page_size = 16;
  d->num_pages = 0;
  d->max_caches = 0;
  d->kv_dtype = PKV_DTYPE_F32;
  d->split_blocks = 0;
}

pkv_status pkv_pool_create(const pkv_pool_desc* desc, pkv_pool** out) {
  if (!desc || !out) return fail(PKV_ERR_INVALID_ARGUMENT, "null desc or out");
  pkv_pool_desc d = *desc;
  if (d.num_layers < 1 || d.num_heads < 1 || d.head_width < 1 || d.page_size < 1 ||
      d.max_context < 1 || d.num_pages < 0 || d.max_caches < 0 || d.num_kv_heads < 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "sizes must be positive");
  if (d.num_kv_heads == 0) d.num_kv_heads = d.num_heads;
  if (d.num_heads % d.num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARGUMENT, "num_heads %d is not a multiple of num_kv_heads %d",
                d.num_heads, d.num_kv_heads);
  if (d.reserved != 0) return fail(PKV_ERR_INVALID_ARGUMENT, "reserved field must be 0");
  if (d.head_width > 1024) return fail(PKV_ERR_INVALID_ARGUMENT, "head_width %d > 1024", d.head_width);
  if (d.kv_dtype != PKV_DTYPE_F32 && d.kv_dtype != PKV_DTYPE_BF16)
    return fail(PKV_ERR_INVALID_ARGUMENT, "unknown kv_dtype %d", d.kv_dtype);
  if (d.flags & ~(PKV_POOL_HOST_ONLY | PKV_POOL_ADDRESS_ORDER))
    return fail(PKV_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", d.flags);
  if (!d.k_storage || !d.v_storage) return fail(PKV_ERR_INVALID_ARGUMENT, "null storage");
  if (!aligned16(d.k_storage) || !aligned16(d.v_storage))
    return fail(PKV_ERR_INVALID_ARGUMENT, "storage not 16-byte aligned");
  if (d.num_pages == 0) d.num_pages = (d.max_context + d.page_size - 1) / d.page_size;
  if (d.max_caches == 0) d.max_caches = 256;
  const int64_t pages_per_cache = ((int64_t)d.max_context + d.page_size - 1) / d.page_size;
  if ((int64_t)d.max_caches * pages_per_cache > std::numeric_limits<int32_t>::max())
    return fail(PKV_ERR_INVALID_ARGUMENT, "max_caches * pages per context overflows");
  const size_t elt = elt_bytes(d.kv_dtype);
  const double layer_bytes =
      (double)d.num_pages * d.num_kv_heads * d.page_size * d.head_width * (double)elt;
  if (layer_bytes * d.num_layers > 9.0e18)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pool larger than 2^63 bytes");
  pkv_pool* p = new (std::nothrow) pkv_pool();
  if (!p) return fail(PKV_ERR_ALLOC, "pool");
  try {
    p->desc = d;
    p->host_only = (d.flags & PKV_POOL_HOST_ONLY) != 0;
    p->elt = elt;
    p->head_bytes = (int64_t)d.page_size * d.head_width * (int64_t)elt;
    p->page_bytes = p->head_bytes * d.num_kv_heads;
    p->layer_bytes = p->page_bytes * d.num_pages;
    p->arena_stride = (int32_t)pages_per_cache;
    p->free_stack.resize(d.num_pages);
    for (int32_t i = 0; i < d.num_pages; ++i) p->free_stack[i] = i;
    if (!(d.flags & PKV_POOL_ADDRESS_ORDER)) {
      uint64_t s = d.free_list_seed;
      for (int32_t i = d.num_pages - 1; i > 0; --i) {
        const uint64_t j = ((splitmix_next(s) >> 32) * (uint64_t)(i + 1)) >> 32;
        std::swap(p->free_stack[i], p->free_stack[(size_t)j]);
      }
    }
    std::reverse(p->free_stack.begin(), p->free_stack.end());  // first lease = first listed ID
    p->owner.assign(d.num_pages, kFree);
    p->refs.assign(d.num_pages, 0);
    p->free_slots.resize(d.max_caches);
    for (int32_t i = 0; i < d.max_caches; ++i) p->free_slots[i] = d.max_caches - 1 - i;
    p->txn_plan.pool = p;
    p->txn_plan.internal = true;
    p->call_plan.pool = p;
    p->call_plan.internal = true;
    p->prefill_plan.pool = p;
    p->prefill_plan.internal = true;
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(PKV_ERR_ALLOC, "pool metadata");
  }
  *out = p;
  return ok();
}

pkv_status pkv_pool_destroy(pkv_pool* p) {
  if (!p) return fail(PKV_ERR_INVALID_ARGUMENT, "null pool");
  if (p->live_caches > 0 || p->live_plans > 0 || p->raw_leased > 0)
    return fail(PKV_ERR_BAD_STATE, "pool still has %d caches, %d plans, %d raw pages",
                p->live_caches, p->live_plans, p->raw_leased);
  plan_release(&p->txn_plan);
  plan_release(&p->call_plan);
  plan_release(&p->prefill_plan);
  for (const auto& t : p->timed) {
    (void)hipEventSynchronize(t.end);
    p->spare.push_back(t.start);
    p->spare.push_back(t.end);
  }
  for (hipEvent_t e : p->spare) (void)hipEventDestroy(e);
  if (p->d_arena) (void)hipFree(p->d_arena);
  delete p;
  return ok();
}

pkv_status pkv_pool_get_desc(const pkv_pool* p, pkv_pool_desc* out) {
  if (!p || !out) return fail(PKV_ERR_INVALID_ARGUMENT, "null argument");
  *out = p->desc;
  return ok();
}

pkv_status pkv_pool_get_counters(const pkv_pool* p, pkv_counters* out) {
  if (!p || !out) return fail(PKV_ERR_INVALID_ARGUMENT, "null argument");
  *out = p->counters;
  out->pages_free = (int32_t)p->free_stack.size();
  out->pages_leased = p->desc.num_pages - out->pages_free;
  out->pages_shared = 0;
  for (int32_t r : p->refs) out->pages_shared += r > 1;
  return ok();
}

pkv_status pkv_pool_set_option(pkv_pool* p, int32_t option, int64_t value) {
  if (!p) return fail(PKV_ERR_INVALID_ARGUMENT, "null pool");
  switch (option) {
    case PKV_OPT_SPLIT_BLOCKS:
      if (value < -1 || value > (1 << 24)) return fail(PKV_ERR_INVALID_ARGUMENT, "split_blocks");
      p->desc.split_blocks = (int32_t)value;
      p->opt_gen += 1;
      return ok();
    case PKV_OPT_MERGE_MODE:
      if (value != pkv::kMergeSeparate && value != pkv::kMergeAuto &&
          value != pkv::kMergeLastArriver)
        return fail(PKV_ERR_INVALID_ARGUMENT, "merge mode %lld", (long long)value);
      p->merge_mode = (int32_t)value;
      p->opt_gen += 1;
      return ok();
    case PKV_OPT_WAVES:
      if (value != 0 && value != 4 && value != 8 && value != 16)
        return fail(PKV_ERR_INVALID_ARGUMENT, "waves %lld", (long long)value);
      p->waves_option = (int32_t)value;
      p->opt_gen += 1;
      return ok();
    case PKV_OPT_PROFILING:
      if (value != 0 && value != 1) return fail(PKV_ERR_INVALID_ARGUMENT, "profiling %lld", (long long)value);
      p->profiling = value == 1;
      return ok();
    case PKV_OPT_VALIDATE:
      if (value != 0 && value != 1) return fail(PKV_ERR_INVALID_ARGUMENT, "validate %lld", (long long)value);
      p->validate = value == 1;
      return ok();
    default:
      return fail(PKV_ERR_INVALID_ARGUMENT, "unknown option %d", option);
  }
}

pkv_status pkv_pool_get_profile(pkv_pool* p, pkv_profile* out, int32_t reset) {
  if (!p || !out) return fail(PKV_ERR_INVALID_ARGUMENT, "null argument");
  for (const auto& t : p->timed) {
    PKV_HIP_TRY(hipEventSynchronize(t.end));
    float ms = 0.f;
    PKV_HIP_TRY(hipEventElapsedTime(&ms, t.start, t.end));
    if (t.kind == pkv_pool::kTimedMerge) {
      p->profile.merge_launches += 1;
      p->profile.merge_ms += ms;
    } else if (t.kind == pkv_pool::kTimedPrefill) {
      p->profile.prefill_launches += 1;
      p->profile.prefill_ms += ms;
    } else {
      p->profile.attention_launches += 1;
      p->profile.attention_ms += ms;
    }
    p->spare.push_back(t.start);
    p->spare.push_back(t.end);
  }
  p->timed.clear();
  *out = p->profile;
  if (reset) p->profile = pkv_profile{};
  return ok();
}

pkv_status pkv_page_lease(pkv_pool* p, int32_t* page) {
  if (!p || !page) return fail(PKV_ERR_INVALID_ARGUMENT, "null argument");
  if (p->free_stack.empty()) return fail(PKV_ERR_OUT_OF_PAGES, "no free page");
  *page = lease_page(p, kRaw);
  p->raw_leased += 1;
  return ok();
}

pkv_status pkv_page_release(pkv_pool* p, int32_t page) {
  if (!p) return fail(PKV_ERR_INVALID_ARGUMENT, "null pool");
  if (page < 0 || page >= p->desc.num_pages)
    return fail(PKV_ERR_INVALID_ARGUMENT, "page %d out of range", page);
  if (p->owner[page] != kRaw) return fail(PKV_ERR_INVALID_ARGUMENT, "page %d is not raw-leased", page);
  release_page(p, page);
  p->raw_leased -= 1;
  return ok();
}

pkv_status pkv_cache_create(pkv_pool* p, int32_t max_context, pkv_cache** out) {
  if (!p || !out) return fail(PKV_ERR_INVALID_ARGUMENT, "null argument");
  if (max_context < 1 || max_context > p->desc.max_context)
    return fail(PKV_ERR_INVALID_ARGUMENT, "max_context %d outside [1, %d]", max_context,
                p->desc.max_context);
  if (p->free_slots.empty())
    return fail(PKV_ERR_BAD_STATE, "all %d cache slots in use", p->desc.max_caches);
  pkv_cache* c = new (std::nothrow) pkv_cache();
  if (!c) return fail(PKV_ERR_ALLOC, "cache");
  try {
    c->pages.reserve((max_context + p->desc.page_size - 1) / p->desc.page_size);
    c->appended.assign(p->desc.num_layers, 0);
  } catch (const std::bad_alloc&) {
    delete c;
    return fail(PKV_ERR_ALLOC, "cache");
  }
  c->pool = p;
  c->max_context = max_context;
  c->slot = p->free_slots.back();
  p->free_slots.pop_back();
  p->live_caches += 1;
  *out = c;
  return ok();
}

static void cache_return_pages(pkv_cache* c) {
  for (auto it = c->pages.rbegin(); it != c->pages.rend(); ++it) release_page(c->pool, *it);
  c->pages.clear();
}

pkv_status pkv_cache_destroy(pkv_cache* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARGUMENT, "null cache");
  pkv_pool* p = c->pool;
  if (c->pending) p->counters.aborted_tokens += (uint64_t)c->pending_count;
  if (c->pending && c->cow_logical >= 0) release_page(p, c->cow_old);
  cache_return_pages(c);
  p->free_slots.push_back(c->slot);
  p->live_caches -= 1;
  p->txn_plan.key.clear();  // slot may be reused: never reuse a plan keyed on it
  delete c;
  return ok();
}

pkv_status pkv_cache_reset(pkv_cache* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARGUMENT, "null cache");
  if (c->pending) return fail(PKV_ERR_BAD_STATE, "reset with a pending token; abort it first");
  cache_return_pages(c);
  c->len = 0;
  return ok();
}

int32_t pkv_cache_size(const pkv_cache* c) { return c ? c->len : -1; }
int32_t pkv_cache_capacity(const pkv_cache* c) { return c ? c->max_context : -1; }
int32_t pkv_cache_block_size(const pkv_cache* c) { return c ? c->pool->desc.page_size : -1; }

pkv_status pkv_cache_page_table(const pkv_cache* c, int32_t* out, int32_t cap, int32_t* n_out) {
  if (!c || !n_out) return fail(PKV_ERR_INVALID_ARGUMENT, "null argument");
  const int32_t n = (int32_t)c->pages.size();
  if (n > 0 && (!out || cap < n))
    return fail(PKV_ERR_INVALID_ARGUMENT, "page table has %d entries, cap %d", n, cap);
  if (n > 0) std::memcpy(out, c->pages.data(), n * sizeof(int32_t));
  *n_out = n;
  return ok();
}

static bool needs_cow(const pkv_cache* c);
static int32_t copy_on_write(pkv_cache* c);

pkv_status pkv_cache_grow(pkv_cache* c, int32_t n_tokens, void* stream) {
  if (!c) return fail(PKV_ERR_INVALID_ARGUMENT, "null cache");
  if (n_tokens < 0) return fail(PKV_ERR_INVALID_ARGUMENT, "negative n_tokens");
  if (c->pending) return fail(PKV_ERR_BAD_STATE, "grow with a pending token");
  if ((int64_t)c->len + n_tokens > c->max_context)
    return fail(PKV_ERR_CAPACITY_EXHAUSTED, "length %d + %d exceeds capacity %d", c->len,
                n_tokens, c->max_context);
  pkv_pool* p = c->pool;
  const int32_t S = p->desc.page_size;
  const bool cow = n_tokens > 0 && needs_cow(c);
  const int32_t need = (c->len + n_tokens + S - 1) / S - (int32_t)c->pages.size();
  if (need + (cow ? 1 : 0) > (int32_t)p->free_stack.size())
    return fail(PKV_ERR_OUT_OF_PAGES, "need %d pages, %zu free", need + (cow ? 1 : 0),
                p->free_stack.size());
  if (cow) {
    // The private copy of the shared last page is enqueued on the caller's
    // stream, so the rows the caller then writes on that stream land after
    // it, and it reads the source after every earlier write there.  The
    // source stays allocated: another holder still has it.
    hipStream_t s = static_cast<hipStream_t>(stream);
    pkv_status st = ensure_device(p, s);
    if (st != PKV_OK) return st;
    const int32_t old = c->pages[c->len / S];
    copy_on_write(c);
    if ((st = flush_copies(p, s)) != PKV_OK) return st;
    release_page(p, old);
  }
  for (int32_t i = 0; i < need; ++i) {
    const int32_t page = lease_page(p, kCache);
    record_patch(c, (int32_t)c->pages.size(), page);
    c->pages.push_back(page);
  }
  c->len += n_tokens;
  return ok();
}

// Whether writing position len of cache c needs a private copy of its last
// page first: the page is partly filled and shared with another holder.
static bool needs_cow(const pkv_cache* c) {
  if (c->len == 0) return false;
  const int32_t S = c->pool->desc.page_size;
  return c->len % S != 0 && c->pool->refs[c->pages[c->len / S]] > 1;
}

// Pages a begin of `count` positions must lease for cache c (a copy-on-write
// page included).
static int32_t pages_for(const pkv_cache* c, int32_t count) {
  const int32_t S = c->pool->desc.page_size;
  return (int32_t)(((int64_t)c->len + count + S - 1) / S - ((int64_t)c->len + S - 1) / S) +
         (needs_cow(c) ? 1 : 0);
}

// Replaces the shared, partly filled last page of c by a private copy (a new
// page, its contents queued for copying).  The caller keeps the cache's
// reference on the old page until the copy can no longer be undone or
// cancelled (commit or abort of the transaction; grow after the copy ran).
// Returns the logical page, or -1 when none is needed.
static int32_t copy_on_write(pkv_cache* c) {
  if (!needs_cow(c)) return -1;
  pkv_pool* p = c->pool;
  const int32_t lp = c->len / p->desc.page_size;
  const int32_t old = c->pages[lp];
  const int32_t page = lease_page(p, kCache);
  p->copies.push_back({old, page});
  c->pages[lp] = page;
  record_patch(c, lp, page);
  p->counters.cow_copies += 1;
  return lp;
}

static pkv_status check_begin(const pkv_cache* c, int32_t count, int32_t i) {
  if (count < 1) return fail(PKV_ERR_INVALID_ARGUMENT, "caches[%d]: count %d < 1", i, count);
  if (c->pending) return fail(PKV_ERR_BAD_STATE, "caches[%d]: a token is already pending", i);
  if ((int64_t)c->len + count > c->max_context)
    return fail(PKV_ERR_CAPACITY_EXHAUSTED, "caches[%d]: length %d + %d exceeds capacity %d", i,
                c->len, count, c->max_context);
  return PKV_OK;
}

// Reserves positions len..len+count-1; the caller has checked the state and
// that enough pages are free.
static int32_t begin_unchecked(pkv_cache* c, int32_t count) {
  pkv_pool* p = c->pool;
  const bool cow = needs_cow(c);
  const int32_t need = pages_for(c, count) - (cow ? 1 : 0);
  c->cow_old = cow ? c->pages[c->len / p->desc.page_size] : -1;
  c->cow_logical = copy_on_write(c);
  for (int32_t i = 0; i < need; ++i) {
    const int32_t page = lease_page(p, kCache);
    record_patch(c, (int32_t)c->pages.size(), page);
    c->pages.push_back(page);
  }
  c->pending = true;
  c->pending_pos = c->len;
  c->pending_count = count;
  c->pending_new_pages = need;
  std::fill(c->appended.begin(), c->appended.end(), 0);
  c->appended_count = 0;
  return c->pending_pos;
}

pkv_status pkv_cache_fork(const pkv_cache* src, int32_t n_tokens, int32_t max_context,
                          pkv_cache** out) {
  if (!src || !out) return fail(PKV_ERR_INVALID_ARGUMENT, "null argument");
  if (src->pending) return fail(PKV_ERR_BAD_STATE, "fork of a cache with a pending token");
  if (n_tokens < 0 || n_tokens > src->len)
    return fail(PKV_ERR_INVALID_ARGUMENT, "n_tokens %d outside [0, %d]", n_tokens, src->len);
  if (max_context < n_tokens)
    return fail(PKV_ERR_INVALID_ARGUMENT, "max_context %d below n_tokens %d", max_context,
                n_tokens);
  pkv_pool* p = src->pool;
  pkv_cache* c = nullptr;
  pkv_status st = pkv_cache_create(p, max_context, &c);
  if (st != PKV_OK) return st;
  const int32_t np = (n_tokens + p->desc.page_size - 1) / p->desc.page_size;
  for (int32_t i = 0; i < np; ++i) {
    const int32_t page = src->pages[i];
    p->refs[page] += 1;
    record_patch(c, i, page);
    c->pages.push_back(page);
  }
  c->len = n_tokens;
  *out = c;
  return ok();
}

pkv_status pkv_begin_tokens(pkv_cache* c, int32_t count, int32_t* position) {
  if (!c) return fail(PKV_ERR_INVALID_ARGUMENT, "null cache");
  pkv_status st = check_begin(c, count, 0);
  if (st != PKV_OK) return st;
  const int32_t need = pages_for(c, count);
  if (need > (int32_t)c->pool->free_stack.size())
    return fail(PKV_ERR_OUT_OF_PAGES, "%d pages needed, %zu free", need,
                c->pool->free_stack.size());
  const int32_t pos = begin_unchecked(c, count);
  if (position) *position = pos;
  return ok();
}

pkv_status pkv_begin_token(pkv_cache* c, int32_t* position) {
  return pkv_begin_tokens(c, 1, position);
}

static pkv_status check_batch(pkv_cache* const* caches, int32_t n) {
  if (!caches || n < 1) return fail(PKV_ERR_INVALID_ARGUMENT, "need at least one cache");
  for (int32_t i = 0; i < n; ++i) {
    if (!caches[i]) return fail(PKV_ERR_INVALID_ARGUMENT, "caches[%d] is null", i);
    if (caches[i]->pool != caches[0]->pool)
      return fail(PKV_ERR_INVALID_ARGUMENT, "caches[%d] belongs to another pool", i);
  }
  if (n > 1) {
    std::vector<const pkv_cache*> sorted(caches, caches + n);
    std::sort(sorted.begin(), sorted.end());
    if (std::adjacent_find(sorted.begin(), sorted.end()) != sorted.end())
      return fail(PKV_ERR_INVALID_ARGUMENT, "a cache appears twice in the batch");
  }
  return PKV_OK;
}

pkv_status pkv_begin_tokens_batched(pkv_cache* const* caches, int32_t n, const int32_t* counts,
                                    int32_t* positions) {
  pkv_status st = check_batch(caches, n);
  if (st != PKV_OK) return st;
  pkv_pool* p = caches[0]->pool;
  int64_t pages = 0;
  for (int32_t i = 0; i < n; ++i) {
    const int32_t count = counts ? counts[i] : 1;
    if ((st = check_begin(caches[i], count, i)) != PKV_OK) return st;
    pages += pages_for(caches[i], count);
  }
  if (pages > (int64_t)p->free_stack.size())
    return fail(PKV_ERR_OUT_OF_PAGES, "%lld pages needed, %zu free", (long long)pages,
                p->free_stack.size());
  for (int32_t i = 0; i < n; ++i) {
    const int32_t pos = begin_unchecked(caches[i], counts ? counts[i] : 1);
    if (positions) positions[i] = pos;
  }
  return ok();
}

pkv_status pkv_begin_token_batched(pkv_cache* const* caches, int32_t n, int32_t* positions) {
  return pkv_begin_tokens_batched(caches, n, nullptr, positions);
}

pkv_status pkv_commit_token_batched(pkv_cache* const* caches, int32_t n) {
  pkv_status st = check_batch(caches, n);
  if (st != PKV_OK) return st;
  const int32_t L = caches[0]->pool->desc.num_layers;
  for (int32_t i = 0; i < n; ++i) {
    const pkv_cache* c = caches[i];
    if (!c->pending) return fail(PKV_ERR_BAD_STATE, "caches[%d]: no pending token", i);
    if (c->appended_count != L)
      return fail(PKV_ERR_BAD_STATE, "caches[%d]: only %d of %d layers appended", i,
                  c->appended_count, L);
  }
  for (int32_t i = 0; i < n; ++i) pkv_commit_token(caches[i]);
  return ok();
}

pkv_status pkv_append_and_attend(pkv_cache* c, int32_t layer, const void* q, const void* k,
                                 const void* v, float* out, void* stream) {
  if (!c) return fail(PKV_ERR_INVALID_ARGUMENT, "null cache");
  return txn_step(&c, 1, layer, q, k, v, out, stream);
}

pkv_status pkv_append_and_attend_batched(pkv_cache* const* caches, int32_t n, int32_t layer,
                                         const void* q, const void* k, const void* v,
                                         float* out, void* stream) {
  return txn_step(caches, n, layer, q, k, v, out, stream);
}

pkv_status pkv_commit_token(pkv_cache* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARGUMENT, "null cache");
  if (!c->pending) return fail(PKV_ERR_BAD_STATE, "no pending token");
  pkv_pool* p = c->pool;
  if (c->appended_count != p->desc.num_layers)
    return fail(PKV_ERR_BAD_STATE, "only %d of %d layers appended", c->appended_count,
                p->desc.num_layers);
  const uint64_t lanes = (uint64_t)p->desc.num_layers * p->desc.num_heads;
  for (int32_t i = 0; i < c->pending_count; ++i)
    p->counters.score_cells += lanes * (uint64_t)(c->pending_pos + i + 1);
  c->len = c->pending_pos + c->pending_count;
  c->pending = false;
  if (c->cow_logical >= 0) release_page(p, c->cow_old);  // the copy is the cache's now
  c->cow_logical = c->cow_old = -1;
  p->counters.committed_tokens += (uint64_t)c->pending_count;
  p->counters.cache_appends += (uint64_t)p->desc.num_layers * c->pending_count;
  return ok();
}

pkv_status pkv_abort_token(pkv_cache* c) {
  if (!c) return fail(PKV_ERR_INVALID_ARGUMENT, "null cache");
  if (!c->pending) return fail(PKV_ERR_BAD_STATE, "no pending token");
  pkv_pool* p = c->pool;
  for (int32_t i = 0; i < c->pending_new_pages; ++i) {
    release_page(p, c->pages.back());
    c->pages.pop_back();
  }
  if (c->cow_logical >= 0) {
    // back to the shared page (the transaction's hold on it becomes the
    // cache's again); the private copy goes, cancelling its copy if queued
    const int32_t copy = c->pages[c->cow_logical];
    c->pages[c->cow_logical] = c->cow_old;
    record_patch(c, c->cow_logical, c->cow_old);
    release_page(p, copy);
    c->cow_logical = c->cow_old = -1;
  }
  c->pending = false;
  c->pool->counters.aborted_tokens += (uint64_t)c->pending_count;
  return ok();
}

pkv_status pkv_plan_create(pkv_pool* p, pkv_plan** out) {
  if (!p || !out) return fail(PKV_ERR_INVALID_ARGUMENT, "null argument");
  pkv_plan* pl = new (std::nothrow) pkv_plan();
  if (!pl) return fail(PKV_ERR_ALLOC, "plan");
  pl->pool = p;
  p->live_plans += 1;
  *out = pl;
  return ok();
}

pkv_status pkv_plan_destroy(pkv_plan* pl) {
  if (!pl || pl->internal) return fail(PKV_ERR_INVALID_ARGUMENT, "null or internal plan");
  pl->pool->live_plans -= 1;
  plan_release(pl);
  delete pl;
  return ok();
}

pkv_status pkv_plan_build(pkv_plan* pl, int32_t n, const int32_t* seq_lens, int32_t pt_stride,
                          void* stream) {
  if (!pl || !seq_lens || n < 1 || pt_stride < 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "null plan/seq_lens or non-positive n/pt_stride");
  std::vector<int32_t> rows(n);
  for (int32_t r = 0; r < n; ++r) rows[r] = r;
  pkv_status st = plan_build(pl, n, rows.data(), seq_lens, pt_stride,
                             static_cast<hipStream_t>(stream));
  return st == PKV_OK ? ok() : st;
}

int32_t pkv_plan_num_chunks(const pkv_plan* pl) {
  return (pl && pl->built) ? pl->num_items : 0;
}

static pkv_status plan_ready(const pkv_plan* pl, int32_t layer, const int32_t* page_table,
                             void* stream) {
  if (!pl) return fail(PKV_ERR_INVALID_ARGUMENT, "null plan");
  if (!pl->built) return fail(PKV_ERR_BAD_STATE, "plan not built");
  pkv_status st = check_layer(pl->pool, layer);
  if (st != PKV_OK) return st;
  if (!page_table) return fail(PKV_ERR_INVALID_ARGUMENT, "page_table is null");
  return ensure_device(pl->pool, static_cast<hipStream_t>(stream));
}

pkv_status pkv_plan_decode_attention(pkv_plan* pl, int32_t layer, const void* q,
                                     const int32_t* page_table, float* out, void* stream) {
  pkv_status st = plan_ready(pl, layer, page_table, stream);
  if (st != PKV_OK) return st;
  if ((st = check_ptr(q, "q")) != PKV_OK || (st = check_ptr(out, "out")) != PKV_OK) return st;
  if ((st = validate_plan_table(pl, page_table, static_cast<hipStream_t>(stream))) != PKV_OK)
    return st;
  st = run_attention(pl, layer, page_table, q, nullptr, nullptr, out, false,
                     static_cast<hipStream_t>(stream));
  return st == PKV_OK ? ok() : st;
}

pkv_status pkv_plan_kv_append(pkv_plan* pl, int32_t layer, const int32_t* page_table,
                              const void* k, const void* v, void* stream) {
  pkv_status st = plan_ready(pl, layer, page_table, stream);
  if (st != PKV_OK) return st;
  if ((st = check_ptr(k, "k")) != PKV_OK || (st = check_ptr(v, "v")) != PKV_OK) return st;
  if ((st = validate_plan_table(pl, page_table, static_cast<hipStream_t>(stream))) != PKV_OK)
    return st;
  if (pl->pool->host_only) return ok();
  AttnArgs a = make_args(pl, layer, page_table, nullptr, k, v, nullptr, false);
  PKV_HIP_TRY(pkv::launch_kv_append(a, pl->pool->desc.kv_dtype, pl->n,
                                    static_cast<hipStream_t>(stream)));
  return ok();
}

pkv_status pkv_plan_append_and_attend(pkv_plan* pl, int32_t layer, const int32_t* page_table,
                                      const void* q, const void* k, const void* v, float* out,
                                      void* stream) {
  pkv_status st = plan_ready(pl, layer, page_table, stream);
  if (st != PKV_OK) return st;
  if ((st = check_ptr(q, "q")) != PKV_OK || (st = check_ptr(k, "k")) != PKV_OK ||
      (st = check_ptr(v, "v")) != PKV_OK || (st = check_ptr(out, "out")) != PKV_OK)
    return st;
  if ((st = validate_plan_table(pl, page_table, static_cast<hipStream_t>(stream))) != PKV_OK)
    return st;
  st = run_attention(pl, layer, page_table, q, k, v, out, true, static_cast<hipStream_t>(stream));
  return st == PKV_OK ? ok() : st;
}

pkv_status pkv_decode_attention(pkv_pool* p, int32_t layer, int32_t n, const void* q,
                                const int32_t* page_table, int32_t pt_stride,
                                const int32_t* seq_lens, float* out, void* stream) {
  if (!p || !seq_lens || n < 1 || pt_stride < 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "null pool/seq_lens or non-positive n/pt_stride");
  pkv_status st = check_layer(p, layer);
  if (st != PKV_OK) return st;
  if (!page_table) return fail(PKV_ERR_INVALID_ARGUMENT, "page_table is null");
  if ((st = check_ptr(q, "q")) != PKV_OK || (st = check_ptr(out, "out")) != PKV_OK) return st;
  std::vector<int32_t> rows(n);
  for (int32_t r = 0; r < n; ++r) rows[r] = r;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = plan_build(&p->call_plan, n, rows.data(), seq_lens, pt_stride, s)) != PKV_OK) return st;
  if ((st = validate_plan_table(&p->call_plan, page_table, s)) != PKV_OK) return st;
  st = run_attention(&p->call_plan, layer, page_table, q, nullptr, nullptr, out, false, s);
  return st == PKV_OK ? ok() : st;
}

pkv_status pkv_decode_attention_noalloc(pkv_pool* p, int32_t layer, int32_t n, const void* q,
                                        const int32_t* page_table, int32_t pt_stride,
                                        const int32_t* seq_lens, float* out, void* stream) {
  static_assert(PKV_NOALLOC_SCRATCH_BYTES == pkv::kScratchBytes, "scratch size");
  static_assert(PKV_NOALLOC_MAX_REQUESTS == pkv::kScratchMaxReqs, "scratch requests");
  static_assert(PKV_NOALLOC_MAX_CHUNKS == pkv::kScratchMaxItems, "scratch chunks");
  static_assert(PKV_NOALLOC_MAX_COUNTERS * sizeof(int32_t) == pkv::kScratchCountersBytes,
                "scratch counters");
  static_assert(PKV_NOALLOC_MAX_PARTIAL_FLOATS * sizeof(float) == pkv::kScratchPartialsBytes,
                "scratch partials");
  if (!p || !seq_lens || n < 1 || pt_stride < 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "null pool/seq_lens or non-positive n/pt_stride");
  pkv_status st = check_layer(p, layer);
  if (st != PKV_OK) return st;
  if (!page_table) return fail(PKV_ERR_INVALID_ARGUMENT, "page_table is null");
  if ((st = check_ptr(q, "q")) != PKV_OK || (st = check_ptr(out, "out")) != PKV_OK) return st;
  const int64_t H = p->desc.num_heads, D = p->desc.head_width;
  if (n > pkv::kScratchMaxReqs)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%d requests exceed the scratch's %d", n,
                pkv::kScratchMaxReqs);
  if ((int64_t)n * H > PKV_NOALLOC_MAX_COUNTERS)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%d requests x %lld heads exceed the scratch's %d "
                "merge counters", n, (long long)H, PKV_NOALLOC_MAX_COUNTERS);
  const int64_t max_len = (int64_t)pt_stride * p->desc.page_size;
  int64_t total_blocks = 0;
  int32_t max_blocks = 0;
  uint64_t rows_attended = 0;
  for (int32_t r = 0; r < n; ++r) {
    if (seq_lens[r] < 1 || seq_lens[r] > max_len)
      return fail(PKV_ERR_INVALID_ARGUMENT, "seq_lens[%d]=%d outside [1, %lld]", r, seq_lens[r],
                  (long long)max_len);
    const int32_t b = (seq_lens[r] + pkv::kBlockRows - 1) / pkv::kBlockRows;
    total_blocks += b;
    max_blocks = std::max(max_blocks, b);
    rows_attended += (uint64_t)seq_lens[r];
  }
  // The plan of pkv_decode_attention, built into the fixed arrays.
  const SplitChoice choice = choose_split(p, n, total_blocks, max_blocks);
  int32_t m = 0, slots = 0, nmerge = 0;
  for (int32_t r = 0; r < n; ++r) {
    const int32_t blocks = (seq_lens[r] + pkv::kBlockRows - 1) / pkv::kBlockRows;
    const int32_t nsplit = (int32_t)(((int64_t)blocks + choice.chunk - 1) / choice.chunk);
    if ((int64_t)m + nsplit > pkv::kScratchMaxItems)
      return fail(PKV_ERR_INVALID_ARGUMENT, "the plan needs more than the scratch's %d chunks",
                  pkv::kScratchMaxItems);
    na_reqs[r] = ReqEntry{r, seq_lens[r], nsplit, nsplit > 1 ? slots : -1};
    if (nsplit > 1) {
      slots += nsplit;
      na_merge[nmerge++] = r;
    }
    int32_t b0 = 0;
    for (int32_t s = 0; s < nsplit; ++s) {
      const int32_t b1 = chunk_end(choice, blocks, nsplit, s, b0);
      na_items[m++] = WorkItem{r, b0, b1, s, na_reqs[r]};
      b0 = b1;
    }
  }
  if ((int64_t)slots * H * (D + 2) > PKV_NOALLOC_MAX_PARTIAL_FLOATS)
    return fail(PKV_ERR_INVALID_ARGUMENT, "%d split chunks x %lld heads x %lld floats exceed the "
                "scratch's %d partial floats", slots, (long long)H, (long long)(D + 2),
                PKV_NOALLOC_MAX_PARTIAL_FLOATS);
  if ((int64_t)m * H > std::numeric_limits<int32_t>::max())
    return fail(PKV_ERR_INVALID_ARGUMENT, "%d chunks x %lld heads exceed one launch", m,
                (long long)H);
  sort_longest_first(na_items, na_tmp, m);
  p->counters.kv_bytes_read += rows_attended * (uint64_t)p->desc.num_kv_heads * 2ull *
                               (uint64_t)D * p->elt;
  if (p->host_only) return ok();

  int dev = 0;
  PKV_HIP_TRY(hipGetDevice(&dev));
  if (p->device >= 0 && dev != p->device)
    return fail(PKV_ERR_INVALID_ARGUMENT, "pool lives on device %d, current device is %d",
                p->device, dev);
  void* base = nullptr;
  PKV_HIP_TRY(pkv::scratch_address(dev, &base));
  char* scratch = static_cast<char*>(base);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool inline_plan = n <= pkv::kInlineReqs && m <= pkv::kInlineItems;
  const int32_t merge_mode = plan_merge_mode(p, rows_attended);
  const bool separate = slots > 0 && merge_mode == pkv::kMergeSeparate;
  char* d_meta = scratch + pkv::kScratchMetaOffset;
  if (!inline_plan || separate) {
    // one copy from fixed host memory: requests, work items, split requests
    const size_t rb = (size_t)n * sizeof(ReqEntry), ib = (size_t)m * sizeof(WorkItem);
    std::memcpy(na_stage, na_reqs, rb);
    std::memcpy(na_stage + rb, na_items, ib);
    std::memcpy(na_stage + rb + ib, na_merge, (size_t)nmerge * sizeof(int32_t));
    PKV_HIP_TRY(hipMemcpyAsync(d_meta, na_stage, rb + ib + (size_t)nmerge * sizeof(int32_t),
                               hipMemcpyHostToDevice, s));
  }
  int32_t* d_counters = reinterpret_cast<int32_t*>(scratch + pkv::kScratchCountersOffset);
  if (slots > 0 && !separate)  // the last-arriver merge counts from zero
    PKV_HIP_TRY(pkv::launch_zero_i32(d_counters, (int64_t)n * H, s));
  const PlanView view{na_reqs, n, na_items, m, pt_stride, choice.waves, merge_mode, inline_plan,
                      d_meta, reinterpret_cast<float*>(scratch + pkv::kScratchPartialsOffset),
                      d_counters};
  const AttnArgs a = make_args_view(p, view, layer, page_table, q, nullptr, nullptr, out, false);
  PKV_HIP_TRY(pkv::launch_attention(a, p->desc.kv_dtype, m, s, nullptr));
  if (separate) PKV_HIP_TRY(pkv::launch_merge(a, nmerge, s));
  return ok();
}

pkv_status pkv_prefill_attention(pkv_pool* p, int32_t layer, int32_t n,
                                 const int32_t* page_table, int32_t pt_stride,
                                 const int32_t* starts, const int32_t* counts, const void* q,
                                 const void* k, const void* v, float* out, void* stream) {
  if (!p || !starts || !counts || n < 1 || pt_stride < 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "null pool/starts/counts or non-positive n/pt_stride");
  pkv_status st = check_layer(p, layer);
  if (st != PKV_OK) return st;
  if (!page_table) return fail(PKV_ERR_INVALID_ARGUMENT, "page_table is null");
  if ((st = check_ptr(q, "q")) != PKV_OK || (st = check_ptr(k, "k")) != PKV_OK ||
      (st = check_ptr(v, "v")) != PKV_OK || (st = check_ptr(out, "out")) != PKV_OK)
    return st;
  std::vector<int32_t> rows(n), used(n);
  for (int32_t r = 0; r < n; ++r) {
    rows[r] = r;
    if (counts[r] < 1 || starts[r] < 0 ||
        (int64_t)starts[r] + counts[r] > (int64_t)pt_stride * p->desc.page_size)
      return fail(PKV_ERR_INVALID_ARGUMENT, "request %d: rows [%d, %d + %d) outside [0, %lld)", r,
                  starts[r], starts[r], counts[r], (long long)pt_stride * p->desc.page_size);
    used[r] = (starts[r] + counts[r] + p->desc.page_size - 1) / p->desc.page_size;
  }
  if ((st = validate_table(p, page_table, pt_stride, n, rows.data(), used.data(),
                           static_cast<hipStream_t>(stream))) != PKV_OK)
    return st;
  st = run_prefill(p, n, rows.data(), starts, counts, pt_stride, layer, page_table, q, k, v, out,
                   static_cast<hipStream_t>(stream));
  return st == PKV_OK ? ok() : st;
}

pkv_status pkv_kv_append(pkv_pool* p, int32_t layer, int32_t n, const int32_t* page_table,
                         int32_t pt_stride, const int32_t* positions, const void* k,
                         const void* v, void* stream) {
  if (!p || !positions || n < 1 || pt_stride < 1)
    return fail(PKV_ERR_INVALID_ARGUMENT, "null pool/positions or non-positive n/pt_stride");
  pkv_status st = check_layer(p, layer);
  if (st != PKV_OK) return st;
  if (!page_table) return fail(PKV_ERR_INVALID_ARGUMENT, "page_table is null");
  if ((st = check_ptr(k, "k")) != PKV_OK || (st = check_ptr(v, "v")) != PKV_OK) return st;
  std::vector<int32_t> rows(n), lens(n);
  for (int32_t r = 0; r < n; ++r) {
    if (positions[r] < 0) return fail(PKV_ERR_INVALID_ARGUMENT, "positions[%d] < 0", r);
    rows[r] = r;
    lens[r] = positions[r] + 1;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if ((st = plan_build(&p->call_plan, n, rows.data(), lens.data(), pt_stride, s)) != PKV_OK)
    return st;
  if ((st = validate_plan_table(&p->call_plan, page_table, s)) != PKV_OK) return st;
  if (p->host_only) return ok();
  AttnArgs a = make_args(&p->call_plan, layer, page_table, nullptr, k, v, nullptr, false);
  PKV_HIP_TRY(pkv::launch_kv_append(a, p->desc.kv_dtype, n, s));
  return ok();
}

}  // extern "C"
