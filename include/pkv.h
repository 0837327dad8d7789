/*
 * pkv.h — paged KV-cache decode attention for AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpkv.  Plain C types only: sizes are int32_t/size_t, device
 * memory is passed as `void*` / typed pointers obtained from the HIP runtime
 * (for example from torch tensors' data_ptr()), and a stream is a `void*`
 * holding a hipStream_t (NULL = the default stream).
 *
 * What the library computes (sources cited by page title and section):
 *
 *  - riftco-transformer "Incremental Serving", section "Paged KV-cache layout":
 *    a pool owns, for every layer, key pages and value pages laid out
 *    [physical_page, head, page_offset, head_width]; a request owns a logical
 *    page table; one physical page ID addresses the matching page in every
 *    layer; pages are leased lazily as a sequence grows and returned on reset
 *    or destroy; the default page holds 16 tokens; a block count of 0 sizes
 *    the pool for one maximum-length context.
 *  - same page, section "Request flow": per token, begin reserves the next
 *    position, each layer appends its K/V row and attends with a [1,H,1,d_h]
 *    query, commit makes the position visible, abort leaves the visible
 *    length unchanged.
 *  - learn_llm ch.38 "cached generation", section "Prepare every block, then
 *    commit every cache together": the newest query scores the retained rows
 *    and the new row (len+1 rows) with dot(q,k)/sqrt(d_h), applies a stable
 *    softmax and mixes the value rows.
 *
 * Conventions
 *  - Every function returning pkv_status returns PKV_OK (0) on success.  On
 *    any error the library state is unchanged and pkv_last_error() describes
 *    the failure (a thread-local string owned by the library).
 *  - Not thread-safe: the caller serialises all calls on one pool and its
 *    caches (as the pages require external synchronisation of the raw C ABI,
 *    section "Stable C and Python sessions").
 *  - Host state changes take effect when the call returns.  Device work is
 *    enqueued on the given stream; results are valid once it completes.  All
 *    device work for one pool must be issued on one stream, or ordered by the
 *    caller.
 *  - Device outputs are float32; K/V, q, k and v use the pool dtype.  Every
 *    device pointer must be 16-byte aligned (INVALID_ARGUMENT otherwise).
 *  - Gathered K/V tensors are never exposed; only the pool and the context.
 *  - Device memory the library owns (the page-table arena, plan buffers) is
 *    allocated on first use and grows by doubling; a replaced buffer stays
 *    allocated until its plan or pool is destroyed, because freeing device
 *    memory waits for the whole device.  No call except the destroys (and
 *    pkv_pool_get_profile, which waits for its timing events) waits for the
 *    device; pkv_plan_build waits only for its own previous upload's copy.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pkv_status {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARGUMENT = 1, /* bad pointer, size, index or geometry       */
  PKV_ERR_BAD_STATE = 2,        /* call not allowed in the current state      */
  PKV_ERR_OUT_OF_PAGES = 3,     /* the pool has no free page                  */
  PKV_ERR_CAPACITY_EXHAUSTED = 4, /* the cache is at its maximum context      */
  PKV_ERR_ALLOC = 5,            /* host or device allocation failed           */
  PKV_ERR_DEVICE = 6            /* a HIP runtime call failed                  */
} pkv_status;

typedef enum pkv_dtype {
  PKV_DTYPE_F32 = 0,  /* IEEE binary32                                      */
  PKV_DTYPE_BF16 = 1  /* bfloat16, the upper half of a binary32             */
} pkv_dtype;

/* Pool flag: host state only.  No device memory is allocated or touched and
 * no work is enqueued; device-facing calls validate their arguments, update
 * the host state exactly as usual and leave every output buffer unwritten.
 * For exercising the page allocator and the token transaction without a GPU;
 * storage pointers are recorded, never dereferenced. */
#define PKV_POOL_HOST_ONLY 1u

/* Pool flag: lease pages in address order.  The initial free list holds
 * pages 0, 1, 2, ... (the first lease is page 0) instead of the seeded
 * shuffle, and free_list_seed is ignored.  A cache grown in one call, or
 * caches grown one after another, then hold runs of consecutive pages, so
 * the loads of one request touch few address-translation pages (far fewer
 * translation-cache misses on pools of many gigabytes).  Pages released
 * later are reused last-in, first-out as usual. */
#define PKV_POOL_ADDRESS_ORDER 2u

typedef struct pkv_pool pkv_pool;
typedef struct pkv_cache pkv_cache;
typedef struct pkv_plan pkv_plan;

/* Pool geometry and storage.
 * k_storage and v_storage are caller-owned device buffers, each holding
 * num_layers * num_pages * H_kv * page_size * head_width elements of
 * kv_dtype, laid out [layer][physical_page][kv_head][page_offset][head_width]
 * and 16-byte aligned.  They must stay alive until pkv_pool_destroy.
 * Queries and contexts have num_heads heads; K/V rows (the k and v of an
 * append, the pool pages) have H_kv heads.  The pages describe H_kv ==
 * num_heads; with fewer K/V heads ("Rollout Serving, Caching, and Batching",
 * key-value cache section, which allows them for grouped- and multi-query
 * models) each K/V head serves num_heads / H_kv consecutive query heads. */
typedef struct pkv_pool_desc {
  int32_t num_layers;     /* L >= 1                                           */
  int32_t num_heads;      /* H >= 1                                           */
  int32_t head_width;     /* d_h, 1..1024                                     */
  int32_t page_size;      /* tokens per page; default 16                      */
  int32_t num_pages;      /* P; 0 = ceil(max_context / page_size)             */
  int32_t max_context;    /* largest context of any cache of this pool        */
  int32_t max_caches;     /* live caches at once (device page-table rows); 0 = 256 */
  int32_t kv_dtype;       /* pkv_dtype                                        */
  int32_t split_blocks;   /* split-K chunk in 16-row blocks (a request of B
                             blocks splits into ceil(B / split_blocks) even
                             chunks); 0 = automatic, -1 = never split          */
  int32_t flags;          /* PKV_POOL_* bits; 0 by default                     */
  int32_t num_kv_heads;   /* K/V heads H_kv; 0 = num_heads.  num_heads must be
                             a multiple: query head h reads K/V head
                             h / (num_heads / H_kv) (grouped-query attention;
                             1 K/V head = multi-query)                        */
  int32_t reserved;       /* 0                                                 */
  void* k_storage;
  void* v_storage;
  uint64_t free_list_seed; /* seeds the shuffle of the initial free list      */
} pkv_pool_desc;

/* Work counters of a pool, summed over its committed tokens.
 * score_cells: one per (layer, head, attended row) of each committed token —
 * the cached newest-query score row of learn_llm ch.38, section "Count
 * attention-score cells, not total runtime". */
typedef struct pkv_counters {
  uint64_t committed_tokens;
  uint64_t aborted_tokens;
  uint64_t cache_appends;     /* layer rows appended by committed tokens     */
  uint64_t score_cells;
  uint64_t kv_bytes_read;     /* algorithmic K/V bytes read by attention launches */
  int32_t pages_free;
  int32_t pages_leased;
  uint64_t cow_copies;        /* shared pages copied before a write            */
  int32_t pages_shared;       /* pages held by more than one holder now        */
  int32_t reserved;
} pkv_counters;

/* Kernel timing of one pool, collected while PKV_OPT_PROFILING is on: HIP
 * events recorded on the launch stream immediately before and after each
 * decode attention kernel (and each separate merge kernel), and each
 * matrix-core prefill attention kernel.  algorithmic_bytes sums what the
 * decode launches must move: the K/V rows read from the pool, q, the
 * appended rows (read and written) and the float32 context.  prefill_flops
 * sums the prefill launches' score and value products, 4 * d_h per (query
 * row, query head, attended row). */
typedef struct pkv_profile {
  uint64_t attention_launches;
  double attention_ms;
  uint64_t merge_launches;
  double merge_ms;
  uint64_t algorithmic_bytes;
  uint64_t prefill_launches;
  double prefill_ms;
  uint64_t prefill_flops;
} pkv_profile;

/* Tunables of a pool (pkv_pool_set_option). */
typedef enum pkv_option {
  PKV_OPT_SPLIT_BLOCKS = 1, /* as pkv_pool_desc.split_blocks                   */
  PKV_OPT_MERGE_MODE = 2,   /* how split requests merge their chunks: 2: the
                               last-arriving chunk merges inside the
                               attention kernel; 0: a separate merge kernel
                               after it; 1 (default): per plan, 0 when its
                               launches read at least 1 GiB of K/V, else 2    */
  PKV_OPT_PROFILING = 3,    /* 1: record kernel timing events; 0: stop         */
  PKV_OPT_WAVES = 4,        /* waves per workgroup of the fast paths: 4, 8,
                               16 (the multi-head kernel for d_h <= 64; other
                               kernels then take 8), or 0
                               (default) to choose per kernel and batch (the
                               plan then picks its split as well)               */
  PKV_OPT_VALIDATE = 5      /* 1: debug mode -- before a call that takes a
                               caller page table enqueues anything, read back
                               each request's entries up to the last row the
                               call touches and reject any outside
                               [0, num_pages) with INVALID_ARGUMENT (this
                               waits for the stream); 0 (default): the caller
                               guarantees the entries.  Not applied by the
                               allocation-free call.                            */
} pkv_option;

/* Library version "major.minor.patch"; static string.  ("Incremental
 * Serving", Stable C and Python sessions: the C surface reports its ABI
 * version.) */
const char* pkv_version(void);

/* Message for the last error on this thread ("" if none); owned by the
 * library, valid until the next call on this thread.  ("Incremental
 * Serving", Stable C and Python sessions: status codes plus a last-error
 * string, no exceptions across the ABI.) */
const char* pkv_last_error(void);

/* ------------------------------------------------------------------ pool -- */

/* Defaults: page_size 16, num_pages 0, max_caches 0 (=256), dtype F32,
 * split_blocks 0, flags 0, seed 0, null storage.  Mirrors the session-options init of
 * "Incremental Serving", section "Stable C and Python sessions". */
void pkv_pool_desc_init(pkv_pool_desc* desc);

/* Creates a pool over caller storage ("Incremental Serving", Paged KV-cache
 * layout: one shared pool of per-layer key and value pages, one physical page
 * ID valid in every layer, a block count of 0 sizing the pool for one
 * maximum context).  The free list holds every page ID in a seeded random
 * order.  Touches no device: device resources are created on the first
 * device call, on the device current at that moment.  *out is owned by the
 * caller until pkv_pool_destroy.
 * Errors: INVALID_ARGUMENT (null desc/out/storage, storage not 16-byte
 * aligned, non-positive sizes, head_width > 1024, unknown dtype or flags);
 * ALLOC. */
pkv_status pkv_pool_create(const pkv_pool_desc* desc, pkv_pool** out);

/* Destroys the pool and frees its device memory (which waits for the
 * device).  ("Incremental Serving", Stable C and Python sessions: a shared
 * object is rejected while anything created from it is alive.)  Errors:
 * BAD_STATE while any cache or plan of the pool is alive or any raw page is
 * leased. */
pkv_status pkv_pool_destroy(pkv_pool* pool);

/* The resolved geometry (num_pages, max_caches filled in; "Incremental
 * Serving", Paged KV-cache layout).  Errors: INVALID_ARGUMENT (null). */
pkv_status pkv_pool_get_desc(const pkv_pool* pool, pkv_pool_desc* out);

/* Work counters (learn_llm ch.38, section "Count attention-score cells, not
 * total runtime": appends and cached score cells of committed tokens) and the
 * pool's page occupancy.  Errors: INVALID_ARGUMENT (null). */
pkv_status pkv_pool_get_counters(const pkv_pool* pool, pkv_counters* out);

/* Sets one pkv_option; a plan built before an option that changes chunking
 * or workgroup shape (split blocks, waves, merge mode) is rebuilt by its
 * next build.  Errors: INVALID_ARGUMENT (unknown option or value). */
pkv_status pkv_pool_set_option(pkv_pool* pool, int32_t option, int64_t value);

/* Waits for the recorded timing events, sums them into *out and, if reset,
 * clears the record.  Errors: DEVICE. */
pkv_status pkv_pool_get_profile(pkv_pool* pool, pkv_profile* out, int32_t reset);

/* Raw page lease/release, for callers that keep their own page tables and
 * use the batched calls below ("Incremental Serving", Paged KV-cache layout:
 * pages are leased from the shared pool and returned to it).  *page receives
 * a physical page ID in [0, num_pages).  Errors: OUT_OF_PAGES;
 * INVALID_ARGUMENT for a page that is out of range or not raw-leased. */
pkv_status pkv_page_lease(pkv_pool* pool, int32_t* page);
pkv_status pkv_page_release(pkv_pool* pool, int32_t page);

/* ------------------------------------------------------- request caches -- */

/* Creates an empty request cache (length 0, no pages): a request-local
 * logical-to-physical page table over the pool ("Incremental Serving", Paged
 * KV-cache layout).  max_context <= the pool's.  *out is owned by the caller
 * until pkv_cache_destroy.  Errors: INVALID_ARGUMENT; BAD_STATE when
 * max_caches caches live. */
pkv_status pkv_cache_create(pkv_pool* pool, int32_t max_context, pkv_cache** out);

/* Returns every page (a pending token's included) and frees the handle
 * ("Incremental Serving", Paged KV-cache layout: pages return to the pool
 * when a cache is destroyed).  Errors: INVALID_ARGUMENT (null). */
pkv_status pkv_cache_destroy(pkv_cache* cache);

/* Length back to 0, every page returned, handle kept ("Incremental
 * Serving", Paged KV-cache layout: pages return on reset; learn_llm ch.38:
 * reset keeps the allocation).  Pages return in the reverse of their lease
 * order, so replaying the same tokens leases the same pages again.  Errors:
 * BAD_STATE while a token is pending. */
pkv_status pkv_cache_reset(pkv_cache* cache);

/* Committed length, maximum context, page size (tokens); -1 for a null
 * cache ("Incremental Serving", Stable C and Python sessions: a session
 * reports its size, capacity and block size). */
int32_t pkv_cache_size(const pkv_cache* cache);
int32_t pkv_cache_capacity(const pkv_cache* cache);
int32_t pkv_cache_block_size(const pkv_cache* cache);

/* Copies the logical page table (pages held, a pending token's included) into
 * out[0..cap) (host memory); *n_out receives the number of entries
 * ("Incremental Serving", Paged KV-cache layout: the request-local table).
 * Errors: INVALID_ARGUMENT when cap is too small (nothing written). */
pkv_status pkv_cache_page_table(const pkv_cache* cache, int32_t* out, int32_t cap,
                                int32_t* n_out);

/* Extends the committed length by n_tokens rows whose K/V bytes the caller
 * writes itself (a bulk prefill writer), leasing the pages they need
 * ("Incremental Serving", Paged KV-cache layout: pages are leased as a
 * sequence grows).  When the last page is shared and partly filled, its
 * private copy is enqueued on `stream` (a hipStream_t, NULL = the default
 * stream): rows the caller then writes on that stream land after the copy.
 * Errors: BAD_STATE (token pending), CAPACITY_EXHAUSTED, OUT_OF_PAGES. */
pkv_status pkv_cache_grow(pkv_cache* cache, int32_t n_tokens, void* stream);

/* A new cache that shares the first n_tokens rows of src (0 <= n_tokens <=
 * its committed length): it holds references to src's first
 * ceil(n_tokens / page_size) pages instead of copies, and its length is
 * n_tokens.  Full shared pages are never written again (writes go only to
 * positions >= length); the first write into a shared, partly filled page
 * -- by either cache -- first gives the writer a private copy of that page
 * (every layer's K and V), queued on the stream of the writer's next layer
 * call (or of pkv_cache_grow), and abort undoes it.
 * A page returns to the free list when its last holder lets it go.
 * ("Incremental Serving", Current scope: paged storage alone does not share
 * pages between matching prompts or manage prefixes by copy-on-write; this
 * is that mechanism, with the choice of which prefix to share left to the
 * caller.)  Errors: BAD_STATE (src has a pending token, or no cache slot is
 * free), INVALID_ARGUMENT (n_tokens out of range, max_context below
 * n_tokens or above the pool's). */
pkv_status pkv_cache_fork(const pkv_cache* src, int32_t n_tokens, int32_t max_context,
                          pkv_cache** out);

/* --------------------------------------------------- token transaction -- */

/* Reserves position = length; leases a page when the position starts one
 * ("Incremental Serving", Request flow: begin reserves the next logical
 * position; Paged KV-cache layout: lazy lease; Stable C and Python sessions:
 * a full context is reported, not cropped).  *position (may be null)
 * receives the position.  Errors: BAD_STATE (already pending),
 * CAPACITY_EXHAUSTED, OUT_OF_PAGES. */
pkv_status pkv_begin_token(pkv_cache* cache, int32_t* position);

/* Reserves a chunk of count >= 1 positions length..length+count-1 as one
 * transaction (a batched prefill chunk) and leases the pages they need;
 * pkv_begin_token is count = 1.  The layer calls then take count rows, and
 * row i of the chunk attends causally to rows 0..length+i -- what count
 * token-at-a-time steps compute.  Commit makes all count positions visible;
 * abort drops all of them and returns the pages this begin leased.
 * ("Incremental Serving", Paged KV-cache layout: a later batched prefill
 * writes the same paged cache that decode attention reads.)
 * *position receives length.  Errors: INVALID_ARGUMENT (count < 1),
 * BAD_STATE (already pending), CAPACITY_EXHAUSTED (length + count over the
 * capacity), OUT_OF_PAGES. */
pkv_status pkv_begin_tokens(pkv_cache* cache, int32_t count, int32_t* position);

/* One layer of the pending token (or chunk of count tokens) ("Incremental
 * Serving", Request flow: each layer appends its K/V row, then attends;
 * learn_llm ch.38, "Prepare every block, then commit every cache together":
 * the query scores the retained rows and the new one, len+1 rows, with
 * dot(q, k)/sqrt(d_h), stable softmax, weighted value rows): writes k and v
 * ([count,H_kv,d_h], pool dtype, device) into the pool at the pending
 * positions, then attends with q ([count,H,d_h]), row i over rows
 * 0..length+i, writing out ([count,H,d_h] float32).  For one token these are
 * the [1,H,1,d_h] tensors of "Incremental Serving", Request flow.
 * Errors: BAD_STATE (no pending token, layer already appended),
 * INVALID_ARGUMENT (layer out of range, null pointer), DEVICE. */
pkv_status pkv_append_and_attend(pkv_cache* cache, int32_t layer, const void* q,
                                 const void* k, const void* v, float* out, void* stream);

/* Makes the pending position(s) visible ("Incremental Serving", Request
 * flow; learn_llm ch.38: every block prepares before any cache commits, so
 * all layers must have appended).  Errors: BAD_STATE (nothing pending, or
 * some layer not appended; the caller may then abort). */
pkv_status pkv_commit_token(pkv_cache* cache);

/* Drops the pending token or chunk: length unchanged ("Incremental Serving",
 * Request flow), the pages leased by its begin returned (learn_llm ch.38:
 * a rejected step commits no state change).  Rows written into the pages by
 * the aborted layers stay as unspecified bytes beyond the length.  Errors:
 * BAD_STATE (nothing pending). */
pkv_status pkv_abort_token(pkv_cache* cache);

/* begin_token on n caches of one pool, all or none: on any error no cache
 * changes ("Incremental Serving", Request flow, for a batch of requests;
 * learn_llm ch.38: rejected operations leave committed state unchanged).  positions (may be null) receives the n reserved positions.
 * Errors: as pkv_begin_token (the first failing cache is named in the
 * message); OUT_OF_PAGES when the n begins together need more pages than are
 * free; INVALID_ARGUMENT for a repeated cache or mixed pools. */
pkv_status pkv_begin_token_batched(pkv_cache* const* caches, int32_t n, int32_t* positions);

/* begin_tokens on n caches, counts[i] positions for caches[i] (counts may be
 * null: one each; host array), all or none ("Incremental Serving", Request
 * flow and Paged KV-cache layout's batched prefill).  Errors: as pkv_begin_tokens, and
 * OUT_OF_PAGES when the begins together need more pages than are free. */
pkv_status pkv_begin_tokens_batched(pkv_cache* const* caches, int32_t n, const int32_t* counts,
                                    int32_t* positions);

/* commit_token on n caches, all or none ("Incremental Serving", Request
 * flow; learn_llm ch.38: commit every cache together).  Errors: as
 * pkv_commit_token. */
pkv_status pkv_commit_token_batched(pkv_cache* const* caches, int32_t n);

/* The same layer step for n pending caches of one pool in one launch set
 * (the Request flow of "Incremental Serving" for many requests at once):
 * q is [T,H,d_h], k and v are [T,H_kv,d_h] (pool dtype), out is [T,H,d_h]
 * float32, where T sums the caches' pending counts (T = n for single
 * tokens) and the rows of caches[i] follow those of caches[0..i).  All
 * caches are validated before any work is enqueued.  Errors: as pkv_append_and_attend, per cache; INVALID_ARGUMENT
 * for a repeated cache or caches of different pools. */
pkv_status pkv_append_and_attend_batched(pkv_cache* const* caches, int32_t n, int32_t layer,
                                         const void* q, const void* k, const void* v,
                                         float* out, void* stream);

/* ------------------------------------------- batched calls on page tables -- */

/* A split plan: per-request attended lengths turned into a device work list
 * (split-K chunks, longest first) plus partial buffers ("Rollout Serving,
 * Caching, and Batching", batching section: ragged lengths in one batch and
 * length-aware grouping).  Build it once per decode step and reuse it for
 * every layer.  The plan owns its device buffers; destroying it frees them
 * (which waits for the device).  Errors: INVALID_ARGUMENT (null; destroy of
 * a library-internal plan); ALLOC. */
pkv_status pkv_plan_create(pkv_pool* pool, pkv_plan** out);
pkv_status pkv_plan_destroy(pkv_plan* plan);

/* seq_lens: host array of n attended lengths t_r >= 1 (the newest row
 * included), each at most pt_stride * page_size (learn_llm ch.38: the
 * newest query reads the whole retained prefix, which grows with t).  A plan of at most 48
 * requests and 64 work items travels in the kernel arguments; a larger one
 * (or one the separate merge kernel reads) is uploaded on the stream.  Errors: INVALID_ARGUMENT (n < 1, t_r < 1 or too long); ALLOC. */
pkv_status pkv_plan_build(pkv_plan* plan, int32_t n, const int32_t* seq_lens,
                          int32_t pt_stride, void* stream);

/* Number of split chunks of the built plan (0 if not built or null). */
int32_t pkv_plan_num_chunks(const pkv_plan* plan);

/* Batched decode attention (learn_llm ch.38, the incremental mixture:
 * softmax(q K^T / sqrt(d_h)) V for the newest query; "Incremental Serving",
 * Paged KV-cache layout: rows reached through a logical-to-physical page
 * table): for each request r, q[r] ([H,d_h], pool dtype, device) attends to
 * rows 0..t_r-1 of its pages; page_table is a device int32 array
 * [n][pt_stride] of physical page IDs (request r's logical page i at
 * page_table[r*pt_stride + i], each in [0, num_pages); entries past the
 * request's pages are never read).  out: [n,H,d_h] float32, device.
 * Errors: INVALID_ARGUMENT (null or misaligned pointer, layer out of
 * range), BAD_STATE (plan not built), DEVICE. */
pkv_status pkv_plan_decode_attention(pkv_plan* plan, int32_t layer, const void* q,
                                     const int32_t* page_table, float* out, void* stream);

/* Batched append ("Incremental Serving", Request flow: the new K/V row
 * becomes part of the cache; Paged KV-cache layout: row j at page
 * pt[j / S], slot j % S): writes k[r], v[r] ([n,H_kv,d_h], pool dtype,
 * device) into row t_r-1 of each request's pages, a byte copy.  Errors: as
 * pkv_plan_decode_attention. */
pkv_status pkv_plan_kv_append(pkv_plan* plan, int32_t layer, const int32_t* page_table,
                              const void* k, const void* v, void* stream);

/* Both in one launch: append row t_r-1, then attend over rows 0..t_r-1 (the
 * append-then-attend order of "Incremental Serving", Request flow).  Errors:
 * as pkv_plan_decode_attention. */
pkv_status pkv_plan_append_and_attend(pkv_plan* plan, int32_t layer,
                                      const int32_t* page_table, const void* q,
                                      const void* k, const void* v, float* out,
                                      void* stream);

/* One-call form of pkv_plan_decode_attention that builds the pool's
 * internal plan from host seq_lens (t_r >= 1, at most pt_stride * page_size;
 * an empty prefix has no softmax, so t_r = 0 is rejected).  Errors:
 * INVALID_ARGUMENT (n < 1, a length out of range, null or misaligned
 * pointer), ALLOC, DEVICE. */
pkv_status pkv_decode_attention(pkv_pool* pool, int32_t layer, int32_t n, const void* q,
                                const int32_t* page_table, int32_t pt_stride,
                                const int32_t* seq_lens, float* out, void* stream);

/* For callers that cannot allocate memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): pkv_decode_attention
 * with no allocation of any kind, device or host.  Same arguments, checks,
 * plan, kernels and result (bit for bit) as pkv_decode_attention; the split
 * plan, the merge arrival counters and the split-K partials live in a
 * library-owned device scratch array of PKV_NOALLOC_SCRATCH_BYTES per GPU
 * (held from library load until the process ends), and the plan is built in
 * fixed host arrays.  Limits: n <= PKV_NOALLOC_MAX_REQUESTS, at most
 * PKV_NOALLOC_MAX_CHUNKS split chunks, n * num_heads <=
 * PKV_NOALLOC_MAX_COUNTERS, and (split chunks) * num_heads * (head_width + 2)
 * <= PKV_NOALLOC_MAX_PARTIAL_FLOATS; beyond them INVALID_ARGUMENT, with
 * nothing enqueued.  Every call on one GPU shares that GPU's scratch (and the
 * host arrays), which keeps the last call's contents: calls must not
 * overlap -- two calls in flight on different streams, or from different
 * threads, race.  A plan above 48 requests or 64 chunks is copied into the
 * scratch from pageable host memory (so the call returns once the copy has
 * read it); PKV_OPT_PROFILING records nothing for this call.  Errors: as
 * pkv_decode_attention, and DEVICE. */
#define PKV_NOALLOC_SCRATCH_BYTES 33554432
#define PKV_NOALLOC_MAX_REQUESTS 4096
#define PKV_NOALLOC_MAX_CHUNKS 32768
#define PKV_NOALLOC_MAX_COUNTERS 262144
#define PKV_NOALLOC_MAX_PARTIAL_FLOATS 7602176
pkv_status pkv_decode_attention_noalloc(pkv_pool* pool, int32_t layer, int32_t n,
                                        const void* q, const int32_t* page_table,
                                        int32_t pt_stride, const int32_t* seq_lens, float* out,
                                        void* stream);

/* Batched prefill on caller page tables: request r appends counts[r] >= 1
 * rows at positions starts[r]..starts[r]+counts[r]-1 (starts[r] >= 0, the
 * last position below pt_stride * page_size), then each of them attends
 * causally, row i over rows 0..starts[r]+i (the pages' token-at-a-time
 * result, computed for the whole chunk; "Incremental Serving", Paged
 * KV-cache layout names this batched prefill).  Rows are packed request
 * after request: q [T,H,d_h], k and v [T,H_kv,d_h] (pool dtype), out
 * [T,H,d_h] float32, T = sum of counts; starts and counts are host arrays.
 * Rows 0..starts[r]-1 must already be in the pages.  Errors:
 * INVALID_ARGUMENT (a range outside the table, a null pointer). */
pkv_status pkv_prefill_attention(pkv_pool* pool, int32_t layer, int32_t n,
                                 const int32_t* page_table, int32_t pt_stride,
                                 const int32_t* starts, const int32_t* counts, const void* q,
                                 const void* k, const void* v, float* out, void* stream);

/* One-call form of pkv_plan_kv_append ("Incremental Serving", Request flow
 * and Paged KV-cache layout): positions is a host array of n row indices;
 * row positions[r] of request r is written, so 0 <= positions[r] <
 * pt_stride * page_size.  Errors: INVALID_ARGUMENT. */
pkv_status pkv_kv_append(pkv_pool* pool, int32_t layer, int32_t n,
                         const int32_t* page_table, int32_t pt_stride,
                         const int32_t* positions, const void* k, const void* v,
                         void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
