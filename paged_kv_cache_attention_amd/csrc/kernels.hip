// gfx950 kernels of libpkv: paged decode attention (the vector-ALU fast and
// generic paths, and the matrix-core path for grouped K/V heads), the
// log-sum-exp merge of split-K partials, the K/V row append, copy-on-write
// page copies and the page-table patch.  Prefill kernels live in
// prefill.hip.
//
// What is computed (learn_llm ch.38 "cached generation", section "Prepare
// every block, then commit every cache together"): for one request, layer and
// head, the newest query q scores each attended row j with dot(q, k_j)/sqrt(d_h),
// a stable softmax turns the scores into weights and the context is the
// weighted sum of the value rows.  Rows are found through the request's page
// table in pages laid out [physical_page, head, page_offset, head_width]
// ("Incremental Serving", section "Paged KV-cache layout").
//
// Arithmetic: float32 throughout (bf16 K/V widen exactly; the grouped-head
// matrix path multiplies bf16 operands exactly and rounds the softmax weights
// to bf16 for the value product, summing the same rounded weights for the
// normaliser).  Scores are kept in
// log2 units (q is pre-multiplied by log2(e)/sqrt(d_h)) so every exponential is
// one v_exp_f32.  Softmax is online: each lane group keeps a running maximum m,
// a running sum l of 2^(s-m) and an accumulator of 2^(s-m) v; groups, waves and
// split-K chunks combine by rescaling to the larger maximum.
#include <cfloat>
#include <cstdint>
#include <initializer_list>
#include <type_traits>

#include <hip/hip_runtime.h>

#include "pkv_internal.h"

namespace pkv {
namespace {

struct bf16_t {
  uint16_t bits;
};

template <typename T>
struct KVTraits;

// Element i of a K/V or q row as float (the generic kernel's scalar reads).
template <>
struct KVTraits<float> {
  __device__ static inline float load1(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
  }
};

template <>
struct KVTraits<bf16_t> {
  __device__ static inline float load1(const void* p, int64_t i) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<const uint16_t*>(p)[i]) << 16);
  }
};

// The work item of this workgroup and request entry r of the plan.  The item
// is uniform across the workgroup; readfirstlane keeps its fields in scalar
// registers whichever source it came from.
__device__ inline WorkItem plan_item(const AttnArgs& a, int idx) {
  WorkItem w = a.num_inline ? a.inline_items[idx] : a.items[idx];
  w.req = __builtin_amdgcn_readfirstlane(w.req);
  w.blk_begin = __builtin_amdgcn_readfirstlane(w.blk_begin);
  w.blk_end = __builtin_amdgcn_readfirstlane(w.blk_end);
  w.split = __builtin_amdgcn_readfirstlane(w.split);
  w.rq.pt_row = __builtin_amdgcn_readfirstlane(w.rq.pt_row);
  w.rq.seq_len = __builtin_amdgcn_readfirstlane(w.rq.seq_len);
  w.rq.nsplit = __builtin_amdgcn_readfirstlane(w.rq.nsplit);
  w.rq.partial_base = __builtin_amdgcn_readfirstlane(w.rq.partial_base);
  return w;
}
__device__ inline WorkItem plan_item(const AttnArgs& a) { return plan_item(a, blockIdx.x); }
__device__ inline ReqEntry plan_req(const AttnArgs& a, int r) {
  return a.num_inline ? a.inline_reqs[r] : a.reqs[r];
}

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Rotate within a 16-lane DPP row (row_ror:N has control 0x120 + N).
template <int CTRL>
__device__ inline float dpp_ror(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row gets the total.
__device__ inline float row16_sum(float x) {
  x += dpp_ror<0x128>(x);
  x += dpp_ror<0x124>(x);
  x += dpp_ror<0x122>(x);
  x += dpp_ror<0x121>(x);
  return x;
}

__device__ inline float wave_max(float x) {
  for (int off = 32; off >= 1; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}

__device__ inline float wave_sum(float x) {
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Read-only view of a page-table row for wave-uniform lookups.  Page tables
// are never written while an attention kernel runs (patches are applied by an
// earlier kernel on the stream), so uniform reads may go through the scalar
// data cache: they then wait on the scalar counter, not on the vector-memory
// counter that tracks K/V loads in flight.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

__device__ inline const_i32_ptr as_const(const int32_t* p) {
  return (const_i32_ptr)(p);
}

// Raw buffer access to one 16-row block: the descriptor (scalar registers)
// holds the block's base address and a 4 KiB range; each load adds a 32-bit
// lane offset.  Offsets past the range would read as zero instead of faulting.
// Word 3 selects 32-bit data format for untyped loads on gfx9-family parts.
constexpr int kBufferWord3 = 0x00020000;

__device__ inline __amdgpu_buffer_rsrc_t block_rsrc(const char* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, bytes, kBufferWord3);
}

// Cache policy of the K/V block loads.  A workgroup that is the only reader
// of its blocks streams them non-temporally (measured on MI355X: 9-12% more
// HBM bandwidth on the large batches, e.g. 6.39 against 5.81 TB/s for 256
// requests of 32 heads); where several workgroups read the same K/V head's
// blocks at about the same time (head_tiles > 1), the later reads hit L2,
// and ordinary loads keep them there (non-temporal loads measured 19% slower
// for one K/V head under 32 query heads).
constexpr int kLoadShared = 0;  // ordinary loads
constexpr int kLoadStream = 2;  // non-temporal ("nt")

template <int CP>
__device__ inline uint4 load_b128(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, CP);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// A lane's share of one K/V row on the fast path: VB bytes (8, 16 or 32) as
// 32-bit words, so that 16 lanes hold a row of 128, 256 or 512 bytes.  Every
// index below is a compile-time constant after unrolling (the words stay in
// registers).
template <int VB>
struct RowVec {
  static constexpr int kWords = VB / 4;
  uint32_t w[kWords];

  __device__ static inline RowVec zero() {
    RowVec v;
#pragma unroll
    for (int k = 0; k < kWords; ++k) v.w[k] = 0;
    return v;
  }
  __device__ static inline RowVec select(bool c, const RowVec& a, const RowVec& b) {
    RowVec v;
#pragma unroll
    for (int k = 0; k < kWords; ++k) v.w[k] = c ? a.w[k] : b.w[k];
    return v;
  }
  // Buffer load at a lane byte offset (16-byte pieces are adjacent) plus a
  // wave-uniform offset `soff`, with cache policy CP.  The buffer's range
  // check is not guaranteed to include `soff`, so a caller that relies on it
  // to drop reads past the range passes the whole offset in `off`.
  template <int CP>
  __device__ static inline RowVec load(__amdgpu_buffer_rsrc_t r, uint32_t off, int soff = 0) {
    RowVec v;
    if constexpr (VB == 8) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, soff, CP);
      v.w[0] = x[0];
      v.w[1] = x[1];
    } else {
#pragma unroll
      for (int h = 0; h < VB / 16; ++h) {
        const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, (int)(off + 16 * h), soff, CP);
#pragma unroll
        for (int k = 0; k < 4; ++k) v.w[4 * h + k] = x[k];
      }
    }
    return v;
  }
  __device__ static inline RowVec load(const char* p) {
    RowVec v;
    if constexpr (VB == 8) {
      const uint2 x = *reinterpret_cast<const uint2*>(p);
      v.w[0] = x.x;
      v.w[1] = x.y;
    } else {
#pragma unroll
      for (int h = 0; h < VB / 16; ++h) {
        const uint4 x = *reinterpret_cast<const uint4*>(p + 16 * h);
        v.w[4 * h] = x.x;
        v.w[4 * h + 1] = x.y;
        v.w[4 * h + 2] = x.z;
        v.w[4 * h + 3] = x.w;
      }
    }
    return v;
  }
  __device__ inline void store(char* p) const {
    if constexpr (VB == 8) {
      *reinterpret_cast<uint2*>(p) = make_uint2(w[0], w[1]);
    } else {
#pragma unroll
      for (int h = 0; h < VB / 16; ++h)
        *reinterpret_cast<uint4*>(p + 16 * h) =
            make_uint4(w[4 * h], w[4 * h + 1], w[4 * h + 2], w[4 * h + 3]);
    }
  }
};

// Elements of a RowVec as float (float32: one per word; bf16: two per word,
// low half first).
template <typename T, int VB>
__device__ inline void unpack_row(const RowVec<VB>& v, float* f) {
#pragma unroll
  for (int k = 0; k < VB / 4; ++k) {
    if constexpr (std::is_same<T, float>::value) {
      f[k] = __uint_as_float(v.w[k]);
    } else {
      f[2 * k] = __uint_as_float(v.w[k] << 16);
      f[2 * k + 1] = __uint_as_float(v.w[k] & 0xFFFF0000u);
    }
  }
}

template <bool COHERENT>
__device__ inline float load_part(const float* p) {
  if constexpr (COHERENT) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return *p;
}

__device__ inline void store_part(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Second pass of split-K for one (request, head), by one whole wave:
// o = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s with M = max_s m_s.
// Splits go 64 at a time, lane j holding split g0 + j: the lanes load their
// (m, l) pair while every lane also issues the loads of its columns for all
// splits of the group, so a group costs one memory round trip.  Weights reach
// the column sums through wave shuffles; a running maximum rescales across
// groups.  The order of every sum is fixed, so the result does not depend on
// which chunk finished last.  COHERENT reads use agent-scope atomic loads
// (partials written by other workgroups inside the same kernel).  MAXC bounds
// the columns per lane: head_width <= 64 * MAXC.
template <int MAXC, bool COHERENT>
__device__ void merge_wave(const AttnArgs& a, int req, const ReqEntry& rq, int h, int lane) {
  constexpr int UNROLL = 8;
  const int D = a.head_width;
  const int H = a.num_heads;
  const int ns = rq.nsplit;
  const int ncol = (D + 63) / 64;
  const int64_t stride = (int64_t)H * (D + 2);
  const float* base = a.partials + ((int64_t)rq.partial_base * H + h) * (D + 2);
  float M = -FLT_MAX, L = 0.f;
  float o[MAXC];
#pragma unroll
  for (int v = 0; v < MAXC; ++v) o[v] = 0.f;
  for (int g0 = 0; g0 < ns; g0 += 64) {
    const int gn = min(64, ns - g0);
    const bool mine = lane < gn;
    const float* ps = base + (int64_t)(g0 + (mine ? lane : 0)) * stride;
    const float m_s = mine ? load_part<COHERENT>(ps) : -FLT_MAX;
    const float l_s = mine ? load_part<COHERENT>(ps + 1) : 0.f;
    const float gm = wave_max(m_s);
    const float newM = fmaxf(M, gm);
    const float scale = fast_exp2(M - newM);
    M = newM;
    const float w = mine ? fast_exp2(m_s - M) : 0.f;
    L = fmaf(L, scale, wave_sum(l_s * w));
#pragma unroll
    for (int v = 0; v < MAXC; ++v) {
      if (v < ncol) {
        const int d = lane + 64 * v;
        const float* col = base + (int64_t)g0 * stride + 2 + (d < D ? d : 0);
        float x = o[v] * scale;
        for (int s = 0; s < gn; s += UNROLL) {
          float av[UNROLL];
#pragma unroll
          for (int j = 0; j < UNROLL; ++j)
            av[j] = (s + j < gn) ? load_part<COHERENT>(col + (int64_t)(s + j) * stride) : 0.f;
#pragma unroll
          for (int j = 0; j < UNROLL; ++j) x = fmaf(av[j], __shfl(w, s + j), x);
        }
        o[v] = x;
      }
    }
  }
  const float inv = 1.0f / L;
  float* out = a.out + ((int64_t)req * H + h) * D;
#pragma unroll
  for (int v = 0; v < MAXC; ++v) {
    const int d = lane + 64 * v;
    if (v < ncol && d < D) out[d] = o[v] * inv;
  }
}

// Ends one (chunk, head), called once per chunk by one whole wave.  A request
// with one chunk writes its context; a split request writes a partial
// (m, l, acc).  In kMergeLastArriver mode the chunk that arrives last at the
// (request, head) counter then merges all partials and returns the counter to
// zero for the next launch; in kMergeSeparate mode merge_kernel does that
// afterwards.  Lane-held column e is col0 + e * CSTRIDE, present when own_cols
// and below the head width; the merge holds MCOLS columns per lane
// (head_width <= 64 * MCOLS).
template <int NCOL, int CSTRIDE, int MCOLS>
__device__ inline void finish_chunk(const AttnArgs& a, const WorkItem& it, const ReqEntry& rq,
                                    int h, int lane, bool own_cols, int col0, float m, float l,
                                    const float* acc) {
  const int D = a.head_width;
  const int H = a.num_heads;
  auto has = [&](int e) { return own_cols && col0 + e * CSTRIDE < D; };
  if (rq.nsplit == 1) {
    const float inv = 1.0f / l;
    float* o = a.out + ((int64_t)it.req * H + h) * D + col0;
#pragma unroll
    for (int e = 0; e < NCOL; ++e)
      if (has(e)) o[e * CSTRIDE] = acc[e] * inv;
    return;
  }
  float* part = a.partials + ((int64_t)(rq.partial_base + it.split) * H + h) * (D + 2);
  if (a.merge_mode == kMergeSeparate) {
#pragma unroll
    for (int e = 0; e < NCOL; ++e)
      if (has(e)) part[2 + col0 + e * CSTRIDE] = acc[e];
    if (lane == 0) {
      part[0] = m;
      part[1] = l;
    }
    return;
  }
  // Last-arriver merge.  Agent-scope stores write through to the
  // device-coherent level; waiting for every outstanding memory operation
  // orders them before the counter increment that publishes them.  The last
  // arriver reads with agent-scope loads, which are served from that level.
#pragma unroll
  for (int e = 0; e < NCOL; ++e)
    if (has(e)) store_part(part + 2 + col0 + e * CSTRIDE, acc[e]);
  if (lane == 0) {
    store_part(part, m);
    store_part(part + 1, l);
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  int* counter = a.merge_count + (int64_t)it.req * H + h;
  int prev = 0;
  if (lane == 0) prev = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  prev = __shfl(prev, 0);
  if (prev != rq.nsplit - 1) return;
  if (lane == 0) (void)__hip_atomic_exchange(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  merge_wave<MCOLS, true>(a, it.req, rq, h, lane);
}

// Work item, K/V head and head tile of a workgroup.  The 1-D grid holds one
// workgroup per (item, K/V head, tile), where `tiles` workgroups share the
// query heads of a K/V head.  Consecutive (item, K/V head) units walk the K/V
// heads of one item before the next item, so the plan's longest-first item
// order holds across the whole grid and the short chunks are dispatched last
// (a 2-D grid would repeat the whole item order once per K/V head).  The
// tiles of one unit sit 8 workgroup IDs apart: workgroups are dealt to the 8
// XCDs round-robin, so they share an XCD, start together and read the same
// K/V blocks at about the same time, and the later reads can hit that XCD's
// L2.  Bijective: each group of up to 8 units takes 8 x tiles consecutive IDs.
struct GridUnit {
  int item, kvh, tile;
};
__device__ inline GridUnit grid_unit(const AttnArgs& a) {
  const int tiles = a.head_tiles;
  const int id = blockIdx.x;
  int u = id, tile = 0;
  if (tiles > 1) {
    const int n = gridDim.x / tiles;
    const int span = 8 * tiles;
    const int q = id / span, r = id - q * span;
    const int m = min(8, n - 8 * q);
    u = 8 * q + r % m;
    tile = r / m;
  }
  return {u / a.num_kv_heads, u % a.num_kv_heads, tile};
}

// ---------------------------------------------------------------------------
// Fast path: rows of 128, 256 or 512 bytes (bf16 d_h = 64, 128, 256; f32
// d_h = 32, 64, 128), pages a multiple of 16 rows.  A workgroup of WAVES
// waves serves one (chunk, K/V head) and the G query heads that share that
// K/V head: its waves form WAVES/WPG head groups of HPW query heads each, and
// the WPG waves of a group interleave the chunk's 16-row blocks, so each head
// group loads every K/V byte of the chunk once for its HPW query heads (with
// one head group, once for all G).  Multi-head attention is G = 1 (HPW = 1,
// WPG = WAVES).  A block is one contiguous 4 KiB slab of K and one of V.
// Lane (g, c): row i*4+g of each of the 4 loads, VB = row bytes / 16 bytes at
// column c, so one load instruction reads four whole rows and the 16 lanes of
// a DPP row hold one K/V row (512-byte rows take two 16-byte loads per lane).
// PAD: the head width is narrower than D (rows of a whole number of VB-byte
// lane shares, e.g. bf16 d_h = 96 in D = 128): row bytes come from the
// arguments, and the lanes past a row's end load no q, contribute nothing to
// the row sums and store nothing.  Each 16-lane group keeps its own online-softmax state per
// query head; groups merge in-wave, the waves of a head group in LDS.
template <typename T, int D, int WAVES, int HPW, int WPG, bool PAD, int CP>
__global__ __launch_bounds__(64 * WAVES) void attend_fast_kernel(AttnArgs a) {
  constexpr int VB = D * (int)sizeof(T) / 16;  // bytes of a row per lane
  static_assert(VB == 8 || VB == 16 || VB == 32, "rows of 128, 256 or 512 bytes");
  using Vec = RowVec<VB>;
  constexpr int EPL = VB / (int)sizeof(T);  // elements of a row per lane
  constexpr int LPR = 16;                  // lanes per row (one DPP row)
  constexpr int RPI = 64 / LPR;            // rows per load instruction
  constexpr int NI = kBlockRows / RPI;     // load instructions per block
  constexpr int NG = WAVES / WPG;          // head groups per workgroup
  static_assert(NG * WPG == WAVES, "waves must split evenly into head groups");
  constexpr int G = NG * HPW;              // query heads per K/V head

  // Work item, K/V head kvh and which of head_tiles consecutive shares of G
  // query heads this workgroup serves (one share unless the group exceeds
  // what one workgroup holds or has an odd factor).
  const int tiles = a.head_tiles;
  const GridUnit gu = grid_unit(a);
  const WorkItem it = plan_item(a, gu.item);
  const ReqEntry rq = it.rq;
  const int kvh = gu.kvh;
  const int tile = gu.tile;
  const int lane = threadIdx.x & 63;
  // Wave-uniform: block indices, page-table reads and branches stay scalar, so
  // the page lookups go through the scalar cache and never wait on the
  // vector-memory counter that tracks the K/V loads in flight.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hg = wave / WPG;               // head group of this wave
  const int sub = wave % WPG;              // its place among the group's waves
  const int qh0 = (kvh * tiles + tile) * G + hg * HPW;  // first query head of this wave
  const int g = lane / LPR;
  const int c = lane % LPR;
  const int DW = PAD ? a.head_width : D;            // elements of a row
  const int ROW_BYTES = DW * (int)sizeof(T);
  const bool lane_on = !PAD || c * VB < ROW_BYTES;  // this lane's share lies in the row
  const int t = rq.seq_len;
  const int S = a.page_size;
  const const_i32_ptr pt = as_const(a.page_table + (int64_t)rq.pt_row * a.pt_stride);
  const int64_t kvrow_bytes =
      (((int64_t)it.req * a.num_kv_heads + kvh) * DW) * (int64_t)sizeof(T);
  const int64_t head_off = (int64_t)kvh * a.head_bytes;
  const int last_blk = (t - 1) / kBlockRows;
  const bool fused = a.fuse_append != 0 && it.blk_end > last_blk;

  float qf[HPW][EPL];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    const int64_t qrow_bytes = (((int64_t)it.req * a.num_heads + qh0 + j) * DW) * (int64_t)sizeof(T);
    Vec qv = Vec::zero();
    if (lane_on) qv = Vec::load(static_cast<const char*>(a.q) + qrow_bytes + c * VB);
    unpack_row<T>(qv, qf[j]);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[j][e] *= a.scale_log2e;
  }

  // With the fused append, the wave of each head group that takes the
  // request's last block (the edge wave) substitutes the new row from the
  // inputs there.  It loads that row now and parks it in LDS once the first
  // K/V loads are issued, so no registers hold it through the block loop;
  // head group 0's edge wave of tile 0 also writes it to its page slot.
  const bool edge_wave = fused && sub == (last_blk - it.blk_begin) % WPG;
  __shared__ __align__(16) uint32_t s_new[NG][2][LPR * Vec::kWords];
  Vec knew = Vec::zero(), vnew = Vec::zero();
  if (edge_wave && lane_on) {
    knew = Vec::load(static_cast<const char*>(a.k_new) + kvrow_bytes + c * VB);
    vnew = Vec::load(static_cast<const char*>(a.v_new) + kvrow_bytes + c * VB);
  }
  auto park_new_row = [&]() {
    if (g == 0) {
#pragma unroll
      for (int k = 0; k < Vec::kWords; ++k) {
        s_new[hg][0][c * Vec::kWords + k] = knew.w[k];
        s_new[hg][1][c * Vec::kWords + k] = vnew.w[k];
      }
    }
    if (hg == 0 && tile == 0 && g == 0 && lane_on) {
      const int pos = t - 1;
      const int64_t slot = (int64_t)pt[pos / S] * a.page_bytes + head_off +
                           (int64_t)(pos % S) * ROW_BYTES + c * VB;
      knew.store(a.k_layer + slot);
      vnew.store(a.v_layer + slot);
    }
  };

  // Physical page of a wave-uniform block index (clamped into the request's
  // blocks so a look-ahead read past the end stays inside the table).
  auto page_of = [&](int b) -> int32_t {
    b = min(b, last_blk);
    return pt[(b * kBlockRows) / S];
  };
  // Lane byte offsets inside a 16-row block: the block base is wave-uniform
  // (scalar registers) and each load adds an unsigned 32-bit lane offset.
  // Whole rows stay inside the block, so load i passes its i * RPI rows as a
  // scalar offset and one register serves all loads; padded rows read past
  // the row into bytes the range check must drop at the block's end, so each
  // load keeps its whole offset in a register.
  uint32_t lane_off[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) lane_off[i] = (uint32_t)((i * RPI + g) * ROW_BYTES + c * VB);
  auto load_block = [&](int b, int32_t page, Vec* kk, Vec* vv) {
    const int row0 = b * kBlockRows;
    const int64_t base = (int64_t)page * a.page_bytes + head_off + (int64_t)(row0 % S) * ROW_BYTES;
    const auto rk = block_rsrc(a.k_layer + base, kBlockRows * ROW_BYTES);
    const auto rv = block_rsrc(a.v_layer + base, kBlockRows * ROW_BYTES);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      if constexpr (PAD) {
        kk[i] = Vec::template load<CP>(rk, lane_off[i]);
        vv[i] = Vec::template load<CP>(rv, lane_off[i]);
      } else {
        kk[i] = Vec::template load<CP>(rk, lane_off[0], i * RPI * ROW_BYTES);
        vv[i] = Vec::template load<CP>(rv, lane_off[0], i * RPI * ROW_BYTES);
      }
    }
  };

  float m[HPW], l[HPW];
  float acc[HPW][EPL];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    m[j] = -FLT_MAX;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[j][e] = 0.f;
  }

  // EDGE is a compile-time tag: the masked variant exists only as its own
  // code path, entered by a scalar branch for the request's last block.
  auto step = [&](int b, Vec* kk, Vec* vv, auto edge_tag) {
    constexpr bool edge = decltype(edge_tag)::value;
    bool valid[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) valid[i] = true;
    if constexpr (edge) {
      // The request's last block: rows >= t are masked (their bytes may be
      // anything), and with a fused append row t-1 comes from k_new/v_new
      // (parked in LDS by this wave).
      Vec k_row = Vec::zero(), v_row = Vec::zero();
      if (fused) {
#pragma unroll
        for (int k = 0; k < Vec::kWords; ++k) {
          k_row.w[k] = s_new[hg][0][c * Vec::kWords + k];
          v_row.w[k] = s_new[hg][1][c * Vec::kWords + k];
        }
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int row = b * kBlockRows + i * RPI + g;
        const bool is_new = fused && row == t - 1;
        valid[i] = row < t;
        kk[i] = Vec::select(is_new, k_row, kk[i]);
        vv[i] = Vec::select(valid[i], Vec::select(is_new, v_row, vv[i]), Vec::zero());
      }
    }
    float s[HPW][NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float kf[EPL];
      unpack_row<T>(kk[i], kf);
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        float d = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) d = fmaf(qf[j][e], kf[e], d);
        if constexpr (PAD) d = lane_on ? d : 0.f;  // bytes past the row may be anything
        s[j][i] = row16_sum(d);
        if constexpr (edge) {
          if (!valid[i]) s[j][i] = -INFINITY;
        }
      }
    }
    float p[HPW][NI];
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      float mb = s[j][0];
#pragma unroll
      for (int i = 1; i < NI; ++i) mb = fmaxf(mb, s[j][i]);
      const float mn = fmaxf(m[j], mb);
      const float alpha = fast_exp2(m[j] - mn);
      float ps = 0.f;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        p[j][i] = fast_exp2(s[j][i] - mn);
        ps += p[j][i];
      }
      l[j] = fmaf(l[j], alpha, ps);
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[j][e] *= alpha;
      m[j] = mn;
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float vf[EPL];
      unpack_row<T>(vv[i], vf);
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[j][e] = fmaf(p[j][i], vf[e], acc[j][e]);
      }
    }
  };

  // Software pipeline over this wave's blocks first, first+WPG, ..., wave_last:
  // the K/V loads of the next block are issued before the current block is
  // computed, and the page ID of the block after that is read one step
  // ahead (its index clamped to wave_last, so the read stays inside the
  // table).  The wave's final block issues no look-ahead load: with chunks
  // of a few blocks per wave, a clamped reload of the final block would add
  // a third or half again to the wave's load requests (measured 1-2% on the
  // launch).  Only a wave's final block can be the request's last block (the
  // masked "edge" step).
  {
    const int end = it.blk_end;
    const int first = it.blk_begin + sub;
    if (first < end) {
      const int wave_last = first + ((end - 1 - first) / WPG) * WPG;
      Vec ka[NI], va[NI], kb[NI], vb[NI];
      load_block(first, page_of(first), ka, va);
      if (edge_wave) park_new_row();
      int32_t p_next = page_of(min(first + WPG, wave_last));
      for (int b = first;; b += 2 * WPG) {
        const int b1 = b + WPG;
        if (b1 <= wave_last) load_block(b1, p_next, kb, vb);
        p_next = page_of(min(b + 2 * WPG, wave_last));
        if (b == last_blk)
          step(b, ka, va, std::true_type{});
        else
          step(b, ka, va, std::false_type{});
        if (b1 > wave_last) break;
        const int b2 = b + 2 * WPG;
        if (b2 <= wave_last) load_block(b2, p_next, ka, va);
        p_next = page_of(min(b + 3 * WPG, wave_last));
        if (b1 == last_blk)
          step(b1, kb, vb, std::true_type{});
        else
          step(b1, kb, vb, std::false_type{});
        if (b2 > wave_last) break;
      }
    }
  }

  // Merge the four 16-lane groups of the wave (lanes differing in bits 4, 5).
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float mo = __shfl_xor(m[j], off);
      const float lo = __shfl_xor(l[j], off);
      const float mx = fmaxf(m[j], mo);
      const float wa = fast_exp2(m[j] - mx), wb = fast_exp2(mo - mx);
      l[j] = l[j] * wa + lo * wb;
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        const float ao = __shfl_xor(acc[j][e], off);
        acc[j][e] = acc[j][e] * wa + ao * wb;
      }
      m[j] = mx;
    }
  }

  // Merge the waves of each head group through LDS; the group's first wave
  // finishes its HPW query heads.
  __shared__ float s_m[WAVES][HPW], s_l[WAVES][HPW];
  __shared__ float s_acc[WAVES][HPW][D];
  if (lane < LPR) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
#pragma unroll
      for (int e = 0; e < EPL; ++e) s_acc[wave][j][c * EPL + e] = acc[j][e];
      if (lane == 0) {
        s_m[wave][j] = m[j];
        s_l[wave][j] = l[j];
      }
    }
  }
  __syncthreads();
  if (sub == 0) {
    const int w0 = hg * WPG;
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      float mx = s_m[w0][j];
#pragma unroll
      for (int w = 1; w < WPG; ++w) mx = fmaxf(mx, s_m[w0 + w][j]);
      float wt[WPG];
      float lsum = 0.f;
#pragma unroll
      for (int w = 0; w < WPG; ++w) {
        wt[w] = fast_exp2(s_m[w0 + w][j] - mx);
        lsum = fmaf(s_l[w0 + w][j], wt[w], lsum);
      }
      float o[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) {
        float x = 0.f;
#pragma unroll
        for (int w = 0; w < WPG; ++w) x = fmaf(s_acc[w0 + w][j][c * EPL + e], wt[w], x);
        o[e] = x;
      }
      finish_chunk<EPL, 1, (D + 63) / 64>(a, it, rq, qh0 + j, lane, lane < LPR, c * EPL, mx, lsum,
                                          o);
    }
  }
}

// ---------------------------------------------------------------------------
// Grouped K/V heads on matrix cores: bf16, d_h = 128, pages of a multiple of
// 16 rows, G = 4, 8 or 16 query heads per workgroup (a share of a larger
// group, see head_share).  With G query heads reading every K/V row, the
// score and value products of a 16-row block are small dense contractions
// (G x 128 by 128 x 16, G x 16 by 16 x 128), so they run on MFMA and the
// vector ALUs keep only the softmax.
//
// Workgroup = W waves (4, or 8 for G = 8 and 16) on one (chunk, K/V head);
// wave w takes blocks w, w+W, ... of the chunk, for all G heads (rows of the
// MFMA tiles; G < 16 pads with repeats of the last head, whose results are
// dropped).  Per block:
//   S^T = K Q^T on 16x16x32 MFMA: A = 16 keys x 32 dims of K, straight from
//     memory (lane l: key l%16, dims 8(l/16)..+7 of a 32-dim slice); B = the
//     G query rows held in registers.  Lane l gets, for head row l%16, the
//     scores of keys 4(l/16)..4(l/16)+3.
//   O^T += V^T P^T on 16x16x16 MFMA: B = P^T is exactly that score layout;
//     A = 16 dims x 16 keys of V^T.  A lane loads keys 4(l/16)..+3 with dims
//     NT (l%16)..+NT-1 (NT = D/16); taking row r of context tile dt to be
//     dim NT r + dt makes its A operand those four keys' dim NT (l%16) + dt,
//     packed from its own registers (no transposition through memory).
//     Lane l accumulates, for head row l%16, dims NT (4(l/16) + j) + dt, so
//     the online-softmax rescale never leaves the lane.
// Waves run independently until the end, then combine through LDS; each wave
// publishes G / W of the heads (finish_heads: the contexts, or split-K
// partials and the last-arriver merge, all heads of a wave at once).
// Reductions across the four 16-lane rows of a wave on the vector ALU
// (gfx950 permlane swaps): with both operands x, permlane16_swap returns rows
// (0,0,2,2) and (1,1,3,3), permlane32_swap the low half twice and the high
// half twice; combining the two gives every lane the result over lanes
// l, l^16 (then l^32), added in the same order in every lane.
__device__ inline float xor16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ inline float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Ends one chunk for NH heads of a wave at once (lanes 0..15 hold columns
// col0..col0+NCOL-1 of each head's context).  Unsplit requests write contexts;
// split ones store all NH partials, order them with one wait, publish them
// with NH counter increments issued back to back, and merge each head whose
// last partial this chunk was -- one memory round trip per step instead of
// one per head.
template <int NH, int NCOL>
__device__ void finish_heads(const AttnArgs& a, const WorkItem& it, const ReqEntry& rq,
                             const int* heads, int lane, int col0, const float* m,
                             const float* l, const float (*o)[NCOL]) {
  const int D = a.head_width;
  const int H = a.num_heads;
  const bool own = lane < 16;
  if (rq.nsplit == 1) {
#pragma unroll
    for (int k = 0; k < NH; ++k) {
      const float inv = 1.0f / l[k];
      float* out = a.out + ((int64_t)it.req * H + heads[k]) * D + col0;
      if (own) {
#pragma unroll
        for (int e = 0; e < NCOL; ++e) out[e] = o[k][e] * inv;
      }
    }
    return;
  }
  const bool coherent = a.merge_mode != kMergeSeparate;
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    float* part = a.partials + ((int64_t)(rq.partial_base + it.split) * H + heads[k]) * (D + 2);
    if (own) {
#pragma unroll
      for (int e = 0; e < NCOL; ++e) {
        if (coherent)
          store_part(part + 2 + col0 + e, o[k][e]);
        else
          part[2 + col0 + e] = o[k][e];
      }
    }
    if (lane == 0) {
      if (coherent) {
        store_part(part, m[k]);
        store_part(part + 1, l[k]);
      } else {
        part[0] = m[k];
        part[1] = l[k];
      }
    }
  }
  if (!coherent) return;
  // As in finish_chunk: agent-scope stores, then wait for every outstanding
  // memory operation before the counter increments that publish them.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_waitcnt(0);
  int prev[NH];
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    prev[k] = 0;
    if (lane == 0)
      prev[k] = __hip_atomic_fetch_add(a.merge_count + (int64_t)it.req * H + heads[k], 1,
                                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    if (__shfl(prev[k], 0) != rq.nsplit - 1) continue;
    if (lane == 0)
      (void)__hip_atomic_exchange(a.merge_count + (int64_t)it.req * H + heads[k], 0,
                                  __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    merge_wave<(16 * NCOL + 63) / 64, true>(a, it.req, rq, heads[k], lane);
  }
}

// The block loop of the grouped matrix-core kernels, for one wave: blocks
// first, first+W, ..., wave_last of the chunk (index j: block first + W j),
// the next block's loads always issued before the current one is computed.
// Only the final block can be the request's last (masked) block, so it is
// peeled off the loop: the loop body is one unmasked step per buffer and the
// context stays in the same registers throughout.  Page IDs come 64 blocks
// at a time in one vector load (lane i: block j0 + i) and are picked out with
// readlane, so issuing a block's loads never waits on a page-table round
// trip.  load_block(b, page, Buf&) issues a block's loads; step(b, Buf&,
// edge_tag) computes it.
template <int W, typename Buf, typename LoadFn, typename StepFn>
__device__ __forceinline__ void group_block_loop(const AttnArgs& a, const WorkItem& it,
                                                 const ReqEntry& rq, int wave, int lane,
                                                 int last_blk, LoadFn& load_block, StepFn& step) {
  const int end = it.blk_end;
  const int first = it.blk_begin + wave;
  if (first >= end) return;
  const int S = a.page_size;
  const int wave_last = first + ((end - 1 - first) / W) * W;
  const int nj = (wave_last - first) / W + 1;
  const bool edge = wave_last == last_blk;
  int32_t pv = 0;
  int j0 = 0;
  auto fetch_pages = [&](int jf) {
    const int bb = min(first + W * (jf + lane), wave_last);
    pv = a.page_table[(int64_t)rq.pt_row * a.pt_stride + (bb * kBlockRows) / S];
    j0 = jf;
    // Complete the load here, so that no later use of pv (after this rare
    // branch rejoins the loop) waits on the K/V loads in flight.
    __builtin_amdgcn_s_waitcnt(0);
  };
  auto page_at = [&](int jj) -> int32_t { return __builtin_amdgcn_readlane(pv, jj - j0); };
  auto blk = [&](int jj) { return first + W * jj; };
  Buf ba, bb;
  fetch_pages(0);
  load_block(first, page_at(0), ba);
  int jc = 0;
  for (; jc + 2 < nj; jc += 2) {  // blocks jc and jc + 1 both precede the final one
    if (jc + 2 - j0 > 63) fetch_pages(jc + 1);
    load_block(blk(jc + 1), page_at(jc + 1), bb);
    step(blk(jc), ba, std::false_type{});
    load_block(blk(jc + 2), page_at(jc + 2), ba);
    step(blk(jc + 1), bb, std::false_type{});
  }
  if (jc + 2 == nj) {
    if (jc + 1 - j0 > 63) fetch_pages(jc + 1);
    load_block(wave_last, page_at(jc + 1), bb);
    step(blk(jc), ba, std::false_type{});
    if (edge)
      step(wave_last, bb, std::true_type{});
    else
      step(wave_last, bb, std::false_type{});
  } else if (edge) {
    step(wave_last, ba, std::true_type{});
  } else {
    step(wave_last, ba, std::false_type{});
  }
}

template <int G, int W, int D, int CP>
__global__ __launch_bounds__(64 * W, D == 256 ? 1 : 8 / W) void attend_group_mfma_kernel(AttnArgs a) {
  constexpr int ROW_BYTES = D * 2;
  static_assert(D == 64 || D == 128 || D == 256, "head widths 64, 128 or 256");
  constexpr int ND = D / 32;     // 32-dim slices of the score product
  constexpr int NT = D / 16;     // 16-dim tiles of the context (and dims per lane of V)
  constexpr int VB = 2 * NT;     // bytes of a V row per lane
  using VVec = RowVec<VB>;
  static_assert(G == 4 || G == 8 || G == 16, "groups of 4, 8 or 16 heads");
  static_assert((W == 4 || W == 8) && G % W == 0, "4 or 8 waves, each publishing G / W heads");
  // Per wave: the final partial context [16 rows][D].
  __shared__ __attribute__((aligned(16))) float s_acc[W][16][D];
  __shared__ float s_m[W][16], s_l[W][16];

  const int tiles = a.head_tiles;  // shares of G query heads per K/V head, as in the fast kernel
  const GridUnit gu = grid_unit(a);
  const WorkItem it = plan_item(a, gu.item);
  const ReqEntry rq = it.rq;
  const int kvh = gu.kvh;
  const int tile = gu.tile;
  const int qbase = (kvh * tiles + tile) * G;  // first query head of this workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 15;
  const int g = lane >> 4;
  const int t = rq.seq_len;
  const int S = a.page_size;
  const const_i32_ptr pt = as_const(a.page_table + (int64_t)rq.pt_row * a.pt_stride);
  const int64_t head_off = (int64_t)kvh * a.head_bytes;
  const int last_blk = (t - 1) / kBlockRows;
  const bool fused = a.fuse_append != 0 && it.blk_end > last_blk;
  const int64_t kvrow = ((int64_t)it.req * a.num_kv_heads + kvh) * ROW_BYTES;

  bf16x8_t qf[ND];
  {
    const int64_t qrow = ((int64_t)it.req * a.num_heads + qbase + min(ql, G - 1)) * ROW_BYTES;
#pragma unroll
    for (int dc = 0; dc < ND; ++dc)
      qf[dc] = __builtin_bit_cast(
          bf16x8_t, *reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) + qrow +
                                                    (4 * dc + g) * 16));
  }
  if (fused && wave == 0 && lane < ROW_BYTES / 16 && tile == 0) {
    const int pos = t - 1;
    const int64_t slot = (int64_t)pt[pos / S] * a.page_bytes + head_off +
                         (int64_t)(pos % S) * ROW_BYTES + lane * 16;
    *reinterpret_cast<uint4*>(a.k_layer + slot) =
        *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + kvrow + lane * 16);
    *reinterpret_cast<uint4*>(a.v_layer + slot) =
        *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + kvrow + lane * 16);
  }

  // K: lane (key ql, dims 32 dc + 8 g); V: lane (keys 4 g + i, dims NT ql..+NT-1).
  struct Buf {
    uint4 k[ND];
    VVec v[4];
  };
  auto load_block = [&](int b, int32_t page, Buf& x) {
    uint4* kk = x.k;
    VVec* vv = x.v;
    const int row0 = b * kBlockRows;
    const int64_t base = (int64_t)page * a.page_bytes + head_off + (int64_t)(row0 % S) * ROW_BYTES;
    const auto rk = block_rsrc(a.k_layer + base, kBlockRows * ROW_BYTES);
    const auto rv = block_rsrc(a.v_layer + base, kBlockRows * ROW_BYTES);
#pragma unroll
    for (int i = 0; i < ND; ++i)
      kk[i] = load_b128<CP>(rk, (uint32_t)(ql * ROW_BYTES + (4 * i + g) * 16));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vv[i] = VVec::template load<CP>(rv, (uint32_t)((4 * g + i) * ROW_BYTES + ql * VB));
  };

  float m = -INFINITY, l = 0.f;
  f32x4_t acc[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int b, Buf& x, auto edge_tag) {
    constexpr bool edge = decltype(edge_tag)::value;
    uint4* kk = x.k;
    VVec* vv = x.v;
    bool valid_k[4] = {true, true, true, true};
    if constexpr (edge) {
      // The request's last block: keys >= t are masked and their V rows
      // zeroed (stale bytes may be anything, NaN and Inf patterns included:
      // a masked score is replaced, never added to); with a fused append,
      // key t-1 comes from the inputs.
      const int row0 = b * kBlockRows;
      if (fused && row0 + ql == t - 1) {
#pragma unroll
        for (int i = 0; i < ND; ++i)
          kk[i] = *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + kvrow +
                                                  (4 * i + g) * 16);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = row0 + 4 * g + i;
        if (fused && key == t - 1)
          vv[i] = VVec::load(static_cast<const char*>(a.v_new) + kvrow + ql * VB);
        if (key >= t) vv[i] = VVec::zero();
        valid_k[i] = key < t;
      }
    }
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dc = 0; dc < ND; ++dc)
      c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, kk[dc]), qf[dc], c,
                                                   0, 0, 0);
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = (!edge || valid_k[j]) ? c[j] : -INFINITY;
    float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    const float cand = xor32_max(xor16_max(mb)) * a.scale_log2e;
    // Lazy rescale: a head's running maximum moves (and its context and sum
    // are rescaled) only when some head of the wave sees a block maximum more
    // than kSlack above its own, so the weights exp2(s - m) stay below
    // 2^kSlack, which float32 sums and bf16 weights carry as well as values
    // below 1.  The branch is wave-uniform and rare after the first block
    // (which always moves m from -inf); the context stays in the matrix
    // accumulators in between.
    constexpr float kSlack = 8.f;
    if (__builtin_expect(__any(cand > m + kSlack), 0)) {
      const float mn = fmaxf(m, cand);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
      m = mn;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) acc[dt] *= alpha;
    }
    // The weights are rounded to bf16 for the value product, and the running
    // sum adds those same rounded weights, so numerator and denominator use
    // one set of weights (the softmax normalises exactly what it mixes).
    typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
    bf16x4_t pb4;
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      pb4[j] = (__bf16)fast_exp2(fmaf(sc[j], a.scale_log2e, -m));
      ps += (float)pb4[j];
    }
    l += xor32_sum(xor16_sum(ps));
    const s16x4_t pb = __builtin_bit_cast(s16x4_t, pb4);
    // Value tile dt, row r is dim NT r + dt, so the A operand of lane (ql, g)
    // -- dim NT ql + dt of keys 4g .. 4g+3 -- is its own V data, packed.
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) {
      const int w = dt >> 1;
      const uint32_t sel = (dt & 1) ? 0x07060302u : 0x05040100u;  // high or low halves
      uint2 x;
      x.x = __builtin_amdgcn_perm(vv[1].w[w], vv[0].w[w], sel);
      x.y = __builtin_amdgcn_perm(vv[3].w[w], vv[2].w[w], sel);
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, x), pb,
                                                          acc[dt], 0, 0, 0);
    }
  };

  group_block_loop<W, Buf>(a, it, rq, wave, lane, last_blk, load_block, step);

  // Combine the waves through LDS (lane (ql, g) holds dims NT (4 g + j) + dt
  // of head ql), then each wave publishes heads wave, wave + W, ...
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) s_acc[wave][ql][NT * (4 * g + j) + dt] = acc[dt][j];
  if (g == 0) {
    s_m[wave][ql] = m;
    s_l[wave][ql] = l;
  }
  __syncthreads();
  constexpr int NH = G / W;
  const int c0 = (lane & 15) * NT;
  int heads[NH];
  float hm[NH], hl[NH], ho[NH][NT];
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    const int r = wave + W * k;
    heads[k] = qbase + r;
    float mx = s_m[0][r];
#pragma unroll
    for (int w = 1; w < W; ++w) mx = fmaxf(mx, s_m[w][r]);
    float wt[W], lsum = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      wt[w] = s_m[w][r] == -INFINITY ? 0.f : fast_exp2(s_m[w][r] - mx);
      lsum = fmaf(s_l[w][r], wt[w], lsum);
    }
#pragma unroll
    for (int e = 0; e < NT; ++e) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) x = fmaf(s_acc[w][r][c0 + e], wt[w], x);
      ho[k][e] = x;
    }
    hm[k] = mx;
    hl[k] = lsum;
  }
  finish_heads<NH, NT>(a, it, rq, heads, lane, c0, hm, hl, ho);
}

// ---------------------------------------------------------------------------
// Grouped K/V heads on matrix cores in float32: d_h = 32, 64 or 128, pages of
// a multiple of 16 rows, G = 4, 8 or 16 query heads per workgroup, W waves
// interleaving the chunk's blocks as in the bf16 kernel.  Both products run
// on v_mfma_f32_16x16x4_f32 (A: lane l holds A[l%16][l/16]; B: B[l/16][l%16];
// C: C[4(l/16)+j][l%16]); since a contraction may visit its index in any
// order, the orders are chosen so that every operand is a lane's own
// contiguous data:
//   S^T = K Q^T, step s (of D/4): k index g <-> dim (D/4) g + s.  Lane
//     (ql, g) holds dims (D/4) g .. +D/4-1 of key ql's K row and of head
//     ql's q row, and gets the scores of keys 4g .. 4g+3 for head ql.
//   O^T += V^T P^T, step s (of 4): k index g <-> key 4g + s, which is the
//     lane's own score element s; output tile t, row r <-> dim (D/16) r + t,
//     so lane (ql, g) holds dims (D/16) ql .. +D/16-1 of V rows 4g + s and
//     accumulates dims (D/16)(4g + j) + t of head ql.
// No LDS staging: K and V go from memory straight into the MFMA operands.
template <int G, int W, int D, int CP>
__global__ __launch_bounds__(64 * W, D == 128 ? 1 : 8 / W) void attend_group_f32_kernel(AttnArgs a) {
  constexpr int ROW_BYTES = D * 4;
  static_assert(D == 32 || D == 64 || D == 128, "head widths 32, 64 or 128");
  constexpr int KD = D / 4;      // score steps, and dims of a K or q row per lane
  constexpr int NT = D / 16;     // context tiles, and dims of a V row per lane
  using KVec = RowVec<KD * 4>;
  using VVec = RowVec<NT * 4>;
  static_assert(G == 4 || G == 8 || G == 16, "groups of 4, 8 or 16 heads");
  static_assert((W == 4 || W == 8) && G % W == 0, "4 or 8 waves, each publishing G / W heads");
  __shared__ __attribute__((aligned(16))) float s_acc[W][16][D];
  __shared__ float s_m[W][16], s_l[W][16];

  const int tiles = a.head_tiles;
  const GridUnit gu = grid_unit(a);
  const WorkItem it = plan_item(a, gu.item);
  const ReqEntry rq = it.rq;
  const int kvh = gu.kvh;
  const int tile = gu.tile;
  const int qbase = (kvh * tiles + tile) * G;  // first query head of this workgroup
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 15;
  const int g = lane >> 4;
  const int t = rq.seq_len;
  const int S = a.page_size;
  const const_i32_ptr pt = as_const(a.page_table + (int64_t)rq.pt_row * a.pt_stride);
  const int64_t head_off = (int64_t)kvh * a.head_bytes;
  const int last_blk = (t - 1) / kBlockRows;
  const bool fused = a.fuse_append != 0 && it.blk_end > last_blk;
  const int64_t kvrow = ((int64_t)it.req * a.num_kv_heads + kvh) * ROW_BYTES;

  float qf[KD];
  {
    const int64_t qrow = ((int64_t)it.req * a.num_heads + qbase + min(ql, G - 1)) * ROW_BYTES;
    const KVec v = KVec::load(static_cast<const char*>(a.q) + qrow + g * KD * 4);
#pragma unroll
    for (int s = 0; s < KD; ++s) qf[s] = __uint_as_float(v.w[s]);
  }
  if (fused && wave == 0 && lane < ROW_BYTES / 16 && tile == 0) {
    const int pos = t - 1;
    const int64_t slot = (int64_t)pt[pos / S] * a.page_bytes + head_off +
                         (int64_t)(pos % S) * ROW_BYTES + lane * 16;
    *reinterpret_cast<uint4*>(a.k_layer + slot) =
        *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + kvrow + lane * 16);
    *reinterpret_cast<uint4*>(a.v_layer + slot) =
        *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + kvrow + lane * 16);
  }

  struct Buf {
    KVec k;       // key ql, dims KD g ..
    VVec v[4];    // keys 4 g + s, dims NT ql ..
  };
  auto load_block = [&](int b, int32_t page, Buf& x) {
    const int row0 = b * kBlockRows;
    const int64_t base = (int64_t)page * a.page_bytes + head_off + (int64_t)(row0 % S) * ROW_BYTES;
    const auto rk = block_rsrc(a.k_layer + base, kBlockRows * ROW_BYTES);
    const auto rv = block_rsrc(a.v_layer + base, kBlockRows * ROW_BYTES);
    x.k = KVec::template load<CP>(rk, (uint32_t)(ql * ROW_BYTES + g * KD * 4));
#pragma unroll
    for (int s = 0; s < 4; ++s)
      x.v[s] = VVec::template load<CP>(rv, (uint32_t)((4 * g + s) * ROW_BYTES + ql * NT * 4));
  };

  float m = -INFINITY, l = 0.f;
  f32x4_t acc[NT];
#pragma unroll
  for (int dt = 0; dt < NT; ++dt) acc[dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto step = [&](int b, Buf& x, auto edge_tag) {
    constexpr bool edge = decltype(edge_tag)::value;
    bool valid_k[4] = {true, true, true, true};
    if constexpr (edge) {
      // The request's last block: keys >= t are masked (their scores
      // replaced, so NaN or Inf bytes in unwritten slots cannot reach the
      // sums) and their V rows zeroed; with a fused append, key t-1 comes
      // from the inputs.
      const int row0 = b * kBlockRows;
      if (fused && row0 + ql == t - 1)
        x.k = KVec::load(static_cast<const char*>(a.k_new) + kvrow + g * KD * 4);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int key = row0 + 4 * g + s;
        if (fused && key == t - 1)
          x.v[s] = VVec::load(static_cast<const char*>(a.v_new) + kvrow + ql * NT * 4);
        if (key >= t) x.v[s] = VVec::zero();
        valid_k[s] = key < t;
      }
    }
    f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KD; ++s)
      c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.k.w[s]), qf[s], c, 0, 0, 0);
    float sc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) sc[j] = (!edge || valid_k[j]) ? c[j] : -INFINITY;
    float mb = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    const float cand = xor32_max(xor16_max(mb)) * a.scale_log2e;
    // Lazy rescale, as in the bf16 kernel.
    constexpr float kSlack = 8.f;
    if (__builtin_expect(__any(cand > m + kSlack), 0)) {
      const float mn = fmaxf(m, cand);
      const float alpha = fast_exp2(m - mn);
      l *= alpha;
      m = mn;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) acc[dt] *= alpha;
    }
    float p[4], ps = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      p[j] = fast_exp2(fmaf(sc[j], a.scale_log2e, -m));
      ps += p[j];
    }
    l += xor32_sum(xor16_sum(ps));
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        acc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(x.v[s].w[dt]), p[s],
                                                       acc[dt], 0, 0, 0);
  };

  group_block_loop<W, Buf>(a, it, rq, wave, lane, last_blk, load_block, step);

  // Combine the waves through LDS (lane (ql, g) holds dims NT (4 g + j) + dt
  // of head ql), then each wave publishes heads wave, wave + W, ...
#pragma unroll
  for (int dt = 0; dt < NT; ++dt)
#pragma unroll
    for (int j = 0; j < 4; ++j) s_acc[wave][ql][NT * (4 * g + j) + dt] = acc[dt][j];
  if (g == 0) {
    s_m[wave][ql] = m;
    s_l[wave][ql] = l;
  }
  __syncthreads();
  constexpr int NH = G / W;
  const int c0 = (lane & 15) * NT;
  int heads[NH];
  float hm[NH], hl[NH], ho[NH][NT];
#pragma unroll
  for (int k = 0; k < NH; ++k) {
    const int r = wave + W * k;
    heads[k] = qbase + r;
    float mx = s_m[0][r];
#pragma unroll
    for (int w = 1; w < W; ++w) mx = fmaxf(mx, s_m[w][r]);
    float wt[W], lsum = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
      wt[w] = s_m[w][r] == -INFINITY ? 0.f : fast_exp2(s_m[w][r] - mx);
      lsum = fmaf(s_l[w][r], wt[w], lsum);
    }
#pragma unroll
    for (int e = 0; e < NT; ++e) {
      float x = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) x = fmaf(s_acc[w][r][c0 + e], wt[w], x);
      ho[k][e] = x;
    }
    hm[k] = mx;
    hl[k] = lsum;
  }
  finish_heads<NH, NT>(a, it, rq, heads, lane, c0, hm, hl, ho);
}

// ---------------------------------------------------------------------------
// Generic path: any head width up to 1024, any page size, any query-head
// group size.  One wave per (chunk, query head), reading its group's K/V
// head.  Tiles of 64 rows: lane j scores row j of the tile, the wave
// reduces max and sum, then lanes sweep head-width columns accumulating the
// weighted value rows.
template <typename T>
__global__ __launch_bounds__(64) void attend_generic_kernel(AttnArgs a) {
  using KV = KVTraits<T>;
  constexpr int MAXV = 16;  // columns per lane: head_width <= 64 * MAXV
  extern __shared__ float smem[];
  const int D = a.head_width;
  float* qs = smem;         // [D]
  float* ps = smem + D;     // [64]

  const WorkItem it = plan_item(a);
  const ReqEntry rq = it.rq;
  const int h = blockIdx.y;                                  // query head
  const int group = a.num_heads / a.num_kv_heads;
  const int kvh = h / group;                                 // its K/V head
  const int lane = threadIdx.x;
  const int t = rq.seq_len;
  const int S = a.page_size;
  const int32_t* pt = a.page_table + (int64_t)rq.pt_row * a.pt_stride;
  const int64_t qrow = ((int64_t)it.req * a.num_heads + h) * D;
  const int64_t kvrow = ((int64_t)it.req * a.num_kv_heads + kvh) * D;
  const int64_t head_off = (int64_t)kvh * a.head_bytes;
  const int64_t row_bytes = (int64_t)D * sizeof(T);
  const int row_begin = it.blk_begin * kBlockRows;
  const int row_end = min(it.blk_end * kBlockRows, t);
  const bool fused = a.fuse_append != 0 && row_end == t;

  for (int d = lane; d < D; d += 64) qs[d] = KV::load1(a.q, qrow + d) * a.scale_log2e;
  if (fused && h % group == 0) {
    // One query head of the group writes the new K/V row.
    const int pos = t - 1;
    const int64_t slot = (int64_t)pt[pos / S] * a.page_bytes + head_off + (int64_t)(pos % S) * row_bytes;
    for (int d = lane; d < D; d += 64) {
      reinterpret_cast<T*>(a.k_layer + slot)[d] = static_cast<const T*>(a.k_new)[kvrow + d];
      reinterpret_cast<T*>(a.v_layer + slot)[d] = static_cast<const T*>(a.v_new)[kvrow + d];
    }
  }
  __syncthreads();

  auto row_ptr = [&](const char* layer, int row) -> const void* {
    return layer + (int64_t)pt[row / S] * a.page_bytes + head_off + (int64_t)(row % S) * row_bytes;
  };

  float m = -FLT_MAX, l = 0.f;
  float acc[MAXV];
#pragma unroll
  for (int v = 0; v < MAXV; ++v) acc[v] = 0.f;

  for (int row0 = row_begin; row0 < row_end; row0 += 64) {
    const int row = row0 + lane;
    const bool valid = row < row_end;
    float s = -INFINITY;
    if (valid) {
      const bool is_new = fused && row == t - 1;
      const void* kp = is_new ? static_cast<const void*>(static_cast<const T*>(a.k_new) + kvrow)
                              : row_ptr(a.k_layer, row);
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qs[d], KV::load1(kp, d), dot);
      s = dot;
    }
    const float mn = fmaxf(m, wave_max(s));
    const float alpha = fast_exp2(m - mn);
    const float p = valid ? fast_exp2(s - mn) : 0.f;
    l = l * alpha + wave_sum(p);
    m = mn;
    ps[lane] = p;
    __syncthreads();
#pragma unroll
    for (int v = 0; v < MAXV; ++v) acc[v] *= alpha;
    const int nrows = min(64, row_end - row0);
    for (int j = 0; j < nrows; ++j) {
      const int rj = row0 + j;
      const void* vp = (fused && rj == t - 1)
                           ? static_cast<const void*>(static_cast<const T*>(a.v_new) + kvrow)
                           : row_ptr(a.v_layer, rj);
      const float pj = ps[j];
#pragma unroll
      for (int v = 0; v < MAXV; ++v) {
        const int d = lane + 64 * v;
        if (d < D) acc[v] = fmaf(pj, KV::load1(vp, d), acc[v]);
      }
    }
    __syncthreads();
  }

  // This lane holds columns lane, lane + 64, ...
  finish_chunk<MAXV, 64, MAXV>(a, it, rq, h, lane, true, lane, m, l, acc);
}

// ---------------------------------------------------------------------------
// Second pass of kMergeSeparate: one wave per (split request, head); lanes
// hold columns lane, lane + 64, ...
__global__ __launch_bounds__(64) void merge_kernel(AttnArgs a) {
  const int req = a.merge_reqs[blockIdx.x];
  const ReqEntry rq = a.reqs[req];
  merge_wave<16, false>(a, req, rq, blockIdx.y, threadIdx.x);
}

// ---------------------------------------------------------------------------
// Append: row t-1 of request r, K/V head h <- k[r][h][:], v[r][h][:] (bit copy).
template <typename W>
__global__ __launch_bounds__(64) void kv_append_kernel(AttnArgs a) {
  const int r = blockIdx.x;
  const int h = blockIdx.y;
  const ReqEntry rq = plan_req(a, r);
  const int pos = rq.seq_len - 1;
  const int S = a.page_size;
  const int D = a.head_width;
  const int32_t* pt = a.page_table + (int64_t)rq.pt_row * a.pt_stride;
  const int64_t dst = (int64_t)pt[pos / S] * a.page_bytes + (int64_t)h * a.head_bytes +
                      (int64_t)(pos % S) * D * (int64_t)sizeof(W);
  const int64_t src = ((int64_t)r * a.num_kv_heads + h) * D;
  W* kd = reinterpret_cast<W*>(a.k_layer + dst);
  W* vd = reinterpret_cast<W*>(a.v_layer + dst);
  const W* ks = static_cast<const W*>(a.k_new) + src;
  const W* vs = static_cast<const W*>(a.v_new) + src;
  for (int d = threadIdx.x; d < D; d += 64) {
    kd[d] = ks[d];
    vd[d] = vs[d];
  }
}

// One workgroup per (copy, layer, K or V): the page's bytes of that layer.
// Pages of a multiple of 16 bytes move 16 bytes per lane, others 2.
__global__ __launch_bounds__(256) void page_copy_kernel(char* k_storage, char* v_storage,
                                                        int64_t layer_bytes, int64_t page_bytes,
                                                        CopyBatch b) {
  char* base = (blockIdx.z == 0 ? k_storage : v_storage) + (int64_t)blockIdx.y * layer_bytes;
  const char* src = base + (int64_t)b.src[blockIdx.x] * page_bytes;
  char* dst = base + (int64_t)b.dst[blockIdx.x] * page_bytes;
  if (page_bytes % 16 == 0) {
    for (int64_t i = threadIdx.x; i < page_bytes / 16; i += 256)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  } else {
    for (int64_t i = threadIdx.x; i < page_bytes / 2; i += 256)
      reinterpret_cast<uint16_t*>(dst)[i] = reinterpret_cast<const uint16_t*>(src)[i];
  }
}

__global__ __launch_bounds__(256) void patch_kernel(int32_t* arena, PatchBatch b) {
  const int i = threadIdx.x;
  if (i < b.count) arena[b.offset[i]] = b.value[i];
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* p, int64_t count) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count; i += (int64_t)gridDim.x * 256)
    p[i] = 0;
}

// Streams the K/V blocks non-temporally when each is read by one
// workgroup only (see kLoadStream).
template <typename T, int D, int WAVES, int HPW, int WPG, bool PAD = false>
hipError_t launch_fast_shape(const AttnArgs& a, int num_items, hipStream_t stream) {
  const dim3 grid(num_items * a.head_tiles * a.num_kv_heads), block(64 * WAVES);
  if (a.head_tiles == 1)
    hipLaunchKernelGGL((attend_fast_kernel<T, D, WAVES, HPW, WPG, PAD, kLoadStream>), grid, block,
                       0, stream, a);
  else
    hipLaunchKernelGGL((attend_fast_kernel<T, D, WAVES, HPW, WPG, PAD, kLoadShared>), grid, block,
                       0, stream, a);
  return hipGetLastError();
}

// The grouped matrix-core kernels, with the load policy by head tiles.
template <int G, int W, int D>
void launch_group_mfma_shape(const AttnArgs& a, dim3 grid, hipStream_t stream) {
  if (a.head_tiles == 1)
    hipLaunchKernelGGL((attend_group_mfma_kernel<G, W, D, kLoadStream>), grid, dim3(64 * W), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((attend_group_mfma_kernel<G, W, D, kLoadShared>), grid, dim3(64 * W), 0,
                       stream, a);
}
template <int G, int W, int D>
void launch_group_f32_shape(const AttnArgs& a, dim3 grid, hipStream_t stream) {
  if (a.head_tiles == 1)
    hipLaunchKernelGGL((attend_group_f32_kernel<G, W, D, kLoadStream>), grid, dim3(64 * W), 0,
                       stream, a);
  else
    hipLaunchKernelGGL((attend_group_f32_kernel<G, W, D, kLoadShared>), grid, dim3(64 * W), 0,
                       stream, a);
}

// Workgroup shape by query heads per workgroup (1, 2, 4, 8, 16).  Up to four
// heads per wave, every wave of the workgroup carries the whole share, so
// each K/V block is loaded once and serves all of its query heads; the waves
// split the chunk's blocks.  Shares of 8 and 16 split over 2 and 4 head groups
// of four (each block loaded by 2 or 4 waves): more heads per wave would
// exceed the register file.  512-byte rows hold twice the registers per
// block, so there a wave carries at most two heads and shares stop at 8.
// One head per workgroup runs on 4, 8 or (d_h <= 64) 16 waves.
template <typename T, int D>
hipError_t launch_fast(const AttnArgs& a, int share, int num_items, hipStream_t stream) {
  constexpr bool wide = D * sizeof(T) == 512;
  switch (share) {
    case 1:
      if constexpr (D <= 64)
        if (a.waves == 16) return launch_fast_shape<T, D, 16, 1, 16>(a, num_items, stream);
      return a.waves >= 8 ? launch_fast_shape<T, D, 8, 1, 8>(a, num_items, stream)
                          : launch_fast_shape<T, D, 4, 1, 4>(a, num_items, stream);
    case 2:
      return launch_fast_shape<T, D, 4, 2, 4>(a, num_items, stream);
    case 4:
      if constexpr (wide) return launch_fast_shape<T, D, 4, 2, 2>(a, num_items, stream);
      else return launch_fast_shape<T, D, 4, 4, 4>(a, num_items, stream);
    case 8:
      if constexpr (wide) return launch_fast_shape<T, D, 4, 2, 1>(a, num_items, stream);
      else return launch_fast_shape<T, D, 4, 4, 2>(a, num_items, stream);
    default:
      if constexpr (wide) return hipErrorInvalidValue;  // shares of wide rows stop at 8
      else return launch_fast_shape<T, D, 4, 4, 1>(a, num_items, stream);
  }
}

// Row bytes of the fast path's widths (0 when the width has no fast shape).
static int fast_row_bytes(int dtype, int head_width) {
  if (dtype == kDtypeF32 && (head_width == 32 || head_width == 64 || head_width == 128))
    return head_width * 4;
  if (dtype == kDtypeBF16 && (head_width == 64 || head_width == 128 || head_width == 256))
    return head_width * 2;
  return 0;
}

// For a width without its own fast shape: the fast width D whose rows hold
// it, when its row is a whole number of that width's lane shares (0 if none).
static int padded_width(int dtype, int head_width) {
  const int elt = dtype == kDtypeF32 ? 4 : 2;
  const int rb = head_width * elt;
  for (int vb : {8, 16, 32})
    if (rb <= 16 * vb) return rb % vb == 0 && rb > 8 * vb ? 16 * vb / elt : 0;
  return 0;
}

// Padded widths run shares of one or two query heads (larger groups as
// several workgroups of two).
template <typename T, int D>
hipError_t launch_fast_padded(const AttnArgs& a, int share, int num_items, hipStream_t stream) {
  if (share == 2) return launch_fast_shape<T, D, 4, 2, 4, true>(a, num_items, stream);
  return a.waves >= 8 ? launch_fast_shape<T, D, 8, 1, 8, true>(a, num_items, stream)
                      : launch_fast_shape<T, D, 4, 1, 4, true>(a, num_items, stream);
}

template <typename T>
hipError_t launch_generic(const AttnArgs& a, int num_items, hipStream_t stream) {
  const size_t lds = (size_t)(a.head_width + 64) * sizeof(float);
  hipLaunchKernelGGL((attend_generic_kernel<T>), dim3(num_items, a.num_heads), dim3(64), lds,
                     stream, a);
  return hipGetLastError();
}

}  // namespace

// Query heads per workgroup for a group of `group` query heads per K/V head:
// the largest of `shares` (descending) that divides it.  A group above the
// largest share, or with an odd factor, takes several workgroups per K/V
// head; they read the same K/V blocks (the later reads mostly hit in cache).
static int head_share(int group, std::initializer_list<int> shares) {
  for (int s : shares)
    if (group % s == 0) return s;
  return 0;
}

bool group_mfma_supported(int dtype, int head_width, int page_size, int group) {
  if (page_size % kBlockRows != 0 || group % 4 != 0) return false;
  if (dtype == kDtypeBF16) return head_width == 64 || head_width == 128 || head_width == 256;
  if (dtype == kDtypeF32) return head_width == 32 || head_width == 64 || head_width == 128;
  return false;
}

// The float32 grouped matrix-core kernel: shares of 16, 8 or 4 heads, eight
// waves for shares of 8 and 16 unless PKV_OPT_WAVES asks for four.
template <int D>
hipError_t launch_group_f32(const AttnArgs& a, int share, dim3 grid, hipStream_t stream) {
  const bool eight = a.waves != 4;
  switch (share) {
    case 4:
      launch_group_f32_shape<4, 4, D>(a, grid, stream);
      break;
    case 8:
      if (eight)
        launch_group_f32_shape<8, 8, D>(a, grid, stream);
      else
        launch_group_f32_shape<8, 4, D>(a, grid, stream);
      break;
    default:
      if (eight)
        launch_group_f32_shape<16, 8, D>(a, grid, stream);
      else
        launch_group_f32_shape<16, 4, D>(a, grid, stream);
      break;
  }
  return hipGetLastError();
}

// The grouped matrix-core kernel for one head width: 16, 8 or 4 query heads
// per workgroup; eight waves for shares of 8 and 16 unless PKV_OPT_WAVES asks
// for four (d_h = 256 stays at four: eight waves' LDS would leave one
// workgroup per CU).
template <int D>
hipError_t launch_group(const AttnArgs& a, int share, dim3 grid, hipStream_t stream) {
  const bool eight = a.waves != 4 && D != 256;
  switch (share) {
    case 4:
      launch_group_mfma_shape<4, 4, D>(a, grid, stream);
      break;
    case 8:
      if constexpr (D != 256) {
        if (eight) {
          launch_group_mfma_shape<8, 8, D>(a, grid, stream);
          break;
        }
      }
      launch_group_mfma_shape<8, 4, D>(a, grid, stream);
      break;
    default:
      if constexpr (D != 256) {
        if (eight) {
          launch_group_mfma_shape<16, 8, D>(a, grid, stream);
          break;
        }
      }
      launch_group_mfma_shape<16, 4, D>(a, grid, stream);
      break;
  }
  return hipGetLastError();
}

bool fast_width_native(int dtype, int head_width) { return fast_row_bytes(dtype, head_width) != 0; }

hipError_t launch_zero_i32(int32_t* p, int64_t count, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  const int64_t blocks = (count + 255) / 256;
  hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)(blocks < 1024 ? blocks : 1024)), dim3(256), 0,
                     stream, p, count);
  return hipGetLastError();
}

bool fast_path_supported(int dtype, int head_width, int page_size, int group) {
  if (page_size % kBlockRows != 0 || group < 1) return false;
  return fast_row_bytes(dtype, head_width) != 0 || padded_width(dtype, head_width) != 0;
}

hipError_t launch_attention(const AttnArgs& args, int dtype, int num_items, hipStream_t stream,
                            KernelPath* path_out) {
  AttnArgs a = args;
  const int group = a.num_heads / a.num_kv_heads;
  if (group_mfma_supported(dtype, a.head_width, a.page_size, group)) {
    if (path_out) *path_out = KernelPath::kFast;
    const int share = head_share(group, {16, 8, 4});
    a.head_tiles = group / share;
    const dim3 grid(num_items * a.head_tiles * a.num_kv_heads);
    if (dtype == kDtypeF32) {
      switch (a.head_width) {
        case 32: return launch_group_f32<32>(a, share, grid, stream);
        case 64: return launch_group_f32<64>(a, share, grid, stream);
        default: return launch_group_f32<128>(a, share, grid, stream);
      }
    }
    switch (a.head_width) {
      case 64: return launch_group<64>(a, share, grid, stream);
      case 128: return launch_group<128>(a, share, grid, stream);
      default: return launch_group<256>(a, share, grid, stream);
    }
  }
  const bool fast = fast_path_supported(dtype, a.head_width, a.page_size, group);
  if (path_out) *path_out = fast ? KernelPath::kFast : KernelPath::kGeneric;
  if (fast && fast_row_bytes(dtype, a.head_width) == 0) {
    const int share = head_share(group, {2, 1});
    a.head_tiles = group / share;
    const int dp = padded_width(dtype, a.head_width);
    if (dtype == kDtypeF32) {
      switch (dp) {
        case 32: return launch_fast_padded<float, 32>(a, share, num_items, stream);
        case 64: return launch_fast_padded<float, 64>(a, share, num_items, stream);
        default: return launch_fast_padded<float, 128>(a, share, num_items, stream);
      }
    }
    switch (dp) {
      case 64: return launch_fast_padded<bf16_t, 64>(a, share, num_items, stream);
      case 128: return launch_fast_padded<bf16_t, 128>(a, share, num_items, stream);
      default: return launch_fast_padded<bf16_t, 256>(a, share, num_items, stream);
    }
  }
  if (fast) {
    const int share = fast_row_bytes(dtype, a.head_width) == 512
                          ? head_share(group, {8, 4, 2, 1})
                          : head_share(group, {16, 8, 4, 2, 1});
    a.head_tiles = group / share;
    if (dtype == kDtypeF32) {
      switch (a.head_width) {
        case 32: return launch_fast<float, 32>(a, share, num_items, stream);
        case 64: return launch_fast<float, 64>(a, share, num_items, stream);
        default: return launch_fast<float, 128>(a, share, num_items, stream);
      }
    }
    switch (a.head_width) {
      case 64: return launch_fast<bf16_t, 64>(a, share, num_items, stream);
      case 128: return launch_fast<bf16_t, 128>(a, share, num_items, stream);
      default: return launch_fast<bf16_t, 256>(a, share, num_items, stream);
    }
  }
  a.head_tiles = 1;
  return dtype == kDtypeF32 ? launch_generic<float>(a, num_items, stream)
                            : launch_generic<bf16_t>(a, num_items, stream);
}

hipError_t launch_merge(const AttnArgs& a, int num_split_reqs, hipStream_t stream) {
  hipLaunchKernelGGL(merge_kernel, dim3(num_split_reqs, a.num_heads), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_kv_append(const AttnArgs& a, int dtype, int num_reqs, hipStream_t stream) {
  if (dtype == kDtypeF32) {
    hipLaunchKernelGGL(kv_append_kernel<uint32_t>, dim3(num_reqs, a.num_kv_heads), dim3(64), 0,
                       stream, a);
  } else {
    hipLaunchKernelGGL(kv_append_kernel<uint16_t>, dim3(num_reqs, a.num_kv_heads), dim3(64), 0,
                       stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_page_copies(char* k_storage, char* v_storage, int64_t layer_bytes,
                              int64_t page_bytes, int32_t num_layers, const CopyBatch& b,
                              hipStream_t stream) {
  hipLaunchKernelGGL(page_copy_kernel, dim3(b.count, num_layers, 2), dim3(256), 0, stream,
                     k_storage, v_storage, layer_bytes, page_bytes, b);
  return hipGetLastError();
}

hipError_t launch_patches(int32_t* arena, const PatchBatch& b, hipStream_t stream) {
  hipLaunchKernelGGL(patch_kernel, dim3(1), dim3(256), 0, stream, arena, b);
  return hipGetLastError();
}

}  // namespace pkv
