// Batched prefill on matrix cores: causal attention of a chunk of new rows
// over a request's paged prefix and the chunk itself.
//
// Source: riftco-transformer "Incremental Serving", section "Paged KV-cache
// layout": the pages leave a batched prefill kernel to later work, one that
// may use FlashAttention while writing the same paged cache that decode
// attention reads.  Row i of a chunk starting at position `start` computes the
// newest-query result at attended length start+i+1 (learn_llm ch.38, the
// incremental mixture: scores q.k/sqrt(d_h), stable softmax, weighted values).
//
// Unlike decode, a chunk has many query rows per key row, so the score and
// value products are dense contractions: 128 query rows share every K/V block
// staged in LDS, and both products run on MFMA (bf16 in, float32 accumulate).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pkv_internal.h"

namespace pkv {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

static_assert(kPrefillTileRows == 128, "four waves of 32 query rows");
constexpr int kBlockKeys = 64;     // keys per LDS block
constexpr int kXcds = 8;           // accelerator complex dies of an MI355X

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Page-table reads that are uniform across a wave go through the scalar data
// cache (the table is not written while this kernel runs).
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

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

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  // round to nearest even (the hardware conversion)
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// K and V blocks in LDS: 64 rows of 2 D bytes each (D / 8 chunks of 16
// bytes), row-major, with the chunks of row r stored XOR-swizzled by r mod
// (D / 8).  Lanes reading one chunk column of consecutive rows (the score
// operand), or four rows of one 32-byte span each (the transposing value
// read), then spread over the banks.  Byte offset of chunk c of row r:
template <int D>
__device__ inline int kv_byte(int row, int chunk) {
  return row * (2 * D) + ((chunk ^ (row & (D / 8 - 1))) << 4);
}

// V blocks at head width 128 take another swizzle: chunk c of row r sits at
// position c ^ f(r), f(r) = 2 (r mod 8) + (r / 8 mod 2).  A transposing
// value read serves each half wave (32 lanes) as eight consecutive rows
// reading chunks 2 dt and 2 dt + 1 of each; with f these are 16 distinct
// positions, which cover every bank once, where r mod 16 (K's swizzle) puts
// rows r and r ^ 1 on the same two chunk positions (two-way bank conflicts,
// two extra LDS cycles per read).  Other widths keep kv_byte's swizzle.
template <int D>
__device__ inline int v_swz(int row) {
  if constexpr (D == 128)
    return ((row & 7) << 1) | ((row >> 3) & 1);
  else
    return row & (D / 8 - 1);
}
template <int D>
__device__ inline int v_byte(int row, int chunk) {
  return row * (2 * D) + ((chunk ^ v_swz<D>(row)) << 4);
}

typedef int32_t i32x4_t __attribute__((ext_vector_type(4)));

// One 16-byte-per-lane buffer load straight into LDS: lane i's 16 bytes at
// byte voff(i) of [base, base + bytes) land at LDS byte lds_addr + 16 i
// (reads past `bytes` return zeros).  Inline assembly rather than the
// builtin: the compiler cannot tell which of the two LDS buffers a builtin
// load writes, so it waits for every such load before any LDS read of
// either buffer, which exposes the staging of block k+1 before block k is
// computed.  The block loop's own s_waitcnt and barrier order these loads.
__device__ inline void lds_dma16(const char* base, uint32_t bytes, uint32_t voff,
                                 uint32_t lds_addr) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const i32x4_t rsrc = {(int32_t)(uint32_t)p, (int32_t)((uint32_t)(p >> 32) & 0xFFFFu),
                        (int32_t)bytes, 0x00020000};
  asm volatile(
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds"
      :
      : "v"(voff), "s"(rsrc), "{m0}"(lds_addr)
      : "memory");
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Workgroup: 4 waves on one tile (request, up to 128 consecutive chunk rows)
// and one query head; each wave owns 32 query rows as two sets of 16 (at head
// width 256: 8 waves of one set each, see prefill_waves).  Every
// 64-key block of the rows the tile can see (0 .. the tile's last position)
// goes to LDS by direct buffer-to-LDS loads (no registers, no stores), into
// one of two buffers while the other one is computed on: one barrier per
// block.  The request's last, partial block takes clamped loads through
// registers instead, so no read passes its pages and every row is finite.
//
// Scores are formed transposed, S^T = K Q^T (A operand: 16 keys x 32 dims of
// K from LDS; B operand: Q held in registers), so lane l holds, for query
// l%16 of a set, the scores of keys 4(l/16)..4(l/16)+3 of each 16-key tile.
// Those are exactly the A-operand elements of the value product O = P V when
// the 32 keys of an MFMA step are taken in the order {tile 2c: 4g..4g+3,
// tile 2c+1: 4g..4g+3} for lane group g -- so probabilities never move
// between lanes.  The V operand (8 keys of one dim per lane, in that order)
// comes from row-major V with two transposing LDS reads (ds_read_b64_tr_b16:
// in each 16-lane group, lane j receives halfword j%4 of the 8 bytes that
// lane 4k + j/4 addresses, k = 0..3; lane i addressing key base + i/4, dims
// 16 dt + 4 (i%4)..+3 then hands lane j the dim 16 dt + j of keys base..+3).
// Each K or V fragment read from LDS feeds the MFMAs of both query sets.
// Online softmax per query in log2 units; the running maximum moves lazily
// (only by more than 2^8 in weight, decided by a vote over each lane's own
// maxima) and only then is reduced across the four lane groups with permlane
// swaps; the running sum comes from the matrix cores
// (head width <= 128) or the same swaps (256).  The context accumulates in
// the MFMA output layout (lane l: rows 4(l/16)..+3, column l%16 of each
// 16-column tile), whose per-row scale factors come from the owning lanes by
// shuffle.
//
// PAGE16: pages of exactly 16 rows (a row's page and slot are a shift and a
// mask instead of a division).
// Waves of a prefill workgroup: four with two 16-row query sets each, or, at
// head width 256 (whose context and query registers are twice as many),
// eight with one set each; either way a workgroup covers a 128-row tile.
constexpr int prefill_waves(int D) { return D == 256 ? 8 : 4; }

// Work item (query head, tile) of this workgroup: consecutive items share a
// request's K/V (the tile list is grouped by request).  Workgroups go to the
// eight XCDs round-robin, each with its own L2, so each XCD gets a contiguous
// range of items: tiles that re-read the same K/V rows then share one L2.
__device__ inline int prefill_item() {
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int per = nwg / kXcds, rem = nwg % kXcds;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

template <bool PAGE16, int D>
__global__ __launch_bounds__(64 * prefill_waves(D), 2) void prefill_mfma_kernel(PrefillArgs a) {
  static_assert(D == 64 || D == 128 || D == 256, "head widths 64, 128 and 256");
  constexpr int WAVES = prefill_waves(D);
  constexpr int QS = 8 / WAVES;  // 16-row query sets per wave
  constexpr int kRowBytes = 2 * D;
  constexpr int ND = D / 32;     // 32-dim slices of the score product
  constexpr int NT = D / 16;     // 16-dim tiles of the context
  constexpr int NC = D / 8;      // 16-byte chunks per row
  constexpr int RPI = 64 / NC;   // rows per 1 KiB staging load (4 or 8)
  constexpr int NPART = 64 / RPI / WAVES;  // staging loads per wave and block
  // [buffer][0: K, 1: V][64 rows x 2 D bytes], swizzled as kv_byte (K) and
  // v_byte (V) describe
  __shared__ __attribute__((aligned(16))) char sKV[2][2][kBlockKeys * kRowBytes];

  const int item = prefill_item();
  const int h = item / a.num_tiles;
  const PrefillTile tile = a.tiles[item - h * a.num_tiles];
  const int kvh = h / (a.num_heads / a.num_kv_heads);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ql = lane & 15;
  const int g = lane >> 4;
  const int S = a.page_size;
  const int32_t* pt = a.page_table + (int64_t)tile.pt_row * a.pt_stride;
  const int64_t head_off = (int64_t)kvh * a.head_bytes;
  const int pos0 = tile.start + tile.i0;  // position of the tile's first row

  // This lane's two query rows (rows past the tile's count attend like its
  // last row; their results are not stored).
  const int wrow0 = 16 * QS * wave;
  int my_pos[QS];
  bf16x8_t qf[QS][ND];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int row = min(wrow0 + 16 * qs + ql, tile.nq - 1);
    my_pos[qs] = pos0 + row;
    const int64_t qrow = (int64_t)(tile.off + tile.i0 + row) * a.num_heads + h;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                      qrow * kRowBytes);
#pragma unroll
    for (int dc = 0; dc < ND; ++dc) qf[qs][dc] = as_bf16x8(src[4 * dc + g]);
  }
  const int wave_first_pos = pos0 + min(wrow0, tile.nq - 1);
  const int wave_last_pos = pos0 + min(wrow0 + 16 * QS - 1, tile.nq - 1);
  const bool wave_active = wrow0 < tile.nq;

  // Row sums of the weights.  Up to head width 128 they come from a matrix
  // product of the bf16 weights with a block of ones, so they sit in the
  // context's row layout and sum exactly the weights the value product used
  // (two reductions across lane groups and ~40 vector instructions per block
  // fewer); at 256, where that product measured slower, from a lane-group
  // reduction of the float32 weights.
  constexpr bool kOnesSum = D <= 128;
  float m[QS], l[QS];
  f32x4_t lsum[QS];
  f32x4_t acc[QS][NT];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    m[qs] = -INFINITY;
    l[qs] = 0.f;
    lsum[qs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int qs = 0; qs < QS; ++qs)
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) acc[qs][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Staging of one 64-key block into buffer b.  Wave w, part i covers block
  // rows RPI (WAVES i + w) .. +RPI-1 (RPI = 1024 / row bytes), which lie in
  // one page; lane L takes row RPI (WAVES i + w) + L / NC and LDS chunk position
  // L % NC, i.e. global chunk (L % NC) ^ (row mod NC) of that row, and lands
  // at LDS byte base + 16 L.
  const int lrow = lane / NC;   // row within the part
  const int lpos = lane % NC;   // LDS chunk position
  const const_i32_ptr ptc = (const_i32_ptr)pt;
  auto stage = [&](int key0, int b) {
    if (key0 + kBlockKeys <= tile.key_end) {
      int32_t pg[NPART];
      if constexpr (PAGE16 && RPI * WAVES == 16) {
        // Part i's rows lie in page key0 / 16 + i (key0 is a multiple of 64
        // and RPI * wave < 16): consecutive table entries, which the
        // compiler fetches with one scalar load instead of one round trip
        // per part.
#pragma unroll
        for (int i = 0; i < NPART; ++i) pg[i] = ptc[(key0 >> 4) + i];
      } else {
#pragma unroll
        for (int i = 0; i < NPART; ++i) {
          const int key = key0 + RPI * (WAVES * i + wave);
          pg[i] = ptc[PAGE16 ? key >> 4 : key / S];
        }
      }
      const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(&sKV[b][0][0]);
      const uint32_t lds1 = (uint32_t)reinterpret_cast<uintptr_t>(&sKV[b][1][0]);
#pragma unroll
      for (int i = 0; i < NPART; ++i) {
        const int r0 = RPI * (WAVES * i + wave);   // first block row of the part
        const int key = key0 + r0;
        const int slot0 = PAGE16 ? key & 15 : key - (key / S) * S;
        const int64_t page = (int64_t)pg[i] * a.page_bytes + head_off;
        const int r = r0 + lrow;
        const uint32_t vrow_off = (slot0 + lrow) * kRowBytes;
        lds_dma16(a.k_layer + page, S * kRowBytes, vrow_off + ((lpos ^ (r & (NC - 1))) << 4),
                  lds0 + r0 * kRowBytes);
        lds_dma16(a.v_layer + page, S * kRowBytes, vrow_off + ((lpos ^ v_swz<D>(r)) << 4),
                  lds1 + r0 * kRowBytes);
      }
    } else {
      // Partial block: keys clamped to the last row the tile may read (the
      // clamped rows are masked, and finite, so they add nothing).
      uint4 kx[NPART], vx[NPART];
#pragma unroll
      for (int i = 0; i < NPART; ++i) {
        const int r = RPI * (WAVES * i + wave) + lrow;
        const int key = min(key0 + r, tile.key_end - 1);
        const int page_idx = PAGE16 ? key >> 4 : key / S;
        const int slot = PAGE16 ? key & 15 : key - page_idx * S;
        const int64_t off = (int64_t)pt[page_idx] * a.page_bytes + head_off +
                            (int64_t)slot * kRowBytes;
        kx[i] = *reinterpret_cast<const uint4*>(a.k_layer + off + ((lpos ^ (r & (NC - 1))) << 4));
        vx[i] = *reinterpret_cast<const uint4*>(a.v_layer + off + ((lpos ^ v_swz<D>(r)) << 4));
      }
#pragma unroll
      for (int i = 0; i < NPART; ++i) {
        const int r = RPI * (WAVES * i + wave) + lrow;
        *reinterpret_cast<uint4*>(&sKV[b][0][r * kRowBytes + lpos * 16]) = kx[i];
        *reinterpret_cast<uint4*>(&sKV[b][1][r * kRowBytes + lpos * 16]) = vx[i];
      }
    }
  };
  stage(0, 0);

  const int nblocks = (tile.key_end + kBlockKeys - 1) / kBlockKeys;
  // Up to head width 128 blocks are taken in pairs, which makes the buffer
  // index of each copy a constant: every LDS read address is then a
  // loop-invariant lane offset plus an immediate (d_h 64: 630 -> 608 us,
  // d_h 128: 1005 -> 1001 us on one box).  At 256 the pairs measured 8%
  // slower (2375 -> 2565 us), and the index stays a run-time value.
  constexpr int kPair = D == 256 ? 1 : 2;
  for (int kp = 0; kp < nblocks; kp += kPair)
#pragma unroll
  for (int u = 0; u < kPair; ++u) {
    const int kb = kp + u;
    if (kb >= nblocks) break;
    const int b = kPair == 2 ? u : kb & 1;
    const int key0 = kb * kBlockKeys;
    // This wave's loads and stores into buffer b are complete; the barrier
    // then makes every wave's visible and ends all reads of buffer b ^ 1.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kb + 1 < nblocks) stage(key0 + kBlockKeys, b ^ 1);  // flies during this block's math
    const char* sK = sKV[b][0];
    const char* sV = sKV[b][1];

    // A wave whose queries all precede every key of the block has nothing
    // to add from it (causal), and an empty wave has nothing at all.  Block 0
    // is never skipped, so every running maximum is finite from then on, and
    // a lane whose query precedes a whole later block keeps it unchanged
    // (scale 1, weights 0).
    if (!wave_active || wave_last_pos < key0) continue;

    // ---- scores S^T = K Q^T: s[qs][kt][j] = q . k(key0 + 16 kt + 4 g + j) ----
    float s[QS][4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4_t c[QS];
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) c[qs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < ND; ++dc) {
        const bf16x8_t kf =
            as_bf16x8(*reinterpret_cast<const uint4*>(sK + kv_byte<D>(16 * kt + ql, 4 * dc + g)));
#pragma unroll
        for (int qs = 0; qs < QS; ++qs)
          c[qs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qs][dc], c[qs], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)  // raw q.k; the log2 scale joins in the exponent
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[qs][kt][j] = c[qs][j];
    }
    // At head width 128 the scheduler is held to eight K reads ahead of the
    // score products (it kept about four, waiting on the LDS five or six
    // times per block): 1009 -> 1000 and 1027 -> 1014 us per launch in
    // alternating runs on two boxes, in the same registers.
    if constexpr (D == 128) {
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);  // LDS reads
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, QS, 0);  // the products of one read
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // the next read
      }
    }
    // causal mask where the block reaches past this wave's first position
    if (key0 + kBlockKeys - 1 > wave_first_pos) {
#pragma unroll
      for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (key0 + 16 * kt + 4 * g + j > my_pos[qs]) s[qs][kt][j] = -INFINITY;
    }
    // This lane's maxima over its 16 keys of the block, in scaled log2 units
    // (the scale is positive, so the maximum of the raw products scales to
    // the maximum of the scores).
    float cand[QS];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float mb = s[qs][0][0];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mb = fmaxf(mb, s[qs][kt][j]);
      cand[qs] = mb * a.scale_log2e;
    }
    // Lazy rescale: the running maxima move (and the context and sums are
    // rescaled) only when some query of the wave sees a block maximum more
    // than kSlack above its own; otherwise the weights exp2(s - m) stay at
    // most 2^kSlack, which float32 sums and bf16 weights carry exactly as
    // well.  The first block always moves them from -inf.  A query's block
    // maximum is the largest of its four lanes' maxima, so the wave-wide
    // vote over lane maxima decides the same; only then are the maxima
    // reduced across the lane groups (every lane of a query then holds the
    // same running maximum).
    constexpr float kSlack = 8.f;
    bool grow = false;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) grow = grow || cand[qs] > m[qs] + kSlack;
    if (__builtin_expect(__any(grow), 0)) {
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        const float mn = fmaxf(m[qs], xor32_max(xor16_max(cand[qs])));
        const float alpha = __builtin_amdgcn_exp2f(m[qs] - mn);
        l[qs] *= alpha;
        m[qs] = mn;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float aj = __shfl(alpha, 4 * g + j);
          lsum[qs][j] *= aj;
#pragma unroll
          for (int dt = 0; dt < NT; ++dt) acc[qs][dt][j] *= aj;
        }
      }
    }
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[qs][kt][j] = __builtin_amdgcn_exp2f(fmaf(s[qs][kt][j], a.scale_log2e, -m[qs]));
          if constexpr (!kOnesSum) ps += s[qs][kt][j];
        }
      if constexpr (!kOnesSum) l[qs] += xor32_sum(xor16_sum(ps));
    }
    // ---- O += P V over two 32-key steps ----
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8_t pf[QS];
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        uint4 pu;
        pu.x = pack_bf16x2(s[qs][2 * kc][0], s[qs][2 * kc][1]);
        pu.y = pack_bf16x2(s[qs][2 * kc][2], s[qs][2 * kc][3]);
        pu.z = pack_bf16x2(s[qs][2 * kc + 1][0], s[qs][2 * kc + 1][1]);
        pu.w = pack_bf16x2(s[qs][2 * kc + 1][2], s[qs][2 * kc + 1][3]);
        pf[qs] = as_bf16x8(pu);
        if constexpr (kOnesSum)
          lsum[qs] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              pf[qs], as_bf16x8(uint4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u}),
              lsum[qs], 0, 0, 0);
      }
      // transposing reads: lane (g, i) addresses key 32 kc + 4 g + i/4 (and
      // + 16), dims 16 dt + 4 (i%4)..+3
      const int vrow = 32 * kc + 4 * g + (ql >> 2);
#pragma unroll
      for (int dt = 0; dt < NT; ++dt) {
        const int chunk = 2 * dt + ((ql & 3) >> 1);
        const int half = (ql & 1) * 8;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(sV + v_byte<D>(vrow, chunk) + half));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(sV + v_byte<D>(vrow + 16, chunk) + half));
        const bf16x8_t vf = __builtin_bit_cast(
            bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int qs = 0; qs < QS; ++qs)
          acc[qs][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[qs], vf, acc[qs][dt], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
#pragma unroll
  for (int qs = 0; qs < QS; ++qs)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wrow0 + 16 * qs + 4 * g + j;
      const float inv = 1.0f / (kOnesSum ? lsum[qs][j] : __shfl(l[qs], 4 * g + j));
      if (row < tile.nq) {
        float* o = a.out + ((int64_t)(tile.off + tile.i0 + row) * a.num_heads + h) * D;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) o[16 * dt + ql] = acc[qs][dt][j] * inv;
      }
    }
}

// ---------------------------------------------------------------------------
// Float32 prefill on matrix cores (v_mfma_f32_16x16x4_f32), head widths 32,
// 64 and 128.  Same tiles, work items, staging and online softmax as the
// bf16 kernel; what differs is the operand layout of 4-deep float32 steps:
//
// Scores S^T = K Q^T, one 16-key tile kt at a time.  For dims 16 q .. 16 q +
// 15 a lane group g supplies dims 16 q + 4 g + t at step t = 0..3, so lane l
// reads four consecutive floats of key 16 kt + l%16 (one 16-byte LDS read
// for four steps) and its query's matching four floats from registers; lane
// l then holds the scores of query l%16 for keys 16 kt + 4 g + j.
// Context O^T = V^T P^T, step j of tile kt taking keys 16 kt + 4 g + j from
// lane group g: the B operand is the lane's own weight for that key and the
// A operand one float of V (key 16 kt + 4 g + j, dim 16 dt + l%16).  Lane l
// accumulates dims 16 dt + 4 g + (0..3) of query l%16, so the softmax's
// per-query rescale is a lane's own scalar and the output row a 16-byte
// store.  K and V sit row-major in LDS, 16-byte chunks XOR-swizzled by row
// so both read patterns spread over the banks.  Weights stay float32.
//
// Keys per LDS block: 64, or 32 at head width 128 (rows of 512 bytes), so
// two buffers of K and V take at most 64 KiB.  Four waves of two 16-row
// query sets, or at head width 128 (twice the context and query registers)
// eight waves of one set; either way a 128-row tile.
constexpr int prefill_f32_waves(int D) { return D == 128 ? 8 : 4; }

template <bool PAGE16, int D>
__global__ __launch_bounds__(64 * prefill_f32_waves(D), 2) void prefill_f32_kernel(PrefillArgs a) {
  static_assert(D == 32 || D == 64 || D == 128, "head widths 32, 64 and 128");
  constexpr int WAVES = prefill_f32_waves(D);
  constexpr int QS = 8 / WAVES;            // 16-row query sets per wave
  constexpr int KB = D == 128 ? 32 : 64;   // keys per LDS block
  constexpr int KT = KB / 16;              // 16-key tiles per block
  constexpr int kRowBytes = 4 * D;
  constexpr int NC = D / 4;                // 16-byte chunks per row
  constexpr int NQ = D / 16;               // 16-dim groups of the score product
  constexpr int NT = D / 16;               // 16-dim tiles of the context
  constexpr int RPI = 64 / NC;             // rows per 1 KiB staging load
  constexpr int NPART = KB / RPI / WAVES;  // staging loads per wave and block
  static_assert(NPART >= 1 && 16 % RPI == 0, "a staging load stays inside one page");
  __shared__ __attribute__((aligned(16))) char sKV[2][2][KB * kRowBytes];
  auto chunk_byte = [](int row, int chunk) {
    return row * kRowBytes + ((chunk ^ (row & (NC - 1))) << 4);
  };

  const int item = prefill_item();
  const int h = item / a.num_tiles;
  const PrefillTile tile = a.tiles[item - h * a.num_tiles];
  const int kvh = h / (a.num_heads / a.num_kv_heads);
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ql = lane & 15;
  const int g = lane >> 4;
  const int S = a.page_size;
  const int32_t* pt = a.page_table + (int64_t)tile.pt_row * a.pt_stride;
  const const_i32_ptr ptc = (const_i32_ptr)pt;
  const int64_t head_off = (int64_t)kvh * a.head_bytes;
  const int pos0 = tile.start + tile.i0;

  // This lane's query rows (rows past the tile's count attend like its last
  // row; their results are not stored) and their dims 16 q + 4 g .. + 3.
  const int wrow0 = 16 * QS * wave;
  int my_pos[QS];
  f32x4_t qf[QS][NQ];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int row = min(wrow0 + 16 * qs + ql, tile.nq - 1);
    my_pos[qs] = pos0 + row;
    const float* src = static_cast<const float*>(a.q) +
                       ((int64_t)(tile.off + tile.i0 + row) * a.num_heads + h) * D;
#pragma unroll
    for (int q = 0; q < NQ; ++q) qf[qs][q] = *reinterpret_cast<const f32x4_t*>(src + 16 * q + 4 * g);
  }
  const int wave_first_pos = pos0 + min(wrow0, tile.nq - 1);
  const int wave_last_pos = pos0 + min(wrow0 + 16 * QS - 1, tile.nq - 1);
  const bool wave_active = wrow0 < tile.nq;

  float m[QS], l[QS];
  f32x4_t acc[QS][NT];
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    m[qs] = -INFINITY;
    l[qs] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NT; ++dt) acc[qs][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Staging of one KB-key block into buffer b, as in the bf16 kernel: wave
  // w, part i covers block rows RPI (WAVES i + w) .. +RPI-1, inside one page;
  // lane L takes row RPI (WAVES i + w) + L / NC and LDS chunk position L % NC.
  const int lrow = lane / NC;
  const int lpos = lane % NC;
  auto stage = [&](int key0, int b) {
    if (key0 + KB <= tile.key_end) {
      int32_t pg[NPART];
#pragma unroll
      for (int i = 0; i < NPART; ++i) {
        const int key = key0 + RPI * (WAVES * i + wave);
        pg[i] = ptc[PAGE16 ? key >> 4 : key / S];
      }
      const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(&sKV[b][0][0]);
      const uint32_t lds1 = (uint32_t)reinterpret_cast<uintptr_t>(&sKV[b][1][0]);
#pragma unroll
      for (int i = 0; i < NPART; ++i) {
        const int r0 = RPI * (WAVES * i + wave);
        const int key = key0 + r0;
        const int slot0 = PAGE16 ? key & 15 : key - (key / S) * S;
        const int64_t page = (int64_t)pg[i] * a.page_bytes + head_off;
        const int r = r0 + lrow;
        const uint32_t voff = (slot0 + lrow) * kRowBytes + ((lpos ^ (r & (NC - 1))) << 4);
        lds_dma16(a.k_layer + page, S * kRowBytes, voff, lds0 + r0 * kRowBytes);
        lds_dma16(a.v_layer + page, S * kRowBytes, voff, lds1 + r0 * kRowBytes);
      }
    } else {
      // Partial block: keys clamped to the last row the tile may read (the
      // clamped rows are masked, and finite, so they add nothing).
      uint4 kx[NPART], vx[NPART];
#pragma unroll
      for (int i = 0; i < NPART; ++i) {
        const int r = RPI * (WAVES * i + wave) + lrow;
        const int key = min(key0 + r, tile.key_end - 1);
        const int page_idx = PAGE16 ? key >> 4 : key / S;
        const int slot = PAGE16 ? key & 15 : key - page_idx * S;
        const int64_t off = (int64_t)pt[page_idx] * a.page_bytes + head_off +
                            (int64_t)slot * kRowBytes + ((lpos ^ (r & (NC - 1))) << 4);
        kx[i] = *reinterpret_cast<const uint4*>(a.k_layer + off);
        vx[i] = *reinterpret_cast<const uint4*>(a.v_layer + off);
      }
#pragma unroll
      for (int i = 0; i < NPART; ++i) {
        const int r = RPI * (WAVES * i + wave) + lrow;
        *reinterpret_cast<uint4*>(&sKV[b][0][r * kRowBytes + lpos * 16]) = kx[i];
        *reinterpret_cast<uint4*>(&sKV[b][1][r * kRowBytes + lpos * 16]) = vx[i];
      }
    }
  };
  stage(0, 0);

  const int nblocks = (tile.key_end + KB - 1) / KB;
  for (int kb = 0; kb < nblocks; ++kb) {
    const int key0 = kb * KB;
    const int b = kb & 1;
    // This wave's loads and stores into buffer b are complete; the barrier
    // then makes every wave's visible and ends all reads of buffer b ^ 1.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (kb + 1 < nblocks) stage(key0 + KB, b ^ 1);
    const char* sK = sKV[b][0];
    const char* sV = sKV[b][1];
    // Causal skip, as in the bf16 kernel (block 0 is never skipped).
    if (!wave_active || wave_last_pos < key0) continue;

    // ---- scores: s[qs][kt][j] = q . k(key0 + 16 kt + 4 g + j) ----
    float s[QS][KT][4];
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      f32x4_t c[QS];
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) c[qs] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int q = 0; q < NQ; ++q) {
        const f32x4_t kf =
            *reinterpret_cast<const f32x4_t*>(sK + chunk_byte(16 * kt + ql, 4 * q + g));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int qs = 0; qs < QS; ++qs)
            c[qs] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[t], qf[qs][q][t], c[qs], 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int qs = 0; qs < QS; ++qs) s[qs][kt][j] = c[qs][j];
    }
    if (key0 + KB - 1 > wave_first_pos) {
#pragma unroll
      for (int qs = 0; qs < QS; ++qs)
#pragma unroll
        for (int kt = 0; kt < KT; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (key0 + 16 * kt + 4 * g + j > my_pos[qs]) s[qs][kt][j] = -INFINITY;
    }
    float cand[QS];
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float mb = s[qs][0][0];
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mb = fmaxf(mb, s[qs][kt][j]);
      cand[qs] = xor32_max(xor16_max(mb)) * a.scale_log2e;
    }
    // Lazy rescale, as in the bf16 kernel; a lane's context belongs to its
    // own query, so the factor needs no exchange.
    constexpr float kSlack = 8.f;
    bool grow = false;
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) grow = grow || cand[qs] > m[qs] + kSlack;
    if (__builtin_expect(__any(grow), 0)) {
#pragma unroll
      for (int qs = 0; qs < QS; ++qs) {
        const float mn = fmaxf(m[qs], cand[qs]);
        const float alpha = __builtin_amdgcn_exp2f(m[qs] - mn);
        l[qs] *= alpha;
        m[qs] = mn;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) acc[qs][dt] *= alpha;
      }
    }
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < KT; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[qs][kt][j] = __builtin_amdgcn_exp2f(fmaf(s[qs][kt][j], a.scale_log2e, -m[qs]));
          ps += s[qs][kt][j];
        }
      l[qs] += xor32_sum(xor16_sum(ps));
    }
    // ---- O^T += V^T P^T, 4 keys per step ----
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int vrow = 16 * kt + 4 * g + j;
#pragma unroll
        for (int dt = 0; dt < NT; ++dt) {
          const float vf = *reinterpret_cast<const float*>(
              sV + chunk_byte(vrow, 4 * dt + (ql >> 2)) + 4 * (ql & 3));
#pragma unroll
          for (int qs = 0; qs < QS; ++qs)
            acc[qs][dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf, s[qs][kt][j], acc[qs][dt], 0, 0, 0);
        }
      }
    // The scheduler is held to sixteen V reads ahead of the value products
    // (d_h 64: 1768 -> 1729 us per launch in alternating runs, 32 and 128
    // within 0.5%; eight ahead slowed d_h 128 by 2%).
    __builtin_amdgcn_sched_group_barrier(0x100, 16, 0);  // LDS reads
#pragma unroll
    for (int i = 0; i < KT * 4 * NT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, QS, 0);  // the products of one read
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // the next read
    }
  }

  if (!wave_active) return;
#pragma unroll
  for (int qs = 0; qs < QS; ++qs) {
    const int row = wrow0 + 16 * qs + ql;
    if (row < tile.nq) {
      const float inv = 1.0f / l[qs];
      float* o = a.out + ((int64_t)(tile.off + tile.i0 + row) * a.num_heads + h) * D + 4 * g;
#pragma unroll
      for (int dt = 0; dt < NT; ++dt)
        *reinterpret_cast<f32x4_t*>(o + 16 * dt) = acc[qs][dt] * inv;
    }
  }
}

// Writes the chunk's new K/V rows into their slots: one workgroup per (tile,
// K/V head), 16 bytes per lane.  It runs before the attention launch, which
// reads the chunk's keys back from the pages (4 KiB contiguous per 16 keys
// of a head, where the packed inputs put consecutive keys H_kv rows apart).
template <int kRowBytes>
__global__ __launch_bounds__(256) void prefill_append_kernel(PrefillArgs a) {
  const PrefillTile tile = a.tiles[blockIdx.x];
  const int kvh = blockIdx.y;
  const int S = a.page_size;
  const int32_t* pt = a.page_table + (int64_t)tile.pt_row * a.pt_stride;
  constexpr int kChunks = kRowBytes / 16;
  for (int c = threadIdx.x; c < tile.nq * kChunks; c += 256) {
    const int i = tile.i0 + c / kChunks;
    const int col = (c % kChunks) * 16;
    const int pos = tile.start + i;
    const int64_t dst = (int64_t)pt[pos / S] * a.page_bytes + (int64_t)kvh * a.head_bytes +
                        (int64_t)(pos % S) * kRowBytes + col;
    const int64_t src = ((int64_t)(tile.off + i) * a.num_kv_heads + kvh) * kRowBytes + col;
    *reinterpret_cast<uint4*>(a.k_layer + dst) =
        *reinterpret_cast<const uint4*>(static_cast<const char*>(a.k_new) + src);
    *reinterpret_cast<uint4*>(a.v_layer + dst) =
        *reinterpret_cast<const uint4*>(static_cast<const char*>(a.v_new) + src);
  }
}

}  // namespace

bool prefill_fast_supported(int dtype, int head_width, int page_size) {
  if (page_size % 16 != 0) return false;
  if (dtype == kDtypeBF16) return head_width == 64 || head_width == 128 || head_width == 256;
  return dtype == kDtypeF32 && (head_width == 32 || head_width == 64 || head_width == 128);
}

// Rows of 128, 256 or 512 bytes (both dtypes' widths above).
hipError_t launch_prefill_append(const PrefillArgs& a, int num_tiles, hipStream_t stream) {
  const dim3 grid(num_tiles, a.num_kv_heads);
  switch (a.head_bytes / a.page_size) {
    case 128: hipLaunchKernelGGL(prefill_append_kernel<128>, grid, dim3(256), 0, stream, a); break;
    case 256: hipLaunchKernelGGL(prefill_append_kernel<256>, grid, dim3(256), 0, stream, a); break;
    default: hipLaunchKernelGGL(prefill_append_kernel<512>, grid, dim3(256), 0, stream, a); break;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_f32(const PrefillArgs& a, int num_tiles, hipStream_t stream) {
  const dim3 block(64 * prefill_f32_waves(D));
  if (a.page_size == 16)
    hipLaunchKernelGGL((prefill_f32_kernel<true, D>), dim3(num_tiles * a.num_heads), block, 0,
                       stream, a);
  else
    hipLaunchKernelGGL((prefill_f32_kernel<false, D>), dim3(num_tiles * a.num_heads), block, 0,
                       stream, a);
  return hipGetLastError();
}

template <int D>
hipError_t launch_prefill_width(const PrefillArgs& a, int num_tiles, hipStream_t stream) {
  const dim3 block(64 * prefill_waves(D));
  if (a.page_size == 16)
    hipLaunchKernelGGL((prefill_mfma_kernel<true, D>), dim3(num_tiles * a.num_heads), block, 0,
                       stream, a);
  else
    hipLaunchKernelGGL((prefill_mfma_kernel<false, D>), dim3(num_tiles * a.num_heads), block, 0,
                       stream, a);
  return hipGetLastError();
}

hipError_t launch_prefill_attention(const PrefillArgs& a, int num_tiles, hipStream_t stream) {
  if (a.dtype == kDtypeF32) {
    switch (a.head_bytes / a.page_size) {
      case 128: return launch_prefill_f32<32>(a, num_tiles, stream);
      case 256: return launch_prefill_f32<64>(a, num_tiles, stream);
      default: return launch_prefill_f32<128>(a, num_tiles, stream);
    }
  }
  switch (a.head_bytes / a.page_size) {
    case 128: return launch_prefill_width<64>(a, num_tiles, stream);
    case 256: return launch_prefill_width<128>(a, num_tiles, stream);
    default: return launch_prefill_width<256>(a, num_tiles, stream);
  }
}

}  // namespace pkv
