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

constexpr int kD = 128;            // head width of this kernel (256-byte bf16 rows)
constexpr int kRowBytes = kD * 2;
static_assert(kPrefillTileRows == 128, "four waves of 32 query rows");
constexpr int kBlockKeys = 64;     // keys per LDS block
constexpr int kKStride = kD + 8;   // bf16 per K row in LDS (272 B: rows 4 banks apart)
constexpr int kVStride = kBlockKeys + 4;  // bf16 per transposed V row in LDS (136 B)
constexpr int kXcds = 8;           // accelerator complex dies of an MI355X

__device__ inline bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

// Page-table reads that are uniform across a wave go through the scalar data
// cache (the table is not written while this kernel runs).
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

// Raw buffer access to one 4 KiB head-page: a scalar base in the descriptor,
// a 32-bit lane offset per load (word 3: 32-bit data format for untyped
// loads on gfx9-family parts).
__device__ inline uint4 page_load(const char* page, uint32_t off) {
  const auto r = __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(page), 0, 16 * kRowBytes,
                                                   0x00020000);
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0));
}

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

// 32-bit word i (a compile-time constant after unrolling) of a 16-byte value.
__device__ inline uint32_t word_of(const uint4& u, int i) {
  return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  // round to nearest even (the hardware conversion)
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Transposed V in LDS: sV[dim][key] with the 4-key groups of each row
// XOR-swizzled by the row's 32-dim band, so the 64 lanes that store one dim
// each (16 dims apart across lanes, 34 banks per row) hit 64 distinct banks;
// readers apply the same swizzle (uniform across a 16-dim tile).
__device__ inline int vt_index(int dim, int key) {
  return dim * kVStride + (((key >> 2) ^ (((dim >> 5) & 3) << 2)) << 2) + (key & 3);
}

// Workgroup: 4 waves on one tile (request, up to 128 consecutive chunk rows)
// and one query head; each wave owns 32 query rows as two sets of 16.  Every
// 64-key block of the rows the tile can see (0 .. the tile's last position)
// is staged in LDS -- K as rows, V transposed -- while the next block's K/V
// are already being fetched into registers.
//
// Scores are formed transposed, S^T = K Q^T (A operand: 16 keys x 32 dims of
// K from LDS; B operand: Q held in registers), so lane l holds, for query
// l%16 of a set, the scores of keys 4(l/16)..4(l/16)+3 of each 16-key tile.
// Those are exactly the A-operand elements of the value product O = P V when
// the 32 keys of an MFMA step are taken in the order {tile 2c: 4g..4g+3,
// tile 2c+1: 4g..4g+3} for lane group g -- so probabilities never move
// between lanes; the transposed V is read in the same key order.  Each K or V
// fragment read from LDS feeds the MFMAs of both query sets.  Online softmax
// per query in log2 units; the running maximum and sum are reduced across
// the four lane groups with shuffles, and the maximum moves lazily (only by
// more than 2^8 in weight).  The context accumulates in the MFMA
// output layout (lane l: rows 4(l/16)..+3, column l%16 of each 16-column
// tile), whose per-row scale factors come from the owning lanes by shuffle.
//
// PAGE16: pages of exactly 16 rows, so a row's page and slot are a shift and
// a mask instead of a division (the lookups run per lane for every load).
template <bool PAGE16>
__global__ __launch_bounds__(256, 2) void prefill_mfma_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[kBlockKeys * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t sV[kD * kVStride];

  // Work item (query head, tile): consecutive items share a request's K/V
  // (the tile list is grouped by request).  Workgroups go to the eight XCDs
  // round-robin, each with its own L2, so each XCD gets a contiguous range of
  // items: tiles that re-read the same K/V rows then share one L2.
  const int nwg = gridDim.x;
  const int xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
  const int per = nwg / kXcds, rem = nwg % kXcds;
  const int item = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
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
  const int wrow0 = 32 * wave;
  int my_pos[2];
  bf16x8_t qf[2][4];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int row = min(wrow0 + 16 * qs + ql, tile.nq - 1);
    my_pos[qs] = pos0 + row;
    const int64_t qrow = (int64_t)(tile.off + tile.i0 + row) * a.num_heads + h;
    const uint4* src = reinterpret_cast<const uint4*>(static_cast<const char*>(a.q) +
                                                      qrow * kRowBytes);
#pragma unroll
    for (int dc = 0; dc < 4; ++dc) qf[qs][dc] = as_bf16x8(src[4 * dc + g]);
  }
  const int wave_first_pos = pos0 + min(wrow0, tile.nq - 1);
  const int wave_last_pos = pos0 + min(wrow0 + 31, tile.nq - 1);
  const bool wave_active = wrow0 < tile.nq;

  float m[2] = {-INFINITY, -INFINITY}, l[2] = {0.f, 0.f};
  f32x4_t acc[2][8];
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) acc[qs][dt] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Global -> register fetch of one block (keys clamped to the last row the
  // tile may read, so no lookup goes past the request's pages).  K chunk
  // c = tid + 256 i is key c/16, bytes 16 (c%16) of its row; V chunk i of a
  // thread is key 2 vpair + i/2, bytes 32 vdg + 16 (i%2).
  const int vpair = tid >> 3;
  const int vdg = tid & 7;
  auto row_off = [&](int key) -> int64_t {
    const int page = PAGE16 ? key >> 4 : key / S;
    const int slot = PAGE16 ? key & 15 : key % S;
    return (int64_t)pt[page] * a.page_bytes + head_off + (int64_t)slot * kRowBytes;
  };
  auto k_src = [&](int key0, int i) -> const uint4* {
    const int c = tid + 256 * i;
    const int key = min(key0 + (c >> 4), tile.key_end - 1);
    return reinterpret_cast<const uint4*>(a.k_layer + row_off(key) + (c & 15) * 16);
  };
  auto v_src = [&](int key0, int i) -> const uint4* {
    const int key = min(key0 + 2 * vpair + (i >> 1), tile.key_end - 1);
    return reinterpret_cast<const uint4*>(a.v_layer + row_off(key) + vdg * 32 + (i & 1) * 16);
  };
  uint4 k0, k1, k2, k3, v0, v1, v2, v3;
  // A block's K/V.  With 16-row pages and all 64 keys visible, K load i is
  // page key0/16 + i for the whole workgroup (thread t: bytes 16 t) and a
  // wave's V rows all lie in page key0/16 + wave: four wave-uniform page
  // reads and constant lane offsets.  Otherwise (other page sizes, or the
  // tile's last, clamped block) every lane looks its row up.
  auto fetch = [&](int key0) {
    if (PAGE16 && key0 + kBlockKeys <= tile.key_end) {
      const const_i32_ptr ptc = (const_i32_ptr)pt;
      const int pg0 = key0 >> 4;
      const char* kp0 = a.k_layer + (int64_t)ptc[pg0] * a.page_bytes + head_off;
      const char* kp1 = a.k_layer + (int64_t)ptc[pg0 + 1] * a.page_bytes + head_off;
      const char* kp2 = a.k_layer + (int64_t)ptc[pg0 + 2] * a.page_bytes + head_off;
      const char* kp3 = a.k_layer + (int64_t)ptc[pg0 + 3] * a.page_bytes + head_off;
      const char* vp = a.v_layer + (int64_t)ptc[pg0 + wave] * a.page_bytes + head_off;
      k0 = page_load(kp0, tid * 16);
      k1 = page_load(kp1, tid * 16);
      k2 = page_load(kp2, tid * 16);
      k3 = page_load(kp3, tid * 16);
      const uint32_t vrow = (uint32_t)(2 * (vpair & 7)) * kRowBytes + vdg * 32;
      v0 = page_load(vp, vrow);
      v1 = page_load(vp, vrow + 16);
      v2 = page_load(vp, vrow + kRowBytes);
      v3 = page_load(vp, vrow + kRowBytes + 16);
    } else {
      k0 = *k_src(key0, 0);
      k1 = *k_src(key0, 1);
      k2 = *k_src(key0, 2);
      k3 = *k_src(key0, 3);
      v0 = *v_src(key0, 0);
      v1 = *v_src(key0, 1);
      v2 = *v_src(key0, 2);
      v3 = *v_src(key0, 3);
    }
  };
  fetch(0);

  const int nblocks = (tile.key_end + kBlockKeys - 1) / kBlockKeys;
  for (int kb = 0; kb < nblocks; ++kb) {
    const int key0 = kb * kBlockKeys;
    __syncthreads();  // every wave is done with the previous block in LDS
    {
      auto store_k = [&](int i, const uint4& u) {
        const int c = tid + 256 * i;
        *reinterpret_cast<uint4*>(&sK[(c >> 4) * kKStride + (c & 15) * 8]) = u;
      };
      store_k(0, k0);
      store_k(1, k1);
      store_k(2, k2);
      store_k(3, k3);
      // V transposed; one 32-bit store per dim holds the key pair (v0, v1:
      // key 2 vpair, dims 16 vdg + 0..15; v2, v3: key 2 vpair + 1).
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t w0 = word_of(e < 8 ? v0 : v1, (e & 7) >> 1);
        const uint32_t w1 = word_of(e < 8 ? v2 : v3, (e & 7) >> 1);
        const uint32_t pair = (e & 1) ? ((w0 >> 16) | (w1 & 0xffff0000u))
                                      : ((w0 & 0xffffu) | (w1 << 16));
        *reinterpret_cast<uint32_t*>(&sV[vt_index(16 * vdg + e, 2 * vpair)]) = pair;
      }
    }
    __syncthreads();
    if (kb + 1 < nblocks) fetch(key0 + kBlockKeys);  // flies during this block's math

    // A wave whose queries all precede every key of the block has nothing
    // to add from it (causal), and an empty wave has nothing at all.  Block 0
    // is never skipped, so every running maximum is finite from then on, and
    // a lane whose query precedes a whole later block keeps it unchanged
    // (scale 1, weights 0).
    if (!wave_active || wave_last_pos < key0) continue;

    // ---- scores S^T = K Q^T: s[qs][kt][j] = q . k(key0 + 16 kt + 4 g + j) ----
    float s[2][4][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      f32x4_t c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int dc = 0; dc < 4; ++dc) {
        const bf16x8_t kf = as_bf16x8(
            *reinterpret_cast<const uint4*>(&sK[(16 * kt + ql) * kKStride + 32 * dc + 8 * g]));
        c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[0][dc], c0, 0, 0, 0);
        c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[1][dc], c1, 0, 0, 0);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {  // raw q.k; the log2 scale joins in the exponent
        s[0][kt][j] = c0[j];
        s[1][kt][j] = c1[j];
      }
    }
    // causal mask where the block reaches past this wave's first position
    if (key0 + kBlockKeys - 1 > wave_first_pos) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (key0 + 16 * kt + 4 * g + j > my_pos[qs]) s[qs][kt][j] = -INFINITY;
    }
    // Block maxima in scaled log2 units (the scale is positive, so the
    // maximum of the raw products scales to the maximum of the scores).
    float cand[2];
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float mb = s[qs][0][0];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) mb = fmaxf(mb, s[qs][kt][j]);
      cand[qs] = xor32_max(xor16_max(mb)) * a.scale_log2e;
    }
    // Lazy rescale: the running maxima move (and the context and sums are
    // rescaled) only when some query of the wave sees a block maximum more
    // than kSlack above its own; otherwise the weights exp2(s - m) stay at
    // most 2^kSlack, which float32 sums and bf16 weights carry exactly as
    // well.  The first block always moves them from -inf.
    constexpr float kSlack = 8.f;
    if (__builtin_expect(__any(cand[0] > m[0] + kSlack || cand[1] > m[1] + kSlack), 0)) {
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        const float mn = fmaxf(m[qs], cand[qs]);
        const float alpha = __builtin_amdgcn_exp2f(m[qs] - mn);
        l[qs] *= alpha;
        m[qs] = mn;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float aj = __shfl(alpha, 4 * g + j);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) acc[qs][dt][j] *= aj;
        }
      }
    }
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      float ps = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          s[qs][kt][j] = __builtin_amdgcn_exp2f(fmaf(s[qs][kt][j], a.scale_log2e, -m[qs]));
          ps += s[qs][kt][j];
        }
      l[qs] += xor32_sum(xor16_sum(ps));
    }
    // ---- O += P V over two 32-key steps ----
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      bf16x8_t pf[2];
#pragma unroll
      for (int qs = 0; qs < 2; ++qs) {
        uint4 pu;
        pu.x = pack_bf16x2(s[qs][2 * kc][0], s[qs][2 * kc][1]);
        pu.y = pack_bf16x2(s[qs][2 * kc][2], s[qs][2 * kc][3]);
        pu.z = pack_bf16x2(s[qs][2 * kc + 1][0], s[qs][2 * kc + 1][1]);
        pu.w = pack_bf16x2(s[qs][2 * kc + 1][2], s[qs][2 * kc + 1][3]);
        pf[qs] = as_bf16x8(pu);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int dim = 16 * dt + ql;
        const uint2 lo = *reinterpret_cast<const uint2*>(&sV[vt_index(dim, 32 * kc + 4 * g)]);
        const uint2 hi =
            *reinterpret_cast<const uint2*>(&sV[vt_index(dim, 32 * kc + 16 + 4 * g)]);
        const bf16x8_t vf = as_bf16x8(uint4{lo.x, lo.y, hi.x, hi.y});
        acc[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[0], vf, acc[0][dt], 0, 0, 0);
        acc[1][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[1], vf, acc[1][dt], 0, 0, 0);
      }
    }
  }

  if (!wave_active) return;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = wrow0 + 16 * qs + 4 * g + j;
      const float inv = 1.0f / __shfl(l[qs], 4 * g + j);
      if (row < tile.nq) {
        float* o = a.out + ((int64_t)(tile.off + tile.i0 + row) * a.num_heads + h) * kD;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[16 * dt + ql] = acc[qs][dt][j] * inv;
      }
    }
}

// Writes the chunk's new K/V rows into their slots: one workgroup per (tile,
// K/V head), 16 bytes per lane.  It runs before the attention launch, which
// reads the chunk's keys back from the pages (4 KiB contiguous per 16 keys
// of a head, where the packed inputs put consecutive keys H_kv rows apart).
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
  return dtype == kDtypeBF16 && head_width == kD && page_size % 16 == 0;
}

hipError_t launch_prefill_append(const PrefillArgs& a, int num_tiles, hipStream_t stream) {
  hipLaunchKernelGGL(prefill_append_kernel, dim3(num_tiles, a.num_kv_heads), dim3(256), 0, stream,
                     a);
  return hipGetLastError();
}

hipError_t launch_prefill_attention(const PrefillArgs& a, int num_tiles, hipStream_t stream) {
  if (a.page_size == 16)
    hipLaunchKernelGGL(prefill_mfma_kernel<true>, dim3(num_tiles * a.num_heads), dim3(256), 0,
                       stream, a);
  else
    hipLaunchKernelGGL(prefill_mfma_kernel<false>, dim3(num_tiles * a.num_heads), dim3(256), 0,
                       stream, a);
  return hipGetLastError();
}

}  // namespace pkv
