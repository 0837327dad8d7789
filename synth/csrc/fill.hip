// Device fill for the seeded input generator: element i of a buffer gets
// table[top 16 bits of SplitMix64 output (start + i) of the stream at key].
// The table bytes come from the host generator, so host and device values
// are bit-identical.  Holds no attention arithmetic.
#include <cstdint>

#include <hip/hip_runtime.h>

namespace {

__device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

template <typename W>
__global__ __launch_bounds__(256) void fill_kernel(W* dst, uint64_t count, uint64_t start,
                                                   uint64_t key, const W* table) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride) {
    const uint64_t bits = mix64(key + (start + i + 1) * 0x9E3779B97F4A7C15ull);
    dst[i] = table[bits >> 48];
  }
}

}  // namespace

// elem_bytes: 4 (float32 table) or 2 (bfloat16 table).  table: 65536 entries
// on the device.  Returns a hipError_t value (0 on success).
extern "C" int synth_fill(void* dst, uint64_t count, uint64_t start, uint64_t key,
                          const void* table, int elem_bytes, void* stream) {
  if (count == 0) return 0;
  if (!dst || !table || (elem_bytes != 2 && elem_bytes != 4)) return (int)hipErrorInvalidValue;
  uint64_t blocks = (count + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (elem_bytes == 4)
    hipLaunchKernelGGL(fill_kernel<uint32_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint32_t*>(dst), count, start, key,
                       static_cast<const uint32_t*>(table));
  else
    hipLaunchKernelGGL(fill_kernel<uint16_t>, dim3((unsigned)blocks), dim3(256), 0, s,
                       static_cast<uint16_t*>(dst), count, start, key,
                       static_cast<const uint16_t*>(table));
  return (int)hipGetLastError();
}
