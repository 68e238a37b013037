// Measurement aid, not a step of the method: a read-only streaming kernel
// that reads a device buffer once with the same 16-byte non-temporal vector
// loads the scoring and attention kernels use, so that a benchmark can time
// the chip's sustained HBM read rate beside them.
#include "moira_common.h"

namespace moira {

constexpr int kStreamWgs = 2048;      // 8 workgroups per compute unit
constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 8;      // 16-byte loads in flight per thread

// Each thread XORs every 16-byte word it reads and stores one word, so the
// loads are live; sink holds kStreamWgs * kStreamThreads words.
__global__ __launch_bounds__(kStreamThreads) void stream_read_kernel(const u32x4_t* __restrict__ src,
                                                                    long long n16,
                                                                    uint32_t* __restrict__ sink) {
  const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
  long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + (kStreamUnroll - 1) * stride < n16; i += kStreamUnroll * stride) {
    u32x4_t v[kStreamUnroll];
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) v[k] = __builtin_nontemporal_load(src + i + k * stride);
#pragma unroll
    for (int k = 0; k < kStreamUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x] = acc;
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  stream_read_kernel<<<kStreamWgs, kStreamThreads, 0, st>>>(
      static_cast<const u32x4_t*>(src), static_cast<long long>(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace moira
