// Internal helpers shared by the gfx950 kernels of libmoira.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moira.h"

namespace moira {

constexpr int kPageSize = 16;
constexpr int kMaxGroup = 16;
constexpr int kMaxPages = 32768;
constexpr int kMaxSegments = 4096;
constexpr float kLog2e = 1.4426950408889634f;

// Arguments every kernel needs about the problem shape (passed by value).
struct Dims {
  int B, H, G, D, ps, max_pages;
  long long num_phys;
  __host__ __device__ int S() const { return B * H; }
  __host__ __device__ int Hq() const { return H * G; }
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

template <typename T> struct KvElem;
template <> struct KvElem<float> {
  static __device__ __forceinline__ float to_f32(float x) { return x; }
};
template <> struct KvElem<uint16_t> {
  static __device__ __forceinline__ float to_f32(uint16_t x) { return bf16_bits_to_f32(x); }
};

__device__ __forceinline__ void set_status(int32_t* status, int bits) {
  if (status) atomicOr(status, bits);
}

// Validated request length: seq_lens[r] if it lies in [0, max_pages*ps],
// else 0 (reported). An empty request has no pages.
__device__ __forceinline__ int checked_len(const int32_t* seq_lens, int r, const Dims& d,
                                           int32_t* status, bool report) {
  int L = seq_lens[r];
  if (L < 0 || L > d.max_pages * d.ps) {
    if (report) set_status(status, MOIRA_ST_BAD_LEN);
    return 0;
  }
  return L;
}

// Validated physical page id: -1 if out of range.
__device__ __forceinline__ long long checked_phys(const int32_t* block_table, int r, int p,
                                                  const Dims& d, int32_t* status) {
  long long phys = block_table[static_cast<long long>(r) * d.max_pages + p];
  if (phys < 0 || phys >= d.num_phys) {
    set_status(status, MOIRA_ST_BAD_PAGE);
    return -1;
  }
  return phys;
}

// ---- wave64 / block reductions ------------------------------------------
template <typename T>
__device__ __forceinline__ T shfl_xor_t(T v, int m) {
  return __shfl_xor(v, m, 64);
}
__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  return __shfl_xor(v, m, 64);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    unsigned long long o = shfl_xor_u64(v, m);
    v = o > v ? o : v;
  }
  return v;
}
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    unsigned long long o = shfl_xor_u64(v, m);
    v = o < v ? o : v;
  }
  return v;
}
__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_u64(v, m);
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
// Inclusive prefix sum across the 64 lanes of a wave.
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    T u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

}  // namespace moira
