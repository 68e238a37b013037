// Internal helpers shared by the gfx950 kernels of libmoira.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moira.h"

namespace moira {

constexpr int kPageSize = 16;
constexpr int kMaxGroup = 16;
constexpr int kMaxPages = 16384;
constexpr int kMaxSegments = 4096;
// Size of the static device scratch of moira_select_pages_noalloc (per GPU).
constexpr size_t kNoAllocScratchBytes = size_t(32) << 20;
constexpr float kLog2e = 1.4426950408889634f;

// Arguments every kernel needs about the problem shape (passed by value).
struct Dims {
  int B, H, G, D, ps, max_pages;
  long long num_phys;
  int sbf;   // page summaries stored as bf16
  int sf8;   // page summaries stored as OCP FP8 E4M3 (neither flag: fp32)
  __host__ __device__ int S() const { return B * H; }
  __host__ __device__ int Hq() const { return H * G; }
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// fp32 -> bf16, round to nearest, ties to even (the 16 dropped bits decide;
// page means are finite, so no NaN case arises)
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

// fp32 -> OCP FP8 E4M3 (bias 7, 3 fraction bits, largest finite 448, no
// infinities), nearest with ties to even, magnitudes from 448 up saturating
// to 448. A value of exponent e (clamped below at -6, the smallest normal
// exponent) lies on the grid of quantum 2^(e-3); the scaling by a power of
// two is exact, so rintf (ties to even) makes the one rounding.
__device__ __forceinline__ uint8_t f32_to_e4m3_rne(float f) {
  const uint32_t sign = (__float_as_uint(f) >> 24) & 0x80u;
  const float a = fabsf(f);
  if (!(a < 448.0f)) return static_cast<uint8_t>(sign | 0x7Eu);   // 448 = 1.75 * 2^8
  int ex;
  (void)frexpf(a, &ex);            // a = m 2^ex, m in [0.5, 1); 0 gives ex = 0
  int e = ex - 1;
  if (e < -6) e = -6;
  int q = static_cast<int>(rintf(ldexpf(a, 3 - e)));   // 0 .. 16
  if (q >= 16) {                   // carried into the next binade
    ++e;
    q = 8;
  }
  if (q >= 8) return static_cast<uint8_t>(sign | static_cast<uint32_t>((e + 7) << 3) | static_cast<uint32_t>(q - 8));
  return static_cast<uint8_t>(sign | static_cast<uint32_t>(q));    // subnormal or zero
}

// A page summary element: the fp64 mean rounded once to fp32 and, for bf16
// (E4M3) summaries, that fp32 value rounded once more to bf16 (E4M3).
__device__ __forceinline__ void store_summary(void* summaries, long long idx, double mean, int sbf,
                                              int sf8) {
  const float f = static_cast<float>(mean);
  if (sbf) static_cast<uint16_t*>(summaries)[idx] = f32_to_bf16_rne(f);
  else if (sf8) static_cast<uint8_t*>(summaries)[idx] = f32_to_e4m3_rne(f);
  else static_cast<float*>(summaries)[idx] = f;
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

// ---- lane pairs by gfx950's permlane swaps (VALU, no LDS crossbar) --------
// lo / hi receive the values of lanes l & ~16 and l | 16 (l & 31 and l | 32):
// the lane itself and its partner at distance 16 (32), lower lane first, so
// that a symmetric combination of the two is the same in both lanes.
__device__ __forceinline__ void lane_pair16(float v, float& lo, float& hi) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(p[0]);
  hi = __uint_as_float(p[1]);
}
__device__ __forceinline__ void lane_pair32(float v, float& lo, float& hi) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  lo = __uint_as_float(p[0]);
  hi = __uint_as_float(p[1]);
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

// ---- DPP wave primitives (gfx9 row_shr / row_bcast): inclusive scans whose
// steps stay inside the VALU, without LDS-crossbar shuffles. Lanes whose DPP
// source lies outside the row read 0 (bound_ctrl), the identity of add and of
// unsigned max.
template <int CTRL, int RM = 0xf, int BM = 0xf>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, RM, BM, true));
}
template <int CTRL, int RM = 0xf, int BM = 0xf>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long v) {
  const uint32_t lo = dpp32<CTRL, RM, BM>(static_cast<uint32_t>(v));
  const uint32_t hi = dpp32<CTRL, RM, BM>(static_cast<uint32_t>(v >> 32));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
// inclusive prefix sum over the 64 lanes (row_shr 1,2,4,8 then row_bcast 15, 31)
__device__ __forceinline__ unsigned long long dpp_incl_add_u64(unsigned long long x) {
  x += dpp64<0x111>(x);
  x += dpp64<0x112>(x);
  x += dpp64<0x114>(x);
  x += dpp64<0x118>(x);
  x += dpp64<0x142, 0xa>(x);
  x += dpp64<0x143, 0xc>(x);
  return x;
}
__device__ __forceinline__ uint32_t dpp_incl_add_u32(uint32_t x) {
  x += dpp32<0x111>(x);
  x += dpp32<0x112>(x);
  x += dpp32<0x114>(x);
  x += dpp32<0x118>(x);
  x += dpp32<0x142, 0xa>(x);
  x += dpp32<0x143, 0xc>(x);
  return x;
}
// Sum over the wave (the same in every lane) and inclusive prefix sum across
// the 64 lanes, both from the DPP scan: six VALU steps instead of six
// LDS-crossbar shuffles.
__device__ __forceinline__ int wave_sum_i32(int v) {
  return __builtin_amdgcn_readlane(static_cast<int>(dpp_incl_add_u32(static_cast<uint32_t>(v))), 63);
}
template <typename T>
__device__ __forceinline__ T wave_incl_scan(T v) {
  static_assert(sizeof(T) == 4, "32-bit lane values");
  return __builtin_bit_cast(T, dpp_incl_add_u32(__builtin_bit_cast(uint32_t, v)));
}
// inclusive prefix max (unsigned); lane 63 holds the wave maximum
__device__ __forceinline__ unsigned long long dpp_incl_max_u64(unsigned long long x) {
  unsigned long long y;
  y = dpp64<0x111>(x); x = y > x ? y : x;
  y = dpp64<0x112>(x); x = y > x ? y : x;
  y = dpp64<0x114>(x); x = y > x ? y : x;
  y = dpp64<0x118>(x); x = y > x ? y : x;
  y = dpp64<0x142, 0xa>(x); x = y > x ? y : x;
  y = dpp64<0x143, 0xc>(x); x = y > x ? y : x;
  return x;
}
__device__ __forceinline__ unsigned long long lane63_u64(unsigned long long x) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x)), 63);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x >> 32)), 63);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
__device__ __forceinline__ unsigned long long wave_max_dpp_u64(unsigned long long x) {
  return lane63_u64(dpp_incl_max_u64(x));
}
__device__ __forceinline__ unsigned long long wave_sum_dpp_u64(unsigned long long x) {
  return lane63_u64(dpp_incl_add_u64(x));
}
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  return __longlong_as_double(static_cast<long long>(
      dpp64<CTRL>(static_cast<unsigned long long>(__double_as_longlong(v)))));
}
// Value of lane t ^ M, for groups of 2M aligned lanes, with direction-free
// DPP patterns: quad_perm for M = 1, 2; row_half_mirror then a quad reversal
// (lane 8a + 4b + c reads 8a + 4(1-b) + c) for M = 4; row_ror by 8, half of
// a 16-lane row, for M = 8; an LDS-crossbar shuffle for M = 16.
template <int M>
__device__ __forceinline__ double xor_lane_f64(double v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16, "partner distance");
  if constexpr (M == 1) return dpp_f64<0xB1>(v);                // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp_f64<0x4E>(v);           // quad_perm [2,3,0,1]
  else if constexpr (M == 4) return dpp_f64<0x1B>(dpp_f64<0x141>(v));  // half mirror, quad_perm [3,2,1,0]
  else if constexpr (M == 8) return dpp_f64<0x128>(v);          // row_ror 8
  else return __shfl_xor(v, 16, 64);
}

// One halving level of group_reduce_scatter_f64: of the K values, the lane
// keeps those whose index has bit 0 equal to `bit` and adds the partner's
// copies of them; the other half goes to the partner. Kept value k2 becomes
// index k2 of the next level.
template <int M, int K>
__device__ __forceinline__ void rs_level_f64(double* v, bool bit) {
#pragma unroll
  for (int k2 = 0; k2 < K / 2; ++k2) {
    const double lo = v[2 * k2], hi = v[2 * k2 + 1];
    const double keep = bit ? hi : lo;
    const double send = bit ? lo : hi;
    v[k2] = keep + xor_lane_f64<M>(send);
  }
}

// Sums over aligned groups of N consecutive lanes of G values per lane
// (G <= N, both powers of two, N <= 32): lane t of a group (t = lane % N)
// returns the group's sum of value t % G. The first log2 G levels halve the
// values held (reduce-scatter), the rest add the partner's copy of the same
// value, so the G sums cost about G + log2(N / G) additions per lane instead
// of G log2 N.
template <int G, int N>
__device__ __forceinline__ double group_reduce_scatter_f64(double (&v)[G], int t) {
  static_assert(G <= N && N <= 32, "one value per lane at most");
  if constexpr (G >= 2) rs_level_f64<1, G>(v, t & 1);
  if constexpr (G >= 4) rs_level_f64<2, G / 2>(v, t & 2);
  if constexpr (G >= 8) rs_level_f64<4, G / 4>(v, t & 4);
  if constexpr (G >= 16) rs_level_f64<8, G / 8>(v, t & 8);
  double x = v[0];
  if constexpr (G <= 1 && N >= 2) x += xor_lane_f64<1>(x);
  if constexpr (G <= 2 && N >= 4) x += xor_lane_f64<2>(x);
  if constexpr (G <= 4 && N >= 8) x += xor_lane_f64<4>(x);
  if constexpr (G <= 8 && N >= 16) x += xor_lane_f64<8>(x);
  if constexpr (G <= 16 && N >= 32) x += xor_lane_f64<16>(x);
  return x;
}

}  // namespace moira
