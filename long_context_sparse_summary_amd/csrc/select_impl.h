// Coverage-rule page selection (MOIRA abstract: for every request, layer, KV
// head and step keep the smallest set of pages whose estimated attention mass
// reaches a fraction gamma).
//
// Two kernels per call:
//  * score (chip-wide, grid = runs of 64-page chunks x segments): for each page the
//    G logits l_h = scale * q_h . kbar_p in fp64 from the fp32 summary, and the
//    page's unnormalised mass w_p = n_p * sum_h exp(l_h) packed into one
//    64-bit order-preserving key (a 12-bit biased binary exponent over the
//    52-bit fraction of the significand). The key depends on the page's own
//    data only, so pages with equal inputs get equal keys and the index tie
//    rule decides between them. Each workgroup also bins its pages into
//    2048 bands of 1/64 octave below a reference key R (the largest key of
//    the previous call on this workspace, stored there) and adds their
//    masses, quantised to exact integers of 2^-F relative to 2^(exp(R)+2),
//    to a per-segment band histogram (LDS, then device atomics: integer
//    sums, so the result does not depend on order).
//  * cut (one workgroup per (request, KV head)): a prefix scan of the band
//    histogram finds the band in which the ranked running mass reaches
//    gamma * total; the pages of that band are compacted into LDS and
//    resolved by a mass-weighted radix select on their keys (8-bit digits),
//    the last <= 64 ranked pairwise with exact ties by page index. This
//    yields a threshold key T and the number of pages of key T to keep (in
//    page order); one block scan writes the kept pages in ascending order.
//    R only steers the binning: when it is unusable (first call, a key more
//    than two octaves above it, or R so far above this call's largest key
//    that the quantised masses would lose resolution) or the boundary band
//    is crowded, the same
//    exact selection runs as a radix select over the keys held in registers
//    (blocked layout, thread t owns pages [tE, tE+E)). The cut stores its
//    largest key as the next R and clears the histogram, so a workspace must
//    be zero-filled before its first call and is ready again after every
//    call.
#pragma once

#include <climits>
#include <type_traits>

#include "moira_common.h"

namespace moira {

constexpr int kScoreChunk = 64;        // pages per score chunk (one lane each in the mass pass)
constexpr int kBands = 2048;           // level-1 bands per segment
constexpr int kBandShift = 46;         // key >> 46: exponent + 6 fraction bits
constexpr int kBandHeadroom = 64;      // one octave of bands above the reference
constexpr int kCutBins = 256;          // digit bins of the in-workgroup radix levels
constexpr int kCandCap = 512;          // boundary-band pages resolved in LDS
constexpr int kRefSlack = 10;          // max bits of mass resolution lost to a high reference
constexpr unsigned long long kMask52 = (1ull << 52) - 1;

// Device workspace of moira_select_pages. The band histogram, the range
// flag and the reference key exist twice and alternate between calls: call
// n scores into parity p (read from `par`), its cut reads parity p, clears
// parity p^1 for call n+1 and stores the new reference and p^1. The score
// kernel copies the reference and parity it used into cur_ref / cur_par, so
// no workgroup of a cut reads a word that another workgroup of the same cut
// writes.
struct SelectWs {
  unsigned long long* hq;      // [S][2][kBands] quantised mass per band, per parity
  unsigned int* hc;            // [S][2][kBands] pages per band, per parity
  unsigned long long* keys;    // [S][max_pages]
  unsigned long long* cmax;    // [S][ceil(max_pages / kScoreChunk)] largest key per score chunk
  unsigned long long* ref;     // [S] reference key R for the next call
  unsigned long long* cur_ref; // [S] reference key the current call scored with
  unsigned int* par;           // [S] parity of the next call
  unsigned int* cur_par;       // [S] parity of the current call
  unsigned int* flag;          // [S][2] bit 0: a key exceeded the fixed-point range
  unsigned int* arrive;        // [S] scoring workgroups of the current call that have
                               // finished (fused select; 0 between calls)
  int fresh;                   // 1: ignore the stored reference keys (exact select)
  unsigned int bytes;          // size of the whole workspace (it starts at hq)
};

__host__ __device__ inline size_t select_ws_bytes(int S, int max_pages) {
  const size_t nch = (static_cast<size_t>(max_pages) + kScoreChunk - 1) / kScoreChunk;
  return static_cast<size_t>(S) *
         (static_cast<size_t>(kBands) * 24 + static_cast<size_t>(max_pages) * 8 + nch * 8 + 48);
}

inline SelectWs select_ws(void* base, int S, int max_pages) {
  SelectWs w;
  const size_t nch = (static_cast<size_t>(max_pages) + kScoreChunk - 1) / kScoreChunk;
  unsigned char* p = static_cast<unsigned char*>(base);
  w.hq = reinterpret_cast<unsigned long long*>(p);   // first: 16-byte pairs stay aligned
  p += static_cast<size_t>(S) * kBands * 16;
  w.hc = reinterpret_cast<unsigned int*>(p);
  p += static_cast<size_t>(S) * kBands * 8;
  w.keys = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * max_pages * 8;
  w.cmax = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * nch * 8;
  w.ref = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * 8;
  w.cur_ref = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * 8;
  w.par = reinterpret_cast<unsigned int*>(p);
  p += static_cast<size_t>(S) * 4;
  w.cur_par = reinterpret_cast<unsigned int*>(p);
  p += static_cast<size_t>(S) * 4;
  w.flag = reinterpret_cast<unsigned int*>(p);
  p += static_cast<size_t>(S) * 8;
  w.arrive = reinterpret_cast<unsigned int*>(p);
  w.fresh = 0;
  w.bytes = static_cast<unsigned int>(select_ws_bytes(S, max_pages));
  return w;
}

// Workspace loads of the cut. In the fused select the cut runs in the last
// scoring workgroup of a segment to finish, on data other workgroups (on
// other XCDs, whose L2 caches are not coherent with this one) wrote with
// write-through agent-scope stores and atomics. It reads them with the
// device-scope (sc1) cache policy, which takes the value at the device's
// coherence point. The loads go through a buffer resource over the
// workspace, so that they stay independent of each other in flight (the
// compiler waits after every agent-scope atomic load, one at a time).
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kCpolSc1 = 16;               // cache policy: device scope
__device__ __forceinline__ __amdgpu_buffer_rsrc_t ws_rsrc(const SelectWs& ws) {
  return __builtin_amdgcn_make_buffer_rsrc(static_cast<void*>(ws.hq), 0,
                                           static_cast<int>(ws.bytes), kBufferWord3);
}
__device__ __forceinline__ int ws_off(const SelectWs& ws, const void* p) {
  return static_cast<int>(static_cast<const char*>(p) - reinterpret_cast<const char*>(ws.hq));
}
template <bool COH>
__device__ __forceinline__ unsigned long long ws_ld(const SelectWs& ws, __amdgpu_buffer_rsrc_t rs,
                                                    const unsigned long long* p) {
  if constexpr (COH)
    return __builtin_bit_cast(unsigned long long,
                              __builtin_amdgcn_raw_buffer_load_b64(rs, ws_off(ws, p), 0, kCpolSc1));
  else return *p;
}
template <bool COH>
__device__ __forceinline__ unsigned int ws_ld(const SelectWs& ws, __amdgpu_buffer_rsrc_t rs,
                                              const unsigned int* p) {
  if constexpr (COH) return __builtin_amdgcn_raw_buffer_load_b32(rs, ws_off(ws, p), 0, kCpolSc1);
  else return *p;
}
// 16 bytes at p (16-byte aligned)
template <bool COH>
__device__ __forceinline__ u32x4_t ws_ld4(const SelectWs& ws, __amdgpu_buffer_rsrc_t rs, const void* p) {
  if constexpr (COH)
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, ws_off(ws, p), 0, kCpolSc1));
  else return *static_cast<const u32x4_t*>(p);
}

// A value every lane holds alike, moved into a scalar register (LDS loads are
// vector loads even at a uniform address).
__device__ __forceinline__ unsigned int uni(unsigned int x) {
  return static_cast<unsigned int>(__builtin_amdgcn_readfirstlane(static_cast<int>(x)));
}
__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ unsigned long long uni(unsigned long long x) {
  return static_cast<unsigned long long>(uni(static_cast<unsigned int>(x))) |
         (static_cast<unsigned long long>(uni(static_cast<unsigned int>(x >> 32))) << 32);
}

// Number of set bits of a wave mask below this lane.
__device__ __forceinline__ unsigned int lanes_below(unsigned long long m) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<unsigned int>(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<unsigned int>(m), 0u));
}

// Slot of this lane in an LDS list that the lanes with `pred` append to: one
// LDS atomic per wave (same-address LDS atomics from every lane serialise).
// Every lane of the wave must call it.
__device__ __forceinline__ int wave_append(bool pred, int* counter) {
  const unsigned long long m = __builtin_amdgcn_ballot_w64(pred);
  int base = 0;
  if ((threadIdx.x & 63) == 0 && m) base = atomicAdd(counter, static_cast<int>(__popcll(m)));
  base = __builtin_amdgcn_readfirstlane(base);
  return base + static_cast<int>(lanes_below(m));
}

// Quantised mass of a key: floor(w * 2^(F - eref)) for a key of binary
// exponent <= eref (w = (1 + frac/2^52) * 2^E). Zero once the shift passes 63.
__device__ __forceinline__ unsigned long long key_mass(unsigned long long key, long long eref,
                                                       int F) {
  const long long ek = static_cast<long long>(key >> 52);
  const long long sh = 52 - F + (eref - ek);
  if (sh >= 64) return 0ull;
  return ((1ull << 52) | (key & kMask52)) >> sh;
}

// Fractional bits of the fixed-point masses of a segment with P pages: the
// sum of P masses, each < 2^(F+1), stays below 2^63.
__device__ __forceinline__ int mass_frac_bits(int P) {
  const int clog = P > 1 ? 32 - __clz(P - 1) : 0;
  return min(52, 62 - clog);
}

// Band of a key below the reference: 0 = heaviest. Monotone non-increasing
// in the key.
__device__ __forceinline__ int band_of(unsigned long long key, unsigned long long ref) {
  const long long b = static_cast<long long>(ref >> kBandShift) + kBandHeadroom -
                      static_cast<long long>(key >> kBandShift);
  return b < 0 ? 0 : (b > kBands - 1 ? kBands - 1 : static_cast<int>(b));
}

// Exponent the fixed-point masses are taken relative to (two octaves above R).
__device__ __forceinline__ long long ref_exponent(unsigned long long ref) {
  return static_cast<long long>(ref >> 52) + 2;
}

// Key of delta times the mass a key encodes (delta in (0, 1]); 0 when that
// falls below the key range. The power-of-two part of the mass is exact, so
// the one rounding is that of the fp64 product delta * mantissa.
__device__ __forceinline__ unsigned long long delta_key(unsigned long long key, double delta) {
  if (key == 0ull) return 0ull;
  const long long biased = static_cast<long long>(key >> 52);
  const double mant = __longlong_as_double(static_cast<long long>((key & kMask52) | (1023ull << 52)));
  const double y = mant * delta;   // the mass is mant * 2^(biased - 2048)
  if (!(y > 0.0)) return 0ull;
  int ex;
  const double m = frexp(y, &ex);  // y = m 2^ex, m in [0.5, 1)
  const long long b2 = biased + ex - 1;
  if (b2 < 0) return 0ull;
  return (static_cast<unsigned long long>(b2) << 52) |
         (static_cast<unsigned long long>(__double_as_longlong(2.0 * m)) & kMask52);
}

template <typename QT> struct QLoad;
template <> struct QLoad<float> {
  static __device__ __forceinline__ double get(const float* q, long long i) { return q[i]; }
};
template <> struct QLoad<uint16_t> {
  static __device__ __forceinline__ double get(const uint16_t* q, long long i) {
    return bf16_bits_to_f32(q[i]);
  }
};

// Lane geometry of the score kernel: LPP lanes share a page, each holding
// DL = D / LPP dimensions of q for all G heads in fp64 registers (G * DL <= 64
// doubles where LPP <= 32 allows) and DL floats of the page's summary row per
// step. A wave step scores PPS = 64 / LPP pages; NS = LPP steps cover a
// 64-page chunk, and up to DEPTH steps of summary loads are in flight. (Fewer
// lanes per page cost registers for q but save cross-lane sums, which
// dominate the step once the loads are in flight.)
// Lane geometry of the score kernel for head_dim D, group capacity G and
// summary elements of SB bytes (4: fp32, 2: bf16, 1: E4M3). LPP lanes share
// a page, each holding DL = D / LPP of its dimensions in pieces of PW
// contiguous elements (one 16-byte load; 8 bytes for bf16 when DL < 8; 16, 8
// or 4 bytes for E4M3).
template <int D, int G, int SB>
struct ScoreGeom {
  static constexpr int pow2_at_least(int x) { return x <= 1 ? 1 : 2 * pow2_at_least((x + 1) / 2); }
  static constexpr int by_q = pow2_at_least((D * G + 63) / 64);
  static constexpr int lpp0 = by_q > D / 16 ? by_q : D / 16;
  static constexpr int lpp_cap = D / 4 < 32 ? D / 4 : 32;  // at least one 4-element piece per lane
  static constexpr int LPP = lpp0 > lpp_cap ? lpp_cap : lpp0;
  static constexpr int PPS = 64 / LPP;
  static constexpr int NS = kScoreChunk / PPS;
  static constexpr int DL = D / LPP;
  static constexpr int PW = SB == 4 ? 4                                   // elements per piece
                           : SB == 2 ? (DL >= 8 ? 8 : 4)
                                     : (DL >= 16 ? 16 : (DL >= 8 ? 8 : 4));
  static constexpr int NP = DL / PW;                            // pieces per lane and page
  static constexpr int RW = PW * SB / 4;                        // 32-bit registers per piece
  static constexpr int LGS = G % 2 == 0 ? G + 1 : G;  // padded logit row (doubles)
  // registers left for loads after q (2 G DL), the sums (2 G) and ~40 others
  static constexpr int budget = 248 - 2 * G * DL - 2 * G - 40;
  static constexpr int steps_fit = budget / (RW * NP);
  static constexpr int pow2_at_most(int x) { return x < 2 ? 1 : 2 * pow2_at_most(x / 2); }
  static constexpr int DEPTH = pow2_at_most(steps_fit < NS ? steps_fit : NS);
  static_assert(LPP >= 4 && LPP <= 32 && NP >= 1 && DL % PW == 0, "score lane geometry");
  static_assert(DEPTH >= 2 && NS % DEPTH == 0, "load ring aligns with chunks");
};

// One summary piece: RW 32-bit registers holding PW fp32 or bf16 elements.
template <typename ST, int PW> struct SumPiece;
template <> struct SumPiece<float, 4> {
  using Raw = u32x4_t;
  static __device__ __forceinline__ void widen(const Raw& v, double (&x)[4]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = static_cast<double>(__uint_as_float(v[e]));
  }
};
template <> struct SumPiece<uint16_t, 8> {
  using Raw = u32x4_t;
  static __device__ __forceinline__ void widen(const Raw& v, double (&x)[8]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[2 * e] = static_cast<double>(__uint_as_float(v[e] << 16));
      x[2 * e + 1] = static_cast<double>(__uint_as_float(v[e] & 0xffff0000u));
    }
  }
};
template <> struct SumPiece<uint16_t, 4> {
  using Raw = u32x2_t;
  static __device__ __forceinline__ void widen(const Raw& v, double (&x)[4]) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      x[2 * e] = static_cast<double>(__uint_as_float(v[e] << 16));
      x[2 * e + 1] = static_cast<double>(__uint_as_float(v[e] & 0xffff0000u));
    }
  }
};

// E4M3 summaries (OCP FP8): gfx950's packed conversion decodes two codes of
// a word (bytes 0-1, or 2-3) into fp32 exactly; fp32 -> fp64 is exact.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void e4m3_word(uint32_t w, double* x) {
  const f32x2_t lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const f32x2_t hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  x[0] = static_cast<double>(lo[0]);
  x[1] = static_cast<double>(lo[1]);
  x[2] = static_cast<double>(hi[0]);
  x[3] = static_cast<double>(hi[1]);
}
template <> struct SumPiece<uint8_t, 16> {
  using Raw = u32x4_t;
  static __device__ __forceinline__ void widen(const Raw& v, double (&x)[16]) {
#pragma unroll
    for (int e = 0; e < 4; ++e) e4m3_word(v[e], x + 4 * e);
  }
};
template <> struct SumPiece<uint8_t, 8> {
  using Raw = u32x2_t;
  static __device__ __forceinline__ void widen(const Raw& v, double (&x)[8]) {
    e4m3_word(v[0], x);
    e4m3_word(v[1], x + 4);
  }
};
template <> struct SumPiece<uint8_t, 4> {
  using Raw = uint32_t;
  static __device__ __forceinline__ void widen(const Raw& v, double (&x)[4]) { e4m3_word(v, x); }
};

// Four query elements: loaded as stored (load), widened to fp64 later (widen).
template <typename QT> struct QLoad4;
template <> struct QLoad4<float> {
  using Raw = float4;
  static __device__ __forceinline__ Raw load(const float* q, long long i) {
    return *reinterpret_cast<const float4*>(q + i);
  }
  static __device__ __forceinline__ Raw zero() { return make_float4(0.f, 0.f, 0.f, 0.f); }
  static __device__ __forceinline__ void widen(const Raw& v, double (&o)[4]) {
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct QLoad4<uint16_t> {
  using Raw = uint2;
  static __device__ __forceinline__ Raw load(const uint16_t* q, long long i) {
    return *reinterpret_cast<const uint2*>(q + i);
  }
  static __device__ __forceinline__ Raw zero() { return make_uint2(0u, 0u); }
  static __device__ __forceinline__ void widen(const Raw& v, double (&o)[4]) {
    o[0] = __uint_as_float(v.x << 16);
    o[1] = __uint_as_float(v.x & 0xffff0000u);
    o[2] = __uint_as_float(v.y << 16);
    o[3] = __uint_as_float(v.y & 0xffff0000u);
  }
};

// ---- block-wide helpers for the cut kernel (NT threads, NT/64 waves) --------
template <int NT>
struct CutShared {
  unsigned long long hq[kCutBins];
  unsigned long long red[2][NT / 64];
  unsigned int redu[NT / 64];
  unsigned long long bc[2];
  int bci[4];
  unsigned long long ck[2][kCandCap];   // candidate keys, double-buffered
  int cp[2][kCandCap];                  // candidate page ids
  unsigned long long zk[kCandCap];      // boundary-band keys as gathered (split cut)
  int zp[kCandCap];                     // and their pages
  int ncl;                              // candidates written to the next buffer
  unsigned long long tk;                // threshold key T
  int take;                             // pages of key T kept, in page order
};


// Each helper: DPP wave step, one LDS slot per wave, barrier, every thread
// folds the NT/64 slots, barrier (so the slots can be reused at once).
template <int NT>
__device__ __forceinline__ unsigned long long block_max_u64(unsigned long long v, CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  const unsigned long long w = wave_max_dpp_u64(v);
  if ((threadIdx.x & 63) == 0) sh.red[0][threadIdx.x >> 6] = w;
  __syncthreads();
  unsigned long long m = sh.red[0][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) m = sh.red[0][i] > m ? sh.red[0][i] : m;
  __syncthreads();
  return m;
}
template <int NT>
__device__ __forceinline__ void block_minmax_u64(unsigned long long& lo, unsigned long long& hi,
                                                 CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  const unsigned long long wl = ~wave_max_dpp_u64(~lo);
  const unsigned long long wh = wave_max_dpp_u64(hi);
  if ((threadIdx.x & 63) == 0) {
    sh.red[0][threadIdx.x >> 6] = wl;
    sh.red[1][threadIdx.x >> 6] = wh;
  }
  __syncthreads();
  lo = sh.red[0][0];
  hi = sh.red[1][0];
#pragma unroll
  for (int i = 1; i < NW; ++i) {
    lo = sh.red[0][i] < lo ? sh.red[0][i] : lo;
    hi = sh.red[1][i] > hi ? sh.red[1][i] : hi;
  }
  __syncthreads();
}
template <int NT>
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  const unsigned long long w = wave_sum_dpp_u64(v);
  if ((threadIdx.x & 63) == 0) sh.red[0][threadIdx.x >> 6] = w;
  __syncthreads();
  unsigned long long t = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) t += sh.red[0][i];
  __syncthreads();
  return t;
}
template <int NT>
__device__ __forceinline__ unsigned long long block_excl_scan_u64(unsigned long long v,
                                                                  unsigned long long* total,
                                                                  CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  const unsigned long long incl = dpp_incl_add_u64(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) sh.red[0][wave] = incl;
  __syncthreads();
  unsigned long long before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const unsigned long long x = sh.red[0][i];
    before += i < wave ? x : 0ull;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}
template <int NT>
__device__ __forceinline__ unsigned int block_excl_scan_u32(unsigned int v, unsigned int* total,
                                                            CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  const unsigned int incl = dpp_incl_add_u32(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) sh.redu[wave] = incl;
  __syncthreads();
  unsigned int before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const unsigned int x = sh.redu[i];
    before += i < wave ? x : 0u;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

__device__ __forceinline__ unsigned long long gamma_target(double gamma, unsigned long long Z) {
  unsigned long long tau;
  const double zt = gamma * static_cast<double>(Z);
  if (!(zt < 18446744073709551615.0)) tau = Z;
  else tau = static_cast<unsigned long long>(ceil(zt));
  if (tau > Z) tau = Z;
  if (tau < 1) tau = 1;
  return tau;
}

// Resolve the candidates held in sh.ck/sh.cp[buf] (count n <= kCandCap;
// every other kept page ranks above them and has mass A in total): leaves
// the threshold key in sh.tk and the number of key-T pages to keep (in page
// order) in sh.take. Wave 0 does the whole resolve, lane l holding
// candidates l, l + 64, ...: each mass-weighted radix level (histogram of
// the 8 key bits below the candidates' common prefix, its prefix sums, the
// compaction of the boundary digit) stays inside the one wave, whose LDS
// operations complete in order, so no level waits at a block barrier. Once
// at most 64 candidates are left they are ranked pairwise. When the caller
// knows that every candidate has the same key >> (pshift + 8), equal to
// pbase >> 8 (the pages of one interior band), the first level takes its
// digit at pshift without the min/max pass. Every thread of the block calls
// it; one barrier at the end publishes the result.
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long x, int l) {
  const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x)), l);
  const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(x >> 32)), l);
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// Candidates ranked pairwise once a level leaves no more than this many
// (one per lane).
constexpr int kPairwiseMax = 64;

template <int NT>
__device__ void resolve_wave(int n, int buf, unsigned long long A, unsigned long long tau,
                             long long eref, int F, bool unit, CutShared<NT>& sh, int pshift,
                             unsigned long long pbase) {
  constexpr int R = kCandCap / 64;   // candidates per lane
  // weight of a candidate: its quantised mass, or 1 when pages are counted
  auto wgt = [&](unsigned long long x) -> unsigned long long {
    return unit ? 1ull : key_mass(x, eref, F);
  };
  const int lane = threadIdx.x & 63;
  const unsigned long long ltmask = (1ull << lane) - 1ull;
  auto finish = [&](unsigned long long T, int take) {
    if (lane == 0) {
      sh.tk = T;
      sh.take = take;
    }
  };
  if (n > kCandCap) n = kCandCap;   // never more: the gathers stop at kCandCap
  if (n <= 0) {  // not reachable while A < tau <= A + total: keep every page
    finish(0ull, 0);
    return;
  }
#pragma unroll 1
  for (int level = 0; level < 12; ++level) {
    if (n <= kPairwiseMax) {
      // pairwise ranking: c' ranks before c if its key is larger, or equal
      // with a lower page index; lane c walks the others by reading their
      // registers; integer sums are exact
      const unsigned long long mk = lane < n ? sh.ck[buf][lane] : 0ull;
      const int mp = lane < n ? sh.cp[buf][lane] : 0;
      const unsigned long long mw = lane < n ? wgt(mk) : 0ull;
      unsigned long long acc = A;
#pragma unroll 4
      for (int c = 0; c < n; ++c) {
        const unsigned long long ok = readlane_u64(mk, c);
        const int op = __builtin_amdgcn_readlane(mp, c);
        const unsigned long long ow = readlane_u64(mw, c);
        if (ok > mk || (ok == mk && op < mp)) acc += ow;
      }
      const bool kept = lane < n && acc < tau;
      const unsigned long long T = ~wave_max_dpp_u64(kept ? ~mk : 0ull);
      const unsigned long long bal = __ballot(kept && mk == T);
      finish(T, static_cast<int>(__popcll(bal)));
      return;
    }
    unsigned long long x[R];
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int i = lane + 64 * k;
      x[k] = i < n ? sh.ck[buf][i] : 0ull;
    }
    int shift;
    unsigned long long base, lo;
    if (level == 0 && pshift >= 0) {
      shift = pshift;
      base = pbase;
      lo = readlane_u64(x[0], 0);   // some candidate's key (n > 64)
    } else {
      unsigned long long hi = 0ull;
      lo = ~0ull;
#pragma unroll
      for (int k = 0; k < R; ++k) {
        if (lane + 64 * k < n) {
          lo = x[k] < lo ? x[k] : lo;
          hi = x[k] > hi ? x[k] : hi;
        }
      }
      lo = ~wave_max_dpp_u64(~lo);
      hi = wave_max_dpp_u64(hi);
      if (lo == hi) {  // all candidates share one key: ties rank by page index
        const unsigned long long qv = wgt(lo);
        const unsigned long long t = qv ? (tau - A + qv - 1) / qv : static_cast<unsigned long long>(n);
        finish(lo, static_cast<int>(t < static_cast<unsigned long long>(n) ? t : n));
        return;
      }
      // mass-weighted histogram on the 8 key bits below the common prefix
      const int hb = 63 - __clzll(static_cast<long long>(lo ^ hi));
      shift = hb > 7 ? hb - 7 : 0;
      base = lo >> shift;
    }
    static_assert(kCutBins == 4 * 64, "four digit bins per lane");
#pragma unroll
    for (int j = 0; j < 4; ++j) sh.hq[4 * lane + j] = 0ull;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      if (lane + 64 * k < n) atomicAdd(&sh.hq[static_cast<int>((x[k] >> shift) - base)], wgt(x[k]));
    }
    unsigned long long h[4];
    unsigned long long lsum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      h[j] = sh.hq[4 * lane + j];
      lsum += h[j];
    }
    const unsigned long long incl = dpp_incl_add_u64(lsum);
    const unsigned long long all = lane63_u64(incl);
    unsigned long long below = incl - lsum;   // mass of the digits below 4 lane
    int bstar = -1;
    unsigned long long anew = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const unsigned long long Sb = all - below;   // mass of digits >= 4 lane + j
      const unsigned long long Sb1 = Sb - h[j];    // mass of digits > 4 lane + j
      if (A + Sb >= tau && A + Sb1 < tau) {
        bstar = 4 * lane + j;
        anew = A + Sb1;
      }
      below += h[j];
    }
    const unsigned long long found = __ballot(bstar >= 0);
    if (found == 0ull) {  // not reachable while A < tau <= A + total: keep all candidates
      finish(lo, n);
      return;
    }
    const int src = static_cast<int>(__ffsll(static_cast<long long>(found))) - 1;
    bstar = __builtin_amdgcn_readlane(bstar, src);
    A = readlane_u64(anew, src);
    // the boundary digit's candidates, compacted into the other buffer
    int o = 0;
#pragma unroll
    for (int k = 0; k < R; ++k) {
      const int i = lane + 64 * k;
      const bool hit = i < n && static_cast<int>((x[k] >> shift) - base) == bstar;
      const unsigned long long m = __ballot(hit);
      if (hit) {
        const int dst = o + static_cast<int>(__popcll(m & ltmask));
        sh.ck[buf ^ 1][dst] = x[k];
        sh.cp[buf ^ 1][dst] = sh.cp[buf][i];
      }
      o += static_cast<int>(__popcll(m));
    }
    n = o;
    buf ^= 1;
  }
  finish(0ull, 0);  // unreachable: 64-bit keys are exhausted within 8 levels
}

template <int NT>
__device__ void resolve_lds(int n, int buf, unsigned long long A, unsigned long long tau,
                            long long eref, int F, bool unit, CutShared<NT>& sh, int pshift = -1,
                            unsigned long long pbase = 0ull) {
  if (threadIdx.x < 64) resolve_wave<NT>(n, buf, A, tau, eref, F, unit, sh, pshift, pbase);
  __syncthreads();
}

// The cut of one segment (request, KV head). Keys stay in registers, in one
// of two layouts:
//  * one workgroup per segment (SPLIT = false): wave w owns pages
//    [64 E w, 64 E (w+1)), lane l holding pages 64 E w + 64 e + l (e < E),
//    so page order is (wave, e, lane);
//  * C workgroups per segment (SPLIT = true), workgroup r writing the kept
//    pages of its own range [2 NT r, 2 NT (r+1)). Each still holds every key
//    of the segment (slot e of wave w: pages (e/2) 2NT + 128 w + 64 (e%2) + l)
//    and loads its own range once more as two slots in (wave, e, lane) order.
// Every workgroup of a segment derives the same threshold from the same keys.
// One LDS exchange gives the largest key and the prefix sums of the band
// histogram; the boundary band's pages are gathered into LDS with wave
// ballots and resolved there. Without a usable reference, or with a crowded
// band, an exact radix select runs over the keys in registers instead. The
// kept set is every page above the threshold key T plus the first `take`
// pages of key T in page order. Ballot counts give each lane the ascending
// position of every kept page it writes: a split workgroup adds the number of
// kept pages before its range, counted from the boundary-band candidates and
// the heavier bands. Range 0 then stores the list length, clears the other
// parity's histogram and range flag for the next call, and records the
// call's largest key as the next reference. Uniform control flow: every
// thread of the block calls it.
template <int NT, int EMAX, bool SPLIT, int RULE, bool COH = false>
__device__ __forceinline__ void cut_segment(const Dims& d, const SelectWs& ws, int s, int r, int C,
                                            const int32_t* __restrict__ seq_lens, double param, int32_t* __restrict__ page_lists,
                                            int32_t* __restrict__ list_lens, unsigned long long ref,
                                            unsigned int par, CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  constexpr int BPT = kBands / NT;  // level-1 bands owned per thread
  constexpr int RANGE = 2 * NT;     // pages per workgroup range (SPLIT)
  using mask_t = typename std::conditional<(EMAX > 32), unsigned long long, unsigned int>::type;
  auto popc = [](mask_t m) -> int {
    return sizeof(mask_t) == 8 ? __popcll(static_cast<unsigned long long>(m))
                               : __popc(static_cast<unsigned int>(m));
  };
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rstart = SPLIT ? r * RANGE : 0;
  // first page of the 64-page row slot e holds (the same for the whole wave);
  // every slot is processed, rows past the table hold no valid page
  auto row = [&](int e) -> int {
    return SPLIT ? (e >> 1) * RANGE + wave * 128 + 64 * (e & 1) : (wave * EMAX + e) * 64;
  };
  auto page = [&](int e) -> int { return row(e) + lane; };
  const unsigned long long ltmask = (1ull << lane) - 1ull;
  int32_t* out = page_lists + static_cast<long long>(s) * d.max_pages;

  // every load goes out before the length is known
  const __amdgpu_buffer_rsrc_t rs = ws_rsrc(ws);
  const int Lraw = seq_lens[s / d.H];
  const unsigned long long* kin = ws.keys + static_cast<long long>(s) * d.max_pages;
  unsigned long long kv[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int p = page(e);
    kv[e] = p < d.max_pages ? ws_ld<COH>(ws, rs, kin + p) : 0ull;
  }
  unsigned long long ko[2] = {0ull, 0ull};  // own range, (wave, e, lane) order
  if (SPLIT) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int p = rstart + wave * 128 + 64 * e + lane;
      ko[e] = p < d.max_pages ? ws_ld<COH>(ws, rs, kin + p) : 0ull;
    }
  }
  const int nslot = (d.max_pages + kScoreChunk - 1) / kScoreChunk;
  // both parities of this thread's bands; the parity picks one once it returns
  // this thread's bands [tid BPT, (tid + 1) BPT) of both parities (the
  // fused select knows its parity and loads only that one)
  par &= 1u;
  const unsigned long long* ghq0 = ws.hq + static_cast<long long>(s) * 2 * kBands + tid * BPT;
  const unsigned int* ghc0 = ws.hc + static_cast<long long>(s) * 2 * kBands + tid * BPT;
  unsigned long long bq0[BPT], bq1[BPT];
  unsigned int bc0[BPT], bc1[BPT];
  static_assert(BPT % 4 == 0, "band loads of 16 bytes");
#pragma unroll
  for (int b = 0; b < BPT; b += 4) {
    const int o0 = COH ? static_cast<int>(par) * kBands : 0;
    const u32x4_t qa = ws_ld4<COH>(ws, rs, ghq0 + o0 + b);
    const u32x4_t qb = ws_ld4<COH>(ws, rs, ghq0 + o0 + b + 2);
    const u32x4_t ca = ws_ld4<COH>(ws, rs, ghc0 + o0 + b);
    bq0[b] = qa[0] | (static_cast<unsigned long long>(qa[1]) << 32);
    bq0[b + 1] = qa[2] | (static_cast<unsigned long long>(qa[3]) << 32);
    bq0[b + 2] = qb[0] | (static_cast<unsigned long long>(qb[1]) << 32);
    bq0[b + 3] = qb[2] | (static_cast<unsigned long long>(qb[3]) << 32);
#pragma unroll
    for (int k = 0; k < 4; ++k) bc0[b + k] = ca[k];
    if constexpr (!COH) {
      const u32x4_t qc = ws_ld4<COH>(ws, rs, ghq0 + kBands + b);
      const u32x4_t qd = ws_ld4<COH>(ws, rs, ghq0 + kBands + b + 2);
      const u32x4_t cb = ws_ld4<COH>(ws, rs, ghc0 + kBands + b);
      bq1[b] = qc[0] | (static_cast<unsigned long long>(qc[1]) << 32);
      bq1[b + 1] = qc[2] | (static_cast<unsigned long long>(qc[3]) << 32);
      bq1[b + 2] = qd[0] | (static_cast<unsigned long long>(qd[1]) << 32);
      bq1[b + 3] = qd[2] | (static_cast<unsigned long long>(qd[3]) << 32);
#pragma unroll
      for (int k = 0; k < 4; ++k) bc1[b + k] = cb[k];
    } else {
#pragma unroll
      for (int k = 0; k < 4; ++k) {   // already this call's parity
        bq1[b + k] = bq0[b + k];
        bc1[b + k] = bc0[b + k];
      }
    }
  }
  const unsigned int fl0 = ws_ld<COH>(ws, rs, ws.flag + 2 * s);
  const unsigned int fl1 = ws_ld<COH>(ws, rs, ws.flag + 2 * s + 1);
  unsigned long long cm = tid < nslot ? ws_ld<COH>(ws, rs, ws.cmax + static_cast<long long>(s) * nslot + tid) : 0ull;
  // the rule parameter and the list pointer (kernel arguments) are fetched
  // from the argument segment now, while the loads above are in flight,
  // instead of at their first use after the exchange
  asm volatile("" ::"s"(param), "s"(out));
  if (tid == 0) {
    sh.bci[0] = -1;
    sh.ncl = 0;
  }

  int L = Lraw;
  if (L < 1 || L > d.max_pages * d.ps) L = 0;
  const int P = (L + d.ps - 1) / d.ps;
  if (P == 0) {  // nothing was scored: the histograms are untouched
    if (tid == 0 && r == 0) list_lens[s] = 0;
    return;
  }
  const unsigned int flagged = par ? fl1 : fl0;
  unsigned long long bq[BPT];
  unsigned int bcnt[BPT];
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    bq[b] = par ? bq1[b] : bq0[b];
    bcnt[b] = par ? bc1[b] : bc0[b];
  }
  const int nch = (P + kScoreChunk - 1) / kScoreChunk;
  if (tid >= nch) cm = 0;
  // lanes of slot e that hold a page of the segment: a prefix of the wave
  auto vmask = [&](int e) -> unsigned long long {
    const int n = P - row(e);
    return n >= 64 ? ~0ull : (n <= 0 ? 0ull : (1ull << n) - 1ull);
  };
  // the same as a per-lane slot mask, for the fallback paths
  mask_t valid = 0;
  auto make_valid = [&]() {
#pragma unroll
    for (int e = 0; e < EMAX; ++e) valid |= mask_t((vmask(e) >> lane) & 1ull) << e;
  };

  // ---- one exchange: largest key, band-histogram prefix sums (of page
  // counts instead of masses when the rule keeps the k heaviest pages)
  constexpr bool unit = RULE == MOIRA_RULE_TOPK;
  unsigned long long own = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) own += unit ? static_cast<unsigned long long>(bcnt[b]) : bq[b];
  const unsigned long long incl = dpp_incl_add_u64(own);
  const unsigned long long wmax = wave_max_dpp_u64(cm);
  if (lane == 63) sh.red[0][wave] = incl;
  if (lane == 0) sh.red[1][wave] = wmax;
  __syncthreads();
  unsigned long long Z = 0, before = 0, kmax = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const unsigned long long x = sh.red[0][w];
    Z += x;
    before += w < wave ? x : 0ull;
    kmax = sh.red[1][w] > kmax ? sh.red[1][w] : kmax;
  }
  before += incl - own;
  const int F = mass_frac_bits(P);
  // The band histogram is usable when every key fit under the fixed-point
  // range and the reference is not so far above this call's largest key that
  // the quantised masses lose more than kRefSlack bits of resolution.
  const bool ref_ok = ref != 0ull && flagged == 0u &&
                      ref_exponent(ref) - static_cast<long long>(kmax >> 52) <= kRefSlack;

  mask_t sel = 0;
  mask_t cand = 0;
  unsigned long long A = 0;     // mass of pages known to rank above every candidate
  unsigned long long tau;
  long long eref;
  bool threshold = false;       // result given as (T, take) in sh
  bool gathered = false;        // boundary band saved in sh.zk / sh.zp (SPLIT)
  int ngath = 0;
  unsigned int lt_all = 0, lt_before = 0;  // this lane's pages of heavier bands

  // weight of a page in the running sum: quantised mass, or 1 for top-k
  auto wgt = [&](unsigned long long x) -> unsigned long long {
    return unit ? 1ull : key_mass(x, eref, F);
  };
  const unsigned long long kbudget = unit ? static_cast<unsigned long long>(param) : 0ull;
  auto target = [&](unsigned long long total) -> unsigned long long {
    return unit ? (kbudget < total ? kbudget : total) : gamma_target(param, total);
  };

  if constexpr (RULE == MOIRA_RULE_TOPDELTA) {
    // keep the pages whose mass is at least delta times the largest: the
    // keys order like the masses, so this is a threshold key
    if (tid == 0) {
      const unsigned long long thr = delta_key(kmax, param);
      sh.tk = thr ? thr - 1ull : 0ull;   // kept: key > tk, i.e. key >= thr
      sh.take = 0;
      sh.bci[2] = thr == 0ull;           // below the key range: every page
    }
    __syncthreads();
    if (sh.bci[2]) {
      make_valid();
      sel = valid;
    } else {
      threshold = true;
    }
  } else if (unit && kbudget >= static_cast<unsigned long long>(P)) {   // the budget covers the segment
    make_valid();
    sel = valid;
  } else if (ref_ok) {
    // ---- level 1 from the band histogram (bands ascend from the heaviest)
    eref = ref_exponent(ref);
    tau = target(Z);
    unsigned long long run = before;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const unsigned long long prev = run;
      run += unit ? static_cast<unsigned long long>(bcnt[b]) : bq[b];
      if (prev < tau && run >= tau) {
        sh.bci[0] = tid * BPT + b;
        sh.bci[1] = static_cast<int>(bcnt[b]);
        sh.bc[0] = prev;
      }
    }
    __syncthreads();
    const int band = sh.bci[0];
    A = sh.bc[0];
    const int nband = sh.bci[1];
    if (band >= 0 && nband <= kCandCap) {
      // gather the band's pages into LDS and count the pages of heavier
      // bands. The band of a key is a function of key >> kBandShift, clamped
      // at both ends. Each lane counts its own band and heavier-band pages
      // with vector operations on 0/1 integers (wave ballots here would put
      // a dozen scalar instructions per slot on the compute unit's one
      // scalar unit, shared by all eight waves); one wave scan of the lane
      // counts and one LDS atomic per wave then place every lane's
      // candidates. Their order in LDS does not matter: the resolve ranks
      // them by key, and the emission orders the kept pages by page.
      const int t = static_cast<int>(ref >> kBandShift) + kBandHeadroom - band;
      const int khi = band == 0 ? INT_MAX : t;
      const unsigned int klo = static_cast<unsigned int>(band == kBands - 1 ? INT_MIN : t);
      const unsigned int kwid = static_cast<unsigned int>(khi) - klo;
      auto kband = [&](int e) {
        return static_cast<unsigned int>(kv[e] >> 32) >> (kBandShift - 32);
      };
      mask_t bm = 0;          // slots of this lane in the band
      unsigned int nb = 0;    // their number
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        // 1 while this lane's page of slot e lies inside the segment
        const unsigned int vld = static_cast<unsigned int>(lane - (P - row(e))) >> 31;
        const unsigned int off = kband(e) - klo;     // klo <= band key <= khi, wrapped
        const unsigned int inb = vld & (off <= kwid ? 1u : 0u);
        bm |= static_cast<mask_t>(inb) << e;
        nb += inb;
        if (SPLIT) {
          const unsigned int hv = vld & (static_cast<int>(kband(e)) > khi ? 1u : 0u);
          lt_all += hv;
          lt_before += (e >> 1) < r ? hv : 0u;
        }
      }
      const unsigned int incl = static_cast<unsigned int>(dpp_incl_add_u64(nb));
      const unsigned int wn = __builtin_amdgcn_readlane(incl, 63);
      int wbase = 0;
      if (lane == 0 && wn) wbase = atomicAdd(&sh.ncl, static_cast<int>(wn));
      wbase = __builtin_amdgcn_readfirstlane(wbase);
      unsigned int o = static_cast<unsigned int>(wbase) + incl - nb;
      // the band holds at most kCandCap pages (its histogram count said so),
      // so a wave whose slots would overrun the store writes nothing
      if (static_cast<unsigned int>(wbase) + wn <= static_cast<unsigned int>(kCandCap)) {
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
          if (bm >> e & 1u) {
            const int p = page(e);
            sh.ck[0][o] = kv[e];
            sh.cp[0][o] = p;
            if (SPLIT) {
              sh.zk[o] = kv[e];
              sh.zp[o] = p;
            }
            ++o;
          }
        }
      }
      __syncthreads();
      ngath = min(sh.ncl, kCandCap);
      // an interior band's pages share key >> kBandShift = t, so the first
      // radix digit is the next 8 key bits
      const bool interior = band > 0 && band < kBands - 1;
      resolve_lds<NT>(ngath, 0, A, tau, eref, F, unit, sh, interior ? kBandShift - 8 : -1,
                      interior ? static_cast<unsigned long long>(t) << 8 : 0ull);
      threshold = true;
      gathered = SPLIT;
    } else if (band < 0) {       // unreachable while tau <= Z: keep everything
      make_valid();
      sel = valid;
    } else {
      make_valid();
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (valid >> e & 1u) {
          const int b = band_of(kv[e], ref);
          if (b < band) sel |= mask_t(1) << e;
          else if (b == band) cand |= mask_t(1) << e;
        }
      }
    }
  } else {
    // ---- no usable reference: exact masses relative to this call's max
    make_valid();
    eref = static_cast<long long>(kmax >> 52);
    unsigned long long lsum = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (valid >> e & 1u) lsum += wgt(kv[e]);
    }
    cand = valid;
    tau = target(block_sum_u64<NT>(lsum, sh));
  }

  // ---- radix select over the candidate masks (fallback paths); every branch
  // below depends only on block-uniform values
  int ncand = threshold ? 0
                        : static_cast<int>(block_sum_u64<NT>(
                              static_cast<unsigned long long>(popc(cand)), sh));
  bool resolved = threshold || ncand == 0;
#pragma unroll 1
  for (int level = 0; level < 12 && !resolved; ++level) {
    unsigned long long lo = ~0ull, hi = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (cand >> e & 1u) {
        lo = kv[e] < lo ? kv[e] : lo;
        hi = kv[e] > hi ? kv[e] : hi;
      }
    }
    block_minmax_u64<NT>(lo, hi, sh);
    if (lo == hi || ncand <= kCandCap) {
      // few enough (or all equal): finish in LDS as a threshold
      if (tid == 0) sh.ncl = 0;
      __syncthreads();
      if (lo == hi) {
        if (tid == 0) {
          const unsigned long long qv = wgt(lo);
          const unsigned long long t = qv ? (tau - A + qv - 1) / qv : static_cast<unsigned long long>(ncand);
          sh.tk = lo;
          sh.take = static_cast<int>(t < static_cast<unsigned long long>(ncand) ? t : ncand);
        }
        __syncthreads();
      } else {
#pragma unroll
        for (int e = 0; e < EMAX; ++e) {
          const bool c = (cand >> e & 1u) != 0u;
          const int o = wave_append(c, &sh.ncl);
          if (c && o < kCandCap) {
            sh.ck[0][o] = kv[e];
            sh.cp[0][o] = page(e);
          }
        }
        __syncthreads();
        resolve_lds<NT>(ncand, 0, A, tau, eref, F, unit, sh);
      }
      threshold = true;
      resolved = true;
      break;
    }
    // mass-weighted histogram on the 8 key bits below the common prefix
    const int hb = 63 - __clzll(static_cast<long long>(lo ^ hi));
    const int shift = hb > 7 ? hb - 7 : 0;
    const unsigned long long base = lo >> shift;
    for (int b = tid; b < kCutBins; b += NT) sh.hq[b] = 0ull;
    if (tid == 0) sh.bci[0] = -1;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (cand >> e & 1u)
        atomicAdd(&sh.hq[static_cast<int>((kv[e] >> shift) - base)], wgt(kv[e]));
    }
    __syncthreads();
    const unsigned long long mine = tid < kCutBins ? sh.hq[tid] : 0ull;
    unsigned long long all;
    const unsigned long long below = block_excl_scan_u64<NT>(mine, &all, sh);
    if (tid < kCutBins) {
      const unsigned long long Sb = all - below;
      const unsigned long long Sb1 = Sb - mine;
      if (A + Sb >= tau && A + Sb1 < tau) {
        sh.bci[0] = tid;
        sh.bc[0] = A + Sb1;
      }
    }
    __syncthreads();
    const int bstar = sh.bci[0];
    if (bstar < 0) break;  // not reachable while A < tau <= A + total holds
    A = sh.bc[0];
    int kept = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (cand >> e & 1u) {
        const int b = static_cast<int>((kv[e] >> shift) - base);
        if (b > bstar) {
          sel |= mask_t(1) << e;
          cand &= ~(mask_t(1) << e);
        } else if (b < bstar) {
          cand &= ~(mask_t(1) << e);
        } else {
          ++kept;
        }
      }
    }
    ncand = static_cast<int>(block_sum_u64<NT>(static_cast<unsigned long long>(kept), sh));
  }
  if (!resolved) sel |= cand;  // keeps the kept mass >= gamma whatever happened

  unsigned int total;
  if (!SPLIT) {
    // ---- kept set: pages above the threshold key T, then the first `take`
    // pages of key T in page order; page order is (wave, slot, lane). With no
    // threshold (unreachable) the selection mask is kept as it stands.
    const unsigned long long T = threshold ? sh.tk : 0ull;
    const unsigned int take = threshold ? static_cast<unsigned int>(sh.take) : 0u;
    auto gmask = [&](int e) -> unsigned long long {
      return threshold ? __ballot(kv[e] > T) & vmask(e) : __ballot((sel >> e & 1u) != 0u);
    };
    auto emask = [&](int e) -> unsigned long long {
      return threshold ? __ballot(kv[e] == T) & vmask(e) : 0ull;
    };
    unsigned int wg = 0, we = 0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      wg += __popcll(gmask(e));
      we += __popcll(emask(e));
    }
    if (lane == 0) sh.redu[wave] = wg | (we << 16);   // each count < 2^15
    __syncthreads();
    unsigned int gacc = 0, eacc = 0, tg = 0, te = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const unsigned int x = sh.redu[w];
      tg += x & 0xffffu;
      te += x >> 16;
      if (w < wave) {
        gacc += x & 0xffffu;
        eacc += x >> 16;
      }
    }
    const unsigned int ntake = min(take, te);
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      const unsigned long long gm = gmask(e);
      const unsigned long long em = emask(e);
      if (gm | em) {
        const bool g = gm >> lane & 1ull;
        const bool q = em >> lane & 1ull;
        const unsigned int gb = gacc + __popcll(gm & ltmask);
        const unsigned int eb = eacc + __popcll(em & ltmask);
        const unsigned int pos = gb + (g ? min(eb, ntake) : eb);
        if (g || (q && eb < ntake)) out[pos] = page(e);
        gacc += __popcll(gm);
        eacc += __popcll(em);
      }
    }
    total = tg + ntake;
  } else {
    // ---- a threshold for every workgroup of the segment (the unreachable
    // no-threshold case keeps every valid page: T = 0 and no limit on take)
    const bool all = !threshold;
    const unsigned long long T = threshold ? sh.tk : 0ull;
    const unsigned int take = threshold ? static_cast<unsigned int>(sh.take) : 0u;
    // gt / eq pages in total and before this range, as four 16-bit fields
    // (each count <= max_pages <= 16384)
    unsigned long long cnt = 0;
    if (gathered) {
      // every key T page and every band page above T is a gathered candidate;
      // the heavier bands were counted while gathering
      if (tid < ngath) {
        const unsigned long long k = sh.zk[tid];
        const bool early = sh.zp[tid] < rstart;
        const unsigned long long g = k > T, q = k == T;
        cnt = g | (q << 16) | ((early ? g : 0ull) << 32) | ((early ? q : 0ull) << 48);
      }
      cnt += static_cast<unsigned long long>(lt_all) |
             (static_cast<unsigned long long>(lt_before) << 32);
    } else {
      unsigned int ga = 0, qa = 0, gb = 0, qb = 0;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        const unsigned long long vm = vmask(e);
        const unsigned int ng = __popcll(__ballot(all || kv[e] > T) & vm);
        const unsigned int nq = all ? 0u : __popcll(__ballot(kv[e] == T) & vm);
        ga += ng;
        qa += nq;
        gb += (e >> 1) < r ? ng : 0u;
        qb += (e >> 1) < r ? nq : 0u;
      }
      if (lane == 0)
        cnt = static_cast<unsigned long long>(ga) | (static_cast<unsigned long long>(qa) << 16) |
              (static_cast<unsigned long long>(gb) << 32) | (static_cast<unsigned long long>(qb) << 48);
    }
    // ---- this workgroup's range, in (wave, e, lane) order; its per-wave
    // counts travel with the segment counts in one exchange (one barrier)
    const int p0 = rstart + wave * 128 + lane;
    const bool g0 = p0 < P && (all || ko[0] > T);
    const bool q0 = p0 < P && !all && ko[0] == T;
    const bool g1 = p0 + 64 < P && (all || ko[1] > T);
    const bool q1 = p0 + 64 < P && !all && ko[1] == T;
    const unsigned long long gm0 = __ballot(g0), em0 = __ballot(q0);
    const unsigned long long gm1 = __ballot(g1), em1 = __ballot(q1);
    const unsigned int wg = __popcll(gm0) + __popcll(gm1);
    const unsigned int we = __popcll(em0) + __popcll(em1);
    const unsigned long long wcnt = wave_sum_dpp_u64(cnt);
    if (lane == 0) {
      sh.red[0][wave] = wcnt;
      sh.redu[wave] = wg | (we << 16);   // each count <= 128
    }
    __syncthreads();
    unsigned long long z = 0;
    unsigned int gacc = 0, eacc = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      z += sh.red[0][w];
      const unsigned int x = sh.redu[w];
      if (w < wave) {
        gacc += x & 0xffffu;
        eacc += x >> 16;
      }
    }
    const unsigned int ngt = static_cast<unsigned int>(z & 0xffffu);
    const unsigned int neq = static_cast<unsigned int>((z >> 16) & 0xffffu);
    const unsigned int ntake = min(take, neq);
    // consistent counts give total <= P; the clamp keeps every write and the
    // stored length inside the segment's list whatever happens
    total = min(ngt + ntake, static_cast<unsigned int>(P));
    gacc += static_cast<unsigned int>((z >> 32) & 0xffffu);
    eacc += static_cast<unsigned int>(z >> 48);
    {
      const unsigned int gb = gacc + __popcll(gm0 & ltmask);
      const unsigned int eb = eacc + __popcll(em0 & ltmask);
      const unsigned int pos = gb + (g0 ? min(eb, ntake) : eb);
      if ((g0 || (q0 && eb < ntake)) && pos < total) out[pos] = p0;
    }
    gacc += __popcll(gm0);
    eacc += __popcll(em0);
    {
      const unsigned int gb = gacc + __popcll(gm1 & ltmask);
      const unsigned int eb = eacc + __popcll(em1 & ltmask);
      const unsigned int pos = gb + (g1 ? min(eb, ntake) : eb);
      if ((g1 || (q1 && eb < ntake)) && pos < total) out[pos] = p0 + 64;
    }
  }

  // ---- range 0: list length; the other parity is cleared for the next call,
  // which scores against this call's largest key
  if (r == 0) {
    const unsigned int np = par ^ 1u;
    unsigned long long* chq = ws.hq + (static_cast<long long>(s) * 2 + np) * kBands + tid * BPT;
    unsigned int* chc = ws.hc + (static_cast<long long>(s) * 2 + np) * kBands + tid * BPT;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      chq[b] = 0ull;
      chc[b] = 0u;
    }
    if (tid == 0) {
      list_lens[s] = static_cast<int>(total);
      ws.flag[2 * s + np] = 0u;
      ws.ref[s] = kmax;
      ws.par[s] = np;
    }
  }
}

// A score workgroup has at most 8 waves (one workgroup per CU).
constexpr int kScoreMaxWaves = 8;
constexpr int kScoreThreads = 64 * kScoreMaxWaves;


// The cut of one segment inside the fused select, by the segment's last
// scoring workgroup (NT = 512 threads). Same result as cut_segment under the
// coverage rule; written so that every per-slot pass is a handful of
// instructions on wave-uniform masks:
//  * keys stay in registers, slot e of wave w holding the 64 pages of row
//    w EMAX + e (page order is (wave, slot, lane));
//  * the band histogram comes from the scoring workgroups (against the
//    previous call's largest key R), or, when R is unusable, is rebuilt here
//    in LDS against this call's largest key, so that every call finds its
//    boundary band the same way;
//  * the boundary band's pages are resolved in LDS (resolve_lds); a crowded
//    band first narrows by mass-weighted radix levels over the keys in
//    registers;
//  * every path ends with a threshold key T and the number `take` of pages of
//    key T kept in page order, and the emission writes the kept pages
//    ascending from scalar ballot masks and lane prefix counts.
// lq / lc are the scoring kernel's LDS band histogram, free by now.
// lst (LDS, NT EMAX ints) stages the list, which then goes out in coalesced rows.
template <int EMAX>
__device__ void cut_fused(const Dims& d, const SelectWs& ws, int s, int P, double gamma,
                          int32_t* __restrict__ page_lists, int32_t* __restrict__ list_lens,
                          unsigned long long ref, unsigned int par, unsigned long long* lq,
                          unsigned int* lc, int* lst, CutShared<kScoreThreads>& sh) {
  constexpr int NT = kScoreThreads;
  constexpr int NW = NT / 64;
  constexpr int BPT = kBands / NT;
  static_assert(BPT == 4, "four bands per thread");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const __amdgpu_buffer_rsrc_t rs = ws_rsrc(ws);
  const int nslot = (d.max_pages + kScoreChunk - 1) / kScoreChunk;
  const int nch = (P + kScoreChunk - 1) / kScoreChunk;
  // slot e of this wave covers pages [row(e), row(e) + 64); vm(e): its valid lanes
  auto row = [&](int e) -> int { return (wave * EMAX + e) * 64; };
  auto vm = [&](int e) -> unsigned long long {
    const int n = P - row(e);
    return n >= 64 ? ~0ull : (n <= 0 ? 0ull : (1ull << n) - 1ull);
  };
  // slots of this wave that hold any page: the per-slot passes skip the rest
  // (a key past the segment reads 0, so it never compares above a threshold)
  const int erows = uni(min(max((P - wave * EMAX * 64 + 63) / 64, 0), EMAX));

  // ---- every load at once: keys, this parity's four bands, a chunk maximum
  const unsigned long long* kin = ws.keys + static_cast<long long>(s) * d.max_pages;
  unsigned long long kv[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int p = row(e) + lane;
    kv[e] = p < P ? ws_ld<true>(ws, rs, kin + p) : 0ull;
  }
  const long long hb0 = (static_cast<long long>(s) * 2 + par) * kBands + tid * BPT;
  const u32x4_t qa = ws_ld4<true>(ws, rs, ws.hq + hb0);
  const u32x4_t qb = ws_ld4<true>(ws, rs, ws.hq + hb0 + 2);
  const u32x4_t ca = ws_ld4<true>(ws, rs, ws.hc + hb0);
  unsigned long long bq[BPT] = {qa[0] | (static_cast<unsigned long long>(qa[1]) << 32),
                                qa[2] | (static_cast<unsigned long long>(qa[3]) << 32),
                                qb[0] | (static_cast<unsigned long long>(qb[1]) << 32),
                                qb[2] | (static_cast<unsigned long long>(qb[3]) << 32)};
  unsigned int bc[BPT] = {ca[0], ca[1], ca[2], ca[3]};
  const unsigned int flagged = ws_ld<true>(ws, rs, ws.flag + 2 * s + par);
  const unsigned long long cm = tid < nch ? ws_ld<true>(ws, rs, ws.cmax + static_cast<long long>(s) * nslot + tid) : 0ull;

  // ---- largest key and the prefix sums of the band masses (one exchange)
  auto exchange = [&](unsigned long long& Z, unsigned long long& before, unsigned long long& kmax,
                      bool with_max) {
    const unsigned long long own = bq[0] + bq[1] + bq[2] + bq[3];
    const unsigned long long incl = dpp_incl_add_u64(own);
    if (lane == 63) sh.red[0][wave] = incl;
    if (with_max) {
      const unsigned long long wmax = wave_max_dpp_u64(cm);
      if (lane == 0) sh.red[1][wave] = wmax;
    }
    __syncthreads();
    Z = 0;
    before = incl - own;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const unsigned long long x = sh.red[0][w];
      Z += x;
      before += w < wave ? x : 0ull;
      if (with_max) kmax = sh.red[1][w] > kmax ? sh.red[1][w] : kmax;
    }
    __syncthreads();   // sh.red is reused
  };
  unsigned long long Z, before, kmax = 0;
  exchange(Z, before, kmax, true);
  const int F = mass_frac_bits(P);
  const bool usable = ref != 0ull && flagged == 0u &&
                      ref_exponent(ref) - static_cast<long long>(kmax >> 52) <= kRefSlack;
  if (!usable) {
    // rebuild the band histogram here, against this call's largest key
    ref = kmax;
    const long long er = ref_exponent(ref);
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      lq[tid * BPT + b] = 0ull;
      lc[tid * BPT + b] = 0u;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      if (row(e) + lane < P) {
        const int b = band_of(kv[e], ref);
        atomicAdd(&lq[b], key_mass(kv[e], er, F));
        atomicAdd(&lc[b], 1u);
      }
    }
    __syncthreads();
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      bq[b] = lq[tid * BPT + b];
      bc[b] = lc[tid * BPT + b];
    }
    exchange(Z, before, kmax, false);
  }
  const long long eref = ref_exponent(ref);
  const unsigned long long tau = gamma_target(gamma, Z);

  // ---- the band in which the ranked running mass reaches tau
  if (tid == 0) {
    sh.bci[0] = -1;
    sh.ncl = 0;
  }
  __syncthreads();
  {
    unsigned long long run = before;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const unsigned long long prev = run;
      run += bq[b];
      if (prev < tau && run >= tau) {
        sh.bci[0] = tid * BPT + b;
        sh.bci[1] = static_cast<int>(bc[b]);
        sh.bc[0] = prev;
      }
    }
  }
  __syncthreads();
  const int band = uni(sh.bci[0]);
  unsigned long long A = uni(sh.bc[0]);   // mass of the heavier bands
  unsigned long long T = 0ull;         // threshold key
  unsigned int take = 0u;              // pages of key T kept, in page order
  if (band < 0) {
    // not reachable while tau <= Z: keep every page (T = 0, no limit)
    take = 0xffffffffu;
  } else {
    // band membership from key >> kBandShift, clamped at both ends
    const int t = static_cast<int>(ref >> kBandShift) + kBandHeadroom - band;
    const int klo = band == kBands - 1 ? INT_MIN : t;
    const int khi = band == 0 ? INT_MAX : t;
    auto kb = [&](int e) -> int {
      return static_cast<int>(static_cast<unsigned int>(kv[e] >> 32) >> (kBandShift - 32));
    };
    unsigned int cand = 0;   // slots of this lane still in play
    unsigned long long cm_[EMAX];   // the same, per slot, as wave masks
#pragma unroll
    for (int e = 0; e < EMAX; ++e) {
      cm_[e] = 0ull;
      if (e < erows) {
        const bool c = kb(e) >= klo && kb(e) <= khi && row(e) + lane < P;
        cm_[e] = __builtin_amdgcn_ballot_w64(c);
        cand |= c ? 1u << e : 0u;
      }
    }
    int ncand = uni(sh.bci[1]);
    const int ncand0 = ncand;
    bool all_equal = false;   // every candidate left has the same key
    // ---- crowded band: mass-weighted radix levels over the keys in registers
#pragma unroll 1
    for (int level = 0; level < 8 && ncand > kCandCap; ++level) {
      unsigned long long lo = ~0ull, hi = 0ull;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (cand >> e & 1u) {
          lo = kv[e] < lo ? kv[e] : lo;
          hi = kv[e] > hi ? kv[e] : hi;
        }
      }
      block_minmax_u64<NT>(lo, hi, sh);
      if (lo == hi) {
        all_equal = true;
        T = lo;
        break;
      }
      const int hbit = 63 - __clzll(static_cast<long long>(lo ^ hi));
      const int shift = hbit > 7 ? hbit - 7 : 0;
      const unsigned long long base = lo >> shift;
      if (tid < kCutBins) sh.hq[tid] = 0ull;
      if (tid == 0) sh.bci[0] = -1;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < EMAX; ++e)
        if (cand >> e & 1u) atomicAdd(&sh.hq[static_cast<int>((kv[e] >> shift) - base)], key_mass(kv[e], eref, F));
      __syncthreads();
      const unsigned long long mine = tid < kCutBins ? sh.hq[tid] : 0ull;
      unsigned long long all;
      const unsigned long long below = block_excl_scan_u64<NT>(mine, &all, sh);
      if (tid < kCutBins) {
        const unsigned long long Sb = all - below;    // mass of digits >= tid
        const unsigned long long Sb1 = Sb - mine;     // mass of digits > tid
        if (A + Sb >= tau && A + Sb1 < tau) {
          sh.bci[0] = tid;
          sh.bc[0] = A + Sb1;
        }
      }
      __syncthreads();
      const int bstar = sh.bci[0];
      if (bstar < 0) break;   // not reachable while A < tau <= A + total
      A = uni(sh.bc[0]);
      int kept = 0;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (cand >> e & 1u) {
          if (static_cast<int>((kv[e] >> shift) - base) != bstar) cand &= ~(1u << e);
          else ++kept;
        }
      }
      ncand = static_cast<int>(block_sum_u64<NT>(static_cast<unsigned long long>(kept), sh));
#pragma unroll
      for (int e = 0; e < EMAX; ++e) cm_[e] = __builtin_amdgcn_ballot_w64((cand >> e & 1u) != 0u);
    }
    if (all_equal) {
      // ties rank by page index: the first `take` of them reach tau
      const unsigned long long qv = key_mass(T, eref, F);
      const unsigned long long tt = qv ? (tau - A + qv - 1) / qv : static_cast<unsigned long long>(ncand);
      take = static_cast<unsigned int>(tt < static_cast<unsigned long long>(ncand) ? tt : ncand);
    } else {
    // ---- gather the remaining candidates into LDS (one LDS atomic per wave)
    // and resolve them there
    {
      // cm_[e]: the slots that hold candidates (most hold none); the
      // per-slot offsets are prefix sums in scalar registers, so the writes
      // of different slots do not wait on each other
      unsigned int pre[EMAX];
      unsigned int wn = 0;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        pre[e] = wn;
        wn += __popcll(cm_[e]);
      }
      int wbase = 0;
      if (lane == 0 && wn) wbase = atomicAdd(&sh.ncl, static_cast<int>(wn));
      wbase = __builtin_amdgcn_readfirstlane(wbase);
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        if (cand >> e & 1u) {
          const unsigned int o = wbase + pre[e] + lanes_below(cm_[e]);
          if (o < kCandCap) {
            sh.ck[0][o] = kv[e];
            sh.cp[0][o] = row(e) + lane;
          }
        }
      }
    }
    __syncthreads();
    const int ng = min(uni(sh.ncl), kCandCap);
    // the candidates of an interior band not narrowed by a level above share
    // key >> kBandShift = t
    const bool interior = band > 0 && band < kBands - 1 && ncand0 <= kCandCap;
    resolve_lds<NT>(ng, 0, A, tau, eref, F, false, sh, interior ? kBandShift - 8 : -1,
                    interior ? static_cast<unsigned long long>(t) << 8 : 0ull);
    T = uni(sh.tk);
    take = uni(static_cast<unsigned int>(sh.take));
    }
  }

  // ---- emission: pages with key > T, then the first `take` of key T. A
  // page past the segment holds key 0, so it never compares above T and
  // only the key-T masks need the valid lanes. Counts per slot first; their
  // prefix sums (wave-uniform, scalar) then give every slot its offsets, so
  // the writes of different slots are independent.
  unsigned int cg[EMAX], cq[EMAX];
  unsigned int wg = 0, wq = 0;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    cg[e] = e < erows ? __popcll(__builtin_amdgcn_ballot_w64(kv[e] > T)) : 0u;
    cq[e] = e < erows ? __popcll(__builtin_amdgcn_ballot_w64(kv[e] == T) & vm(e)) : 0u;
    wg += cg[e];
    wq += cq[e];
  }
  if (lane == 0) sh.redu[wave] = wg | (wq << 16);   // each count <= 64 EMAX < 2^16
  __syncthreads();
  unsigned int gacc = 0, eacc = 0, ngt = 0, neq = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const unsigned int x = uni(sh.redu[w]);
    ngt += x & 0xffffu;
    neq += x >> 16;
    gacc += w < wave ? (x & 0xffffu) : 0u;
    eacc += w < wave ? (x >> 16) : 0u;
  }
  const unsigned int ntake = min(take, neq);
  const unsigned int total = min(ngt + ntake, static_cast<unsigned int>(P));
  int32_t* out = page_lists + static_cast<long long>(s) * d.max_pages;
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const unsigned int bg = gacc, bq = eacc;   // kept-above and key-T pages before this slot
    gacc += cg[e];
    eacc += cq[e];
    if (e < erows) {
      const bool g = kv[e] > T;
      const bool q = kv[e] == T && ((vm(e) >> lane) & 1ull);
      const unsigned long long gm = __builtin_amdgcn_ballot_w64(g);
      const unsigned long long qm = __builtin_amdgcn_ballot_w64(q);
      // pages of key T before this one (page order); a page above T goes
      // after min(that, ntake) of them, a key-T page is kept while below ntake
      const unsigned int eb = bq + lanes_below(qm);
      const unsigned int pos = bg + lanes_below(gm) + min(eb, ntake);
      if ((g || (q && eb < ntake)) && pos < total) lst[pos] = row(e) + lane;
    }
  }
  __syncthreads();
  for (int i = tid; i < static_cast<int>(total); i += NT) out[i] = lst[i];

  // ---- for the next call: the length, the other parity cleared, R
  const unsigned int np = par ^ 1u;
  const long long cb = (static_cast<long long>(s) * 2 + np) * kBands + tid * BPT;
  *reinterpret_cast<u32x4_t*>(ws.hq + cb) = u32x4_t{0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4_t*>(ws.hq + cb + 2) = u32x4_t{0u, 0u, 0u, 0u};
  *reinterpret_cast<u32x4_t*>(ws.hc + cb) = u32x4_t{0u, 0u, 0u, 0u};
  if (tid == 0) {
    list_lens[s] = static_cast<int>(total);
    ws.flag[2 * s + np] = 0u;
    ws.ref[s] = kmax;
    ws.par[s] = np;
  }
}

// A score workgroup has 8 waves on the fixed single-request grid (one
// workgroup per CU) and 4 on the planned batch grid (two per CU); the kernel
// takes the count from blockDim and is compiled for the larger.

// One request: grid (ceil(nch / (waves cpw)), B*H) over the nch 64-page
// chunks of max_pages; a batch: the planned grid. Each wave
// scores cpw consecutive 64-page chunks of one segment: the summary rows of
// the next DEPTH-1 steps and the block-table entries of the next chunk are in
// flight while a step is computed. Per step the LPP lanes of a page form
// partial dot products for all G heads, summed across the group with DPP
// moves; the logits are staged in LDS so that the per-page tail (softmax mass
// and key, histogram) runs with one lane per page over the whole chunk.
// The workgroup's band counts go to the segment histogram at the end.
// The step's K/V append, done by the score wave that owns the request's tail
// page before it scores (APPEND variant): k_new/v_new of (request, KV head)
// go to token slot seq_lens-1 of the tail page, whose mean key is recomputed
// in fp64 in token order exactly as the append kernel does, stored, and used
// for that page's score instead of the summary row in memory.
struct AppendArgs {
  const uint16_t* k_new;
  const uint16_t* v_new;
  uint16_t* k_pool;
  uint16_t* v_pool;
  void* summaries;    // the tail page's new mean is stored through this pointer
};

// Self-planned split of the score work for a batch of requests, whose
// lengths differ: the workgroups read seq_lens and share the C = H * sum_r
// nch_r chunks (nch_r: 64-page chunks of request r) out by segment. With the
// quota q_c = max(4, ceil(C / (nwg - S))) chunks per workgroup, segment s of
// request r gets n_r = max(1, ceil(nch_r / q_c)) workgroups, so sum n <= C /
// q_c + S <= nwg, and workgroup i of them takes chunks [i nch_r / n_r,
// (i + 1) nch_r / n_r). base (LDS, B ints) receives the first workgroup of
// every request; tmp (LDS, one int per wave) is scratch. Called by every
// thread; false when workgroup w has no segment.
__device__ __forceinline__ int score_chunks_of(const Dims& d, int L) {
  if (L < 0 || L > d.max_pages * d.ps) L = 0;
  const int P = (L + d.ps - 1) / d.ps;
  return (P + kScoreChunk - 1) / kScoreChunk;
}

__device__ bool plan_score_wg(const Dims& d, const int32_t* __restrict__ seq_lens, int nwg, int w,
                              int* base, int* tmp, int& s, int& c_begin, int& c_end, bool& first,
                              int& n_seg) {
  const int B = d.B, H = d.H, S = d.S();
  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int nt = blockDim.x;
  const int per = (B + nt - 1) / nt;
  const int r0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (r0 + i < B) local += score_chunks_of(d, seq_lens[r0 + i]);
  int incl = wave_incl_scan<int>(local);
  if ((tid & 63) == 63) tmp[wave] = incl;
  __syncthreads();
  long long C = 0;
  for (int v = 0; v < nt / 64; ++v) C += tmp[v];
  C *= H;
  long long qc = (C + (nwg - S) - 1) / (nwg - S);
  if (qc < nt / 64) qc = nt / 64;   // at least one chunk per wave
  __syncthreads();   // tmp is reused
  local = 0;
  for (int i = 0; i < per; ++i) {
    if (r0 + i < B) {
      const long long n = (score_chunks_of(d, seq_lens[r0 + i]) + qc - 1) / qc;
      local += H * static_cast<int>(n < 1 ? 1 : n);
    }
  }
  incl = wave_incl_scan<int>(local);
  if ((tid & 63) == 63) tmp[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int v = 0; v < nt / 64; ++v) {
    before += v < wave ? tmp[v] : 0;
    total += tmp[v];
  }
  int run = before + incl - local;
  for (int i = 0; i < per; ++i) {
    if (r0 + i < B) {
      base[r0 + i] = run;
      const long long n = (score_chunks_of(d, seq_lens[r0 + i]) + qc - 1) / qc;
      run += H * static_cast<int>(n < 1 ? 1 : n);
    }
  }
  __syncthreads();
  if (w >= total) return false;
  int lo = 0, hi = B - 1;   // last r with base[r] <= w
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (base[mid] <= w) lo = mid;
    else hi = mid - 1;
  }
  const int r = lo;
  const int n_r = ((r + 1 < B ? base[r + 1] : total) - base[r]) / H;
  const int k = w - base[r];
  const int j = k / n_r;
  const int i = k - j * n_r;
  const int nch = score_chunks_of(d, seq_lens[r]);
  s = r * H + j;
  c_begin = static_cast<int>((static_cast<long long>(i) * nch) / n_r);
  c_end = static_cast<int>((static_cast<long long>(i + 1) * nch) / n_r);
  first = i == 0;
  n_seg = n_r;
  return true;
}

// Outputs of the cut when it runs inside the scoring kernel (fused select).
struct CutArgs {
  double gamma;
  int32_t* page_lists;
  int32_t* list_lens;
};

// CUT_EMAX > 0: the fused select. Page keys and chunk maxima are stored
// through to the device's coherence point (agent-scope stores; the band
// histogram is built with atomics), every workgroup of a segment then counts
// itself in on ws.arrive, and the last one to arrive runs the segment's cut
// (one workgroup, CUT_EMAX key slots per lane), resets the counter and
// leaves the workspace ready for the next call. No workgroup waits on
// another. Needs 8-wave workgroups.
template <typename QT, typename ST, int D, int G, bool APPEND, int CUT_EMAX = 0>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    Dims d, const QT* __restrict__ q, const ST* __restrict__ summaries,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, float scale,
    SelectWs ws, int cpw, int nwg, int sw, AppendArgs app, int32_t* status, CutArgs cut) {
  constexpr bool FUSED = CUT_EMAX > 0;
  // one value from each 64-byte line of the argument segment, asked for at
  // entry: the five lines are fetched together, with one wait, instead of
  // the line holding the append and cut arguments a round trip after the
  // others
  asm volatile("" ::"s"(d.B), "s"(seq_lens), "s"(sw), "s"(status), "s"(gridDim.x), "s"(blockDim.x));
  using Geo = ScoreGeom<D, G, static_cast<int>(sizeof(ST))>;
  constexpr int LPP = Geo::LPP, PPS = Geo::PPS, NS = Geo::NS, DL = Geo::DL;
  constexpr int PW = Geo::PW, NP = Geo::NP;
  constexpr int LGS = Geo::LGS, DEPTH = Geo::DEPTH;
  using Piece = SumPiece<ST, PW>;
  using Raw = typename Piece::Raw;
  __shared__ unsigned long long lq[kBands];
  __shared__ unsigned int lc[kBands];
  __shared__ double lg[kScoreMaxWaves][kScoreChunk * LGS];
  __shared__ int over;
  __shared__ __align__(16) ST tail_sum[APPEND ? D : 1];   // the appended page's new summary
  // the cut's LDS, declared only in the fused variants
  __shared__ __align__(16) unsigned char csh_raw[FUSED ? sizeof(CutShared<kScoreThreads>) : 16];
  __shared__ int cut_list[FUSED ? kScoreThreads * CUT_EMAX : 1];
  __shared__ int last_arriver;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t = lane % LPP;   // dimension slice of this lane
  const int pg = lane / LPP;  // page of a step this lane works on
  // the segment and chunks of this workgroup: a fixed grid (blockIdx.y is
  // the segment; the first sw waves score cpw chunks each, the others only
  // take part in the histogram and the cut) or, with nwg > 0, the batch
  // split planned from seq_lens
  int s = blockIdx.y;
  const int nw = blockDim.x >> 6;        // waves of the workgroup
  const int nsw = sw > 0 && sw < nw ? sw : nw;   // scoring waves of the fixed grid
  int cw0 = blockIdx.x * nsw * cpw;      // first chunk of the workgroup
  int cwe = cw0 + nsw * cpw;             // end of the workgroup's chunks
  int wcpw = cpw;                        // chunks per wave
  bool first = blockIdx.x == 0;          // scores the segment's first chunk
  int n_seg = gridDim.x;                 // workgroups of this segment
  if (nwg > 0) {
    if (!plan_score_wg(d, seq_lens, nwg, blockIdx.x, reinterpret_cast<int*>(lq),
                       reinterpret_cast<int*>(lc), s, cw0, cwe, first, n_seg)) return;
    wcpw = (cwe - cw0 + nw - 1) / nw;
    __syncthreads();   // lq and lc are the histogram again
  }
  const int r = s / d.H;
  const int j = s - r * d.H;
  int c0 = cw0 + wave * wcpw;            // first chunk of this wave
  int cend = cwe;                        // end of this wave's chunks
  if (nwg == 0 && nsw < nw && wave == nsw) {
    // the table's chunks past those of the scoring waves (at most one per
    // workgroup, a short last chunk of the table) go to wave nsw of the
    // first workgroups
    const int nchg = nsw * cpw * static_cast<int>(gridDim.x);
    const int leftover = (d.max_pages + kScoreChunk - 1) / kScoreChunk - nchg;
    if (static_cast<int>(blockIdx.x) < leftover) {
      c0 = nchg + static_cast<int>(blockIdx.x);
      cend = c0 + 1;
    }
  }
  const int32_t* trow = block_table + static_cast<long long>(r) * d.max_pages;

  // every load that does not depend on the request length goes out first.
  // In the split select the length, the reference key and its parity are
  // vector (buffer) loads, waited for where they are first used: as scalar
  // loads they would share one wait with the kernel arguments the table
  // row's address needs (scalar loads return out of order), and the row
  // would go out a round trip later (128k step: 41.35 -> 41.24 us). The
  // fused select measured no faster with vector loads and keeps scalar ones.
  unsigned int Lv, parv;
  u32x2_t refv;
  if constexpr (FUSED) {
    Lv = static_cast<unsigned int>(seq_lens[r]);
    const unsigned long long rv = ws.ref[s];
    refv = u32x2_t{static_cast<uint32_t>(rv), static_cast<uint32_t>(rv >> 32)};
    parv = ws.par[s];
  } else {
    const __amdgpu_buffer_rsrc_t rsl = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(seq_lens), 0, d.B * 4, kBufferWord3);
    Lv = __builtin_amdgcn_raw_buffer_load_b32(rsl, r * 4, 0, 0);
    const __amdgpu_buffer_rsrc_t rsw = ws_rsrc(ws);
    refv = __builtin_amdgcn_raw_buffer_load_b64(rsw, ws_off(ws, ws.ref + s), 0, 0);
    parv = __builtin_amdgcn_raw_buffer_load_b32(rsw, ws_off(ws, ws.par + s), 0, 0);
  }
  // q as stored; widened to fp64 once the first summary loads are out. Only
  // waves with chunks load it (the others never score).
  using QL = QLoad4<QT>;
  typename QL::Raw qraw[G][NP][PW / 4];
  if (c0 < cend) {   // uniform over the wave
    // G is the compiled group capacity; heads d.G .. G-1 are padding with a
    // zero query and take no part in the mass
    const long long qbase = (static_cast<long long>(r) * d.Hq() + static_cast<long long>(j) * d.G) * D;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bool real = g < d.G;           // padding heads read head 0 and are zeroed
      // piece i of this lane covers dimensions (i LPP + t) PW .. + PW
#pragma unroll
      for (int i = 0; i < NP; ++i) {
#pragma unroll
        for (int h = 0; h < PW / 4; ++h)
          qraw[g][i][h] = QL::load(q, qbase + (real ? g : 0) * D + (i * LPP + t) * PW + 4 * h);
      }
    }
  } else {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < NP; ++i)
#pragma unroll
        for (int h = 0; h < PW / 4; ++h) qraw[g][i][h] = QL::zero();
  }
  int raw_next = -1;  // table entry of this lane's page in the next chunk
  if (c0 * kScoreChunk + lane < d.max_pages) raw_next = trow[c0 * kScoreChunk + lane];
  for (int b = tid; b < kBands; b += blockDim.x) {
    lq[b] = 0ull;
    lc[b] = 0u;
  }
  if (tid == 0) over = 0;

  int L = static_cast<int>(uni(Lv));
  // a fresh call scores as if no earlier call had left a reference key: the
  // cut then takes the exact select, and no histogram is read
  const unsigned long long ref =
      ws.fresh ? 0ull : (static_cast<unsigned long long>(uni(refv.y)) << 32) | uni(refv.x);
  const unsigned int par = uni(parv) & 1u;
  if (tid == 0 && first) {   // what this call scores with, for its cut
    ws.cur_ref[s] = ref;
    ws.cur_par[s] = par;
  }
  if (L < 0 || L > d.max_pages * d.ps) {
    if (tid == 0 && first && j == 0) set_status(status, MOIRA_ST_BAD_LEN);
    L = 0;
  }
  const int P = (L + d.ps - 1) / d.ps;
  const int nch = (P + kScoreChunk - 1) / kScoreChunk;
  if (APPEND && L == 0 && tid == 0 && first && j == 0)
    set_status(status, MOIRA_ST_BAD_LEN);   // nothing was advanced: no slot to write
  if (cw0 < nch) {   // uniform over the workgroup; idle workgroups of a fused
                     // select still count themselves in below
  const int c1 = min(min(c0 + wcpw, cend), nch);
  const long long eref = ref_exponent(ref);
  const int F = mass_frac_bits(P);
  const double dscale = static_cast<double>(scale);
  const int nslot = (d.max_pages + kScoreChunk - 1) / kScoreChunk;
  double* lgw = lg[wave];

  // validated physical page of this lane's page in chunk c (-1: none)
  auto phys_of = [&](int raw, int c) -> int {
    const int p = c * kScoreChunk + lane;
    if (p >= P) return -1;
    if (raw < 0 || static_cast<long long>(raw) >= d.num_phys) {
      set_status(status, MOIRA_ST_BAD_PAGE);
      return -1;
    }
    return raw;
  };
  // summary loads of step `st` of a chunk whose per-lane pages are `ph`
  // (non-temporal: every summary row is read once per call)
  auto issue = [&](Raw (&v)[NP], int ph, int st) {
    const int pp = __shfl(ph, st * PPS + pg, 64);
    const long long row = pp >= 0 ? pp : 0;  // a dead page reads page 0 and is ignored
    const Raw* src = reinterpret_cast<const Raw*>(summaries + (row * d.H + j) * D);
#pragma unroll
    for (int i = 0; i < NP; ++i) v[i] = __builtin_nontemporal_load(src + i * LPP + t);
  };

  // the wave's state from its first loads on: the first steps go out before
  // the block barrier that publishes the cleared histogram, which the wave
  // first needs after its first chunk's dot products
  Raw buf[DEPTH][NP];
  int ph_cur = -1;
  int ph_next = -1;
  double qr[G][DL];
  // the tail page (P - 1) and, in APPEND mode, the step's token written
  // into it by the wave that scores it. When the tail page lies in the
  // wave's first chunk its physical page is already in a lane (no extra
  // round trip); its token loads then travel with the first summary loads.
  const int pt = P - 1;
  const int ct = pt / kScoreChunk;                 // its chunk
  const int st_t = (pt - ct * kScoreChunk) / PPS;  // its step in the chunk
  const int pg_t = (pt - ct * kScoreChunk) - st_t * PPS;
  bool tail_ok = false;
  if (c0 < c1) {  // uniform over the wave
    ph_cur = phys_of(raw_next, c0);
    raw_next = -1;
    if (c0 + 1 < c1) raw_next = trow[(c0 + 1) * kScoreChunk + lane];
    if (APPEND && ct >= c0 && ct < c1) {
      const int slot = (L - 1) - pt * d.ps;
      // uniform over the wave: kept in a scalar register
      const int phys = __builtin_amdgcn_readfirstlane(
          ct == c0 ? __shfl(ph_cur, pt - c0 * kScoreChunk, 64) : trow[pt]);
      tail_ok = phys >= 0 && static_cast<long long>(phys) < d.num_phys;
      if (!tail_ok) {
        if (lane == 0) set_status(status, MOIRA_ST_BAD_PAGE);
      } else {
        // the tail wave appends before it starts streaming summaries (one
        // round trip; its chunk is the last one, usually short): the new
        // token goes into the pool and the page's mean is recomputed in
        // fp64, token order, exactly as the append kernel does
        const long long page_base = (static_cast<long long>(phys) * d.H + j) * d.ps * D;
        const long long src = (static_cast<long long>(r) * d.H + j) * D;
        const bool act = 2 * lane < D;       // lane l owns dimensions 2l, 2l+1
        const int cc = act ? 2 * lane : 0;
        const uint32_t kn = *reinterpret_cast<const uint32_t*>(app.k_new + src + cc);
        const uint32_t vn = *reinterpret_cast<const uint32_t*>(app.v_new + src + cc);
        uint32_t prev[kPageSize];   // every slot of the page (in bounds); the first `slot` are summed
#pragma unroll
        for (int t2 = 0; t2 < kPageSize; ++t2)
          prev[t2] = *reinterpret_cast<const uint32_t*>(app.k_pool + page_base + static_cast<long long>(t2) * D + cc);
        if (act) {
          *reinterpret_cast<uint32_t*>(app.k_pool + page_base + static_cast<long long>(slot) * D + cc) = kn;
          *reinterpret_cast<uint32_t*>(app.v_pool + page_base + static_cast<long long>(slot) * D + cc) = vn;
          double a0 = 0.0, a1 = 0.0;
#pragma unroll
          for (int t2 = 0; t2 < kPageSize; ++t2) {
            if (t2 < slot) {
              a0 += static_cast<double>(__uint_as_float(prev[t2] << 16));
              a1 += static_cast<double>(__uint_as_float(prev[t2] & 0xffff0000u));
            }
          }
          a0 += static_cast<double>(__uint_as_float(kn << 16));
          a1 += static_cast<double>(__uint_as_float(kn & 0xffff0000u));
          const double n = static_cast<double>(slot + 1);
          const float m0 = static_cast<float>(a0 / n), m1 = static_cast<float>(a1 / n);
          // the tail row is never read through `summaries` after this: its
          // step takes the new summary from LDS
          const long long srow = (static_cast<long long>(phys) * d.H + j) * D + cc;
          if (sizeof(ST) == 2) {
            const uint16_t b0 = f32_to_bf16_rne(m0), b1 = f32_to_bf16_rne(m1);
            *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(app.summaries) + srow) =
                static_cast<uint32_t>(b0) | (static_cast<uint32_t>(b1) << 16);
            reinterpret_cast<uint16_t*>(tail_sum)[cc] = b0;
            reinterpret_cast<uint16_t*>(tail_sum)[cc + 1] = b1;
          } else if (sizeof(ST) == 1) {
            const uint8_t b0 = f32_to_e4m3_rne(m0), b1 = f32_to_e4m3_rne(m1);
            *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(app.summaries) + srow) =
                static_cast<uint16_t>(b0 | (b1 << 8));
            reinterpret_cast<uint8_t*>(tail_sum)[cc] = b0;
            reinterpret_cast<uint8_t*>(tail_sum)[cc + 1] = b1;
          } else {
            *reinterpret_cast<float2*>(static_cast<float*>(app.summaries) + srow) = make_float2(m0, m1);
            reinterpret_cast<float*>(tail_sum)[cc] = m0;
            reinterpret_cast<float*>(tail_sum)[cc + 1] = m1;
          }
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }

#pragma unroll
    for (int k = 0; k < DEPTH - 1; ++k) issue(buf[k], ph_cur, k);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const double keep = g < d.G ? 1.0 : 0.0;
#pragma unroll
      for (int i = 0; i < NP; ++i) {
#pragma unroll
        for (int h = 0; h < PW / 4; ++h) {
          double v[4];
          QL::widen(qraw[g][i][h], v);
#pragma unroll
          for (int e = 0; e < 4; ++e) qr[g][i * PW + 4 * h + e] = v[e] * keep;
        }
      }
    }
  }
  __syncthreads();  // histogram cleared

  if (c0 < c1) {  // uniform over the wave

#pragma unroll 1
    for (int c = c0; c < c1; ++c) {
      if (c + 1 < c1) {
        ph_next = phys_of(raw_next, c + 1);
        raw_next = -1;
        if (c + 2 < c1) raw_next = trow[(c + 2) * kScoreChunk + lane];
      }
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        const int sn = st + DEPTH - 1;
        if (sn < NS) issue(buf[sn % DEPTH], ph_cur, sn);
        else if (c + 1 < c1) issue(buf[sn % DEPTH], ph_next, sn - NS);
        // a step whose pages all lie past the request's end is not scored
        // (its loads went out all the same: the load ring stays in order)
        if (c * kScoreChunk + st * PPS < P) {   // uniform over the wave
        double acc[G];
#pragma unroll
        for (int g = 0; g < G; ++g) acc[g] = 0.0;
        // the freshly appended tail page scores from its new mean (a branch
        // uniform over the wave, taken on one step of one wave)
        if (APPEND && tail_ok && c == ct && st == st_t) {
          if (pg == pg_t) {
#pragma unroll
            for (int i = 0; i < NP; ++i)
              buf[st % DEPTH][i] = *reinterpret_cast<const Raw*>(&tail_sum[(i * LPP + t) * PW]);
          }
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
          double x[PW];
          Piece::widen(buf[st % DEPTH][i], x);
#pragma unroll
          for (int e = 0; e < PW; ++e)
#pragma unroll
            for (int g = 0; g < G; ++g) acc[g] = fma(qr[g][i * PW + e], x[e], acc[g]);
        }
        // lane t < G of the page's lanes ends with head t's logit
        const double mine = group_reduce_scatter_f64<G, LPP>(acc, t);
        if (t < G) lgw[(st * PPS + pg) * LGS + t] = mine;
        }
      }
      // LDS accesses of one wave complete in order; keep the compiler's too
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // one lane per page: mass, key, histogram
      const int p = c * kScoreChunk + lane;
      unsigned long long key = 0;
      if (p < P) {
        if (ph_cur >= 0) {
          double l[G];
          double mu = -INFINITY;
#pragma unroll
          for (int g = 0; g < G; ++g) {
            l[g] = g < d.G ? lgw[lane * LGS + g] * dscale : -INFINITY;   // padding heads: no mass
            mu = fmax(mu, l[g]);
          }
          double part = 0.0;
#pragma unroll
          for (int g = 0; g < G; ++g) part += exp(l[g] - mu);
          const int n = min(d.ps, L - p * d.ps);
          const double v = static_cast<double>(n) * part;         // in [1, 16G]
          double tt = mu * 1.4426950408889634;                     // log2 of exp(mu)
          tt = fmin(fmax(tt, -1.0e6), 1.0e6);
          const double e1 = floor(tt);
          const double x = v * exp2(tt - e1);                       // in [1, 32G)
          int ex;
          const double m = frexp(x, &ex);                           // x = m 2^ex, m in [0.5, 1)
          const long long E = static_cast<long long>(e1) + ex - 1;  // x 2^e1 = (2m) 2^E
          const double mant = 2.0 * m;
          const long long biased = E + 2048;
          if (biased < 0 || biased > 4095) {
            set_status(status, MOIRA_ST_MASS_RANGE);
            key = biased < 0 ? 0ull : ((4095ull << 52) | kMask52);
          } else {
            key = (static_cast<unsigned long long>(biased) << 52) |
                  (static_cast<unsigned long long>(__double_as_longlong(mant)) & kMask52);
          }
        }
        if constexpr (FUSED)
          __hip_atomic_store(ws.keys + static_cast<long long>(s) * d.max_pages + p, key,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
          ws.keys[static_cast<long long>(s) * d.max_pages + p] = key;
        if (static_cast<long long>(key >> 52) > eref) {
          over = 1;
        } else {
          const int b = band_of(key, ref);
          atomicAdd(&lq[b], key_mass(key, eref, F));
          atomicAdd(&lc[b], 1u);
        }
      }
      const unsigned long long cm = wave_max_dpp_u64(key);
      if (lane == 0) {
        if constexpr (FUSED)
          __hip_atomic_store(ws.cmax + static_cast<long long>(s) * nslot + c, cm, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        else
          ws.cmax[static_cast<long long>(s) * nslot + c] = cm;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      ph_cur = ph_next;  // the ring already holds the next chunk's first steps
    }
  }
  __syncthreads();
  unsigned long long* ghq = ws.hq + (static_cast<long long>(s) * 2 + par) * kBands;
  unsigned int* ghc = ws.hc + (static_cast<long long>(s) * 2 + par) * kBands;
  for (int b = tid; b < kBands; b += blockDim.x) {
    const unsigned int c = lc[b];
    if (c) {
      atomicAdd(&ghq[b], lq[b]);
      atomicAdd(&ghc[b], c);
    }
  }
  if (tid == 0 && over) atomicOr(&ws.flag[2 * s + par], 1u);
  }   // cw0 < nch
  if constexpr (FUSED) {
    // every key, chunk maximum and histogram atomic of this workgroup is
    // complete (acknowledged at the coherence point) before it counts itself in
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (tid == 0) {
      const unsigned int before =
          __hip_atomic_fetch_add(ws.arrive + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      last_arriver = before + 1 == static_cast<unsigned int>(n_seg);
    }
    __syncthreads();
    if (!last_arriver) return;
    if (tid == 0) ws.arrive[s] = 0u;   // read again only by the next call
    if (P == 0) {   // nothing was scored: the histograms are untouched
      if (tid == 0) cut.list_lens[s] = 0;
      return;
    }
    cut_fused<(FUSED ? CUT_EMAX : 4)>(d, ws, s, P, cut.gamma, cut.page_lists, cut.list_lens, ref,
                                      par, lq, lc, cut_list,
                                      *reinterpret_cast<CutShared<kScoreThreads>*>(csh_raw));
  }
}

// grid (C, B*H), block kCutThreads: the cut of each segment once its keys
// exist, by C workgroups of one range each (SPLIT) or by one. EMAX (key slots
// per lane) is the smallest multiple of 4 covering the slots the layout
// needs, so the unrolled per-lane passes carry no unused slots.
constexpr int kCutThreads = 512;
constexpr int kCutRange = 2 * kCutThreads;   // pages per range of a split cut
constexpr int kCutSplitMaxWgs = 512;         // split only while all ranges fit at once
// Up to 12 key slots per lane the cut asks for four waves per SIMD (at most
// 128 VGPRs, a few of them spilled), so two workgroups share a CU: batches
// with many short segments then cut in one round over the chip.
template <int EMAX, bool SPLIT, int RULE>
__global__ __launch_bounds__(kCutThreads, (EMAX <= 12 ? 4 : 1)) void cut_kernel(Dims d, SelectWs ws,
                                                          const int32_t* __restrict__ seq_lens,
                                                          double param, int C,
                                                          int32_t* __restrict__ page_lists,
                                                          int32_t* __restrict__ list_lens) {
  __shared__ CutShared<kCutThreads> sh;
  cut_segment<kCutThreads, EMAX, SPLIT, RULE>(d, ws, blockIdx.y, blockIdx.x, C, seq_lens, param,
                                              page_lists, list_lens, ws.cur_ref[blockIdx.y],
                                              ws.cur_par[blockIdx.y], sh);
}

// ---- host side shared by the launchers ----------------------------------------
// Chunks per score wave: each segment's chunks are spread evenly over its
// share of about two waves per SIMD (256 compute units x 4 SIMDs), at least
// one chunk per wave, and never so many that a workgroup's waves would
// not all get chunks. (More, shorter waves measured slower: every workgroup
// clears and flushes its own band histogram.)
constexpr int kScoreTargetWaves = 2048;
constexpr int kScorePlannedWgs = 1024;   // planned grid for a batch (at least 2 S)
inline int score_chunks_per_wave(int nch, int S, int nw) {
  long long wps = kScoreTargetWaves / (S > 0 ? S : 1);   // waves per segment
  if (wps < 1) wps = 1;
  long long c = (nch + wps - 1) / wps;
  const long long share = (nch + nw - 1) / nw;   // every wave of a workgroup gets chunks
  if (c > share) c = share;
  if (c < 1) c = 1;
  return static_cast<int>(c);
}

// Launch shape of the scoring kernel: one request uses a fixed grid (every
// segment has the same length, blockIdx.y is the segment); a batch plans its
// split from seq_lens on the device (nwg > 0).
// On the fixed grid of 8-wave workgroups only the first sw waves score
// (sw = 4: one scoring wave per SIMD) while the grid of such workgroups still
// fits the chip at once, the table's last chunks left over beyond a full
// grid going to one more wave of the first workgroups; otherwise all 8
// score.
constexpr int kChipCUs = 256;   // MI355X compute units
struct ScoreGrid {
  dim3 grid;
  int threads, cpw, nwg, sw;
};
inline ScoreGrid score_grid(const Dims& d, int waves) {
  const int nch = (d.max_pages + kScoreChunk - 1) / kScoreChunk;
  ScoreGrid g;
  g.threads = 64 * waves;
  if (d.B == 1) {
    int sw = waves;
    g.cpw = score_chunks_per_wave(nch, d.S(), waves);
    int gx = (nch + waves * g.cpw - 1) / (waves * g.cpw);
    if (waves == 8) {
      const int c4 = score_chunks_per_wave(nch, d.S(), 4);
      const int gx4 = (nch + 4 * c4 - 1) / (4 * c4);
      if (static_cast<long long>(gx4) * d.S() <= kChipCUs) {
        sw = 4;
        g.cpw = c4;
        gx = gx4;
      } else if (c4 == 1 && nch % 4 != 0 && nch / 4 >= nch % 4 &&
                 static_cast<long long>(nch / 4) * d.S() <= kChipCUs) {
        // one chunk per scoring wave, and the few left over (a table a few
        // pages longer than a multiple of 256 pages) to wave 4 of the first
        // workgroups
        sw = 4;
        g.cpw = 1;
        gx = nch / 4;
      }
    }
    g.sw = sw;
    g.nwg = 0;
    g.grid = dim3(gx, d.S());
  } else {
    g.sw = 0;
    g.cpw = 0;
    g.nwg = 2 * d.S() > kScorePlannedWgs ? 2 * d.S() : kScorePlannedWgs;
    g.grid = dim3(g.nwg, 1);
  }
  return g;
}

// Key slots per lane of the fused select's cut (one 8-wave workgroup holds a
// segment's keys): the smallest multiple of 4 covering max_pages.
inline int fused_cut_slots(const Dims& d) {
  const int e = (d.max_pages + kScoreThreads - 1) / kScoreThreads;
  return (e + 3) / 4 * 4;
}

// The fused select (scoring with the cut in each segment's last workgroup) is
// compiled for bf16 queries at head_dim 128 and group capacities 4 and 8;
// E = fused_cut_slots(d), instantiated in its own translation unit.
template <int E>
hipError_t launch_fused_select_e(const Dims& d, const void* q, const void* summaries,
                                 const int32_t* block_table, const int32_t* seq_lens, float scale,
                                 const SelectWs& ws, const AppendArgs& app, bool append,
                                 const CutArgs& cut, int32_t* status, hipStream_t st) {
  const ScoreGrid g = score_grid(d, kScoreMaxWaves);
  const uint16_t* qq = static_cast<const uint16_t*>(q);
#define MOIRA_FUSED(ST, GG, AP)                                                                  \
  score_kernel<uint16_t, ST, 128, GG, AP, E><<<g.grid, g.threads, 0, st>>>(                   \
      d, qq, static_cast<const ST*>(summaries), block_table, seq_lens, scale, ws, g.cpw, g.nwg, g.sw, \
      app, status, cut)
#define MOIRA_FUSED_G(ST, AP)            \
  do {                                   \
    if (d.G <= 4) MOIRA_FUSED(ST, 4, AP); \
    else MOIRA_FUSED(ST, 8, AP);          \
  } while (0)
  if (d.sbf) {
    if (append) MOIRA_FUSED_G(uint16_t, true);
    else MOIRA_FUSED_G(uint16_t, false);
  } else if (d.sf8) {
    if (append) MOIRA_FUSED_G(uint8_t, true);
    else MOIRA_FUSED_G(uint8_t, false);
  } else {
    if (append) MOIRA_FUSED_G(float, true);
    else MOIRA_FUSED_G(float, false);
  }
#undef MOIRA_FUSED_G
#undef MOIRA_FUSED
  return hipGetLastError();
}

}  // namespace moira
