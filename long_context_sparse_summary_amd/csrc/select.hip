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
#include <climits>
#include <mutex>
#include <type_traits>

#include "moira_common.h"

namespace moira {

constexpr int kScoreChunk = 64;        // pages per score chunk (one per lane quad)
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
  unsigned long long* hq;      // [S][kBands][2] quantised mass per band, per parity
  unsigned int* hc;            // [S][kBands][2] pages per band, per parity
  unsigned long long* keys;    // [S][max_pages]
  unsigned long long* cmax;    // [S][ceil(max_pages / kScoreChunk)] largest key per score chunk
  unsigned long long* ref;     // [S] reference key R for the next call
  unsigned long long* cur_ref; // [S] reference key the current call scored with
  unsigned int* par;           // [S] parity of the next call
  unsigned int* cur_par;       // [S] parity of the current call
  unsigned int* flag;          // [S][2] bit 0: a key exceeded the fixed-point range
  int fresh;                   // 1: ignore the stored reference keys (exact select)
};

__host__ __device__ inline size_t select_ws_bytes(int S, int max_pages) {
  const size_t nch = (static_cast<size_t>(max_pages) + kScoreChunk - 1) / kScoreChunk;
  return static_cast<size_t>(S) *
         (static_cast<size_t>(kBands) * 24 + static_cast<size_t>(max_pages) * 8 + nch * 8 + 32);
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
  w.fresh = 0;
  return w;
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
// summary elements of SB bytes (4: fp32, 2: bf16). LPP lanes share a page,
// each holding DL = D / LPP of its dimensions in pieces of PW contiguous
// elements (one 16-byte load, or 8 bytes for bf16 when DL < 8).
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
  static constexpr int PW = SB == 4 ? 4 : (DL >= 8 ? 8 : 4);   // elements per piece
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

template <typename QT> struct QLoad4;
template <> struct QLoad4<float> {
  static __device__ __forceinline__ void get(const float* q, long long i, double (&o)[4]) {
    const float4 v = *reinterpret_cast<const float4*>(q + i);
    o[0] = v.x; o[1] = v.y; o[2] = v.z; o[3] = v.w;
  }
};
template <> struct QLoad4<uint16_t> {
  static __device__ __forceinline__ void get(const uint16_t* q, long long i, double (&o)[4]) {
    const uint2 v = *reinterpret_cast<const uint2*>(q + i);
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

// Resolve the candidates held in sh.ck/sh.cp[buf] (count n; every other kept
// page ranks above them and has mass A in total): leaves the threshold key in
// sh.tk and the number of key-T pages to keep (in page order) in sh.take.
// Uniform control flow; every thread of the block calls it.
template <int NT>
__device__ void resolve_lds(int n, int buf, unsigned long long A, unsigned long long tau,
                            long long eref, int F, bool unit, CutShared<NT>& sh) {
  // weight of a candidate: its quantised mass, or 1 when pages are counted
  auto wgt = [&](unsigned long long x) -> unsigned long long {
    return unit ? 1ull : key_mass(x, eref, F);
  };
  const int tid = threadIdx.x;
  if (n <= 0) {  // not reachable while A < tau <= A + total: keep every page
    if (tid == 0) {
      sh.tk = 0ull;
      sh.take = 0;
    }
    __syncthreads();
    return;
  }
#pragma unroll 1
  for (int level = 0; level < 12; ++level) {
    if (n <= 64) {
      // pairwise ranking in one wave: c' ranks before c if its key is larger,
      // or equal with a lower page index; integer sums are exact
      if (tid < 64) {
        bool kept = false;
        unsigned long long mk = 0;
        if (tid < n) {
          mk = sh.ck[buf][tid];
          const int mp = sh.cp[buf][tid];
          unsigned long long acc = A;
#pragma unroll 1
          for (int c = 0; c < n; ++c) {
            const unsigned long long ok = sh.ck[buf][c];
            if (ok > mk || (ok == mk && sh.cp[buf][c] < mp)) acc += wgt(ok);
          }
          kept = acc < tau;
        }
        const unsigned long long T = ~wave_max_dpp_u64(kept ? ~mk : 0ull);
        const unsigned long long bal = __ballot(kept && mk == T);
        if (tid == 0) {
          sh.tk = T;
          sh.take = __popcll(bal);
        }
      }
      __syncthreads();
      return;
    }
    unsigned long long lo = ~0ull, hi = 0;
    for (int i = tid; i < n; i += NT) {
      const unsigned long long x = sh.ck[buf][i];
      lo = x < lo ? x : lo;
      hi = x > hi ? x : hi;
    }
    block_minmax_u64<NT>(lo, hi, sh);
    if (lo == hi) {  // all candidates share one key: ties rank by page index
      if (tid == 0) {
        const unsigned long long qv = wgt(lo);
        const unsigned long long t = qv ? (tau - A + qv - 1) / qv : static_cast<unsigned long long>(n);
        sh.tk = lo;
        sh.take = static_cast<int>(t < static_cast<unsigned long long>(n) ? t : n);
      }
      __syncthreads();
      return;
    }
    // mass-weighted histogram on the 8 key bits below the common prefix
    const int hb = 63 - __clzll(static_cast<long long>(lo ^ hi));
    const int shift = hb > 7 ? hb - 7 : 0;
    const unsigned long long base = lo >> shift;
    for (int b = tid; b < kCutBins; b += NT) sh.hq[b] = 0ull;
    if (tid == 0) {
      sh.bci[0] = -1;
      sh.ncl = 0;
    }
    __syncthreads();
    for (int i = tid; i < n; i += NT) {
      const unsigned long long x = sh.ck[buf][i];
      atomicAdd(&sh.hq[static_cast<int>((x >> shift) - base)], wgt(x));
    }
    __syncthreads();
    const unsigned long long mine = tid < kCutBins ? sh.hq[tid] : 0ull;
    unsigned long long all;
    const unsigned long long below = block_excl_scan_u64<NT>(mine, &all, sh);
    if (tid < kCutBins) {
      const unsigned long long Sb = all - below;   // mass of digits >= tid
      const unsigned long long Sb1 = Sb - mine;    // mass of digits > tid
      if (A + Sb >= tau && A + Sb1 < tau) {
        sh.bci[0] = tid;
        sh.bc[0] = A + Sb1;
      }
    }
    __syncthreads();
    const int bstar = sh.bci[0];
    if (bstar < 0) {  // not reachable while A < tau <= A + total: keep all candidates
      if (tid == 0) {
        sh.tk = lo;
        sh.take = n;
      }
      __syncthreads();
      return;
    }
    A = sh.bc[0];
    for (int i = tid; i < n; i += NT) {
      const unsigned long long x = sh.ck[buf][i];
      if (static_cast<int>((x >> shift) - base) == bstar) {
        const int o = atomicAdd(&sh.ncl, 1);
        sh.ck[buf ^ 1][o] = x;
        sh.cp[buf ^ 1][o] = sh.cp[buf][i];
      }
    }
    __syncthreads();
    n = sh.ncl;
    buf ^= 1;
    __syncthreads();
  }
  if (tid == 0) {  // unreachable: 64-bit keys are exhausted within 8 levels
    sh.tk = 0ull;
    sh.take = 0;
  }
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
template <int NT, int EMAX, bool SPLIT, int RULE>
__device__ __forceinline__ void cut_segment(const Dims& d, const SelectWs& ws, int s, int r, int C,
                                            const int32_t* __restrict__ seq_lens, double param, int32_t* __restrict__ page_lists,
                                            int32_t* __restrict__ list_lens, CutShared<NT>& sh) {
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
  const int Lraw = seq_lens[s / d.H];
  const unsigned long long* kin = ws.keys + static_cast<long long>(s) * d.max_pages;
  unsigned long long kv[EMAX];
#pragma unroll
  for (int e = 0; e < EMAX; ++e) {
    const int p = page(e);
    kv[e] = p < d.max_pages ? kin[p] : 0ull;
  }
  unsigned long long ko[2] = {0ull, 0ull};  // own range, (wave, e, lane) order
  if (SPLIT) {
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int p = rstart + wave * 128 + 64 * e + lane;
      ko[e] = p < d.max_pages ? kin[p] : 0ull;
    }
  }
  const int nslot = (d.max_pages + kScoreChunk - 1) / kScoreChunk;
  // both parities of this thread's bands; the parity picks one once it returns
  const unsigned long long* ghq = ws.hq + (static_cast<long long>(s) * kBands + tid * BPT) * 2;
  const unsigned int* ghc = ws.hc + (static_cast<long long>(s) * kBands + tid * BPT) * 2;
  unsigned long long bq0[BPT], bq1[BPT];
  unsigned int bc0[BPT], bc1[BPT];
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    bq0[b] = ghq[2 * b];
    bq1[b] = ghq[2 * b + 1];
    bc0[b] = ghc[2 * b];
    bc1[b] = ghc[2 * b + 1];
  }
  const unsigned long long ref = ws.cur_ref[s];
  const unsigned int par = ws.cur_par[s] & 1u;
  const unsigned int fl0 = ws.flag[2 * s];
  const unsigned int fl1 = ws.flag[2 * s + 1];
  unsigned long long cm = tid < nslot ? ws.cmax[static_cast<long long>(s) * nslot + tid] : 0ull;
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
  unsigned int lt_all = 0, lt_before = 0;  // this wave's pages of heavier bands

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
      // gather the band's pages into LDS (one LDS atomic per wave and slot
      // that holds any) and count the pages of heavier bands. The band of a
      // key is a function of key >> kBandShift, clamped at both ends.
      const int t = static_cast<int>(ref >> kBandShift) + kBandHeadroom - band;
      const int klo = band == kBands - 1 ? INT_MIN : t;
      const int khi = band == 0 ? INT_MAX : t;
#pragma unroll
      for (int e = 0; e < EMAX; ++e) {
        const unsigned long long vm = vmask(e);
        const int kb = static_cast<int>(static_cast<unsigned int>(kv[e] >> 32) >> (kBandShift - 32));
        const unsigned long long le = __ballot(kb <= khi);
        const unsigned long long be = le & __ballot(kb >= klo) & vm;
        if (SPLIT) {
          const unsigned int nl = __popcll(~le & vm);   // heavier bands
          lt_all += nl;
          lt_before += (e >> 1) < r ? nl : 0u;
        }
        if (be) {
          int base = 0;
          if (lane == 0) base = atomicAdd(&sh.ncl, __popcll(be));
          base = __builtin_amdgcn_readfirstlane(base);
          if (be >> lane & 1ull) {
            const int o = base + __popcll(be & ltmask);
            if (o < kCandCap) {
              const int p = page(e);
              sh.ck[0][o] = kv[e];
              sh.cp[0][o] = p;
              if (SPLIT) {
                sh.zk[o] = kv[e];
                sh.zp[o] = p;
              }
            }
          }
        }
      }
      __syncthreads();
      ngath = min(sh.ncl, kCandCap);
      resolve_lds<NT>(ngath, 0, A, tau, eref, F, unit, sh);
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
          if (cand >> e & 1u) {
            const int o = atomicAdd(&sh.ncl, 1);
            if (o < kCandCap) {
              sh.ck[0][o] = kv[e];
              sh.cp[0][o] = page(e);
            }
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
      if (lane == 0) cnt += static_cast<unsigned long long>(lt_all) |
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
    const unsigned long long z = block_sum_u64<NT>(cnt, sh);
    const unsigned int ngt = static_cast<unsigned int>(z & 0xffffu);
    const unsigned int neq = static_cast<unsigned int>((z >> 16) & 0xffffu);
    const unsigned int ntake = min(take, neq);
    // consistent counts give total <= P; the clamp keeps every write and the
    // stored length inside the segment's list whatever happens
    total = min(ngt + ntake, static_cast<unsigned int>(P));

    // ---- this workgroup's range, in (wave, e, lane) order
    const int p0 = rstart + wave * 128 + lane;
    const bool g0 = p0 < P && (all || ko[0] > T);
    const bool q0 = p0 < P && !all && ko[0] == T;
    const bool g1 = p0 + 64 < P && (all || ko[1] > T);
    const bool q1 = p0 + 64 < P && !all && ko[1] == T;
    const unsigned long long gm0 = __ballot(g0), em0 = __ballot(q0);
    const unsigned long long gm1 = __ballot(g1), em1 = __ballot(q1);
    const unsigned int wg = __popcll(gm0) + __popcll(gm1);
    const unsigned int we = __popcll(em0) + __popcll(em1);
    if (lane == 0) sh.redu[wave] = wg | (we << 16);   // each count <= 128
    __syncthreads();
    unsigned int gacc = static_cast<unsigned int>((z >> 32) & 0xffffu);
    unsigned int eacc = static_cast<unsigned int>(z >> 48);
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const unsigned int x = sh.redu[w];
      if (w < wave) {
        gacc += x & 0xffffu;
        eacc += x >> 16;
      }
    }
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
    unsigned long long* chq = ws.hq + (static_cast<long long>(s) * kBands + tid * BPT) * 2 + np;
    unsigned int* chc = ws.hc + (static_cast<long long>(s) * kBands + tid * BPT) * 2 + np;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      chq[2 * b] = 0ull;
      chc[2 * b] = 0u;
    }
    if (tid == 0) {
      list_lens[s] = static_cast<int>(total);
      ws.flag[2 * s + np] = 0u;
      ws.ref[s] = kmax;
      ws.par[s] = np;
    }
  }
}

// A score workgroup has 8 waves on the fixed single-request grid (one
// workgroup per CU) and 4 on the planned batch grid (two per CU); the kernel
// takes the count from blockDim and is compiled for the larger.
constexpr int kScoreMaxWaves = 8;
constexpr int kScoreThreads = 64 * kScoreMaxWaves;

// grid (ceil(ceil(max_pages / 64) / (4 cpw)), B*H), block 256. Each wave
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
                              int* base, int* tmp, int& s, int& c_begin, int& c_end, bool& first) {
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
  if (qc < 4) qc = 4;
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
  return true;
}

template <typename QT, typename ST, int D, int G, bool APPEND>
__global__ __launch_bounds__(kScoreThreads) void score_kernel(
    Dims d, const QT* __restrict__ q, const ST* __restrict__ summaries,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, float scale,
    SelectWs ws, int cpw, int nwg, AppendArgs app, int32_t* status) {
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
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int t = lane % LPP;   // dimension slice of this lane
  const int pg = lane / LPP;  // page of a step this lane works on
  // the segment and chunks of this workgroup: a fixed grid (blockIdx.y is
  // the segment, 4 cpw chunks per workgroup) or, with nwg > 0, the batch
  // split planned from seq_lens
  int s = blockIdx.y;
  const int nw = blockDim.x >> 6;        // waves of the workgroup
  int cw0 = blockIdx.x * nw * cpw;       // first chunk of the workgroup
  int cwe = cw0 + nw * cpw;              // end of the workgroup's chunks
  int wcpw = cpw;                        // chunks per wave
  bool first = blockIdx.x == 0;          // scores the segment's first chunk
  if (nwg > 0) {
    if (!plan_score_wg(d, seq_lens, nwg, blockIdx.x, reinterpret_cast<int*>(lq),
                       reinterpret_cast<int*>(lc), s, cw0, cwe, first)) return;
    wcpw = (cwe - cw0 + nw - 1) / nw;
    __syncthreads();   // lq and lc are the histogram again
  }
  const int r = s / d.H;
  const int j = s - r * d.H;
  const int c0 = cw0 + wave * wcpw;      // first chunk of this wave
  const int32_t* trow = block_table + static_cast<long long>(r) * d.max_pages;

  // every load that does not depend on the request length goes out first
  const int Lraw = seq_lens[r];
  // a fresh call scores as if no earlier call had left a reference key: the
  // cut then takes the exact select, and no histogram is read
  const unsigned long long ref = ws.fresh ? 0ull : ws.ref[s];
  const unsigned int par = ws.par[s] & 1u;
  double qr[G][DL];
  {
    // G is the compiled group capacity; heads d.G .. G-1 are padding with a
    // zero query and take no part in the mass
    const long long qbase = (static_cast<long long>(r) * d.Hq() + static_cast<long long>(j) * d.G) * D;
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const bool real = g < d.G;           // padding heads read head 0 and are zeroed
      const double keep = real ? 1.0 : 0.0;
      // piece i of this lane covers dimensions (i LPP + t) PW .. + PW
#pragma unroll
      for (int i = 0; i < NP; ++i) {
#pragma unroll
        for (int h = 0; h < PW / 4; ++h) {
          double v[4];
          QLoad4<QT>::get(q, qbase + (real ? g : 0) * D + (i * LPP + t) * PW + 4 * h, v);
#pragma unroll
          for (int e = 0; e < 4; ++e) qr[g][i * PW + 4 * h + e] = v[e] * keep;
        }
      }
    }
  }
  int raw_next = -1;  // table entry of this lane's page in the next chunk
  if (c0 * kScoreChunk + lane < d.max_pages) raw_next = trow[c0 * kScoreChunk + lane];
  for (int b = tid; b < kBands; b += blockDim.x) {
    lq[b] = 0ull;
    lc[b] = 0u;
  }
  if (tid == 0) over = 0;
  if (tid == 0 && first) {   // what this call scores with, for its cut
    ws.cur_ref[s] = ref;
    ws.cur_par[s] = par;
  }

  int L = Lraw;
  if (L < 0 || L > d.max_pages * d.ps) {
    if (tid == 0 && first && j == 0) set_status(status, MOIRA_ST_BAD_LEN);
    L = 0;
  }
  const int P = (L + d.ps - 1) / d.ps;
  const int nch = (P + kScoreChunk - 1) / kScoreChunk;
  if (APPEND && L == 0 && tid == 0 && first && j == 0)
    set_status(status, MOIRA_ST_BAD_LEN);   // nothing was advanced: no slot to write
  if (cw0 >= nch) return;  // uniform over the workgroup
  const int c1 = min(min(c0 + wcpw, cwe), nch);
  const long long eref = ref_exponent(ref);
  const int F = mass_frac_bits(P);
  const double dscale = static_cast<double>(scale);
  const int nslot = (d.max_pages + kScoreChunk - 1) / kScoreChunk;
  double* lgw = lg[wave];
  __syncthreads();  // histogram cleared

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

  if (c0 < c1) {  // uniform over the wave
    Raw buf[DEPTH][NP];
    int ph_cur = phys_of(raw_next, c0);
    int ph_next = -1;
    raw_next = -1;
    if (c0 + 1 < c1) raw_next = trow[(c0 + 1) * kScoreChunk + lane];
    // the tail page (P - 1) and, in APPEND mode, the step's token written
    // into it by the wave that scores it. When the tail page lies in the
    // wave's first chunk its physical page is already in a lane (no extra
    // round trip); its token loads then travel with the first summary loads.
    const int pt = P - 1;
    const int ct = pt / kScoreChunk;                 // its chunk
    const int st_t = (pt - ct * kScoreChunk) / PPS;  // its step in the chunk
    const int pg_t = (pt - ct * kScoreChunk) - st_t * PPS;
    bool tail_ok = false;
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
      if (lane == 0) ws.cmax[static_cast<long long>(s) * nslot + c] = cm;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      ph_cur = ph_next;  // the ring already holds the next chunk's first steps
    }
  }
  __syncthreads();
  unsigned long long* ghq = ws.hq + static_cast<long long>(s) * kBands * 2 + par;
  unsigned int* ghc = ws.hc + static_cast<long long>(s) * kBands * 2 + par;
  for (int b = tid; b < kBands; b += blockDim.x) {
    const unsigned int c = lc[b];
    if (c) {
      atomicAdd(&ghq[2 * b], lq[b]);
      atomicAdd(&ghc[2 * b], c);
    }
  }
  if (tid == 0 && over) atomicOr(&ws.flag[2 * s + par], 1u);
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
                                              page_lists, list_lens, sh);
}

// gamma = 1: every page of every segment, in order (no scoring needed).
__global__ __launch_bounds__(1024) void all_pages_kernel(Dims d, const int32_t* __restrict__ seq_lens,
                                                        int32_t* __restrict__ page_lists,
                                                        int32_t* __restrict__ list_lens) {
  const int s = blockIdx.x;
  const int r = s / d.H;
  int L = seq_lens[r];
  if (L < 1 || L > d.max_pages * d.ps) L = 0;
  const int P = (L + d.ps - 1) / d.ps;
  int32_t* out = page_lists + static_cast<long long>(s) * d.max_pages;
  for (int p = threadIdx.x; p < P; p += blockDim.x) out[p] = p;
  if (threadIdx.x == 0) list_lens[s] = P;
}

// ---- host launcher ----------------------------------------------------------
// Chunks per score wave: each segment's chunks are spread evenly over its
// share of about two waves per SIMD (256 compute units x 4 SIMDs), at least
// one chunk per wave, and never so many that a workgroup's waves would
// not all get chunks. (More, shorter waves measured slower: every workgroup
// clears and flushes its own band histogram.)
constexpr int kScoreTargetWaves = 2048;
constexpr int kScorePlannedWgs = 1024;   // planned grid for a batch (at least 2 S)
static int score_chunks_per_wave(int nch, int S, int nw) {
  long long wps = kScoreTargetWaves / (S > 0 ? S : 1);   // waves per segment
  if (wps < 1) wps = 1;
  long long c = (nch + wps - 1) / wps;
  const long long share = (nch + nw - 1) / nw;   // every wave of a workgroup gets chunks
  if (c > share) c = share;
  if (c < 1) c = 1;
  return static_cast<int>(c);
}

template <typename QT, typename ST, int D, bool APPEND>
static void launch_score_d(const Dims& d, const void* q, const void* summaries,
                           const int32_t* block_table, const int32_t* seq_lens, float scale,
                           const SelectWs& ws, const AppendArgs& app, int32_t* status,
                           hipStream_t st) {
  const int nch = (d.max_pages + kScoreChunk - 1) / kScoreChunk;
  // one request: every segment has the same length and a fixed grid is
  // balanced; a batch: the workgroups plan the split from seq_lens
  const int nwv = d.B == 1 ? kScoreMaxWaves : 4;                   // waves per workgroup
  const int cpw = d.B == 1 ? score_chunks_per_wave(nch, d.S(), nwv) : 0;
  const int nwg = d.B == 1 ? 0 : (2 * d.S() > kScorePlannedWgs ? 2 * d.S() : kScorePlannedWgs);
  dim3 grid = d.B == 1 ? dim3((nch + nwv * cpw - 1) / (nwv * cpw), d.S()) : dim3(nwg, 1);
  const QT* qq = static_cast<const QT*>(q);
  const ST* ss = static_cast<const ST*>(summaries);
#define MOIRA_SELECT(GG)                                                                     \
  score_kernel<QT, ST, D, GG, APPEND><<<grid, 64 * nwv, 0, st>>>(                        \
      d, qq, ss, block_table, seq_lens, scale, ws, cpw, nwg, app, status)
  // group capacities 1, 2, 4, 8, 16 (smaller groups run padded)
  if (d.G <= 1) MOIRA_SELECT(1);
  else if (d.G <= 2) MOIRA_SELECT(2);
  else if (d.G <= 4) MOIRA_SELECT(4);
  else if (d.G <= 8) MOIRA_SELECT(8);
  else MOIRA_SELECT(16);
#undef MOIRA_SELECT
}

template <typename ST, bool APPEND>
static void launch_score_s(const Dims& d, int q_dtype, const void* q, const void* summaries,
                           const int32_t* block_table, const int32_t* seq_lens, float scale,
                           const SelectWs& ws, const AppendArgs& app, int32_t* status,
                           hipStream_t st) {
  if (q_dtype == MOIRA_BF16) {
    if (d.D == 128)
      launch_score_d<uint16_t, ST, 128, APPEND>(d, q, summaries, block_table, seq_lens, scale, ws, app, status, st);
    else
      launch_score_d<uint16_t, ST, 64, APPEND>(d, q, summaries, block_table, seq_lens, scale, ws, app, status, st);
  } else {
    if (d.D == 128)
      launch_score_d<float, ST, 128, APPEND>(d, q, summaries, block_table, seq_lens, scale, ws, app, status, st);
    else
      launch_score_d<float, ST, 64, APPEND>(d, q, summaries, block_table, seq_lens, scale, ws, app, status, st);
  }
}

template <bool APPEND>
static void launch_score(const Dims& d, int q_dtype, const void* q, const void* summaries,
                         const int32_t* block_table, const int32_t* seq_lens, float scale,
                         const SelectWs& ws, const AppendArgs& app, int32_t* status,
                         hipStream_t st) {
  if (d.sbf)
    launch_score_s<uint16_t, APPEND>(d, q_dtype, q, summaries, block_table, seq_lens, scale, ws, app, status, st);
  else
    launch_score_s<float, APPEND>(d, q_dtype, q, summaries, block_table, seq_lens, scale, ws, app, status, st);
}

// The cut is split into ranges of kCutRange pages, one workgroup each, when a
// segment spans at least two ranges and every range of every segment fits on
// the chip at once; otherwise one workgroup cuts a whole segment.
template <bool SPLIT, int RULE>
static void launch_cut_e(const Dims& d, const SelectWs& ws, const int32_t* seq_lens, double param,
                         int C, int E, int32_t* page_lists, int32_t* list_lens, hipStream_t st) {
  const dim3 grid(C, d.S());
#define MOIRA_CUT(EM) \
  cut_kernel<EM, SPLIT, RULE><<<grid, kCutThreads, 0, st>>>(d, ws, seq_lens, param, C, page_lists, list_lens)
  if (E <= 4) MOIRA_CUT(4);
  else if (E <= 8) MOIRA_CUT(8);
  else if (E <= 12) MOIRA_CUT(12);
  else if (E <= 16) MOIRA_CUT(16);
  else if (E <= 20) MOIRA_CUT(20);
  else if (E <= 24) MOIRA_CUT(24);
  else if (E <= 28) MOIRA_CUT(28);
  else MOIRA_CUT(32);
#undef MOIRA_CUT
}

template <int RULE>
static void launch_cut_r(const Dims& d, const SelectWs& ws, const int32_t* seq_lens, double param,
                         int32_t* page_lists, int32_t* list_lens, hipStream_t st) {
  const int C = (d.max_pages + kCutRange - 1) / kCutRange;
  if (C >= 2 && static_cast<long long>(C) * d.S() <= kCutSplitMaxWgs)
    launch_cut_e<true, RULE>(d, ws, seq_lens, param, C, 2 * C, page_lists, list_lens, st);
  else
    launch_cut_e<false, RULE>(d, ws, seq_lens, param, 1,
                              (d.max_pages + kCutThreads - 1) / kCutThreads, page_lists, list_lens, st);
}

// The rule is a template argument of the cut, so each rule's kernel carries
// only its own branches.
static void launch_cut(const Dims& d, const SelectWs& ws, const int32_t* seq_lens, int rule,
                       double param, int32_t* page_lists, int32_t* list_lens, hipStream_t st) {
  if (rule == MOIRA_RULE_TOPK)
    launch_cut_r<MOIRA_RULE_TOPK>(d, ws, seq_lens, param, page_lists, list_lens, st);
  else if (rule == MOIRA_RULE_TOPDELTA)
    launch_cut_r<MOIRA_RULE_TOPDELTA>(d, ws, seq_lens, param, page_lists, list_lens, st);
  else
    launch_cut_r<MOIRA_RULE_COVERAGE>(d, ws, seq_lens, param, page_lists, list_lens, st);
}

// Selection under a rule: coverage (param = gamma), the k heaviest pages
// (param = k) or the pages above delta times the largest mass (param =
// delta). Rules that keep every page skip the scoring.
hipError_t launch_select_rule(const Dims& d, int q_dtype, const void* q, const void* summaries,
                              const int32_t* block_table, const int32_t* seq_lens, int rule,
                              double param, float scale, void* workspace, int32_t* page_lists,
                              int32_t* list_lens, int32_t* status, hipStream_t st) {
  const SelectWs ws = select_ws(workspace, d.S(), d.max_pages);
  const bool all = (rule == MOIRA_RULE_COVERAGE && param >= 1.0) ||
                   (rule == MOIRA_RULE_TOPK && param >= static_cast<double>(d.max_pages)) ||
                   (rule == MOIRA_RULE_TOPDELTA && param <= 0.0);
  if (all) {
    all_pages_kernel<<<d.S(), 1024, 0, st>>>(d, seq_lens, page_lists, list_lens);
    return hipGetLastError();
  }
  launch_score<false>(d, q_dtype, q, summaries, block_table, seq_lens, scale, ws, AppendArgs{},
                      status, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_cut(d, ws, seq_lens, rule, param, page_lists, list_lens, st);
  return hipGetLastError();
}

hipError_t launch_select(const Dims& d, int q_dtype, const void* q, const void* summaries,
                         const int32_t* block_table, const int32_t* seq_lens, double gamma,
                         float scale, void* workspace, int32_t* page_lists, int32_t* list_lens,
                         int32_t* status, hipStream_t st) {
  return launch_select_rule(d, q_dtype, q, summaries, block_table, seq_lens, MOIRA_RULE_COVERAGE,
                            gamma, scale, workspace, page_lists, list_lens, status, st);
}

hipError_t launch_append(const Dims& d, int kv_dtype, const void* k_new, const void* v_new,
                         void* k_pool, void* v_pool, void* summaries, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t* status, hipStream_t st);

// Append and select in one step: for bf16 K/V below gamma = 1 the append
// runs inside the score kernel; otherwise the append kernel runs first.
hipError_t launch_append_select(const Dims& d, int kv_dtype, int q_dtype, const void* q,
                                const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                void* summaries, const int32_t* block_table,
                                const int32_t* seq_lens, double gamma, float scale,
                                void* workspace, int32_t* page_lists, int32_t* list_lens,
                                int32_t* status, hipStream_t st) {
  if (kv_dtype != MOIRA_BF16 || gamma >= 1.0) {
    hipError_t e = launch_append(d, kv_dtype, k_new, v_new, k_pool, v_pool, summaries,
                                 block_table, seq_lens, status, st);
    if (e != hipSuccess) return e;
    return launch_select(d, q_dtype, q, summaries, block_table, seq_lens, gamma, scale, workspace,
                         page_lists, list_lens, status, st);
  }
  const SelectWs ws = select_ws(workspace, d.S(), d.max_pages);
  const AppendArgs app{static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
                       static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), summaries};
  launch_score<true>(d, q_dtype, q, summaries, block_table, seq_lens, scale, ws, app, status, st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_cut(d, ws, seq_lens, MOIRA_RULE_COVERAGE, gamma, page_lists, list_lens, st);
  return hipGetLastError();
}

size_t select_workspace_bytes(int S, int max_pages) { return select_ws_bytes(S, max_pages); }

// ---- selection without a caller-provided workspace ----------------------------
// For callers that cannot allocate (code under graph capture, serving loops):
// the workspace lives in a file-scope device array, one copy per GPU, held
// until the process ends. Its address is looked up once per device on the
// first call there (with that device current) and kept; host code uses only
// that address, never the array's name. Every call treats the array's stored
// reference keys as absent (SelectWs::fresh), so whatever an earlier call of
// any shape left there cannot steer the result: the scoring kernel writes
// every word the cut reads, and the cut runs the exact in-workgroup select.
// Calls that overlap on one GPU race on the array.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of this GPU's copy of the scratch array (looked up once).
static hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_select_noalloc(const Dims& d, int q_dtype, const void* q, const void* summaries,
                                 const int32_t* block_table, const int32_t* seq_lens, double gamma,
                                 float scale, int32_t* page_lists, int32_t* list_lens,
                                 int32_t* status, hipStream_t st) {
  if (gamma >= 1.0) {   // every page: no scoring, no workspace
    all_pages_kernel<<<d.S(), 1024, 0, st>>>(d, seq_lens, page_lists, list_lens);
    return hipGetLastError();
  }
  void* base = nullptr;
  hipError_t e = scratch_address(&base);
  if (e != hipSuccess) return e;
  SelectWs ws = select_ws(base, d.S(), d.max_pages);
  ws.fresh = 1;
  launch_score<false>(d, q_dtype, q, summaries, block_table, seq_lens, scale, ws, AppendArgs{},
                      status, st);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch_cut(d, ws, seq_lens, MOIRA_RULE_COVERAGE, gamma, page_lists, list_lens, st);
  return hipGetLastError();
}

}  // namespace moira
