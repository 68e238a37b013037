// Coverage-rule page selection (MOIRA abstract: for every request, layer, KV
// head and step keep the smallest set of pages whose estimated attention mass
// reaches a fraction gamma).
//
// Two kernels per call:
//  * score (chip-wide, grid = 64-page chunks x segments): for each page the
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
#include "moira_common.h"

namespace moira {

constexpr int kScoreChunk = 64;        // pages per score workgroup (one per lane quad)
constexpr int kBands = 2048;           // level-1 bands per segment
constexpr int kBandShift = 46;         // key >> 46: exponent + 6 fraction bits
constexpr int kBandHeadroom = 64;      // one octave of bands above the reference
constexpr int kCutBins = 256;          // digit bins of the in-workgroup radix levels
constexpr int kCandCap = 512;          // boundary-band pages resolved in LDS
constexpr int kRefSlack = 10;          // max bits of mass resolution lost to a high reference
constexpr unsigned long long kMask52 = (1ull << 52) - 1;

// Device workspace of moira_select_pages.
struct SelectWs {
  unsigned long long* keys;    // [S][max_pages]
  unsigned long long* hq;      // [S][kBands] quantised mass per band
  unsigned int* hc;            // [S][kBands] pages per band
  unsigned long long* ref;     // [S] reference key R for the band histogram
  unsigned long long* cmax;    // [S][ceil(max_pages / kScoreChunk)] largest key per score chunk
  unsigned int* flag;          // [S] bit 0: a key exceeded the fixed-point range
};

__host__ __device__ inline size_t select_ws_bytes(int S, int max_pages) {
  const size_t nch = (static_cast<size_t>(max_pages) + kScoreChunk - 1) / kScoreChunk;
  return static_cast<size_t>(S) *
         (static_cast<size_t>(max_pages) * 8 + nch * 8 + static_cast<size_t>(kBands) * 12 + 16);
}

inline SelectWs select_ws(void* base, int S, int max_pages) {
  SelectWs w;
  unsigned char* p = static_cast<unsigned char*>(base);
  w.keys = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * max_pages * 8;
  w.hq = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * kBands * 8;
  w.ref = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * 8;
  w.cmax = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * ((static_cast<size_t>(max_pages) + kScoreChunk - 1) / kScoreChunk) * 8;
  w.hc = reinterpret_cast<unsigned int*>(p);
  p += static_cast<size_t>(S) * kBands * 4;
  w.flag = reinterpret_cast<unsigned int*>(p);
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

template <typename QT> struct QLoad;
template <> struct QLoad<float> {
  static __device__ __forceinline__ double get(const float* q, long long i) { return q[i]; }
};
template <> struct QLoad<uint16_t> {
  static __device__ __forceinline__ double get(const uint16_t* q, long long i) {
    return bf16_bits_to_f32(q[i]);
  }
};

// grid (ceil(max_pages / kScoreChunk), B*H), block 256. Four lanes per page,
// each covering D/4 dimensions as float4 pieces at stride 16 floats.
template <typename QT, int D, int G>
__global__ __launch_bounds__(256) void score_kernel(Dims d, const QT* __restrict__ q,
                                                    const float* __restrict__ summaries,
                                                    const int32_t* __restrict__ block_table,
                                                    const int32_t* __restrict__ seq_lens,
                                                    float scale, SelectWs ws,
                                                    int32_t* status) {
  __shared__ double qs[G * D];
  __shared__ unsigned long long lq[kBands];
  __shared__ unsigned int lc[kBands];
  __shared__ int over;
  __shared__ unsigned long long wmax[4];
  const int s = blockIdx.y;
  const int r = s / d.H;
  const int j = s - r * d.H;
  const int L = checked_len(seq_lens, r, d, status, threadIdx.x == 0 && blockIdx.x == 0 && j == 0);
  if (L == 0) return;
  const int P = (L + d.ps - 1) / d.ps;
  const int c0 = blockIdx.x * kScoreChunk;
  if (c0 >= P) return;
  const long long qbase = (static_cast<long long>(r) * d.Hq() + static_cast<long long>(j) * G) * D;
  for (int i = threadIdx.x; i < G * D; i += blockDim.x) qs[i] = QLoad<QT>::get(q, qbase + i);
  for (int b = threadIdx.x; b < kBands; b += blockDim.x) {
    lq[b] = 0ull;
    lc[b] = 0u;
  }
  if (threadIdx.x == 0) over = 0;
  const unsigned long long ref = ws.ref[s];
  const long long eref = ref_exponent(ref);
  const int F = mass_frac_bits(P);
  __syncthreads();

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int k = lane & 3;
  const int slot = lane >> 2;
  constexpr int NI = D / 16;  // float4 pieces per lane
  const double dscale = static_cast<double>(scale);

  const int p = c0 + wave * 16 + slot;
  const bool live = p < P;
  long long phys = -1;
  if (live) {
    long long raw = block_table[static_cast<long long>(r) * d.max_pages + p];
    if (raw >= 0 && raw < d.num_phys) phys = raw;
    else set_status(status, MOIRA_ST_BAD_PAGE);
  }
  double acc[G];
#pragma unroll
  for (int g = 0; g < G; ++g) acc[g] = 0.0;
  if (phys >= 0) {
    const float4* row = reinterpret_cast<const float4*>(summaries + (phys * d.H + j) * D);
    float4 v[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) v[i] = row[i * 4 + k];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = i * 16 + k * 4;
      const double x0 = v[i].x, x1 = v[i].y, x2 = v[i].z, x3 = v[i].w;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const double* qg = qs + g * D + c;
        acc[g] = fma(qg[0], x0, acc[g]);
        acc[g] = fma(qg[1], x1, acc[g]);
        acc[g] = fma(qg[2], x2, acc[g]);
        acc[g] = fma(qg[3], x3, acc[g]);
      }
    }
  }
  // all-reduce over the 4 lanes of the page
#pragma unroll
  for (int g = 0; g < G; ++g) {
    acc[g] += __shfl_xor(acc[g], 1, 64);
    acc[g] += __shfl_xor(acc[g], 2, 64);
  }
  double mu = -INFINITY;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    acc[g] *= dscale;
    mu = fmax(mu, acc[g]);
  }
  double part = 0.0;
#pragma unroll
  for (int g = 0; g < G; ++g)
    if ((g & 3) == k) part += exp(acc[g] - mu);
  part += __shfl_xor(part, 1, 64);
  part += __shfl_xor(part, 2, 64);
  unsigned long long kreg = 0;
  if (live && k == 0) {
    unsigned long long key = 0;
    if (phys >= 0) {
      const int n = min(d.ps, L - p * d.ps);
      const double v = static_cast<double>(n) * part;         // in [1, 16G]
      double t = mu * 1.4426950408889634;                      // log2 of exp(mu)
      t = fmin(fmax(t, -1.0e6), 1.0e6);
      const double e1 = floor(t);
      const double x = v * exp2(t - e1);                        // in [1, 32G)
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
    kreg = key;
    if (static_cast<long long>(key >> 52) > eref) {
      over = 1;
    } else {
      const int b = band_of(key, ref);
      atomicAdd(&lq[b], key_mass(key, eref, F));
      atomicAdd(&lc[b], 1u);
    }
  }
  __syncthreads();
  unsigned long long* ghq = ws.hq + static_cast<long long>(s) * kBands;
  unsigned int* ghc = ws.hc + static_cast<long long>(s) * kBands;
  for (int b = threadIdx.x; b < kBands; b += blockDim.x) {
    const unsigned int c = lc[b];
    if (c) {
      atomicAdd(&ghq[b], lq[b]);
      atomicAdd(&ghc[b], c);
    }
  }
  const unsigned long long wm = wave_max_dpp_u64(kreg);
  if (lane == 0) wmax[wave] = wm;
  __syncthreads();
  if (threadIdx.x == 0) {
    if (over) atomicOr(&ws.flag[s], 1u);
    unsigned long long m = wmax[0];
    for (int w = 1; w < 4; ++w) m = wmax[w] > m ? wmax[w] : m;
    ws.cmax[static_cast<long long>(s) * ((d.max_pages + kScoreChunk - 1) / kScoreChunk) + blockIdx.x] = m;
  }
}

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
  int ncl;                              // candidates written to the next buffer
  unsigned long long tk;                // threshold key T
  int take;                             // pages of key T kept, in page order
  unsigned int gt[kMaxPages / 32];      // page bitmap: kept regardless of ties
  unsigned int eq[kMaxPages / 32];      // page bitmap: key == T
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
                            long long eref, int F, CutShared<NT>& sh) {
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
            if (ok > mk || (ok == mk && sh.cp[buf][c] < mp)) acc += key_mass(ok, eref, F);
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
        const unsigned long long qv = key_mass(lo, eref, F);
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
      atomicAdd(&sh.hq[static_cast<int>((x >> shift) - base)], key_mass(x, eref, F));
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

// One 1024-thread workgroup per (request, KV head). The segment's keys are
// copied once into LDS (coalesced); thread t owns pages e*NT + t, e < E =
// ceil(P/NT) <= 16, and keeps its candidate / kept flags as bit masks. The
// kept set is written to two LDS page bitmaps (one wave ballot per 64 pages),
// which a blocked pass (thread t owns pages [tE, tE+E)) turns into ascending
// ids, staged in LDS over the keys and copied out coalesced.
constexpr int kCutThreads = 1024;
constexpr int kCutMaxE = kMaxPages / kCutThreads;

__global__ __launch_bounds__(kCutThreads) void cut_kernel(Dims d, SelectWs ws,
                                                          const int32_t* __restrict__ seq_lens,
                                                          double gamma,
                                                          int32_t* __restrict__ page_lists,
                                                          int32_t* __restrict__ list_lens) {
  constexpr int NT = kCutThreads;
  constexpr int NW = NT / 64;
  constexpr int BPT = kBands / NT;  // level-1 bands owned per thread
  static_assert(kCutMaxE <= 32, "per-thread masks are 32-bit");
  __shared__ CutShared<NT> sh;
  extern __shared__ __align__(16) unsigned long long kl[];   // [max_pages] keys, later ids
  using mask_t = unsigned int;
  const int s = blockIdx.x;
  const int r = s / d.H;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  int L = seq_lens[r];
  if (L < 1 || L > d.max_pages * d.ps) L = 0;
  const int P = (L + d.ps - 1) / d.ps;
  int32_t* out = page_lists + static_cast<long long>(s) * d.max_pages;

  if (P == 0 || gamma >= 1.0) {
    for (int p = tid; p < P; p += NT) out[p] = p;
    if (tid == 0) list_lens[s] = P;
    return;
  }
  const int E = (P + NT - 1) / NT;

  // keys into LDS (all loads issued before the first store); this thread's
  // bands; the chunk maxima; the reference
  const unsigned long long* kin = ws.keys + static_cast<long long>(s) * d.max_pages;
  {
    unsigned long long kv[kCutMaxE];
#pragma unroll
    for (int e = 0; e < kCutMaxE; ++e) {
      const int p = e * NT + tid;
      kv[e] = p < P ? kin[p] : 0ull;
    }
#pragma unroll
    for (int e = 0; e < kCutMaxE; ++e) {
      const int p = e * NT + tid;
      if (p < P) kl[p] = kv[e];
    }
  }
  const int nch = (P + kScoreChunk - 1) / kScoreChunk;
  unsigned long long cm = 0;
  if (tid < nch)
    cm = ws.cmax[static_cast<long long>(s) * ((d.max_pages + kScoreChunk - 1) / kScoreChunk) + tid];
  unsigned long long* ghq = ws.hq + static_cast<long long>(s) * kBands + tid * BPT;
  unsigned int* ghc = ws.hc + static_cast<long long>(s) * kBands + tid * BPT;
  unsigned long long bq[BPT];
  unsigned int bcnt[BPT];
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    bq[b] = ghq[b];
    bcnt[b] = ghc[b];
  }
  const unsigned long long ref = ws.ref[s];
  const unsigned int flagged = ws.flag[s];
  const unsigned long long kmax = block_max_u64<NT>(cm, sh);   // also orders the LDS keys
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
  if (tid == 0) {
    sh.bci[0] = -1;
    sh.ncl = 0;
  }

  if (ref_ok) {
    // ---- level 1 from the band histogram (bands ascend from the heaviest)
    eref = ref_exponent(ref);
    unsigned long long own = 0;
#pragma unroll
    for (int b = 0; b < BPT; ++b) own += bq[b];
    unsigned long long Z;
    const unsigned long long before = block_excl_scan_u64<NT>(own, &Z, sh);  // also orders the LDS keys
    tau = gamma_target(gamma, Z);
    unsigned long long run = before;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      const unsigned long long prev = run;
      run += bq[b];
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
    if (band < 0) {              // unreachable while tau <= Z: keep everything
      for (int e = 0; e < E; ++e)
        if (e * NT + tid < P) sel |= mask_t(1) << e;
    } else if (nband <= kCandCap) {
      // compact the band's pages into LDS and resolve them there
      for (int e = 0; e < E; ++e) {
        const int p = e * NT + tid;
        if (p < P && band_of(kl[p], ref) == band) {
          const int o = atomicAdd(&sh.ncl, 1);
          if (o < kCandCap) {
            sh.ck[0][o] = kl[p];
            sh.cp[0][o] = p;
          }
        }
      }
      __syncthreads();
      resolve_lds<NT>(min(sh.ncl, kCandCap), 0, A, tau, eref, F, sh);
      threshold = true;
    } else {
      for (int e = 0; e < E; ++e) {
        const int p = e * NT + tid;
        if (p < P) {
          const int b = band_of(kl[p], ref);
          if (b < band) sel |= mask_t(1) << e;
          else if (b == band) cand |= mask_t(1) << e;
        }
      }
    }
  } else {
    // ---- no usable reference: exact masses relative to this call's max
    eref = static_cast<long long>(kmax >> 52);
    unsigned long long lsum = 0;
    for (int e = 0; e < E; ++e) {
      const int p = e * NT + tid;
      if (p < P) {
        lsum += key_mass(kl[p], eref, F);
        cand |= mask_t(1) << e;
      }
    }
    tau = gamma_target(gamma, block_sum_u64<NT>(lsum, sh));
  }

  // ---- radix select over the candidate masks (fallback paths); every branch
  // below depends only on block-uniform values
  int ncand = static_cast<int>(block_sum_u64<NT>(static_cast<unsigned long long>(__popc(cand)), sh));
  bool resolved = threshold || ncand == 0;
#pragma unroll 1
  for (int level = 0; level < 12 && !resolved; ++level) {
    unsigned long long lo = ~0ull, hi = 0;
    for (int e = 0; e < E; ++e)
      if (cand >> e & 1u) {
        const unsigned long long x = kl[e * NT + tid];
        lo = x < lo ? x : lo;
        hi = x > hi ? x : hi;
      }
    block_minmax_u64<NT>(lo, hi, sh);
    if (lo == hi || ncand <= kCandCap) {
      // few enough (or all equal): finish in LDS as a threshold
      if (tid == 0) sh.ncl = 0;
      __syncthreads();
      for (int e = 0; e < E; ++e)
        if (cand >> e & 1u) {
          const int p = e * NT + tid;
          const int o = atomicAdd(&sh.ncl, 1);
          if (o < kCandCap) {
            sh.ck[0][o] = kl[p];
            sh.cp[0][o] = p;
          }
        }
      __syncthreads();
      if (lo == hi) {
        if (tid == 0) {
          const unsigned long long qv = key_mass(lo, eref, F);
          const unsigned long long t = qv ? (tau - A + qv - 1) / qv : static_cast<unsigned long long>(ncand);
          sh.tk = lo;
          sh.take = static_cast<int>(t < static_cast<unsigned long long>(ncand) ? t : ncand);
        }
        __syncthreads();
      } else {
        resolve_lds<NT>(ncand, 0, A, tau, eref, F, sh);
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
    for (int e = 0; e < E; ++e)
      if (cand >> e & 1u) {
        const unsigned long long x = kl[e * NT + tid];
        atomicAdd(&sh.hq[static_cast<int>((x >> shift) - base)], key_mass(x, eref, F));
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
    for (int e = 0; e < E; ++e)
      if (cand >> e & 1u) {
        const int b = static_cast<int>((kl[e * NT + tid] >> shift) - base);
        if (b > bstar) {
          sel |= mask_t(1) << e;
          cand &= ~(mask_t(1) << e);
        } else if (b < bstar) {
          cand &= ~(mask_t(1) << e);
        } else {
          ++kept;
        }
      }
    ncand = static_cast<int>(block_sum_u64<NT>(static_cast<unsigned long long>(kept), sh));
  }
  if (!resolved) sel |= cand;  // keeps the kept mass >= gamma whatever happened

  // ---- page bitmaps: "gt" = kept outright, "eq" = key == T (kept by rank)
  const unsigned long long T = threshold ? sh.tk : 0ull;
  const int take = threshold ? sh.take : 0;
  for (int e = 0; e < E; ++e) {
    const int p = e * NT + tid;
    const bool v = p < P;
    const unsigned long long x = v ? kl[p] : 0ull;
    const bool g = threshold ? (v && x > T) : ((sel >> e & 1u) != 0);
    const bool q = threshold && v && x == T;
    const unsigned long long gm = __ballot(g);
    const unsigned long long em = __ballot(q);
    if (lane == 0) {
      const int w = (e * NT + wave * 64) >> 5;
      sh.gt[w] = static_cast<unsigned int>(gm);
      sh.gt[w + 1] = static_cast<unsigned int>(gm >> 32);
      sh.eq[w] = static_cast<unsigned int>(em);
      sh.eq[w + 1] = static_cast<unsigned int>(em >> 32);
    }
  }
  __syncthreads();

  // ---- blocked pass in page order: position = gt before + min(eq before, take)
  const int p0 = tid * E;
  unsigned int cg = 0, ce = 0;
  for (int i = 0; i < E; ++i) {
    const int p = p0 + i;
    if (p < P) {
      cg += sh.gt[p >> 5] >> (p & 31) & 1u;
      ce += sh.eq[p >> 5] >> (p & 31) & 1u;
    }
  }
  unsigned int tot;
  const unsigned int pre = block_excl_scan_u32<NT>(cg | (ce << 16), &tot, sh);
  unsigned int gb = pre & 0xffffu;
  unsigned int eb = pre >> 16;
  const unsigned int ntake = min(static_cast<unsigned int>(take), tot >> 16);
  int* ids = reinterpret_cast<int*>(kl);   // keys are no longer read
  for (int i = 0; i < E; ++i) {
    const int p = p0 + i;
    if (p < P) {
      if (sh.gt[p >> 5] >> (p & 31) & 1u) {
        ids[gb + min(eb, ntake)] = p;
        ++gb;
      } else if (sh.eq[p >> 5] >> (p & 31) & 1u) {
        if (eb < ntake) ids[gb + eb] = p;
        ++eb;
      }
    }
  }
  const int total = static_cast<int>((tot & 0xffffu) + ntake);
  __syncthreads();
  for (int i = tid; i < total; i += NT) out[i] = ids[i];
  // clear this thread's bands and the call's largest key for the next call
#pragma unroll
  for (int b = 0; b < BPT; ++b) {
    ghq[b] = 0ull;
    ghc[b] = 0u;
  }
  if (tid == 0) {
    list_lens[s] = total;
    ws.ref[s] = kmax;      // reference for the next call's band histogram
    ws.flag[s] = 0u;
  }
}

// ---- host launcher ----------------------------------------------------------
template <typename QT, int D>
static void launch_score_d(const Dims& d, const void* q, const float* summaries,
                           const int32_t* block_table, const int32_t* seq_lens, float scale,
                           const SelectWs& ws, int32_t* status, hipStream_t st) {
  dim3 grid((d.max_pages + kScoreChunk - 1) / kScoreChunk, d.S());
  const QT* qq = static_cast<const QT*>(q);
#define MOIRA_SCORE(GG) score_kernel<QT, D, GG><<<grid, 256, 0, st>>>(d, qq, summaries, block_table, seq_lens, scale, ws, status)
  switch (d.G) {
    case 1: MOIRA_SCORE(1); break;
    case 2: MOIRA_SCORE(2); break;
    case 3: MOIRA_SCORE(3); break;
    case 4: MOIRA_SCORE(4); break;
    case 5: MOIRA_SCORE(5); break;
    case 6: MOIRA_SCORE(6); break;
    case 7: MOIRA_SCORE(7); break;
    case 8: MOIRA_SCORE(8); break;
    case 9: MOIRA_SCORE(9); break;
    case 10: MOIRA_SCORE(10); break;
    case 11: MOIRA_SCORE(11); break;
    case 12: MOIRA_SCORE(12); break;
    case 13: MOIRA_SCORE(13); break;
    case 14: MOIRA_SCORE(14); break;
    case 15: MOIRA_SCORE(15); break;
    default: MOIRA_SCORE(16); break;
  }
#undef MOIRA_SCORE
}

template <typename QT>
static void launch_score_t(const Dims& d, const void* q, const float* summaries,
                           const int32_t* block_table, const int32_t* seq_lens, float scale,
                           const SelectWs& ws, int32_t* status, hipStream_t st) {
  if (d.D == 128) launch_score_d<QT, 128>(d, q, summaries, block_table, seq_lens, scale, ws, status, st);
  else launch_score_d<QT, 64>(d, q, summaries, block_table, seq_lens, scale, ws, status, st);
}

hipError_t launch_select(const Dims& d, int q_dtype, const void* q, const float* summaries,
                         const int32_t* block_table, const int32_t* seq_lens, double gamma,
                         float scale, void* workspace, int32_t* page_lists, int32_t* list_lens,
                         int32_t* status, hipStream_t st) {
  const int S = d.S();
  const SelectWs ws = select_ws(workspace, S, d.max_pages);
  if (gamma < 1.0) {
    if (q_dtype == MOIRA_BF16)
      launch_score_t<uint16_t>(d, q, summaries, block_table, seq_lens, scale, ws, status, st);
    else
      launch_score_t<float>(d, q, summaries, block_table, seq_lens, scale, ws, status, st);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const size_t dyn = static_cast<size_t>(d.max_pages) * sizeof(unsigned long long);
  // dynamic LDS above the default limit (a host-side attribute, legal during capture)
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&cut_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize,
                                     static_cast<int>(kMaxPages * sizeof(unsigned long long)));
  if (e != hipSuccess) return e;
  cut_kernel<<<S, kCutThreads, dyn, st>>>(d, ws, seq_lens, gamma, page_lists, list_lens);
  return hipGetLastError();
}

size_t select_workspace_bytes(int S, int max_pages) { return select_ws_bytes(S, max_pages); }

}  // namespace moira
