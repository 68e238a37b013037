// Coverage-rule page selection (MOIRA abstract: for every request, layer, KV
// head and step keep the smallest set of pages whose estimated attention mass
// reaches a fraction gamma).
//
// Three kernels:
//  * score (chip-wide, grid = page chunks x segments): for each page, the G
//    logits l_h = scale * q_h . kbar_p in fp64 from the fp32 summary, and the
//    page's unnormalised mass w_p = n_p * sum_h exp(l_h) packed into one
//    64-bit order-preserving key: a 12-bit biased binary exponent over the
//    52-bit fraction of the significand. The key is a function of the page's
//    own data only, so pages with equal inputs get equal keys and the
//    index tie rule decides between them. Each workgroup also stores its
//    chunk's largest key.
//  * hist (chip-wide): masses quantised to exact integers relative to the
//    segment's largest page (F fractional bits), accumulated into a
//    4096-bin histogram per segment whose bins are 1/128-octave bands below
//    the largest key (LDS per workgroup, then device atomics: integer sums,
//    so the result does not depend on order).
//  * cut (one 256-thread workgroup per (request, KV head)): a prefix scan of
//    the histogram finds the band in which the ranked running mass reaches
//    gamma * total; pages in heavier bands are kept, pages in lighter bands
//    dropped, and the band's pages are resolved by a mass-weighted radix
//    select on their keys (8-bit digits in LDS), the last <= 64 ranked
//    pairwise with exact ties by page index. Keys stay in registers
//    (blocked layout: thread t owns pages [tE, tE+E)); kept pages are
//    written in ascending order with one block scan.
#include "moira_common.h"

namespace moira {

constexpr int kScoreChunk = 64;        // pages per score workgroup (one per lane quad)
constexpr int kHistChunk = 256;        // pages per hist workgroup
constexpr int kBins = 4096;            // level-1 bands per segment
constexpr int kBandShift = 45;         // key >> 45: exponent + 7 fraction bits
constexpr int kCutBins = 256;          // digit bins of the in-workgroup radix levels
constexpr unsigned long long kMask52 = (1ull << 52) - 1;

__device__ __forceinline__ unsigned long long fmax_u64_4(const unsigned long long* v) {
  unsigned long long m = v[0];
  for (int i = 1; i < 4; ++i) m = v[i] > m ? v[i] : m;
  return m;
}

// Device workspace of moira_select_pages: keys, per-chunk maxima, histograms.
struct SelectWs {
  unsigned long long* keys;    // [S][max_pages]
  unsigned long long* cmax;    // [S][ceil(max_pages / kScoreChunk)]
  unsigned long long* hq;      // [S][kBins] quantised mass per band
  unsigned int* hc;            // [S][kBins] pages per band
  int nchunks;
};

__host__ __device__ inline size_t select_ws_bytes(int S, int max_pages) {
  const size_t nch = (static_cast<size_t>(max_pages) + kScoreChunk - 1) / kScoreChunk;
  return static_cast<size_t>(S) * (static_cast<size_t>(max_pages) * 8 + nch * 8 + kBins * 12);
}

inline SelectWs select_ws(void* base, int S, int max_pages) {
  SelectWs w;
  w.nchunks = (max_pages + kScoreChunk - 1) / kScoreChunk;
  unsigned char* p = static_cast<unsigned char*>(base);
  w.keys = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * max_pages * 8;
  w.cmax = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * w.nchunks * 8;
  w.hq = reinterpret_cast<unsigned long long*>(p);
  p += static_cast<size_t>(S) * kBins * 8;
  w.hc = reinterpret_cast<unsigned int*>(p);
  return w;
}

__device__ __forceinline__ unsigned long long key_mass(unsigned long long key, long long emax,
                                                       int F) {
  const long long ek = static_cast<long long>(key >> 52);
  const long long sh = 52 - F + (emax - ek);
  if (sh >= 64) return 0ull;
  return ((1ull << 52) | (key & kMask52)) >> sh;
}

// Fractional bits of the fixed-point masses of a segment with P pages: the
// sum of P masses, each < 2^(F+1), stays below 2^63.
__device__ __forceinline__ int mass_frac_bits(int P) {
  const int clog = P > 1 ? 32 - __clz(P - 1) : 0;
  return min(52, 62 - clog);
}

__device__ __forceinline__ int band_of(unsigned long long key, unsigned long long kmax) {
  const unsigned long long b = (kmax >> kBandShift) - (key >> kBandShift);
  return b < kBins - 1 ? static_cast<int>(b) : kBins - 1;
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
  if (blockIdx.x == 0) {  // clear this segment's histogram for the hist kernel
    unsigned long long* hq = ws.hq + static_cast<long long>(s) * kBins;
    unsigned int* hc = ws.hc + static_cast<long long>(s) * kBins;
    for (int i = threadIdx.x; i < kBins; i += blockDim.x) {
      hq[i] = 0ull;
      hc[i] = 0u;
    }
  }
  __syncthreads();
  unsigned long long kloc = 0;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int k = lane & 3;
  const int slot = lane >> 2;
  constexpr int NI = D / 16;  // float4 pieces per lane
  const double dscale = static_cast<double>(scale);

  for (int pass = 0; pass < kScoreChunk / 64; ++pass) {
    const int p = c0 + pass * 64 + wave * 16 + slot;
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
        long long E = static_cast<long long>(e1) + ex - 1;        // x 2^e1 = (2m) 2^E
        const double mant = 2.0 * m;
        long long biased = E + 2048;
        if (biased < 0 || biased > 4095) {
          set_status(status, MOIRA_ST_MASS_RANGE);
          key = biased < 0 ? 0ull : ((4095ull << 52) | kMask52);
        } else {
          key = (static_cast<unsigned long long>(biased) << 52) |
                (static_cast<unsigned long long>(__double_as_longlong(mant)) & kMask52);
        }
      }
      ws.keys[static_cast<long long>(s) * d.max_pages + p] = key;
      kloc = key;
    }
  }
  kloc = wave_max_u64(kloc);
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = kloc;
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long m = wmax[0];
    for (int w = 1; w < 4; ++w) m = wmax[w] > m ? wmax[w] : m;
    ws.cmax[static_cast<long long>(s) * ws.nchunks + blockIdx.x] = m;
  }
}

// grid (ceil(max_pages / kHistChunk), S), 256 threads: one page per thread.
__global__ __launch_bounds__(256) void hist_kernel(Dims d, const int32_t* __restrict__ seq_lens,
                                                   SelectWs ws) {
  __shared__ unsigned long long hq[kBins];
  __shared__ unsigned int hc[kBins];
  __shared__ unsigned long long wmax[4];
  const int s = blockIdx.y;
  const int r = s / d.H;
  int L = seq_lens[r];
  if (L < 1 || L > d.max_pages * d.ps) L = 0;
  const int P = (L + d.ps - 1) / d.ps;
  const int c0 = blockIdx.x * kHistChunk;
  if (c0 >= P) return;
  const int tid = threadIdx.x;
  const int nch = (P + kScoreChunk - 1) / kScoreChunk;
  unsigned long long m = 0;
  for (int c = tid; c < nch; c += blockDim.x) {
    const unsigned long long x = ws.cmax[static_cast<long long>(s) * ws.nchunks + c];
    m = x > m ? x : m;
  }
  const int p = c0 + tid;
  const unsigned long long key = p < P ? ws.keys[static_cast<long long>(s) * d.max_pages + p] : 0ull;
  for (int b = tid; b < kBins; b += blockDim.x) {
    hq[b] = 0ull;
    hc[b] = 0u;
  }
  m = wave_max_u64(m);
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  const unsigned long long kmax = fmax_u64_4(wmax);
  if (p < P) {
    const int b = band_of(key, kmax);
    atomicAdd(&hq[b], key_mass(key, static_cast<long long>(kmax >> 52), mass_frac_bits(P)));
    atomicAdd(&hc[b], 1u);
  }
  __syncthreads();
  unsigned long long* ghq = ws.hq + static_cast<long long>(s) * kBins;
  unsigned int* ghc = ws.hc + static_cast<long long>(s) * kBins;
  for (int b = tid; b < kBins; b += blockDim.x) {
    const unsigned int c = hc[b];
    if (c) {
      atomicAdd(&ghq[b], hq[b]);
      atomicAdd(&ghc[b], c);
    }
  }
}

// ---- block-wide helpers for the cut kernel (NT threads, NT/64 waves) --------
template <int NT>
struct CutShared {
  unsigned long long hq[kCutBins];
  unsigned long long red[2][NT / 64];
  int redi[NT / 64];
  unsigned long long bc[2];
  int bci[2];
  unsigned long long ck[64];
  unsigned long long cq[64];
  int cp[64];
  int cres[64];
};

// Min and max of a u64 over the block (one barrier pair).
template <int NT>
__device__ __forceinline__ void block_minmax_u64(unsigned long long& lo, unsigned long long& hi,
                                                 CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  lo = wave_min_u64(lo);
  hi = wave_max_u64(hi);
  const int lane = threadIdx.x & 63;
  if (lane == 0) {
    sh.red[0][threadIdx.x >> 6] = lo;
    sh.red[1][threadIdx.x >> 6] = hi;
  }
  __syncthreads();
  lo = sh.red[0][0];
  hi = sh.red[1][0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    lo = sh.red[0][w] < lo ? sh.red[0][w] : lo;
    hi = sh.red[1][w] > hi ? sh.red[1][w] : hi;
  }
  __syncthreads();
}
template <int NT>
__device__ __forceinline__ unsigned long long block_sum_u64(unsigned long long v, CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  v = wave_sum_u64(v);
  if ((threadIdx.x & 63) == 0) sh.red[0][threadIdx.x >> 6] = v;
  __syncthreads();
  unsigned long long t = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) t += sh.red[0][w];
  __syncthreads();
  return t;
}
// Exclusive prefix over threads in thread order; *total gets the block sum.
template <int NT>
__device__ __forceinline__ int block_excl_scan_i32(int v, int* total, CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  const int incl = wave_incl_scan<int>(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) sh.redi[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int x = sh.redi[w];
    before += w < wave ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}
template <int NT>
__device__ __forceinline__ unsigned long long block_excl_scan_u64(unsigned long long v,
                                                                  unsigned long long* total,
                                                                  CutShared<NT>& sh) {
  constexpr int NW = NT / 64;
  const unsigned long long incl = wave_incl_scan<unsigned long long>(v);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 63) sh.red[0][wave] = incl;
  __syncthreads();
  unsigned long long before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const unsigned long long x = sh.red[0][w];
    before += w < wave ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// One workgroup of NT threads per (request, KV head); E pages per thread in a
// blocked layout (thread t owns pages [tE, tE+E)), keys kept in registers.
template <int NT, int E>
__global__ __launch_bounds__(NT) void cut_kernel(Dims d, SelectWs ws,
                                                 const int32_t* __restrict__ seq_lens, double gamma,
                                                 int32_t* __restrict__ page_lists,
                                                 int32_t* __restrict__ list_lens) {
  static_assert(E <= 64, "candidate masks are 64-bit");
  constexpr int BPT = kBins / NT;   // level-1 bands owned per thread
  __shared__ CutShared<NT> sh;
  using mask_t = unsigned long long;
  const int s = blockIdx.x;
  const int r = s / d.H;
  const int tid = threadIdx.x;
  int L = seq_lens[r];
  if (L < 1 || L > d.max_pages * d.ps) L = 0;
  const int P = (L + d.ps - 1) / d.ps;
  int32_t* out = page_lists + static_cast<long long>(s) * d.max_pages;
  const int p0 = tid * E;

  if (P == 0 || gamma >= 1.0) {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (p0 + e < P) out[p0 + e] = p0 + e;
    if (tid == 0) list_lens[s] = P;
    return;
  }

  // keys of this thread's pages and this thread's level-1 bands
  unsigned long long key[E];
  mask_t valid = 0;
  const unsigned long long* kin = ws.keys + static_cast<long long>(s) * d.max_pages;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int p = p0 + e;
    key[e] = p < P ? kin[p] : 0ull;
    if (p < P) valid |= mask_t(1) << e;
  }
  unsigned long long bq[BPT];
  unsigned int bcnt[BPT];
  {
    const unsigned long long* ghq = ws.hq + static_cast<long long>(s) * kBins + tid * BPT;
    const unsigned int* ghc = ws.hc + static_cast<long long>(s) * kBins + tid * BPT;
#pragma unroll
    for (int b = 0; b < BPT; ++b) {
      bq[b] = ghq[b];
      bcnt[b] = ghc[b];
    }
  }
  unsigned long long lo = ~0ull, hi = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (valid >> e & 1) {
      lo = key[e] < lo ? key[e] : lo;
      hi = key[e] > hi ? key[e] : hi;
    }
  block_minmax_u64<NT>(lo, hi, sh);
  const unsigned long long kmax = hi;
  const long long emax = static_cast<long long>(kmax >> 52);
  const int F = mass_frac_bits(P);

  // Level 1 from the band histogram: bands ascend from the heaviest.
  unsigned long long own = 0;
#pragma unroll
  for (int b = 0; b < BPT; ++b) own += bq[b];
  unsigned long long Z;
  const unsigned long long before = block_excl_scan_u64<NT>(own, &Z, sh);
  unsigned long long tau;
  {
    const double zt = gamma * static_cast<double>(Z);
    if (!(zt < 18446744073709551615.0)) tau = Z;
    else tau = static_cast<unsigned long long>(ceil(zt));
    if (tau > Z) tau = Z;
    if (tau < 1) tau = 1;
  }
  if (tid == 0) sh.bci[0] = -1;
  __syncthreads();
  {
    unsigned long long run = before;   // mass of all bands before this thread's
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
  }
  __syncthreads();
  const int band = sh.bci[0];
  unsigned long long A = sh.bc[0];    // mass of pages known to rank above every candidate
  int ncand = sh.bci[1];
  __syncthreads();

  mask_t cand = 0;
  mask_t sel = 0;
  if (band < 0) {           // unreachable while tau <= Z: keep everything
    sel = valid;
    ncand = 0;
  } else {
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (valid >> e & 1) {
        const int b = band_of(key[e], kmax);
        if (b < band) sel |= mask_t(1) << e;
        else if (b == band) cand |= mask_t(1) << e;
      }
  }
  bool resolved = ncand == 0;

#pragma unroll 1
  for (int level = 0; level < 12 && !resolved; ++level) {
    lo = ~0ull;
    hi = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (cand >> e & 1) {
        lo = key[e] < lo ? key[e] : lo;
        hi = key[e] > hi ? key[e] : hi;
      }
    block_minmax_u64<NT>(lo, hi, sh);
    if (lo == hi) {
      // Every candidate has the same mass: ties rank by page index.
      const unsigned long long qv = key_mass(lo, emax, F);
      const unsigned long long take = qv ? (tau - A + qv - 1) / qv : ~0ull;
      int total;
      const int pre = block_excl_scan_i32<NT>(__popcll(cand), &total, sh);
      int i = 0;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (cand >> e & 1) {
          if (static_cast<unsigned long long>(pre + i) < take) sel |= mask_t(1) << e;
          ++i;
        }
      resolved = true;
      break;
    }
    if (ncand <= 64) {
      // Rank the last candidates pairwise: c' ranks before c if its key is
      // larger, or equal with a lower page index. Integer sums: exact.
      int total;
      const int pre = block_excl_scan_i32<NT>(__popcll(cand), &total, sh);
      int i = 0;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (cand >> e & 1) {
          const int idx = pre + i;
          if (idx < 64) {
            sh.ck[idx] = key[e];
            sh.cq[idx] = key_mass(key[e], emax, F);
            sh.cp[idx] = p0 + e;
          }
          ++i;
        }
      __syncthreads();
      if (tid < total && tid < 64) {
        const unsigned long long mk = sh.ck[tid];
        const int mp = sh.cp[tid];
        unsigned long long acc = A;
#pragma unroll 1
        for (int c = 0; c < total; ++c) {
          const unsigned long long ok = sh.ck[c];
          if (ok > mk || (ok == mk && sh.cp[c] < mp)) acc += sh.cq[c];
        }
        sh.cres[tid] = acc < tau ? 1 : 0;
      }
      __syncthreads();
      i = 0;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (cand >> e & 1) {
          const int idx = pre + i;
          if (idx < 64 && sh.cres[idx]) sel |= mask_t(1) << e;
          ++i;
        }
      resolved = true;
      break;
    }

    // Mass-weighted histogram of the candidates on the 8 key bits below
    // their common prefix; digits ascend with mass.
    const int hb = 63 - __clzll(static_cast<long long>(lo ^ hi));
    const int shift = hb > 7 ? hb - 7 : 0;
    const unsigned long long base = lo >> shift;
    for (int b = tid; b < kCutBins; b += NT) sh.hq[b] = 0ull;
    if (tid == 0) sh.bci[0] = -1;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (cand >> e & 1) {
        const int b = static_cast<int>((key[e] >> shift) - base);
        atomicAdd(&sh.hq[b], key_mass(key[e], emax, F));
      }
    __syncthreads();
    // S(b) = sum_{b' >= b} hq[b']; the crossing bin b* has A + S(b*) >= tau > A + S(b*+1).
    const unsigned long long mine = tid < kCutBins ? sh.hq[tid] : 0ull;
    unsigned long long all;
    const unsigned long long below = block_excl_scan_u64<NT>(mine, &all, sh);  // sum over bins < tid
    if (tid < kCutBins) {
      const unsigned long long Sb = all - below;       // S(tid)
      const unsigned long long Sb1 = Sb - mine;        // S(tid + 1)
      if (A + Sb >= tau && A + Sb1 < tau) {
        sh.bci[0] = tid;
        sh.bc[0] = A + Sb1;
      }
    }
    __syncthreads();
    const int bstar = sh.bci[0];
    if (bstar < 0) break;  // not reachable while the invariant A < tau <= A + S(0) holds
    A = sh.bc[0];
    int kept = 0;
#pragma unroll
    for (int e = 0; e < E; ++e)
      if (cand >> e & 1) {
        const int b = static_cast<int>((key[e] >> shift) - base);
        if (b > bstar) {
          sel |= mask_t(1) << e;
          cand &= ~(mask_t(1) << e);
        } else if (b < bstar) {
          cand &= ~(mask_t(1) << e);
        } else {
          ++kept;
        }
      }
    int nc;
    block_excl_scan_i32<NT>(kept, &nc, sh);
    ncand = nc;
  }
  if (!resolved) sel |= cand;  // keeps the kept mass >= gamma whatever happened

  int total;
  const int pre = block_excl_scan_i32<NT>(__popcll(sel), &total, sh);
  int i = 0;
#pragma unroll
  for (int e = 0; e < E; ++e)
    if (sel >> e & 1) {
      out[pre + i] = p0 + e;
      ++i;
    }
  if (tid == 0) list_lens[s] = total;
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
    hist_kernel<<<dim3((d.max_pages + kHistChunk - 1) / kHistChunk, S), 256, 0, st>>>(d, seq_lens, ws);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int mp = d.max_pages;
#define MOIRA_CUT(NT, E) cut_kernel<NT, E><<<S, NT, 0, st>>>(d, ws, seq_lens, gamma, page_lists, list_lens)
  if (mp <= 256 * 4) MOIRA_CUT(256, 4);
  else if (mp <= 256 * 8) MOIRA_CUT(256, 8);
  else if (mp <= 256 * 16) MOIRA_CUT(256, 16);
  else if (mp <= 512 * 16) MOIRA_CUT(512, 16);
  else if (mp <= 512 * 24) MOIRA_CUT(512, 24);
  else if (mp <= 512 * 32) MOIRA_CUT(512, 32);
  else MOIRA_CUT(1024, 32);
#undef MOIRA_CUT
  return hipGetLastError();
}

size_t select_workspace_bytes(int S, int max_pages) { return select_ws_bytes(S, max_pages); }

}  // namespace moira
