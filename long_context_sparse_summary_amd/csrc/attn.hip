// Self-planning ragged split-K GQA decode attention and its log-sum-exp
// combine (MOIRA abstract: each workgroup derives its own share of the work
// from the list lengths, so no host-side plan is needed and the step stays
// inside a graph; the split along the sequence and the merge of partial
// states follow FlashDecoding, "Faster than Flash", section 2).
//
// Work split: the per-(request, KV head) page lists are concatenated in
// segment order s = r*H + j into W pages. Workgroup w of N takes pages
// [floor(wW/N), floor((w+1)W/N)); every workgroup builds the list offsets
// itself in LDS and finds its first segment by binary search. For each
// segment its range touches (a "piece") it writes one partial state to slot
// w + s; slots strictly increase along the pieces, so they never collide.
// With at least 8 workgroups per segment (and at most 1024 segments) the
// split is aligned to the segments instead (aligned_quota): every workgroup
// takes a share of one list only and writes its single partial state to
// slot w.
//
// bf16 K/V path (matrix cores, gfx950): one wave per page at a time, four
// waves per workgroup interleaved over the piece's pages.
//   S^T[t][g] = K[t][:] . Q[g][:]   v_mfma_f32_16x16x32_bf16, A = K rows
//                                   (tokens), B = Q^T (group heads, padded
//                                   to 16); D/32 instructions per page.
//   The accumulator layout (lane l: column g = l%16, rows t = 4(l/16)+i) is
//   exactly the A-operand layout of the 16x16x16 product, so the softmax
//   weights feed the next product without any data movement:
//   O[g][8n+c] += P[g][t] V[t][8n+c]  v_mfma_f32_16x16x16_bf16, two
//                                   instructions per c (P as bf16 hi + lo
//                                   parts); lane (n, kg) loads
//                                   16 contiguous bytes of each of its 4
//                                   token rows and two byte permutes build
//                                   each B operand.
// K and V come straight from HBM into registers in operand layout (16-byte
// loads, each row read as contiguous 64-256 byte runs); the next page's loads
// are issued before the current page is computed. Each K/V byte is read once
// per step, so the loads are non-temporal: they do not displace the lists,
// tables and partial states that other workgroups and the next kernel reuse
// from the caches.
#include "moira_common.h"

namespace moira {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// ---- self-planning prologue ---------------------------------------------
// off[0..S] in LDS: off[s] = sum_{s' < s} clamp(list_lens[s'], 0, max_pages).
__device__ int build_offsets(const int32_t* __restrict__ list_lens, int S, int max_pages,
                             int* off, int* scan_tmp, int32_t* status, bool report) {
  const int nt = blockDim.x;
  const int tid = threadIdx.x;
  const int per = (S + nt - 1) / nt;
  const int s0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s < S) {
      int v = list_lens[s];
      if (v < 0 || v > max_pages) {
        if (report) set_status(status, MOIRA_ST_BAD_LIST);
        v = v < 0 ? 0 : max_pages;
      }
      local += v;
    }
  }
  const int incl = wave_incl_scan<int>(local);
  const int wave = tid >> 6;
  const int nw = (nt + 63) >> 6;
  if ((tid & 63) == 63) scan_tmp[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < nw; ++w) {
    before += w < wave ? scan_tmp[w] : 0;
    total += scan_tmp[w];
  }
  int run = before + incl - local;
  for (int i = 0; i < per; ++i) {
    const int s = s0 + i;
    if (s < S) {
      off[s] = run;
      int v = list_lens[s];
      v = v < 0 ? 0 : (v > max_pages ? max_pages : v);
      run += v;
    }
  }
  if (tid == 0) off[S] = total;
  __syncthreads();
  return total;
}

// Last s in [0, S) with off[s] <= x (x < off[S]).
__device__ __forceinline__ int find_segment(const int* off, int S, int x) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (off[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// ---- bf16 K/V, matrix-core kernel ----------------------------------------
template <int D, bool QF32>
struct MfmaTile {
  static constexpr int KK = D / 32;     // 16x16x32 products per page for S^T
  static constexpr int NN = D / 16;     // 16x16x16 products per page for O
  static constexpr int VB = D / 16;     // bf16 values per lane per V token row
  // page buffers per wave (K and V of a page: D/4 registers per lane): four
  // fit in the registers of two waves per SIMD, but not beside the second
  // set of Q fragments that fp32 queries need
  static constexpr int NB = QF32 ? 3 : 4;
};

// Workgroups that get work: at most one per kMinPagesPerWG listed pages (one
// page per wave), so a step whose lists are short still spreads over the chip
// while no wave idles. The combine derives the same count from the same list
// lengths.
constexpr int kMinPagesPerWG = 4;
__device__ __forceinline__ int effective_wgs(int W, int N) {
  const int want = (W + kMinPagesPerWG - 1) / kMinPagesPerWG;
  return want < 1 ? 1 : (want < N ? want : N);
}

// Segment-aligned split, used when there are at least 8 workgroups per
// segment: segment s gets n_s = ceil(len_s / q) workgroups of its own, with
// q = max(ceil(W / (N - S)), kMinPagesPerWG) pages at most per workgroup, so
// that sum_s n_s <= W / q + S <= N. No workgroup then spans two lists (which
// would run the dependent start of a piece, list -> table -> K/V, twice in a
// row), at the price of up to N / (N - S) <= 8/7 times the mean pages per
// workgroup. Up to kAlignedMaxSegments segments, so that its LDS table of
// first workgroups stays small. Returns q, or 0 for the plain even split.
constexpr int kAlignedMaxSegments = 1024;
__host__ __device__ __forceinline__ bool aligned_possible(int N, int S) {
  return S <= kAlignedMaxSegments && N >= 8 * S;
}
__device__ __forceinline__ int aligned_quota(int W, int N, int S) {
  if (W <= 0 || !aligned_possible(N, S)) return 0;
  const int q = (W + (N - S) - 1) / (N - S);
  return q > kMinPagesPerWG ? q : kMinPagesPerWG;
}

// The listed pages [a, b) of workgroup w (global indices into the
// concatenated lists), its first segment s and the slot of the partial state
// of the piece in segment s: w + s for the even split (slots increase along
// the pieces), w for the aligned split (one piece per workgroup). Builds
// off[0..S] (list offsets) and, for the aligned split, wb[0..S] (first
// workgroup of each segment) in LDS. Called by every thread; false when w
// has no work.
struct WgWork {
  int a, b, s, slot_seg;   // slot = w + slot_seg * s
};

__device__ bool plan_workgroup(const int32_t* __restrict__ list_lens, const Dims& d, int N, int w,
                               int* off, int* wb, int* scan_tmp, int32_t* status, WgWork& wk) {
  const int S = d.S();
  const int W = build_offsets(list_lens, S, d.max_pages, off, scan_tmp, status, w == 0);
  const int q = aligned_quota(W, N, S);
  if (q == 0) {
    const int Ne = effective_wgs(W, N);
    if (w >= Ne) return false;
    wk.a = static_cast<int>((static_cast<long long>(w) * W) / Ne);
    wk.b = static_cast<int>((static_cast<long long>(w + 1) * W) / Ne);
    if (wk.a >= wk.b) return false;
    wk.s = find_segment(off, S, wk.a);
    wk.slot_seg = 1;
    return true;
  }
  // wb[] = exclusive prefix of n_s, scanned like off[]
  const int nt = blockDim.x;
  const int tid = threadIdx.x;
  const int per = (S + nt - 1) / nt;
  const int s0 = tid * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int t = s0 + i;
    if (t < S) local += (off[t + 1] - off[t] + q - 1) / q;
  }
  const int incl = wave_incl_scan<int>(local);
  const int wave = tid >> 6;
  const int nw = (nt + 63) >> 6;
  if ((tid & 63) == 63) scan_tmp[wave] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int v = 0; v < nw; ++v) {
    before += v < wave ? scan_tmp[v] : 0;
    total += scan_tmp[v];
  }
  int run = before + incl - local;
  for (int i = 0; i < per; ++i) {
    const int t = s0 + i;
    if (t < S) {
      wb[t] = run;
      run += (off[t + 1] - off[t] + q - 1) / q;
    }
  }
  if (tid == 0) wb[S] = total;
  __syncthreads();
  if (w >= total) return false;
  const int sg = find_segment(wb, S, w);
  const int i = w - wb[sg];
  const int n = wb[sg + 1] - wb[sg];
  const int len = off[sg + 1] - off[sg];
  wk.a = off[sg] + static_cast<int>((static_cast<long long>(i) * len) / n);
  wk.b = off[sg] + static_cast<int>((static_cast<long long>(i + 1) * len) / n);
  wk.s = sg;
  wk.slot_seg = 0;
  return wk.a < wk.b;
}

// The same plan for at most 64 segments, computed by each wave on its own in
// registers: lane t holds segment t, so the list offsets are a wave scan,
// and the segment of a list position or a workgroup is a ballot over the
// non-decreasing prefixes. No LDS and no barrier: the waves start on their
// pages as soon as the list lengths arrive. offl / offh receive off[t] /
// off[t + 1] of lane t. Called by every thread; false when w has no work.
__device__ bool plan_workgroup_wave(const int32_t* __restrict__ list_lens, const Dims& d, int N,
                                    int w, int32_t* status, WgWork& wk, int& offl, int& offh) {
  const int S = d.S();
  const int lane = threadIdx.x & 63;
  int v = 0;
  if (lane < S) {
    v = list_lens[lane];
    if (v < 0 || v > d.max_pages) {
      if (w == 0) set_status(status, MOIRA_ST_BAD_LIST);
      v = v < 0 ? 0 : d.max_pages;
    }
  }
  const int incl = wave_incl_scan<int>(v);
  const int W = __builtin_amdgcn_readlane(incl, 63);
  offl = incl - v;
  offh = incl;
  const int q = aligned_quota(W, N, S);
  if (q == 0) {
    const int Ne = effective_wgs(W, N);
    if (w >= Ne) return false;
    wk.a = static_cast<int>((static_cast<long long>(w) * W) / Ne);
    wk.b = static_cast<int>((static_cast<long long>(w + 1) * W) / Ne);
    if (wk.a >= wk.b) return false;
    // last segment with off[s] <= a: the lanes with off[t] <= a are a prefix
    wk.s = __popcll(__ballot(lane < S && offl <= wk.a)) - 1;
    wk.slot_seg = 1;
    return true;
  }
  const int n = lane < S ? (v + q - 1) / q : 0;   // workgroups of segment t
  const int wincl = wave_incl_scan<int>(n);
  const int total = __builtin_amdgcn_readlane(wincl, 63);
  if (w >= total) return false;
  // last segment whose first workgroup is <= w
  const int sg = __popcll(__ballot(lane < S && wincl - n <= w)) - 1;
  const int i = w - __builtin_amdgcn_readlane(wincl - n, sg);
  const int ns = __builtin_amdgcn_readlane(n, sg);
  const int len = __builtin_amdgcn_readlane(v, sg);
  const int o = __builtin_amdgcn_readlane(offl, sg);
  wk.a = o + static_cast<int>((static_cast<long long>(i) * len) / ns);
  wk.b = o + static_cast<int>((static_cast<long long>(i + 1) * len) / ns);
  wk.s = sg;
  wk.slot_seg = 0;
  return wk.a < wk.b;
}

struct LseState {
  float m;      // log2-domain maximum, -inf when empty
  float l;      // sum of l_i 2^(m_i - m)
  float4 o;     // sum of o_i 2^(m_i - m)
};

__device__ __forceinline__ LseState lse_merge(const LseState& a, const LseState& b) {
  const float M = fmaxf(a.m, b.m);
  if (M == -INFINITY) return a;
  const float fa = a.m == -INFINITY ? 0.f : exp2f(a.m - M);
  const float fb = b.m == -INFINITY ? 0.f : exp2f(b.m - M);
  LseState r;
  r.m = M;
  r.l = fa * a.l + fb * b.l;
  r.o = make_float4(fa * a.o.x + fb * b.o.x, fa * a.o.y + fb * b.o.y,
                    fa * a.o.z + fb * b.o.z, fa * a.o.w + fb * b.o.w);
  return r;
}

// The state of lane l ^ 8 (DPP row rotation by 8), and the states of the
// lane pair at distance 16 or 32, lower lane first (permlane swaps).
__device__ __forceinline__ LseState lse_xor8(const LseState& a) {
  auto f = [](float v) { return __uint_as_float(dpp32<0x128>(__float_as_uint(v))); };
  LseState r;
  r.m = f(a.m);
  r.l = f(a.l);
  r.o = make_float4(f(a.o.x), f(a.o.y), f(a.o.z), f(a.o.w));
  return r;
}
template <int M>
__device__ __forceinline__ void lse_pair(const LseState& a, LseState& lo, LseState& hi) {
  static_assert(M == 16 || M == 32, "permlane distance");
  auto pr = [](float v, float& x, float& y) {
    if constexpr (M == 16) lane_pair16(v, x, y);
    else lane_pair32(v, x, y);
  };
  pr(a.m, lo.m, hi.m);
  pr(a.l, lo.l, hi.l);
  pr(a.o.x, lo.o.x, hi.o.x);
  pr(a.o.y, lo.o.y, hi.o.y);
  pr(a.o.z, lo.o.z, hi.o.z);
  pr(a.o.w, lo.o.w, hi.o.w);
}

// ---- merge inside the attention kernel (moira_ragged_decode_attn_combine) ----
// The last workgroup to finish a piece of a segment merges the segment's
// partial states itself. They were written by other workgroups, on other
// XCDs whose L2 caches are not coherent with this one, through write-through
// agent-scope stores; they are read back with the device-scope (sc1) cache
// policy through buffer resources, so that the loads stay in flight together
// (the compiler waits after every agent-scope atomic load, one at a time).
constexpr int kBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format
constexpr int kCpolSc1 = 16;               // cache policy: device scope
constexpr int kMergeBatch = 16;            // pieces per round of loads and thread

// Pieces of segment s as the attention workgroups planned them (off and wb
// in LDS): slot of piece 0 and their number.
__device__ __forceinline__ void piece_span(const int* off, const int* wb, int q, int W, int N,
                                           int s, long long& slot0, int& np) {
  if (q > 0) {   // aligned split: the segment's own workgroups, slot = w
    slot0 = wb[s];
    np = wb[s + 1] - wb[s];
    return;
  }
  const int Ne = effective_wgs(W, N);
  auto wg_of = [&](long long x) -> long long {   // largest w with floor(wW/Ne) <= x
    const long long v = ((x + 1) * Ne - 1) / W;
    return v < Ne - 1 ? v : Ne - 1;
  };
  const long long w0 = wg_of(off[s]);
  slot0 = w0 + s;
  np = static_cast<int>(wg_of(static_cast<long long>(off[s + 1]) - 1) - w0 + 1);
}

// Merge the np partial states of segment s (slots slot0 .. slot0 + np - 1)
// into out with all NT threads: thread (pg, u) takes column quad u of the
// G x D outputs and the pieces pg, pg + PG, ..., kMergeBatch per round of
// loads; the PG piece groups are then merged in LDS (red: NT * 6 floats).
template <int NT>
__device__ void merge_segment(const Dims& d, int s, long long slot0, int np,
                              const float* partial_o, const float* partial_ml, long long nslots,
                              float* __restrict__ out, float* red) {
  const int G = d.G;
  const int D = d.D;
  const int U = G * D / 4;            // column quads (G D <= 1024: U <= 256)
  const int PG = NT / U;              // piece groups
  const int tid = threadIdx.x;
  const int pg = tid / U;
  const int u = tid - pg * U;
  const bool act = pg < PG;
  const int g = (4 * u) / D;
  const int col = 4 * u - g * D;
  const __amdgpu_buffer_rsrc_t ro = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(partial_o), 0, static_cast<int>(nslots * G * D * 4), kBufferWord3);
  const __amdgpu_buffer_rsrc_t rm = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<float*>(partial_ml), 0, static_cast<int>(nslots * G * 2 * 4), kBufferWord3);
  LseState st;
  st.m = -INFINITY;
  st.l = 0.f;
  st.o = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int i0 = act ? pg : np; i0 < np; i0 += PG * kMergeBatch) {
    float2 ml[kMergeBatch];
    float4 o[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const int i = i0 + k * PG;
      ml[k] = make_float2(-INFINITY, 0.f);
      o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < np) {
        const long long slot = slot0 + i;
        const u32x2_t a = __builtin_bit_cast(
            u32x2_t, __builtin_amdgcn_raw_buffer_load_b64(rm, static_cast<int>((slot * G + g) * 8), 0, kCpolSc1));
        const u32x4_t b = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(ro, static_cast<int>(((slot * G + g) * D + col) * 4), 0, kCpolSc1));
        ml[k] = make_float2(__uint_as_float(a[0]), __uint_as_float(a[1]));
        o[k] = make_float4(__uint_as_float(b[0]), __uint_as_float(b[1]), __uint_as_float(b[2]), __uint_as_float(b[3]));
      }
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      LseState t;
      t.m = ml[k].x;
      t.l = ml[k].y;
      t.o = o[k];
      st = lse_merge(st, t);
    }
  }
  if (act) {
    red[tid * 6 + 0] = st.m;
    red[tid * 6 + 1] = st.l;
    red[tid * 6 + 2] = st.o.x;
    red[tid * 6 + 3] = st.o.y;
    red[tid * 6 + 4] = st.o.z;
    red[tid * 6 + 5] = st.o.w;
  }
  __syncthreads();
  if (act && pg == 0) {
    for (int j = 1; j < PG; ++j) {
      const float* x = red + (j * U + u) * 6;
      LseState t;
      t.m = x[0];
      t.l = x[1];
      t.o = make_float4(x[2], x[3], x[4], x[5]);
      st = lse_merge(st, t);
    }
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    const int r = s / d.H;
    const int j = s - r * d.H;
    float* dst = out + (static_cast<long long>(r) * d.Hq() + static_cast<long long>(j) * G + g) * D + col;
    *reinterpret_cast<float4*>(dst) = make_float4(st.o.x * inv, st.o.y * inv, st.o.z * inv, st.o.w * inv);
  }
  __syncthreads();
}

template <int KK>
struct PageRegs {
  u32x4_t k[KK];
  u32x4_t v[4];
  long long base;   // element offset of the (page, KV head) block, -1 = none
  int n;            // tokens in the page
};

// Waves per workgroup: 8 (one workgroup per CU) when the waves' partial
// states fit the LDS merge buffer, G*D <= 1024 floats each, else 4 (two per
// CU), a template parameter of the kernel. Either way the register
// budget is that of two waves per SIMD, which holds the page buffers
// (MfmaTile::NB) without spilling.
constexpr int kAttnMaxWaves = 8;
__host__ __device__ inline int attn_waves(const Dims& d) {
  return d.G * d.D <= 1024 ? 8 : 4;
}
// COMB: the merge of each segment's partial states runs in the last
// workgroup to finish one of its pieces (arrival counters in `counters`,
// one per segment, zero between calls), which writes the segment's output.
template <int D, bool QF32, int NW, bool COMB = false>
__global__ __launch_bounds__(64 * NW, 2) void attn_mfma_kernel(
    Dims d, const void* __restrict__ qv, const uint16_t* __restrict__ k_pool,
    const uint16_t* __restrict__ v_pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_lists,
    const int32_t* __restrict__ list_lens, float scale_log2, int N,
    float* __restrict__ partial_o, float* __restrict__ partial_ml, int32_t* status,
    unsigned int* __restrict__ counters, float* __restrict__ out) {
  using T = MfmaTile<D, QF32>;
  // one value from each 64-byte line of the argument segment the plan reads
  // (the workgroup size sits in the third), asked for at entry so that the
  // lines are fetched together with one wait
  asm volatile("" ::"s"(d.B), "s"(list_lens), "s"(blockDim.x));
  extern __shared__ __align__(16) unsigned char smem[];
  const int S = d.S();
  const int G = d.G;
  int* off = reinterpret_cast<int*>(smem);
  int* wb = off + (S + 1);                                      // aligned split only
  int* scan_tmp = wb + (aligned_possible(N, S) ? S + 1 : 0);
  float* wm = reinterpret_cast<float*>(scan_tmp + 8);
  float* wl = wm + kAttnMaxWaves * kMaxGroup;
  float* wo = wl + kAttnMaxWaves * kMaxGroup;   // [waves][G][D]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  constexpr int nw = NW;                 // waves of the workgroup
  const int l16 = lane & 15;
  const int kg = lane >> 4;
  const int w = blockIdx.x;

  WgWork wk;
  // up to 64 segments (and no merge in this kernel) every wave plans on its
  // own in registers; otherwise the workgroup plans in LDS
  const bool wave_plan = !COMB && S <= 64;
  int offl = 0, offh = 0;
  const bool has_work =
      wave_plan ? plan_workgroup_wave(list_lens, d, N, w, status, wk, offl, offh)
                : plan_workgroup(list_lens, d, N, w, off, wb, scan_tmp, status, wk);
  auto off_lo = [&](int t) { return wave_plan ? __builtin_amdgcn_readlane(offl, t) : off[t]; };
  auto off_hi = [&](int t) { return wave_plan ? __builtin_amdgcn_readlane(offh, t) : off[t + 1]; };
  __shared__ int last_arriver;
  if constexpr (COMB) {
    // a segment with an empty list has no piece: workgroup 0 writes its zeros
    if (w == 0) {
      for (int t = 0; t < S; ++t) {
        if (off[t + 1] == off[t]) {
          const int r = t / d.H;
          const int j = t - r * d.H;
          float* dst = out + (static_cast<long long>(r) * d.Hq() + static_cast<long long>(j) * G) * D;
          for (int i = tid; i < G * D; i += blockDim.x) dst[i] = 0.f;
        }
      }
    }
  }
  if (!has_work) return;
  int a = wk.a;
  const int b = wk.b;
  int s = wk.s;
  const long long head_stride = static_cast<long long>(d.ps) * D;

  while (a < b) {
    while (off_hi(s) <= a) ++s;          // skip empty lists
    const int hi = min(b, off_hi(s));
    const int li0 = a - off_lo(s);
    const int li1 = hi - off_lo(s);
    const int r = s / d.H;
    const int j = s - r * d.H;
    int L = seq_lens[r];
    if (L < 1 || L > d.max_pages * d.ps) L = 0;
    const int P = (L + d.ps - 1) / d.ps;
    const int nlast = L - (P - 1) * d.ps;
    const int32_t* plist = page_lists + static_cast<long long>(s) * d.max_pages;
    const int32_t* trow = block_table + static_cast<long long>(r) * d.max_pages;
    const long long head_base = static_cast<long long>(j) * head_stride;

    // Q fragments (B operand of S^T): lane (g = l16, kg) holds dims
    // [32kk + 8kg, +8) of query head j*G + g; heads >= G are zero.
    bf16x8_t qh[T::KK], ql[T::KK];
    {
      const long long qrow = (static_cast<long long>(r) * d.Hq() + static_cast<long long>(j) * G + l16) * D;
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
        const int c = 32 * kk + 8 * kg;
        if (QF32) {
          float x[8];
          if (l16 < G) {
            const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(qv) + qrow + c);
            const float4 x0 = src[0], x1 = src[1];
            x[0] = x0.x; x[1] = x0.y; x[2] = x0.z; x[3] = x0.w;
            x[4] = x1.x; x[5] = x1.y; x[6] = x1.z; x[7] = x1.w;
          } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) x[i] = 0.f;
          }
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const __bf16 h = static_cast<__bf16>(x[i]);
            qh[kk][i] = h;
            ql[kk][i] = static_cast<__bf16>(x[i] - static_cast<float>(h));
          }
        } else {
          u32x4_t raw = {0u, 0u, 0u, 0u};
          if (l16 < G) raw = *reinterpret_cast<const u32x4_t*>(static_cast<const uint16_t*>(qv) + qrow + c);
          qh[kk] = __builtin_bit_cast(bf16x8_t, raw);
        }
      }
    }

    float m_run = -INFINITY;
    float l_run = 0.f;
    f32x4_t o[T::NN];
#pragma unroll
    for (int nn = 0; nn < T::NN; ++nn) o[nn] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // This wave takes list indices my0, my0 + nw, ...; metadata for up to 64
    // of them is fetched lane-parallel (list entry, then block-table entry).
    const int my0 = li0 + wave;
    const int cnt = my0 < li1 ? (li1 - my0 + nw - 1) / nw : 0;

    auto issue = [&](PageRegs<T::KK>& pr, int k, int m_phys, int m_n, int cc) {
      pr.base = -1;
      pr.n = 0;
      if (k >= cc) return;
      const int phys = __builtin_amdgcn_readlane(m_phys, k);
      const int n = __builtin_amdgcn_readlane(m_n, k);
      if (phys < 0) return;
      const long long base = static_cast<long long>(phys) * d.H * head_stride + head_base;
      pr.base = base;
      pr.n = n;
      const uint16_t* kp = k_pool + base + static_cast<long long>(l16) * D + 8 * kg;
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk)
        pr.k[kk] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(kp + 32 * kk));
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const uint16_t* vp = v_pool + base + static_cast<long long>(4 * kg + s4) * D + T::VB * l16;
        if (D == 128) {
          pr.v[s4] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(vp));
        } else {
          const u32x2_t x = *reinterpret_cast<const u32x2_t*>(vp);
          pr.v[s4] = u32x4_t{x[0], x[1], 0u, 0u};
        }
      }
    };

    auto compute = [&](const PageRegs<T::KK>& pr) {
      if (pr.base < 0) return;
      const int n_cur = pr.n;
      f32x4_t sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < T::KK; ++kk) {
        const bf16x8_t kf = __builtin_bit_cast(bf16x8_t, pr.k[kk]);
        sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qh[kk], sacc, 0, 0, 0);
        if (QF32) sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, ql[kk], sacc, 0, 0, 0);
      }
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) x[i] = (4 * kg + i < n_cur) ? sacc[i] * scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
      {   // the page's maximum for head g over the four token groups
        float lo, hi;
        lane_pair16(mx, lo, hi);
        mx = fmaxf(lo, hi);
        lane_pair32(mx, lo, hi);
        mx = fmaxf(lo, hi);
      }
      const float m_new = fmaxf(m_run, mx);
      const float alpha = exp2f(m_run - m_new);
      // P in fp32, fed to the matrix cores as bf16 hi + lo parts (P - hi is
      // exact in fp32), so the weights keep ~16 significant bits and the
      // result does not depend on how the pages were split.
      bf16x4_t ph, plo;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = exp2f(x[i] - m_new);
        const __bf16 h = static_cast<__bf16>(p);
        ph[i] = h;
        plo[i] = static_cast<__bf16>(p - static_cast<float>(h));
        psum += p;
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * kg + i, 64);
#pragma unroll
      for (int nn = 0; nn < T::NN; ++nn) {
#pragma unroll
        for (int i = 0; i < 4; ++i) o[nn][i] *= ar[i];
      }
      // V operand words: token rows 4kg + s4, zero beyond the page's tokens
      uint32_t vw[4][T::VB / 2];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const bool ok = 4 * kg + s4 < n_cur;
#pragma unroll
        for (int wi = 0; wi < T::VB / 2; ++wi) vw[s4][wi] = ok ? pr.v[s4][wi] : 0u;
      }
#pragma unroll
      for (int nn = 0; nn < T::NN; ++nn) {
        const int wi = nn >> 1;
        const uint32_t sel = (nn & 1) ? 0x07060302u : 0x05040100u;
        u32x2_t bw;
        bw[0] = __builtin_amdgcn_perm(vw[1][wi], vw[0][wi], sel);
        bw[1] = __builtin_amdgcn_perm(vw[3][wi], vw[2][wi], sel);
        const bf16x4_t vf = __builtin_bit_cast(bf16x4_t, bw);
        o[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(ph, vf, o[nn], 0, 0, 0);
        o[nn] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(plo, vf, o[nn], 0, 0, 0);
      }
    };

    for (int c0 = 0; c0 < cnt; c0 += 64) {
      const int cc = min(64, cnt - c0);
      int m_phys = -1, m_n = 0;
      if (lane < cc) {
        const int p = plist[my0 + nw * (c0 + lane)];
        if (p < 0 || p >= P) {
          set_status(status, MOIRA_ST_BAD_LIST);
        } else {
          const int ph = trow[p];
          if (ph < 0 || ph >= d.num_phys) set_status(status, MOIRA_ST_BAD_PAGE);
          else {
            m_phys = ph;
            m_n = (p == P - 1) ? nlast : d.ps;
          }
        }
      }
      // NB page buffers in rotation: NB - 1 pages in flight while one computes
      PageRegs<T::KK> pr[T::NB];
#pragma unroll
      for (int q = 0; q < T::NB; ++q) issue(pr[q], q, m_phys, m_n, cc);
      for (int k = 0; k < cc; k += T::NB) {
#pragma unroll
        for (int q = 0; q < T::NB; ++q) {
          compute(pr[q]);
          issue(pr[q], k + T::NB + q, m_phys, m_n, cc);
        }
      }
    }

    // merge the waves' states of this piece and write one partial
    float l_tot, l_hi;
    lane_pair16(l_run, l_tot, l_hi);
    l_tot += l_hi;
    lane_pair32(l_tot, l_tot, l_hi);
    l_tot += l_hi;
    if (lane < G) {
      wm[wave * kMaxGroup + lane] = m_run;
      wl[wave * kMaxGroup + lane] = l_tot;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int g = 4 * kg + i;
      if (g < G) {
#pragma unroll
        for (int nn = 0; nn < T::NN; ++nn)
          wo[(wave * G + g) * D + (D / 16) * l16 + nn] = o[nn][i];
      }
    }
    __syncthreads();
    const long long slot = static_cast<long long>(w) + static_cast<long long>(wk.slot_seg) * s;
    for (int idx = tid; idx < G * D; idx += blockDim.x) {
      const int g = idx / D;
      const int c = idx - g * D;
      float M = -INFINITY;
#pragma unroll
      for (int v = 0; v < nw; ++v) M = fmaxf(M, wm[v * kMaxGroup + g]);
      float acc = 0.f, lsum = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int v = 0; v < nw; ++v) {
          const float mv = wm[v * kMaxGroup + g];
          const float f = mv == -INFINITY ? 0.f : exp2f(mv - M);
          acc += f * wo[(v * G + g) * D + c];
          lsum += f * wl[v * kMaxGroup + g];
        }
      }
      if constexpr (COMB) {   // written through: another workgroup merges it
        __hip_atomic_store(partial_o + (slot * G + g) * D + c, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (c == 0) {
          __hip_atomic_store(partial_ml + (slot * G + g) * 2, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          __hip_atomic_store(partial_ml + (slot * G + g) * 2 + 1, lsum, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        partial_o[(slot * G + g) * D + c] = acc;
        if (c == 0) {
          partial_ml[(slot * G + g) * 2] = M;
          partial_ml[(slot * G + g) * 2 + 1] = lsum;
        }
      }
    }
    __syncthreads();
    a = hi;
  }
  if constexpr (COMB) {
    // every piece of this workgroup is stored, complete at the coherence
    // point, before it counts itself in on each segment it took part in; the
    // last to arrive at a segment merges it (after the attention loop, so
    // the merge does not add to the loop's registers)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    const int q = aligned_quota(off[S], N, S);
    for (int t = wk.s; t < S && off[t] < b; ++t) {
      if (off[t + 1] <= wk.a || off[t + 1] == off[t]) continue;   // no piece of t here
      long long slot0;
      int np;
      piece_span(off, wb, q, off[S], N, t, slot0, np);
      if (tid == 0) {
        const unsigned int before =
            __hip_atomic_fetch_add(counters + t, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_arriver = before + 1 == static_cast<unsigned int>(np);
      }
      __syncthreads();
      if (last_arriver) {
        if (tid == 0) counters[t] = 0u;   // read again only by the next call
        merge_segment<64 * NW>(d, t, slot0, np, partial_o, partial_ml,
                               static_cast<long long>(N) + S - 1, out, wo);
      }
      __syncthreads();
    }
  }
}

// ---- fp32 K/V kernel (vector ALU) -----------------------------------------
// Same self-planning split; one workgroup walks each piece's pages in order.
constexpr int kValuBatch = 256;   // page metadata fetched per round (one per thread)
template <typename QT>
__global__ __launch_bounds__(256) void attn_valu_kernel(
    Dims d, const QT* __restrict__ q, const float* __restrict__ k_pool,
    const float* __restrict__ v_pool, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_lists,
    const int32_t* __restrict__ list_lens, float scale_log2, int N,
    float* __restrict__ partial_o, float* __restrict__ partial_ml, int32_t* status) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int S = d.S();
  const int G = d.G;
  const int D = d.D;
  int* off = reinterpret_cast<int*>(smem);
  int* wb = off + (S + 1);                                      // aligned split only
  int* scan_tmp = wb + (aligned_possible(N, S) ? S + 1 : 0);
  float* qs = reinterpret_cast<float*>(scan_tmp + 8);   // [G][D]
  float* lg = qs + kMaxGroup * 128;                     // [G][16]
  float* st_m = lg + kMaxGroup * 16;                    // [G]
  float* st_l = st_m + kMaxGroup;
  float* st_a = st_l + kMaxGroup;
  float* ks = st_a + kMaxGroup;                         // [16][D] K rows of a page
  float* vs = ks + 16 * 128;                            // [16][D] V rows of a page
  __shared__ long long pbase[kValuBatch];
  __shared__ int pn[kValuBatch];

  const int tid = threadIdx.x;
  const int w = blockIdx.x;
  WgWork wk;
  if (!plan_workgroup(list_lens, d, N, w, off, wb, scan_tmp, status, wk)) return;
  int a = wk.a;
  const int b = wk.b;
  int s = wk.s;
  const int npairs = G * D;

  while (a < b) {
    while (off[s + 1] <= a) ++s;
    const int hi = min(b, off[s + 1]);
    const int li0 = a - off[s];
    const int li1 = hi - off[s];
    const int r = s / d.H;
    const int j = s - r * d.H;
    int L = seq_lens[r];
    if (L < 1 || L > d.max_pages * d.ps) L = 0;
    const int P = (L + d.ps - 1) / d.ps;
    const int nlast = L - (P - 1) * d.ps;
    const long long qrow = (static_cast<long long>(r) * d.Hq() + static_cast<long long>(j) * G) * D;
    for (int i = tid; i < npairs; i += blockDim.x) {
      if (sizeof(QT) == 2) qs[i] = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(q)[qrow + i]);
      else qs[i] = reinterpret_cast<const float*>(q)[qrow + i];
    }
    if (tid < G) {
      st_m[tid] = -INFINITY;
      st_l[tid] = 0.f;
    }
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
    __syncthreads();
    const int32_t* plist = page_lists + static_cast<long long>(s) * d.max_pages;
    // the pages' list entries and table entries are fetched kValuBatch at a
    // time, one per thread, instead of one dependent pair of loads per page
    for (int c0 = li0; c0 < li1; c0 += kValuBatch) {
      const int cn = min(kValuBatch, li1 - c0);
      if (tid < cn) {
        long long base = -1;
        int n = 0;
        const int p = plist[c0 + tid];
        if (p < 0 || p >= P) {
          set_status(status, MOIRA_ST_BAD_LIST);
        } else {
          const long long phys = block_table[static_cast<long long>(r) * d.max_pages + p];
          if (phys < 0 || phys >= d.num_phys) set_status(status, MOIRA_ST_BAD_PAGE);
          else {
            base = (phys * d.H + j) * static_cast<long long>(d.ps) * D;
            n = (p == P - 1) ? nlast : d.ps;
          }
        }
        pbase[tid] = base;
        pn[tid] = n;
      }
      __syncthreads();
      for (int k = 0; k < cn; ++k) {
        const long long base = pbase[k];
        const int n = pn[k];
        if (base >= 0) {
          // the page's K and V rows into LDS with coalesced loads (rows
          // past its tokens are never read)
          for (int i = tid; i < n * D; i += blockDim.x) {
            ks[i] = k_pool[base + i];
            vs[i] = v_pool[base + i];
          }
          __syncthreads();
          if (tid < G * 16) {
            const int g = tid >> 4;
            const int t = tid & 15;
            float x = -INFINITY;
            if (t < n) {
              const float* kr = ks + t * D;
              const float* qg = qs + g * D;
              float dot = 0.f;
              for (int c = 0; c < D; ++c) dot = fmaf(qg[c], kr[c], dot);
              x = dot * scale_log2;
            }
            lg[g * 16 + t] = x;
          }
          __syncthreads();
          if (tid < G) {
            float mx = -INFINITY;
            for (int t = 0; t < 16; ++t) mx = fmaxf(mx, lg[tid * 16 + t]);
            const float m_old = st_m[tid];
            const float m_new = fmaxf(m_old, mx);
            const float alpha = exp2f(m_old - m_new);
            float ps = 0.f;
            for (int t = 0; t < 16; ++t) {
              const float p = exp2f(lg[tid * 16 + t] - m_new);
              lg[tid * 16 + t] = p;
              ps += p;
            }
            st_l[tid] = st_l[tid] * alpha + ps;
            st_m[tid] = m_new;
            st_a[tid] = alpha;
          }
          __syncthreads();
#pragma unroll
          for (int k2 = 0; k2 < 8; ++k2) {
            const int idx = tid + k2 * 256;
            if (idx < npairs) {
              const int g = idx / D;
              const int c = idx - g * D;
              float v = acc[k2] * st_a[g];
              for (int t = 0; t < n; ++t) v = fmaf(lg[g * 16 + t], vs[t * D + c], v);
              acc[k2] = v;
            }
          }
        }
        __syncthreads();
      }
    }
    const long long slot = static_cast<long long>(w) + static_cast<long long>(wk.slot_seg) * s;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int idx = tid + k * 256;
      if (idx < npairs) {
        const int g = idx / D;
        partial_o[slot * npairs + idx] = acc[k];
        if (idx - g * D == 0) {
          partial_ml[(slot * G + g) * 2] = st_m[g];
          partial_ml[(slot * G + g) * 2 + 1] = st_l[g];
        }
      }
    }
    __syncthreads();
    a = hi;
  }
}

// ---- combine ---------------------------------------------------------------
// The pieces of segment s are the attention workgroup ranges that overlap its
// list (with effective_wgs every such range is non-empty); piece i of s holds
// the partial state in slot slot0 + i, where slot0 is w0 + s for the even
// split (w0: the first such workgroup) and the segment's first workgroup for
// the aligned split. Each thread merges the pieces it loads
// into a local state (max m, rescaled l, rescaled o); the local states are then
// merged with the same algebra.
constexpr int kPieceBatch = 8;

// Merge pieces i0, i0 + stride, ... (< np) of one (segment, head) column quad
// into st, kPieceBatch pieces per round of loads. ml points at piece 0's
// (m, l) pair (piece i at ml[2 i G]), po at piece 0's float4 (piece i at
// po[i G D]).
__device__ __forceinline__ void merge_pieces(LseState& st, const float* ml, const float* po, int np,
                                             int i0, int stride, int G, int D) {
  for (; i0 < np; i0 += stride * kPieceBatch) {
    float2 mlv[kPieceBatch];
    float4 o[kPieceBatch];
#pragma unroll
    for (int k = 0; k < kPieceBatch; ++k) {
      const int i = i0 + k * stride;
      mlv[k] = make_float2(-INFINITY, 0.f);
      o[k] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (i < np) {
        mlv[k] = *reinterpret_cast<const float2*>(ml + 2LL * i * G);
        o[k] = *reinterpret_cast<const float4*>(po + static_cast<long long>(i) * G * D);
      }
    }
    float M = st.m;
#pragma unroll
    for (int k = 0; k < kPieceBatch; ++k) M = fmaxf(M, mlv[k].x);
    if (M != -INFINITY) {
      const float f0 = st.m == -INFINITY ? 0.f : exp2f(st.m - M);
      st.l *= f0;
      st.o = make_float4(st.o.x * f0, st.o.y * f0, st.o.z * f0, st.o.w * f0);
#pragma unroll
      for (int k = 0; k < kPieceBatch; ++k) {
        const float f = mlv[k].x == -INFINITY ? 0.f : exp2f(mlv[k].x - M);
        st.l += f * mlv[k].y;
        st.o.x += f * o[k].x;
        st.o.y += f * o[k].y;
        st.o.z += f * o[k].z;
        st.o.w += f * o[k].w;
      }
      st.m = M;
    }
  }
}

// Pieces of segment s, computed by a whole workgroup of NT threads from
// list_lens exactly as the attention workgroups planned them: the list
// offset of s and the total W come from one block reduction; for the aligned
// split a second reduction counts the workgroups of the segments before s.
// Returns the clamped list length; slot0 (the slot of piece 0; piece i is at
// slot0 + i) and np are set when it is positive.
template <int NT>
__device__ int segment_pieces(const Dims& d, const int32_t* __restrict__ list_lens, int N, int s,
                              long long* red, long long& slot0, int& np) {
  constexpr int NW = NT / 64;
  const int S = d.S();
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  auto clamp_len = [&](int v) { return v < 0 ? 0 : (v > d.max_pages ? d.max_pages : v); };
  if (S <= 64) {
    // one wave holds every list length: each wave derives the pieces by
    // itself with wave reductions, and no block barrier is needed
    const int v = lane < S ? clamp_len(list_lens[lane]) : 0;
    const int Wt = wave_sum_i32(v);
    const int off = wave_sum_i32(lane < s ? v : 0);
    const int len = __shfl(v, s, 64);
    const int q = aligned_quota(Wt, N, S);
    if (q > 0) {
      slot0 = wave_sum_i32(lane < s ? (v + q - 1) / q : 0);
      np = (len + q - 1) / q;
    } else if (len > 0) {
      const int Ne = effective_wgs(Wt, N);
      auto wg_of = [&](long long x) -> long long {
        long long w = ((x + 1) * Ne - 1) / Wt;
        return w < Ne - 1 ? w : Ne - 1;
      };
      const long long w0 = wg_of(off);
      slot0 = w0 + s;
      np = static_cast<int>(wg_of(static_cast<long long>(off) + len - 1) - w0 + 1);
    }
    return len;
  }
  long long before = 0, all = 0;
  int first = 0;   // this thread's first length, kept for the second reduction
  for (int i = tid; i < S; i += NT) {
    const int v = clamp_len(list_lens[i]);
    if (i == tid) first = v;
    all += v;
    if (i < s) before += v;
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    before += __shfl_xor(before, m, 64);
    all += __shfl_xor(all, m, 64);
  }
  if (lane == 0) {
    red[wave] = before;
    red[NW + wave] = all;
  }
  __syncthreads();
  long long off = 0, W = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    off += red[w];
    W += red[NW + w];
  }
  const int len = clamp_len(list_lens[s]);
  const int q = aligned_quota(static_cast<int>(W), N, S);
  if (q > 0) {
    long long wbefore = 0;
    for (int i = tid; i < s; i += NT)
      wbefore += ((i == tid ? first : clamp_len(list_lens[i])) + q - 1) / q;
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) wbefore += __shfl_xor(wbefore, m, 64);
    if (lane == 0) red[2 * NW + wave] = wbefore;
    __syncthreads();
    long long wb = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) wb += red[2 * NW + w];
    slot0 = wb;
    np = (len + q - 1) / q;
    return len;
  }
  if (len > 0) {
    // workgroup whose range holds global page x: largest w with floor(wW/Ne) <= x
    const int Ne = effective_wgs(static_cast<int>(W), N);
    auto wg_of = [&](long long x) -> long long {
      long long v = ((x + 1) * Ne - 1) / W;
      return v < Ne - 1 ? v : Ne - 1;
    };
    const long long w0 = wg_of(off);
    slot0 = w0 + s;
    np = static_cast<int>(wg_of(off + len - 1) - w0 + 1);
  }
  return len;
}

// Few segments with many pieces each (a long context split over many
// workgroups): grid (S, G, D / kCombineCols), one workgroup per (segment,
// query head, 32-column slice). Thread (pg, cq) owns column quad cq of the
// slice and the pieces pg, pg + 32, ..., so one round of loads serves up to
// 256 pieces; the 32 piece groups are merged with three exchanges inside
// each wave and one pass over the four waves in LDS.
constexpr int kCombineThreads = 256;
constexpr int kCombineCols = 32;                          // output columns per workgroup
constexpr int kCombineQuads = kCombineCols / 4;           // float4 column quads
constexpr int kCombineGroups = kCombineThreads / kCombineQuads;  // piece groups (32)

__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    Dims d, const int32_t* __restrict__ list_lens, int N, const float* __restrict__ partial_o,
    const float* __restrict__ partial_ml, float* __restrict__ out) {
  // the partial-state pointers end in the argument segment's second 64-byte
  // line: asked for at entry, both lines are fetched together, not the
  // second one a round trip later, between the list lengths and the loads
  // of the partial states
  asm volatile("" ::"s"(d.B), "s"(out));
  constexpr int NW = kCombineThreads / 64;
  __shared__ long long red[3 * NW];
  __shared__ LseState red_s[NW][kCombineQuads];
  const int s = blockIdx.x;
  const int g = blockIdx.y;
  const int col0 = blockIdx.z * kCombineCols;
  const int G = d.G;
  const int D = d.D;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cq = tid % kCombineQuads;
  const int pg = tid / kCombineQuads;

  long long slot0 = 0;
  int np = 0;
  const int len = segment_pieces<kCombineThreads>(d, list_lens, N, s, red, slot0, np);
  const int r = s / d.H;
  const int j = s - r * d.H;
  float* dst = out + ((static_cast<long long>(r) * d.Hq() + static_cast<long long>(j) * G + g) * D) + col0;
  if (len == 0) {
    if (tid < kCombineCols) dst[tid] = 0.f;
    return;
  }
  const float* ml = partial_ml + (slot0 * G + g) * 2;
  const float* po = partial_o + (slot0 * G + g) * static_cast<long long>(D) + col0 + 4 * cq;

  LseState st;
  st.m = -INFINITY;
  st.l = 0.f;
  st.o = make_float4(0.f, 0.f, 0.f, 0.f);
  merge_pieces(st, ml, po, np, pg, kCombineGroups, G, D);
  // merge the piece groups: lanes cq, cq + 8, ... of a wave, then the waves
  // (the merge is symmetric, so merging the lower lane's state into the
  // upper one's gives both lanes the same result)
  static_assert(kCombineQuads == 8, "exchanges at lane distances 8, 16, 32");
  st = lse_merge(st, lse_xor8(st));
  {
    LseState lo, hi;
    lse_pair<16>(st, lo, hi);
    st = lse_merge(lo, hi);
    lse_pair<32>(st, lo, hi);
    st = lse_merge(lo, hi);
  }
  if (lane < kCombineQuads) red_s[wave][lane] = st;
  __syncthreads();
  if (tid < kCombineQuads) {
    LseState t = red_s[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) t = lse_merge(t, red_s[w][tid]);
    const float inv = t.l > 0.f ? 1.f / t.l : 0.f;
    *reinterpret_cast<float4*>(dst + 4 * tid) = make_float4(t.o.x * inv, t.o.y * inv, t.o.z * inv, t.o.w * inv);
  }
}

// Many segments with few pieces each (a batch of requests): grid S, one
// workgroup of 256 threads per segment. Lane (u8, cq) of wave w owns column
// quad cq of the 32-column units u = 8 w + u8, 8 w + u8 + 32, ... of the
// segment (a unit is one query head's 32-column slice) and walks all pieces
// of its unit itself, 8 per round of loads.
constexpr int kCombineSegThreads = 256;

__global__ __launch_bounds__(kCombineSegThreads) void combine_seg_kernel(
    Dims d, const int32_t* __restrict__ list_lens, int N, const float* __restrict__ partial_o,
    const float* __restrict__ partial_ml, float* __restrict__ out) {
  // both 64-byte lines of the argument segment fetched together at entry
  asm volatile("" ::"s"(d.B), "s"(out));
  constexpr int NW = kCombineSegThreads / 64;
  __shared__ long long red[3 * NW];
  const int s = blockIdx.x;
  const int G = d.G;
  const int D = d.D;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int cq = lane % kCombineQuads;
  const int u8 = lane / kCombineQuads;
  const int slices = D / kCombineCols;
  const int U = G * slices;

  long long slot0 = 0;
  int np = 0;
  const int len = segment_pieces<kCombineSegThreads>(d, list_lens, N, s, red, slot0, np);
  const int r = s / d.H;
  const int j = s - r * d.H;
  float* seg_out = out + (static_cast<long long>(r) * d.Hq() + static_cast<long long>(j) * G) * D;
  for (int u = wave * 8 + u8; u < U; u += NW * 8) {
    const int g = u / slices;
    const int col = (u - g * slices) * kCombineCols + 4 * cq;
    float* dst = seg_out + static_cast<long long>(g) * D + col;
    if (len == 0) {
      *reinterpret_cast<float4*>(dst) = make_float4(0.f, 0.f, 0.f, 0.f);
      continue;
    }
    const float* ml = partial_ml + (slot0 * G + g) * 2;
    const float* po = partial_o + (slot0 * G + g) * static_cast<long long>(D) + col;
    LseState st;
    st.m = -INFINITY;
    st.l = 0.f;
    st.o = make_float4(0.f, 0.f, 0.f, 0.f);
    merge_pieces(st, ml, po, np, 0, 1, G, D);
    const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
    *reinterpret_cast<float4*>(dst) = make_float4(st.o.x * inv, st.o.y * inv, st.o.z * inv, st.o.w * inv);
  }
}

// ---- host launchers ----------------------------------------------------------
hipError_t launch_combine(const Dims& d, const int32_t* list_lens, int N, const float* partial_o,
                          const float* partial_ml, float* out, hipStream_t st);

size_t attn_smem_bytes(const Dims& d, int N, bool mfma, bool comb = false) {
  const size_t S1 = static_cast<size_t>(d.S()) + 1;
  size_t base = (S1 + (aligned_possible(N, d.S()) ? S1 : 0) + 8) * sizeof(int);
  base = (base + 15) & ~static_cast<size_t>(15);
  if (mfma) {
    // the waves' partial states; the in-kernel merge reuses them as 6 floats per thread
    size_t wo = static_cast<size_t>(attn_waves(d)) * d.G * d.D;
    if (comb && wo < static_cast<size_t>(64 * attn_waves(d)) * 6) wo = static_cast<size_t>(64 * attn_waves(d)) * 6;
    return base + (2 * kAttnMaxWaves * kMaxGroup + wo) * sizeof(float);
  }
  return base + (kMaxGroup * 128 + kMaxGroup * 16 + 3 * kMaxGroup + 2 * 16 * 128) * sizeof(float);
}

hipError_t launch_attn(const Dims& d, int kv_dtype, int q_dtype, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* page_lists, const int32_t* list_lens, float scale, int N,
                       float* partial_o, float* partial_ml, int32_t* status, hipStream_t st) {
  const float sl2 = scale * kLog2e;
  if (kv_dtype == MOIRA_BF16) {
    const size_t sm = attn_smem_bytes(d, N, true);
    const uint16_t* kp = static_cast<const uint16_t*>(k_pool);
    const uint16_t* vp = static_cast<const uint16_t*>(v_pool);
#define MOIRA_ATTN(DD, QF)                                                                       \
  do {                                                                                         \
    if (attn_waves(d) == 8)                                                                    \
      attn_mfma_kernel<DD, QF, 8><<<N, 512, sm, st>>>(d, q, kp, vp, block_table, seq_lens,      \
                                                      page_lists, list_lens, sl2, N, partial_o,  \
                                                      partial_ml, status, nullptr, nullptr);     \
    else                                                                                       \
      attn_mfma_kernel<DD, QF, 4><<<N, 256, sm, st>>>(d, q, kp, vp, block_table, seq_lens,      \
                                                      page_lists, list_lens, sl2, N, partial_o,  \
                                                      partial_ml, status, nullptr, nullptr);     \
  } while (0)
    if (d.D == 128) {
      if (q_dtype == MOIRA_BF16) MOIRA_ATTN(128, false);
      else MOIRA_ATTN(128, true);
    } else {
      if (q_dtype == MOIRA_BF16) MOIRA_ATTN(64, false);
      else MOIRA_ATTN(64, true);
    }
#undef MOIRA_ATTN
  } else {
    const size_t sm = attn_smem_bytes(d, N, false);
    const float* kp = static_cast<const float*>(k_pool);
    const float* vp = static_cast<const float*>(v_pool);
    if (q_dtype == MOIRA_BF16)
      attn_valu_kernel<uint16_t><<<N, 256, sm, st>>>(d, static_cast<const uint16_t*>(q), kp, vp, block_table,
                                                     seq_lens, page_lists, list_lens, sl2, N, partial_o,
                                                     partial_ml, status);
    else
      attn_valu_kernel<float><<<N, 256, sm, st>>>(d, static_cast<const float*>(q), kp, vp, block_table,
                                                  seq_lens, page_lists, list_lens, sl2, N, partial_o,
                                                  partial_ml, status);
  }
  return hipGetLastError();
}

// Attention and the merge of the partial states in one launch for bf16 K/V
// when a workgroup is 8 waves (G D <= 1024); otherwise the two kernels.
hipError_t launch_attn_combine(const Dims& d, int kv_dtype, int q_dtype, const void* q,
                               const void* k_pool, const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* page_lists,
                               const int32_t* list_lens, float scale, int N, float* partial_o,
                               float* partial_ml, unsigned int* counters, float* out,
                               int32_t* status, hipStream_t st) {
  if (kv_dtype != MOIRA_BF16 || attn_waves(d) != 8) {
    hipError_t e = launch_attn(d, kv_dtype, q_dtype, q, k_pool, v_pool, block_table, seq_lens,
                               page_lists, list_lens, scale, N, partial_o, partial_ml, status, st);
    if (e != hipSuccess) return e;
    return launch_combine(d, list_lens, N, partial_o, partial_ml, out, st);
  }
  const float sl2 = scale * kLog2e;
  const size_t sm = attn_smem_bytes(d, N, true, true);
  const uint16_t* kp = static_cast<const uint16_t*>(k_pool);
  const uint16_t* vp = static_cast<const uint16_t*>(v_pool);
#define MOIRA_ATTN_C(DD, QF)                                                                      \
  attn_mfma_kernel<DD, QF, 8, true><<<N, 512, sm, st>>>(d, q, kp, vp, block_table, seq_lens,    \
                                                        page_lists, list_lens, sl2, N, partial_o, \
                                                        partial_ml, status, counters, out)
  if (d.D == 128) {
    if (q_dtype == MOIRA_BF16) MOIRA_ATTN_C(128, false);
    else MOIRA_ATTN_C(128, true);
  } else {
    if (q_dtype == MOIRA_BF16) MOIRA_ATTN_C(64, false);
    else MOIRA_ATTN_C(64, true);
  }
#undef MOIRA_ATTN_C
  return hipGetLastError();
}

hipError_t launch_combine(const Dims& d, const int32_t* list_lens, int N, const float* partial_o,
                          const float* partial_ml, float* out, hipStream_t st) {
  // pieces per segment average (N + S) / S: with more than 8 of them the
  // wide kernel spreads each segment over many threads; otherwise one
  // workgroup per segment walks its few pieces per lane
  if (N > 8 * d.S())
    combine_kernel<<<dim3(d.S(), d.G, d.D / kCombineCols), kCombineThreads, 0, st>>>(
        d, list_lens, N, partial_o, partial_ml, out);
  else
    combine_seg_kernel<<<d.S(), kCombineSegThreads, 0, st>>>(d, list_lens, N, partial_o, partial_ml, out);
  return hipGetLastError();
}

}  // namespace moira
