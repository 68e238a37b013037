// KV-cache maintenance kernels: advance the per-request lengths, append the
// step's token into its page, and build page summaries (mean key per page).
//
// Page summary (mean-vector block metadata, "Faster than Flash", section 2,
// dynamic sparse attention): kbar_p = (1/n_p) sum_t k_t over the page's n_p
// tokens, summed in fp64 in token order, divided in fp64, rounded once to
// fp32 (and, for bf16 summaries, that value rounded once to bf16). For bf16 or
// fp32 keys the fp64 sum of at most 16 tokens is exact for any ordinary range
// of values, and the same roundings follow, so appending and rebuilding give
// the same bits.
#include "moira_common.h"

namespace moira {

__global__ void advance_kernel(Dims d, int32_t* seq_lens, int32_t* status) {
  const int cap = d.max_pages * d.ps;
  for (int r = threadIdx.x + blockIdx.x * blockDim.x; r < d.B; r += blockDim.x * gridDim.x) {
    int L = seq_lens[r];
    if (L < 0) {
      set_status(status, MOIRA_ST_BAD_LEN);
    } else if (L >= cap) {
      set_status(status, MOIRA_ST_CAPACITY);
    } else {
      seq_lens[r] = L + 1;
    }
  }
}

// grid (B, H), 256 threads: one workgroup per (request, KV head). The page's
// earlier tokens are loaded in parallel into LDS, then one thread per
// dimension sums them in token order, followed by the new token.
template <typename T>
__global__ __launch_bounds__(256) void append_kernel(Dims d, const T* __restrict__ k_new,
                                                     const T* __restrict__ v_new,
                                                     T* __restrict__ k_pool,
                                                     T* __restrict__ v_pool,
                                                     void* __restrict__ summaries,
                                                     const int32_t* __restrict__ block_table,
                                                     const int32_t* __restrict__ seq_lens,
                                                     int32_t* status) {
  __shared__ float tile[kPageSize * 128];
  const int r = blockIdx.x;
  const int j = blockIdx.y;
  const int L = checked_len(seq_lens, r, d, status, threadIdx.x == 0 && j == 0);
  if (L == 0) {  // nothing was advanced for this request: no slot to write
    if (threadIdx.x == 0 && j == 0) set_status(status, MOIRA_ST_BAD_LEN);
    return;
  }
  const int pos = L - 1;
  const int lp = pos / d.ps;
  const int slot = pos - lp * d.ps;
  const long long phys = block_table[static_cast<long long>(r) * d.max_pages + lp];
  if (phys < 0 || phys >= d.num_phys) {
    if (threadIdx.x == 0) set_status(status, MOIRA_ST_BAD_PAGE);
    return;
  }
  const int D = d.D;
  const long long page_base = (phys * d.H + j) * d.ps * static_cast<long long>(D);
  const long long src = (static_cast<long long>(r) * d.H + j) * D;
  const int nprev = slot * D;
#pragma unroll 4
  for (int idx = threadIdx.x; idx < nprev; idx += blockDim.x)
    tile[idx] = KvElem<T>::to_f32(k_pool[page_base + idx]);
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    const T kv = k_new[src + c];
    k_pool[page_base + static_cast<long long>(slot) * D + c] = kv;
    v_pool[page_base + static_cast<long long>(slot) * D + c] = v_new[src + c];
    double acc = 0.0;
    for (int t = 0; t < slot; ++t) acc += static_cast<double>(tile[t * D + c]);
    acc += static_cast<double>(KvElem<T>::to_f32(kv));
    store_summary(summaries, (phys * d.H + j) * D + c, acc / static_cast<double>(slot + 1), d.sbf,
                  d.sf8);
  }
}

// DPL consecutive elements of one token row as raw bits (one load;
// non-temporal: every K row is read once per build), widened to fp32 when
// summed.
template <typename T, int DPL> struct RowRaw;
template <> struct RowRaw<uint16_t, 2> {
  using R = uint32_t;
  static __device__ __forceinline__ R load(const uint16_t* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
  static __device__ __forceinline__ float get(R u, int e) {
    return __uint_as_float(e == 0 ? u << 16 : u & 0xffff0000u);
  }
};
template <> struct RowRaw<uint16_t, 1> {
  using R = uint32_t;
  static __device__ __forceinline__ R load(const uint16_t* p) {
    return static_cast<uint32_t>(__builtin_nontemporal_load(p));
  }
  static __device__ __forceinline__ float get(R u, int) { return __uint_as_float(u << 16); }
};
template <> struct RowRaw<float, 2> {
  using R = u32x2_t;
  static __device__ __forceinline__ R load(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
  }
  static __device__ __forceinline__ float get(R u, int e) { return __uint_as_float(u[e]); }
};
template <> struct RowRaw<float, 1> {
  using R = uint32_t;
  static __device__ __forceinline__ R load(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
  }
  static __device__ __forceinline__ float get(R u, int) { return __uint_as_float(u); }
};

// The DPL summary elements of a lane, stored with one store.
template <int DPL>
__device__ __forceinline__ void store_summary_run(void* summaries, long long idx, const double (&mean)[DPL],
                                                  int sbf, int sf8) {
  if constexpr (DPL == 2) {
    const float f0 = static_cast<float>(mean[0]), f1 = static_cast<float>(mean[1]);
    if (sbf) {
      *reinterpret_cast<uint32_t*>(static_cast<uint16_t*>(summaries) + idx) =
          static_cast<uint32_t>(f32_to_bf16_rne(f0)) | (static_cast<uint32_t>(f32_to_bf16_rne(f1)) << 16);
    } else if (sf8) {
      *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(summaries) + idx) =
          static_cast<uint16_t>(f32_to_e4m3_rne(f0) | (f32_to_e4m3_rne(f1) << 8));
    } else {
      *reinterpret_cast<float2*>(static_cast<float*>(summaries) + idx) = make_float2(f0, f1);
    }
  } else {
    store_summary(summaries, idx, mean[0], sbf, sf8);
  }
}

// Items (page p, KV head j), numbered p * H + j. A wave takes ipw <= 64
// consecutive items (whole pages' heads, contiguous in the pool), or one item
// (the tail page of one head) when only tail pages are rebuilt. Lane i first
// loads the table entry of the wave's item i, alongside the request length;
// then the wave streams its items with the next item's rows in flight while
// it sums the current one. Lane l owns dimensions [l * DPL, (l + 1) * DPL) and
// sums them in fp64 in token order, so the result is bitwise the append
// kernel's. Every load is in bounds: a page past the request or with a bad
// table entry reads page 0 and stores nothing (a bad entry is reported).
template <typename T, int DPL>
__global__ __launch_bounds__(256) void summaries_kernel(Dims d, const T* __restrict__ k_pool,
                                                        const int32_t* __restrict__ block_table,
                                                        const int32_t* __restrict__ seq_lens,
                                                        void* __restrict__ summaries,
                                                        int tail_only, int ipw, int32_t* status) {
  using RR = RowRaw<T, DPL>;
  using Raw = typename RR::R;
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int H = d.H;
  const int32_t* trow = block_table + static_cast<long long>(r) * d.max_pages;
  const bool report = threadIdx.x == 0 && blockIdx.x == 0;
  long long first;   // the wave's first item
  int cnt;           // and its item count
  int my_raw = 0;    // lane i: table entry of item first + i
  int L;
  if (tail_only) {
    L = checked_len(seq_lens, r, d, status, report);
    if (L == 0 || wave >= H) return;
    const int P = (L + d.ps - 1) / d.ps;
    first = static_cast<long long>(P - 1) * H + wave;
    cnt = 1;
    my_raw = trow[P - 1];
  } else {
    const long long items = static_cast<long long>(d.max_pages) * H;
    first = static_cast<long long>(wave) * ipw;
    if (first >= items) return;
    cnt = static_cast<int>(min(static_cast<long long>(ipw), items - first));
    if (lane < cnt) my_raw = trow[(first + lane) / H];
    L = checked_len(seq_lens, r, d, status, report);
    if (L == 0) return;
  }
  const int P = (L + d.ps - 1) / d.ps;
  const int c0 = lane * DPL < d.D ? lane * DPL : 0;   // idle lanes (D < 64 DPL) read column 0
  const bool act = lane * DPL < d.D;

  auto page_of = [&](int k) { return static_cast<int>((first + k) / H); };
  auto raw_of = [&](int k) { return __builtin_amdgcn_readlane(my_raw, k); };
  auto usable = [&](int k) {
    const int raw = raw_of(k);
    return page_of(k) < P && raw >= 0 && static_cast<long long>(raw) < d.num_phys;
  };
  auto issue = [&](Raw (&b)[kPageSize], int k) {
    const long long it = first + k;
    const int j = static_cast<int>(it - static_cast<long long>(page_of(k)) * H);
    const long long raw = usable(k) ? raw_of(k) : 0;
    const T* src = k_pool + ((raw * H + j) * d.ps) * static_cast<long long>(d.D) + c0;
#pragma unroll
    for (int t = 0; t < kPageSize; ++t) b[t] = RR::load(src + static_cast<long long>(t) * d.D);
  };
  auto finish = [&](const Raw (&b)[kPageSize], int k) {
    const int p = page_of(k);
    if (p >= P) return;   // uniform over the wave
    const int raw = raw_of(k);
    if (raw < 0 || static_cast<long long>(raw) >= d.num_phys) {
      if (lane == 0) set_status(status, MOIRA_ST_BAD_PAGE);
      return;
    }
    const int j = static_cast<int>(first + k - static_cast<long long>(p) * H);
    const int n = min(d.ps, L - p * d.ps);
    double mean[DPL];
#pragma unroll
    for (int e = 0; e < DPL; ++e) {
      double acc = 0.0;
#pragma unroll
      for (int t = 0; t < kPageSize; ++t)
        if (t < n) acc += static_cast<double>(RR::get(b[t], e));
      mean[e] = acc / static_cast<double>(n);
    }
    if (act)
      store_summary_run<DPL>(summaries, (static_cast<long long>(raw) * H + j) * d.D + c0, mean, d.sbf, d.sf8);
  };

  // two row buffers in turn; every issue is unconditional (past the last
  // item it repeats the last one, unused), so each wait counts the same loads
  Raw a[kPageSize], b[kPageSize];
  issue(a, 0);
  for (int k = 0; k < cnt; k += 2) {
    issue(b, min(k + 1, cnt - 1));
    finish(a, k);
    issue(a, min(k + 2, cnt - 1));
    if (k + 1 < cnt) finish(b, k + 1);
  }
}

// ---- host launchers ------------------------------------------------------
hipError_t launch_advance(const Dims& d, int32_t* seq_lens, int32_t* status, hipStream_t st) {
  const int threads = 256;
  const int blocks = (d.B + threads - 1) / threads;
  advance_kernel<<<blocks, threads, 0, st>>>(d, seq_lens, status);
  return hipGetLastError();
}

hipError_t launch_append(const Dims& d, int kv_dtype, const void* k_new, const void* v_new,
                         void* k_pool, void* v_pool, void* summaries,
                         const int32_t* block_table, const int32_t* seq_lens, int32_t* status,
                         hipStream_t st) {
  if (kv_dtype == MOIRA_BF16) {
    append_kernel<uint16_t><<<dim3(d.B, d.H), 256, 0, st>>>(
        d, static_cast<const uint16_t*>(k_new), static_cast<const uint16_t*>(v_new),
        static_cast<uint16_t*>(k_pool), static_cast<uint16_t*>(v_pool), summaries, block_table,
        seq_lens, status);
  } else {
    append_kernel<float><<<dim3(d.B, d.H), 256, 0, st>>>(
        d, static_cast<const float*>(k_new), static_cast<const float*>(v_new),
        static_cast<float*>(k_pool), static_cast<float*>(v_pool), summaries, block_table,
        seq_lens, status);
  }
  return hipGetLastError();
}

hipError_t launch_summaries(const Dims& d, int kv_dtype, const void* k_pool,
                            const int32_t* block_table, const int32_t* seq_lens,
                            void* summaries, int mode, int32_t* status, hipStream_t st) {
  const int tail = mode == MOIRA_SUM_TAIL ? 1 : 0;
  // items per wave: enough waves to keep every SIMD's loads flowing (about
  // 4096 over the chip), each streaming 4 to 32 items (measured at 128k
  // context: 4 items 69, 8 items 64, 16 items 63 us)
  const long long items = static_cast<long long>(d.max_pages) * d.H;
  const long long per = items * d.B / 4096;
  const int ipw = tail ? 1 : static_cast<int>(per < 4 ? 4 : (per > 32 ? 32 : per));
  const long long waves = tail ? d.H : (items + ipw - 1) / ipw;
  const dim3 grid(static_cast<unsigned>((waves + 3) / 4), d.B);
#define MOIRA_SUMS(TT, DPL)                                                                    \
  summaries_kernel<TT, DPL><<<grid, 256, 0, st>>>(d, static_cast<const TT*>(k_pool), block_table, \
                                                  seq_lens, summaries, tail, ipw, status)
  if (kv_dtype == MOIRA_BF16) {
    if (d.D == 128) MOIRA_SUMS(uint16_t, 2);
    else MOIRA_SUMS(uint16_t, 1);
  } else {
    if (d.D == 128) MOIRA_SUMS(float, 2);
    else MOIRA_SUMS(float, 1);
  }
#undef MOIRA_SUMS
  return hipGetLastError();
}

}  // namespace moira
