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
    store_summary(summaries, (phys * d.H + j) * D + c, acc / static_cast<double>(slot + 1), d.sbf);
  }
}

// DPL consecutive elements of one token row, widened to fp32 (one load each;
// non-temporal: every K row is read once per build).
template <typename T, int DPL> struct RowLoad;
template <> struct RowLoad<uint16_t, 2> {
  static __device__ __forceinline__ void get(const uint16_t* p, float (&o)[2]) {
    const uint32_t u = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
    o[0] = __uint_as_float(u << 16);
    o[1] = __uint_as_float(u & 0xffff0000u);
  }
};
template <> struct RowLoad<uint16_t, 1> {
  static __device__ __forceinline__ void get(const uint16_t* p, float (&o)[1]) {
    o[0] = bf16_bits_to_f32(__builtin_nontemporal_load(p));
  }
};
template <> struct RowLoad<float, 2> {
  static __device__ __forceinline__ void get(const float* p, float (&o)[2]) {
    const u32x2_t x = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
    o[0] = __uint_as_float(x[0]);
    o[1] = __uint_as_float(x[1]);
  }
};
template <> struct RowLoad<float, 1> {
  static __device__ __forceinline__ void get(const float* p, float (&o)[1]) {
    o[0] = __builtin_nontemporal_load(p);
  }
};

// One wave per (page, KV head) block, four blocks per workgroup: grid
// (ceil(max_pages * H / 4), B), or (ceil(H / 4), B) for the tail page only.
// Lane l owns dimensions [l * DPL, (l + 1) * DPL) and issues the loads of all
// of the page's token rows at once (each wave load reads one contiguous row),
// then sums them in fp64 in token order, so the result is bitwise the append
// kernel's.
template <typename T, int DPL>
__global__ __launch_bounds__(256) void summaries_kernel(Dims d, const T* __restrict__ k_pool,
                                                        const int32_t* __restrict__ block_table,
                                                        const int32_t* __restrict__ seq_lens,
                                                        void* __restrict__ summaries,
                                                        int tail_only, int32_t* status) {
  const int r = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int L = checked_len(seq_lens, r, d, status, threadIdx.x == 0 && blockIdx.x == 0);
  if (L == 0) return;
  const int P = (L + d.ps - 1) / d.ps;
  const int p = tail_only ? P - 1 : item / d.H;
  const int j = tail_only ? item : item - (item / d.H) * d.H;
  if ((tail_only && item >= d.H) || p >= P) return;   // uniform over the wave
  const long long raw = block_table[static_cast<long long>(r) * d.max_pages + p];
  if (raw < 0 || raw >= d.num_phys) {
    if (lane == 0) set_status(status, MOIRA_ST_BAD_PAGE);
    return;
  }
  const int n = min(d.ps, L - p * d.ps);
  const int c0 = lane * DPL;
  if (c0 >= d.D) return;
  const T* src = k_pool + ((raw * d.H + j) * d.ps) * static_cast<long long>(d.D) + c0;
  float v[kPageSize][DPL];
#pragma unroll
  for (int t = 0; t < kPageSize; ++t) {
#pragma unroll
    for (int e = 0; e < DPL; ++e) v[t][e] = 0.f;
    if (t < n) RowLoad<T, DPL>::get(src + static_cast<long long>(t) * d.D, v[t]);
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) {
    double acc = 0.0;
#pragma unroll
    for (int t = 0; t < kPageSize; ++t)
      if (t < n) acc += static_cast<double>(v[t][e]);
    store_summary(summaries, (raw * d.H + j) * d.D + c0 + e, acc / static_cast<double>(n), d.sbf);
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
  const long long items = tail ? d.H : static_cast<long long>(d.max_pages) * d.H;
  const dim3 grid(static_cast<unsigned>((items + 3) / 4), d.B);
#define MOIRA_SUMS(TT, DPL)                                                                    \
  summaries_kernel<TT, DPL><<<grid, 256, 0, st>>>(d, static_cast<const TT*>(k_pool), block_table, \
                                                  seq_lens, summaries, tail, status)
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
