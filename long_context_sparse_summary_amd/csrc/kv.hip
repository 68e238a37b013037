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

// grid (page chunks, B). tail_only: only the request's last page.
template <typename T>
__global__ __launch_bounds__(256) void summaries_kernel(Dims d, const T* __restrict__ k_pool,
                                                        const int32_t* __restrict__ block_table,
                                                        const int32_t* __restrict__ seq_lens,
                                                        void* __restrict__ summaries,
                                                        int pages_per_block, int tail_only,
                                                        int32_t* status) {
  const int r = blockIdx.y;
  const int L = checked_len(seq_lens, r, d, status, threadIdx.x == 0 && blockIdx.x == 0);
  if (L == 0) return;
  const int P = (L + d.ps - 1) / d.ps;
  int p0, p1;
  if (tail_only) {
    p0 = P - 1;
    p1 = P;
  } else {
    p0 = blockIdx.x * pages_per_block;
    p1 = min(P, p0 + pages_per_block);
  }
  const int HD = d.H * d.D;
  for (int p = p0; p < p1; ++p) {
    const long long raw = block_table[static_cast<long long>(r) * d.max_pages + p];
    if (raw < 0 || raw >= d.num_phys) {
      if (threadIdx.x == 0) set_status(status, MOIRA_ST_BAD_PAGE);
      continue;
    }
    const int n = min(d.ps, L - p * d.ps);
    for (int idx = threadIdx.x; idx < HD; idx += blockDim.x) {
      const int j = idx / d.D;
      const int c = idx - j * d.D;
      const long long page_base = (raw * d.H + j) * d.ps;
      double acc = 0.0;
      for (int t = 0; t < n; ++t)
        acc += static_cast<double>(KvElem<T>::to_f32(k_pool[(page_base + t) * d.D + c]));
      store_summary(summaries, (raw * d.H + j) * d.D + c, acc / static_cast<double>(n), d.sbf);
    }
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
  const int ppb = 4;
  dim3 grid(mode == MOIRA_SUM_TAIL ? 1 : (d.max_pages + ppb - 1) / ppb, d.B);
  const int tail = mode == MOIRA_SUM_TAIL ? 1 : 0;
  if (kv_dtype == MOIRA_BF16) {
    summaries_kernel<uint16_t><<<grid, 256, 0, st>>>(d, static_cast<const uint16_t*>(k_pool),
                                                    block_table, seq_lens, summaries, ppb, tail,
                                                    status);
  } else {
    summaries_kernel<float><<<grid, 256, 0, st>>>(d, static_cast<const float*>(k_pool),
                                                 block_table, seq_lens, summaries, ppb, tail,
                                                 status);
  }
  return hipGetLastError();
}

}  // namespace moira
