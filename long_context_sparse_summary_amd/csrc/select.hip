// Host launchers of the page selection (kernels in select_impl.h).
#include <mutex>

#include "select_impl.h"

namespace moira {

// the fused select's instantiations live in select_fused.hip
#define MOIRA_FUSED_EXTERN(E)                                                                     \
  extern template hipError_t launch_fused_select_e<E>(const Dims&, const void*, const void*,     \
                                                      const int32_t*, const int32_t*, float,     \
                                                      const SelectWs&, const AppendArgs&, bool,  \
                                                      const CutArgs&, int32_t*, hipStream_t);
MOIRA_FUSED_EXTERN(4)
MOIRA_FUSED_EXTERN(8)
#undef MOIRA_FUSED_EXTERN

// The fused select runs the whole cut of a segment in one workgroup, whose
// passes over the segment's keys are bound by that one compute unit's
// instruction issue (about 2 us per pass at 8k pages). It pays off while a
// segment has at most 4096 pages and one request fills the chip (32k
// context: 41.6 against 44.7 us per layer-step); longer segments and batches
// measured faster with the cut as a kernel of its own, split over 1024-page
// ranges (128k: +1.5 us fused; 32 requests of 4k-128k: 266 against 248 us).
// Compiled for bf16 queries, head_dim 128 and groups of up to 8.
static bool fused_select_ok(const Dims& d, int q_dtype) {
  return q_dtype == MOIRA_BF16 && d.D == 128 && d.G <= 8 && d.B == 1 && fused_cut_slots(d) <= 8;
}

static hipError_t launch_fused_select(const Dims& d, const void* q, const void* summaries,
                                      const int32_t* block_table, const int32_t* seq_lens,
                                      float scale, const SelectWs& ws, const AppendArgs& app,
                                      bool append, const CutArgs& cut, int32_t* status,
                                      hipStream_t st) {
#define MOIRA_FUSED_CASE(E)                                                                       \
  case E:                                                                                       \
    return launch_fused_select_e<E>(d, q, summaries, block_table, seq_lens, scale, ws, app,   \
                                    append, cut, status, st);
  switch (fused_cut_slots(d)) {
    MOIRA_FUSED_CASE(4)
    MOIRA_FUSED_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef MOIRA_FUSED_CASE
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

// ---- host launchers ----------------------------------------------------------
template <typename QT, typename ST, int D, bool APPEND>
static void launch_score_d(const Dims& d, const void* q, const void* summaries,
                           const int32_t* block_table, const int32_t* seq_lens, float scale,
                           const SelectWs& ws, const AppendArgs& app, int32_t* status,
                           hipStream_t st) {
  // 8-wave workgroups on the single-request grid (one per CU), 4 on the
  // batch grid (two per CU)
  const ScoreGrid g = score_grid(d, d.B == 1 ? kScoreMaxWaves : 4);
  const dim3 grid = g.grid;
  const int cpw = g.cpw, nwg = g.nwg, sw = g.sw, nwv = g.threads / 64;
  const QT* qq = static_cast<const QT*>(q);
  const ST* ss = static_cast<const ST*>(summaries);
#define MOIRA_SELECT(GG)                                                                     \
  score_kernel<QT, ST, D, GG, APPEND><<<grid, 64 * nwv, 0, st>>>(                        \
      d, qq, ss, block_table, seq_lens, scale, ws, cpw, nwg, sw, app, status, CutArgs{})
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
  else if (d.sf8)
    launch_score_s<uint8_t, APPEND>(d, q_dtype, q, summaries, block_table, seq_lens, scale, ws, app, status, st);
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
  else if (SPLIT && E <= 18) {
    // a split cut holds 2 C slots: 18 for a 128k context with a few pages of
    // headroom (9 ranges)
    if constexpr (SPLIT) MOIRA_CUT(18);
  }
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
  if (rule == MOIRA_RULE_COVERAGE && fused_select_ok(d, q_dtype))
    return launch_fused_select(d, q, summaries, block_table, seq_lens, scale, ws, AppendArgs{},
                               false, CutArgs{param, page_lists, list_lens}, status, st);
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
  if (fused_select_ok(d, q_dtype))
    return launch_fused_select(d, q, summaries, block_table, seq_lens, scale, ws, app, true,
                               CutArgs{gamma, page_lists, list_lens}, status, st);
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
