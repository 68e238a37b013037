// C ABI of libmoira.so: host-side argument checks and launches. Every entry
// point validates its arguments before enqueueing anything, then enqueues on
// the caller's stream only (no allocation, no synchronisation, no device reads
// from the host).
#include <cmath>

#include "moira_common.h"

namespace moira {
hipError_t launch_advance(const Dims& d, int32_t* seq_lens, int32_t* status, hipStream_t st);
hipError_t launch_append(const Dims& d, int kv_dtype, const void* k_new, const void* v_new,
                         void* k_pool, void* v_pool, void* summaries, const int32_t* block_table,
                         const int32_t* seq_lens, int32_t* status, hipStream_t st);
hipError_t launch_summaries(const Dims& d, int kv_dtype, const void* k_pool,
                            const int32_t* block_table, const int32_t* seq_lens, void* summaries,
                            int mode, int32_t* status, hipStream_t st);
hipError_t launch_select(const Dims& d, int q_dtype, const void* q, const void* summaries,
                         const int32_t* block_table, const int32_t* seq_lens, double gamma,
                         float scale, void* workspace, int32_t* page_lists, int32_t* list_lens,
                         int32_t* status, hipStream_t st);
size_t select_workspace_bytes(int S, int max_pages);
hipError_t launch_select_rule(const Dims& d, int q_dtype, const void* q, const void* summaries,
                              const int32_t* block_table, const int32_t* seq_lens, int rule,
                              double param, float scale, void* workspace, int32_t* page_lists,
                              int32_t* list_lens, int32_t* status, hipStream_t st);
hipError_t launch_append_select(const Dims& d, int kv_dtype, int q_dtype, const void* q,
                                const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                void* summaries, const int32_t* block_table,
                                const int32_t* seq_lens, double gamma, float scale,
                                void* workspace, int32_t* page_lists, int32_t* list_lens,
                                int32_t* status, hipStream_t st);
hipError_t launch_attn(const Dims& d, int kv_dtype, int q_dtype, const void* q, const void* k_pool,
                       const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* page_lists, const int32_t* list_lens, float scale, int N,
                       float* partial_o, float* partial_ml, int32_t* status, hipStream_t st);
hipError_t launch_combine(const Dims& d, const int32_t* list_lens, int N, const float* partial_o,
                          const float* partial_ml, float* out, hipStream_t st);
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);
hipError_t launch_attn_combine(const Dims& d, int kv_dtype, int q_dtype, const void* q,
                               const void* k_pool, const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* page_lists,
                               const int32_t* list_lens, float scale, int N, float* partial_o,
                               float* partial_ml, unsigned int* counters, float* out,
                               int32_t* status, hipStream_t st);
hipError_t launch_select_noalloc(const Dims& d, int q_dtype, const void* q, const void* summaries,
                                 const int32_t* block_table, const int32_t* seq_lens, double gamma,
                                 float scale, int32_t* page_lists, int32_t* list_lens,
                                 int32_t* status, hipStream_t st);
}  // namespace moira

using moira::Dims;

namespace {

int check_shape(const moira_shape_t* s, Dims* d) {
  if (!s) return MOIRA_E_NULL;
  if (s->batch < 1 || s->num_kv_heads < 1 || s->group < 1 || s->head_dim < 1 ||
      s->page_size < 1 || s->max_pages < 1 || s->num_phys_pages < 1)
    return MOIRA_E_SHAPE;
  if (s->num_phys_pages > 2147483647LL) return MOIRA_E_SHAPE;
  if ((s->kv_dtype != MOIRA_BF16 && s->kv_dtype != MOIRA_F32) ||
      (s->q_dtype != MOIRA_BF16 && s->q_dtype != MOIRA_F32) ||
      (s->sum_dtype != 0 && s->sum_dtype != MOIRA_BF16 && s->sum_dtype != MOIRA_F32 &&
       s->sum_dtype != MOIRA_FP8_E4M3))
    return MOIRA_E_DTYPE;
  if (s->head_dim != 64 && s->head_dim != 128) return MOIRA_E_UNSUPPORTED;
  if (s->page_size != moira::kPageSize) return MOIRA_E_UNSUPPORTED;
  if (s->group > moira::kMaxGroup) return MOIRA_E_UNSUPPORTED;
  if (s->max_pages > moira::kMaxPages) return MOIRA_E_UNSUPPORTED;
  if (static_cast<long long>(s->batch) * s->num_kv_heads > moira::kMaxSegments)
    return MOIRA_E_UNSUPPORTED;
  d->B = s->batch;
  d->H = s->num_kv_heads;
  d->G = s->group;
  d->D = s->head_dim;
  d->ps = s->page_size;
  d->max_pages = s->max_pages;
  d->num_phys = s->num_phys_pages;
  d->sbf = s->sum_dtype == MOIRA_BF16 ? 1 : 0;
  d->sf8 = s->sum_dtype == MOIRA_FP8_E4M3 ? 1 : 0;
  return MOIRA_OK;
}

int finish(hipError_t e) { return e == hipSuccess ? MOIRA_OK : MOIRA_E_LAUNCH; }

}  // namespace

extern "C" {

const char* moira_strerror(int code) {
  switch (code) {
    case MOIRA_OK: return "ok";
    case MOIRA_E_NULL: return "a required pointer is NULL";
    case MOIRA_E_SHAPE: return "inconsistent or non-positive shape";
    case MOIRA_E_DTYPE: return "unknown dtype";
    case MOIRA_E_GAMMA: return "gamma must lie in (0, 1]";
    case MOIRA_E_UNSUPPORTED: return "shape outside the supported set (head_dim 64/128, page_size 16, group <= 16, max_pages <= 16384, batch*kv_heads <= 4096)";
    case MOIRA_E_LAUNCH: return "HIP launch error";
    case MOIRA_E_ARG: return "invalid scalar argument";
    case MOIRA_E_SCRATCH: return "the selection workspace this shape needs exceeds the library's static scratch (moira_select_pages_noalloc: 32 MiB per GPU)";
    default: return "unknown moira error";
  }
}

int moira_abi_version(void) { return MOIRA_ABI_VERSION; }

int moira_advance_seq_lens(const moira_shape_t* shape, int32_t* seq_lens, int32_t* status,
                           void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!seq_lens) return MOIRA_E_NULL;
  return finish(moira::launch_advance(d, seq_lens, status, static_cast<hipStream_t>(stream)));
}

int moira_append_kv(const moira_shape_t* shape, const void* k_new, const void* v_new,
                    void* k_pool, void* v_pool, void* summaries, const int32_t* block_table,
                    const int32_t* seq_lens, int32_t* status, void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!k_new || !v_new || !k_pool || !v_pool || !summaries || !block_table || !seq_lens)
    return MOIRA_E_NULL;
  return finish(moira::launch_append(d, shape->kv_dtype, k_new, v_new, k_pool, v_pool, summaries,
                                     block_table, seq_lens, status,
                                     static_cast<hipStream_t>(stream)));
}

int moira_page_summaries(const moira_shape_t* shape, const void* k_pool,
                         const int32_t* block_table, const int32_t* seq_lens, void* summaries,
                         int32_t mode, int32_t* status, void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!k_pool || !block_table || !seq_lens || !summaries) return MOIRA_E_NULL;
  if (mode != MOIRA_SUM_ALL && mode != MOIRA_SUM_TAIL) return MOIRA_E_ARG;
  return finish(moira::launch_summaries(d, shape->kv_dtype, k_pool, block_table, seq_lens,
                                        summaries, mode, status,
                                        static_cast<hipStream_t>(stream)));
}

size_t moira_select_workspace_bytes(const moira_shape_t* shape) {
  Dims d;
  if (check_shape(shape, &d)) return 0;
  return moira::select_workspace_bytes(d.S(), d.max_pages);
}

int moira_select_pages(const moira_shape_t* shape, const void* q, const void* summaries,
                       const int32_t* block_table, const int32_t* seq_lens, double gamma,
                       float scale, void* workspace, int32_t* page_lists, int32_t* list_lens,
                       int32_t* status, void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!q || !summaries || !block_table || !seq_lens || !workspace || !page_lists || !list_lens)
    return MOIRA_E_NULL;
  if (!(gamma > 0.0 && gamma <= 1.0)) return MOIRA_E_GAMMA;
  if (!std::isfinite(scale)) return MOIRA_E_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return MOIRA_E_ARG;
  return finish(moira::launch_select(d, shape->q_dtype, q, summaries, block_table, seq_lens, gamma,
                                     scale, workspace, page_lists, list_lens, status,
                                     static_cast<hipStream_t>(stream)));
}

int moira_select_pages_rule(const moira_shape_t* shape, const void* q, const void* summaries,
                            const int32_t* block_table, const int32_t* seq_lens, int32_t rule,
                            double param, float scale, void* workspace, int32_t* page_lists,
                            int32_t* list_lens, int32_t* status, void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!q || !summaries || !block_table || !seq_lens || !workspace || !page_lists || !list_lens)
    return MOIRA_E_NULL;
  if (!std::isfinite(scale) || !std::isfinite(param)) return MOIRA_E_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return MOIRA_E_ARG;
  switch (rule) {
    case MOIRA_RULE_COVERAGE:
      if (!(param > 0.0 && param <= 1.0)) return MOIRA_E_GAMMA;
      break;
    case MOIRA_RULE_TOPK:
      if (!(param >= 1.0) || param != std::floor(param) || param > 2147483647.0) return MOIRA_E_ARG;
      break;
    case MOIRA_RULE_TOPDELTA:
      if (!(param >= 0.0 && param <= 1.0)) return MOIRA_E_ARG;
      break;
    default:
      return MOIRA_E_ARG;
  }
  return finish(moira::launch_select_rule(d, shape->q_dtype, q, summaries, block_table, seq_lens,
                                          rule, param, scale, workspace, page_lists, list_lens,
                                          status, static_cast<hipStream_t>(stream)));
}

int moira_append_select(const moira_shape_t* shape, const void* q, const void* k_new,
                        const void* v_new, void* k_pool, void* v_pool, void* summaries,
                        const int32_t* block_table, const int32_t* seq_lens, double gamma,
                        float scale, void* workspace, int32_t* page_lists, int32_t* list_lens,
                        int32_t* status, void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!q || !k_new || !v_new || !k_pool || !v_pool || !summaries || !block_table || !seq_lens ||
      !workspace || !page_lists || !list_lens)
    return MOIRA_E_NULL;
  if (!(gamma > 0.0 && gamma <= 1.0)) return MOIRA_E_GAMMA;
  if (!std::isfinite(scale)) return MOIRA_E_ARG;
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0) return MOIRA_E_ARG;
  return finish(moira::launch_append_select(d, shape->kv_dtype, shape->q_dtype, q, k_new, v_new,
                                            k_pool, v_pool, summaries, block_table, seq_lens,
                                            gamma, scale, workspace, page_lists, list_lens,
                                            status, static_cast<hipStream_t>(stream)));
}

int moira_select_pages_noalloc(const moira_shape_t* shape, const void* q, const void* summaries,
                               const int32_t* block_table, const int32_t* seq_lens, double gamma,
                               float scale, int32_t* page_lists, int32_t* list_lens,
                               int32_t* status, void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!q || !summaries || !block_table || !seq_lens || !page_lists || !list_lens)
    return MOIRA_E_NULL;
  if (!(gamma > 0.0 && gamma <= 1.0)) return MOIRA_E_GAMMA;
  if (!std::isfinite(scale)) return MOIRA_E_ARG;
  if (moira::select_workspace_bytes(d.S(), d.max_pages) > moira::kNoAllocScratchBytes)
    return MOIRA_E_SCRATCH;
  return finish(moira::launch_select_noalloc(d, shape->q_dtype, q, summaries, block_table, seq_lens,
                                             gamma, scale, page_lists, list_lens, status,
                                             static_cast<hipStream_t>(stream)));
}

size_t moira_partials_slots(const moira_shape_t* shape, int32_t num_workgroups) {
  Dims d;
  if (check_shape(shape, &d) || num_workgroups < 1) return 0;
  return static_cast<size_t>(num_workgroups) + static_cast<size_t>(d.S()) - 1;
}

size_t moira_partials_bytes(const moira_shape_t* shape, int32_t num_workgroups) {
  Dims d;
  if (check_shape(shape, &d) || num_workgroups < 1) return 0;
  const size_t slots = static_cast<size_t>(num_workgroups) + static_cast<size_t>(d.S()) - 1;
  return slots * static_cast<size_t>(d.G) * (static_cast<size_t>(d.D) + 2) * sizeof(float);
}

int moira_ragged_decode_attn(const moira_shape_t* shape, const void* q, const void* k_pool,
                             const void* v_pool, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* page_lists,
                             const int32_t* list_lens, float scale, int32_t num_workgroups,
                             float* partial_o, float* partial_ml, int32_t* status, void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !page_lists || !list_lens ||
      !partial_o || !partial_ml)
    return MOIRA_E_NULL;
  if (!std::isfinite(scale) || num_workgroups < 1 || num_workgroups > 65536) return MOIRA_E_ARG;
  return finish(moira::launch_attn(d, shape->kv_dtype, shape->q_dtype, q, k_pool, v_pool,
                                   block_table, seq_lens, page_lists, list_lens, scale,
                                   num_workgroups, partial_o, partial_ml, status,
                                   static_cast<hipStream_t>(stream)));
}

int moira_ragged_decode_attn_combine(const moira_shape_t* shape, const void* q, const void* k_pool,
                                     const void* v_pool, const int32_t* block_table,
                                     const int32_t* seq_lens, const int32_t* page_lists,
                                     const int32_t* list_lens, float scale, int32_t num_workgroups,
                                     float* partial_o, float* partial_ml, uint32_t* counters,
                                     float* out, int32_t* status, void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !page_lists || !list_lens ||
      !partial_o || !partial_ml || !counters || !out)
    return MOIRA_E_NULL;
  if (!std::isfinite(scale) || num_workgroups < 1 || num_workgroups > 65536) return MOIRA_E_ARG;
  return finish(moira::launch_attn_combine(d, shape->kv_dtype, shape->q_dtype, q, k_pool, v_pool,
                                           block_table, seq_lens, page_lists, list_lens, scale,
                                           num_workgroups, partial_o, partial_ml, counters, out,
                                           status, static_cast<hipStream_t>(stream)));
}

int moira_combine(const moira_shape_t* shape, const int32_t* list_lens, int32_t num_workgroups,
                  const float* partial_o, const float* partial_ml, float* out, void* stream) {
  Dims d;
  int rc = check_shape(shape, &d);
  if (rc) return rc;
  if (!list_lens || !partial_o || !partial_ml || !out) return MOIRA_E_NULL;
  if (num_workgroups < 1 || num_workgroups > 65536) return MOIRA_E_ARG;
  return finish(moira::launch_combine(d, list_lens, num_workgroups, partial_o, partial_ml, out,
                                      static_cast<hipStream_t>(stream)));
}

size_t moira_stream_read_sink_words(void) { return 2048 * 256; }

int moira_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (!src || !sink) return MOIRA_E_NULL;
  if (bytes < 16 || bytes % 16 != 0 || reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return MOIRA_E_ARG;
  return finish(moira::launch_stream_read(src, bytes, sink, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
