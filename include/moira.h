/*
 * moira.h -- C ABI of libmoira.so: coverage-rule sparse paged decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (MOIRA: Mass-Oriented Indexing with Ragged
 * Attention for Long-Context Decoding, abstract): per decode step and per
 * (request, layer, KV head), a coverage selection of KV pages -- the fewest
 * pages whose estimated share of the attention reaches gamma -- followed by
 * split-K attention over the resulting lists of unequal length. The attention
 * kernels derive their split on the device from the list lengths, so no host
 * round trip sits inside a step and a step can be replayed as one graph.
 *
 * The estimator is not defined on the pages; this library takes a page's
 * estimated mass for KV head j as n_p * sum_h exp(scale * q_h . kbar_p), summed
 * over the query heads h of j's GQA group and normalised over the pages of
 * that (request, KV head), where kbar_p is the page's mean key and n_p its
 * token count.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor pointers are DEVICE pointers unless a comment says "host".
 *   The caller allocates every buffer; the library never allocates, never
 *   synchronises and never reads device memory on the host. Every call only
 *   enqueues kernels on `stream` (a hipStream_t passed as void*; NULL is the
 *   legacy default stream), so every call can be captured in a HIP graph.
 *   Grid sizes depend only on the shape and on `num_workgroups`, never on
 *   device data.
 * - Layouts (row-major, innermost last):
 *     k_pool, v_pool  [num_phys_pages][num_kv_heads][page_size][head_dim]
 *                      element type kv_dtype
 *     summaries       [num_phys_pages][num_kv_heads][head_dim], sum_dtype
 *     block_table     [batch][max_pages] int32 physical page ids
 *     seq_lens        [batch] int32, tokens in the cache INCLUDING the token
 *                      appended by the current step
 *     q               [batch][num_kv_heads * group][head_dim], q_dtype;
 *                      query head h uses KV head h / group
 *     k_new, v_new    [batch][num_kv_heads][head_dim], kv_dtype
 *     page_lists      [batch][num_kv_heads][max_pages] int32 logical page ids
 *     list_lens       [batch][num_kv_heads] int32
 *     out             [batch][num_kv_heads * group][head_dim] float32
 *   Logical page p of request r holds tokens [p*page_size,
 *   min((p+1)*page_size, seq_lens[r])) and lives in physical page
 *   block_table[r][p].
 * - Return value: MOIRA_OK (0) or a negative MOIRA_E_* code. Codes other than
 *   MOIRA_E_LAUNCH come from host-side argument checks made before anything is
 *   enqueued. Problems that only device data reveals (a bad page id, a length
 *   out of range) never fault: the affected item is skipped and a MOIRA_ST_*
 *   bit is OR-ed into *status, if status is non-NULL (an int32 device word the
 *   caller clears and reads back).
 * - Concurrency: calls that write the same buffers must be ordered on one
 *   stream. The library itself keeps no device state between calls. The one
 *   caller-owned buffer that does carry something from call to call is the
 *   selection workspace: it keeps each (request, KV head)'s largest page key,
 *   which the next selection uses to bin masses. That value steers speed only,
 *   never the result, but it makes calls that share a workspace
 *   order-dependent in time, so they must not overlap.
 */
#ifndef MOIRA_H
#define MOIRA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOIRA_ABI_VERSION 5

/* Element types. MOIRA_FP8_E4M3 (OCP FP8 E4M3: 4 exponent bits, bias 7, 3
 * fraction bits, no infinities, largest finite 448) is for page summaries
 * only. */
enum moira_dtype { MOIRA_BF16 = 1, MOIRA_F32 = 2, MOIRA_FP8_E4M3 = 3 };

enum moira_status_code {
  MOIRA_OK = 0,
  MOIRA_E_NULL = -1,        /* a required pointer is NULL */
  MOIRA_E_SHAPE = -2,       /* inconsistent or non-positive sizes */
  MOIRA_E_DTYPE = -3,       /* unknown dtype */
  MOIRA_E_GAMMA = -4,       /* gamma outside (0, 1] or NaN */
  MOIRA_E_UNSUPPORTED = -5, /* size outside the compiled set */
  MOIRA_E_LAUNCH = -6,      /* the HIP runtime reported an error */
  MOIRA_E_ARG = -7,         /* other invalid scalar argument */
  MOIRA_E_SCRATCH = -8      /* the shape needs more than the static scratch holds */
};

/* Bits OR-ed into the optional device status word. */
enum moira_device_status {
  MOIRA_ST_CAPACITY = 1,    /* advancing would exceed max_pages*page_size tokens */
  MOIRA_ST_BAD_LEN = 2,     /* seq_lens[r] outside [0, max_pages*page_size], or 0 at append */
  MOIRA_ST_BAD_PAGE = 4,    /* block-table id outside [0, num_phys_pages) */
  MOIRA_ST_BAD_LIST = 8,    /* page-list entry or list length out of range */
  MOIRA_ST_MASS_RANGE = 16  /* a page's mass exponent left the 12-bit key range */
};

/* Selection rules over the same estimated page masses (moira_select_pages_rule). */
enum moira_select_rule {
  MOIRA_RULE_COVERAGE = 0,  /* smallest set reaching a mass fraction gamma (MOIRA abstract) */
  MOIRA_RULE_TOPK = 1,      /* the k heaviest pages: a fixed budget */
  MOIRA_RULE_TOPDELTA = 2   /* pages of mass >= delta * the largest page mass */
};

enum moira_summary_mode {
  MOIRA_SUM_ALL = 0,        /* every page of every request */
  MOIRA_SUM_TAIL = 1        /* only the last page of each request */
};

/* Problem shape, read (host memory) at call time and never retained.
 * Supported: head_dim in {64, 128}; page_size == 16; 1 <= group <= 16;
 * 1 <= max_pages <= 16384; batch * num_kv_heads <= 4096. */
typedef struct moira_shape {
  int32_t batch;           /* B: requests */
  int32_t num_kv_heads;    /* H_kv */
  int32_t group;           /* G: query heads per KV head */
  int32_t head_dim;        /* D */
  int32_t page_size;       /* tokens per page (16) */
  int32_t max_pages;       /* row stride of block_table and page_lists */
  int64_t num_phys_pages;  /* pages in the KV pool */
  int32_t kv_dtype;        /* MOIRA_BF16 or MOIRA_F32 (k_pool, v_pool, k_new, v_new) */
  int32_t q_dtype;         /* MOIRA_BF16 or MOIRA_F32 */
  int32_t sum_dtype;       /* page summaries: MOIRA_F32 (or 0), MOIRA_BF16 or MOIRA_FP8_E4M3 */
} moira_shape_t;

/* Message for a MOIRA_* return code (static string). */
const char* moira_strerror(int code);

/* MOIRA_ABI_VERSION of the loaded library. */
int moira_abi_version(void);

/* Start of a decode step: seq_lens[r] += 1 for every request, so that the
 * step's new token is counted. A request already holding
 * max_pages*page_size tokens (or with a negative length) is left unchanged
 * and sets MOIRA_ST_CAPACITY (MOIRA_ST_BAD_LEN). Call once per step, before
 * the per-layer calls. */
int moira_advance_seq_lens(const moira_shape_t* shape, int32_t* seq_lens,
                           int32_t* status, void* stream);

/* Append the step's token: write k_new/v_new of every (request, KV head) at
 * token position seq_lens[r]-1 of its page and refresh that page's summary
 * (mean key, summed in fp64 over the page's tokens in token order, divided by
 * the token count, rounded once to fp32; with sum_dtype MOIRA_BF16 that fp32
 * value is rounded once more, to the nearest bf16 with ties to even, and
 * stored as bf16; with MOIRA_FP8_E4M3, to the nearest E4M3 value with ties
 * to even, magnitudes from 448 up stored as 448). The result is bitwise equal to a
 * full rebuild by moira_page_summaries. The page-summary metadata follows the
 * mean-vector block metadata listed in "Faster than Flash" (section 2,
 * dynamic sparse attention); maintaining it on append is the indexing the
 * MOIRA title names. seq_lens is not modified. */
int moira_append_kv(const moira_shape_t* shape, const void* k_new, const void* v_new,
                    void* k_pool, void* v_pool, void* summaries,
                    const int32_t* block_table, const int32_t* seq_lens,
                    int32_t* status, void* stream);

/* Rebuild page summaries from the K pool (after a prefill or after KV was
 * written by other code). mode: MOIRA_SUM_ALL or MOIRA_SUM_TAIL. A page's
 * summary is its mean key, the mean-vector block metadata of "Faster than
 * Flash" (section 2, dynamic sparse attention), which the MOIRA abstract's
 * estimated page mass is computed from; same arithmetic and rounding as
 * moira_append_kv (fp64 token-order sum, one rounding to fp32, for bf16 or
 * E4M3 summaries one more to that type). Reads every listed page of every request once
 * (MOIRA_SUM_ALL) or only each request's last page (MOIRA_SUM_TAIL). */
int moira_page_summaries(const moira_shape_t* shape, const void* k_pool,
                         const int32_t* block_table, const int32_t* seq_lens,
                         void* summaries, int32_t mode, int32_t* status, void* stream);

/* Bytes of device workspace moira_select_pages needs for this shape: page
 * keys (8 bytes per (request, KV head, page)) plus, per (request, KV head),
 * two 2048-band mass histograms used by alternate calls, reference keys and
 * per-chunk key maxima. 0 on a bad shape. */
size_t moira_select_workspace_bytes(const moira_shape_t* shape);

/* Coverage-rule page selection (MOIRA abstract). For every (request r, KV
 * head j): masses of all P_r = ceil(seq_lens[r]/page_size) pages from the
 * stored summaries (logits in fp64), pages ranked by mass descending with
 * ties by page index ascending, and the first k* kept, k* the smallest k whose
 * running mass reaches gamma * (total mass). Running sums are exact integer
 * sums of masses quantised to 2^-F of the largest page mass,
 * F = min(52, 62 - ceil(log2 P_r)). Writes the kept page ids in ascending
 * order to page_lists[r][j][0..k*) and k* to list_lens[r][j]. gamma == 1 keeps
 * every page. `workspace` holds moira_select_workspace_bytes(shape) bytes, is
 * 16-byte aligned (MOIRA_E_ARG otherwise) and must be zero-filled before its
 * first use; every call leaves it ready for the next one. Between calls it
 * keeps each (request, KV head)'s largest key, which the next call uses to
 * bin masses chip-wide; that value only affects speed, never the result (an
 * unusable value falls back to an exact in-workgroup radix select). Calls
 * that share a workspace must not overlap. q may be bf16 or fp32; summaries
 * are fp32, bf16 or E4M3 (shape->sum_dtype), read exactly into fp64. */
int moira_select_pages(const moira_shape_t* shape, const void* q, const void* summaries,
                       const int32_t* block_table, const int32_t* seq_lens,
                       double gamma, float scale, void* workspace,
                       int32_t* page_lists, int32_t* list_lens,
                       int32_t* status, void* stream);

/* Page selection under another rule, for comparing rules on the same
 * kernels ("Faster than Flash", section 1, Figure 1): the same masses as
 * moira_select_pages, ranked the same way (mass descending, page index
 * ascending), and the same outputs. rule / param:
 *   MOIRA_RULE_COVERAGE  param = gamma in (0, 1]: identical to moira_select_pages;
 *   MOIRA_RULE_TOPK      param = k, a whole number >= 1: the k heaviest pages
 *                        (all P_r pages when k >= P_r);
 *   MOIRA_RULE_TOPDELTA  param = delta in [0, 1]: every page whose mass is at
 *                        least delta times the segment's largest page mass
 *                        (delta * that mass taken in fp64; delta = 0 keeps
 *                        every page).
 * Other values return MOIRA_E_ARG. Workspace rules as for moira_select_pages. */
int moira_select_pages_rule(const moira_shape_t* shape, const void* q, const void* summaries,
                            const int32_t* block_table, const int32_t* seq_lens,
                            int32_t rule, double param, float scale, void* workspace,
                            int32_t* page_lists, int32_t* list_lens,
                            int32_t* status, void* stream);

/* moira_select_pages for callers that cannot allocate device memory or pass a
 * workspace: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation. Same arguments minus the workspace, same results:
 * the workspace is a static device array inside the library, 32 MiB per GPU,
 * held by every GPU the library runs on until the process ends. A shape whose
 * workspace (moira_select_workspace_bytes) exceeds it returns
 * MOIRA_E_SCRATCH before anything is enqueued. The library looks up that
 * GPU's copy of the array on the first call on each device (make that first
 * call outside graph capture); it allocates nothing, ever. Every call ignores
 * what earlier calls left in the array (no reference key is carried, so
 * each call takes the exact in-workgroup select); calls that overlap on one
 * GPU race on the array and must be ordered. */
int moira_select_pages_noalloc(const moira_shape_t* shape, const void* q, const void* summaries,
                               const int32_t* block_table, const int32_t* seq_lens,
                               double gamma, float scale, int32_t* page_lists,
                               int32_t* list_lens, int32_t* status, void* stream);

/* moira_append_kv followed by moira_select_pages, as one call with the union
 * of their arguments and the same results bit for bit (pools, summaries,
 * lists, workspace state). For bf16 K/V below gamma = 1 it is a single
 * launch of the selection's scoring kernel, in which the wave that scores a
 * request's tail page first writes the step's token and recomputes that
 * page's mean; otherwise the append runs as its own kernel first. */
int moira_append_select(const moira_shape_t* shape, const void* q, const void* k_new,
                        const void* v_new, void* k_pool, void* v_pool, void* summaries,
                        const int32_t* block_table, const int32_t* seq_lens,
                        double gamma, float scale, void* workspace,
                        int32_t* page_lists, int32_t* list_lens,
                        int32_t* status, void* stream);

/* Number of split-K partial slots moira_ragged_decode_attn may write for
 * num_workgroups workgroups: num_workgroups + batch*num_kv_heads - 1.
 * partial_o needs slots*group*head_dim floats, partial_ml slots*group*2
 * floats. 0 on a bad shape or num_workgroups < 1. */
size_t moira_partials_slots(const moira_shape_t* shape, int32_t num_workgroups);

/* Bytes of the split-K partial states for num_workgroups workgroups:
 * slots * group * (head_dim + 2) * 4, i.e. partial_o followed by partial_ml
 * (partial_ml at byte offset slots*group*head_dim*4, a multiple of 256, so one
 * allocation of this size can hold both). 0 on a bad shape or
 * num_workgroups < 1. */
size_t moira_partials_bytes(const moira_shape_t* shape, int32_t num_workgroups);

/* Self-planning ragged split-K GQA decode attention (MOIRA abstract). The
 * per-(request, KV head) lists are concatenated in (r, j) order into W pages,
 * and the workgroups plan their shares on the device from list_lens:
 * - N < 8*S or S > 1024 (S = batch*num_kv_heads): workgroup w of the N =
 *   num_workgroups takes pages [floor(wW/N'), floor((w+1)W/N')), N' =
 *   min(N, ceil(W/4)), and for each list it touches writes one partial state
 *   to slot w + (r*num_kv_heads + j);
 * - N >= 8*S and S <= 1024: with q = max(ceil(W/(N-S)), 4), list s gets ceil(len_s/q)
 *   workgroups of its own (at most N in all), which split it evenly; each
 *   writes one partial state to slot w.
 * A workgroup is 8 waves when group*head_dim <= 1024 (one workgroup per CU:
 * num_workgroups = 256 fills an MI355X once), else 4 waves (two per CU).
 * A partial state is partial_ml = (m, l) and
 * partial_o = o for each of the group's query heads, with m the maximum of
 * scale*q.k*log2(e) over the piece's tokens, l = sum 2^(that - m) and
 * o = sum 2^(that - m) v (unnormalised). This is the sequence-parallel
 * split of FlashDecoding ("Faster than Flash", section 2) made ragged-aware.
 * Page-list entries must be ascending, unique and < P_r. Attention is exact
 * softmax over the listed pages' tokens (fp32 accumulation; bf16 K/V use the
 * matrix cores with P split into bf16 high and low parts). */
int moira_ragged_decode_attn(const moira_shape_t* shape, const void* q,
                             const void* k_pool, const void* v_pool,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* page_lists, const int32_t* list_lens,
                             float scale, int32_t num_workgroups,
                             float* partial_o, float* partial_ml,
                             int32_t* status, void* stream);

/* moira_ragged_decode_attn followed by moira_combine, with the same results,
 * in one launch where it can: for bf16 K/V with group*head_dim <= 1024, the
 * last attention workgroup to finish a piece of a (request, KV head) merges
 * that segment's partial states into out itself (no workgroup waits on
 * another), so the step loses a kernel boundary; otherwise the two kernels
 * run in turn. The merge sits behind two device-scope round trips (the
 * arrival count, then loads of the partial states past the per-XCD L2s)
 * that cost more on MI355X than the boundary they remove: the two calls
 * are the faster path; this one is for callers that want a single launch.
 * counters: [batch][num_kv_heads] uint32 device words,
 * zero-filled before the first call and left zero by every call; calls that
 * share them must not overlap. partial_o / partial_ml as for
 * moira_ragged_decode_attn, out as for moira_combine. A list of length 0
 * yields zeros. */
int moira_ragged_decode_attn_combine(const moira_shape_t* shape, const void* q,
                                     const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const int32_t* page_lists, const int32_t* list_lens,
                                     float scale, int32_t num_workgroups, float* partial_o,
                                     float* partial_ml, uint32_t* counters, float* out,
                                     int32_t* status, void* stream);

/* Log-sum-exp merge of the partial states of each (request, KV head) into
 * out (fp32, normalised): for each query head, M = max m_i, L = sum l_i
 * 2^(m_i - M), out = sum 2^(m_i - M) o_i / L over the pieces i of its list.
 * This is the merge step of the sequence-parallel decode split ("Faster than
 * Flash", section 2), over the ragged per-head lists of the MOIRA abstract.
 * Re-derives the pieces from list_lens exactly as moira_ragged_decode_attn
 * did; num_workgroups must be the value given to that call. A list of length
 * 0 yields zeros. partial_o, partial_ml: as written by that call (read
 * only); out: [batch][num_kv_heads * group][head_dim] fp32, written whole. */
int moira_combine(const moira_shape_t* shape, const int32_t* list_lens,
                  int32_t num_workgroups, const float* partial_o,
                  const float* partial_ml, float* out, void* stream);

/* ---- measurement aid (not a step of the method) ------------------------ */

/* Words of the sink buffer moira_stream_read writes (one per thread). */
size_t moira_stream_read_sink_words(void);

/* Reads `bytes` of device memory at src once, front to back, with the 16-byte
 * non-temporal vector loads the scoring and attention kernels use, and stores
 * one XOR word per thread into sink (moira_stream_read_sink_words() uint32
 * words, device memory). A benchmark times it as the sustained HBM read
 * ceiling beside the method's kernels. src 16-byte aligned and bytes a
 * positive multiple of 16 (MOIRA_E_ARG otherwise). */
int moira_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOIRA_H */
