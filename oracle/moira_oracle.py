"""Plain, slow fp64 CPU oracle for coverage-rule sparse paged decode attention.

TEST INFRASTRUCTURE. This module is the checker, not the product: only the
test suite, the smoke check and the benchmark's CPU-baseline leg may import or
call it. It shares no code, table or helper with the HIP library and imports
nothing from the product package; both sides only consume the same seeded
inputs.

What it computes (sources are the pages' titles and sections):

* "MOIRA: Mass-Oriented Indexing with Ragged Attention for Long-Context
  Decoding", abstract: for every request, layer, KV head and decode step a
  coverage rule keeps the smallest set of KV pages whose estimated attention
  mass reaches a fraction gamma; attention then reads only those pages.
* The abstract names an "estimated attention mass" but does not define the
  estimator. The reading taken here: a page is summarised by its mean key
  (the mean-vector block metadata listed in "Faster than Flash", section 2,
  dynamic sparse attention); the unnormalised mass of page p for KV head j is
  n_p * sum_h exp(scale * q_h . kbar_p), summed over the query heads h that
  share KV head j, and the masses are normalised over the pages of that
  (request, KV head).
* Ranking is by mass, descending; equal masses rank by page index,
  ascending. The kept set is the first k* ranked pages, k* the smallest k
  whose running sum of normalised masses is >= gamma. gamma >= 1 keeps every
  page.
* Attention over the kept pages is exact softmax attention restricted to
  their tokens, with no correction for the mass left out. Split-K partial
  states (m, l, o) and their log-sum-exp merge follow the sequence-parallel
  decoding of FlashDecoding ("Faster than Flash", section 2, hardware-aware
  exact attention).

Precision: every step runs in fp64 on values upcast exactly from the inputs.
One exception, by design: selection is a floating-point decision that yields
integers (page ids), so the oracle takes it from the same stored page
summaries the kernel reads -- the fp64 page mean rounded once to fp32, and
for bf16 (or OCP FP8 E4M3) summaries that fp32 value rounded once more to
bf16 (or E4M3), nearest with ties to even, E4M3 saturating at 448
(``stored_summaries``). Everything after that rounding is fp64 again.

Parity status per function (pins live in tests/test_oracle_pins.py):
    page_means            pinned (closed forms, incremental == batch)
    stored_summaries      pinned (exact fp32 rounding of the mean; bf16
                          rounding against torch's conversion and hand ties)
    e4m3_round            pinned (hand-derived grid points, ties, subnormals
                          and saturation; torch's float8_e4m3fn conversion in
                          range; idempotent and monotone)
    page_masses           pinned (softmax special case, closed forms, golden)
    coverage_select       pinned (brute force, minimality, nesting, golden)
    topk_select           pinned (brute force over subsets, ties, bounds)
    topdelta_select       pinned (special cases, nesting, scale invariance, golden)
    select_pages          pinned (composition of the above)
    select_pages_rule     pinned (every rule through the dispatcher on
                          hand-derived masses; rows past the request ignored)
    sparse_attention      pinned (torch SDPA in fp64, closed forms)
    attention_partial /
    combine_partials      pinned (merge of any partition == unsplit SDPA)
    OracleHead            pinned (incremental summaries == page_means;
                          select_rule on a head whose means are hand-derived)
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "num_pages",
    "page_token_counts",
    "page_means",
    "e4m3_round",
    "stored_summaries",
    "page_logits",
    "page_masses",
    "coverage_select",
    "topk_select",
    "topdelta_select",
    "select_pages",
    "select_pages_rule",
    "page_tokens",
    "sparse_attention",
    "attention_partial",
    "combine_partials",
    "OracleHead",
]


# --------------------------------------------------------------------------
# Pages (MOIRA abstract: the KV cache is read in pages; the page size is not
# stated on the pages, every workload here uses 16 tokens).
# --------------------------------------------------------------------------
def num_pages(seq_len: int, page_size: int) -> int:
    """P = ceil(L / page_size): number of pages that hold L tokens."""
    return (int(seq_len) + page_size - 1) // page_size


def page_token_counts(seq_len: int, page_size: int) -> np.ndarray:
    """n_p for p = 0..P-1: page_size for full pages, the remainder for the tail."""
    P = num_pages(seq_len, page_size)
    n = np.full(P, page_size, dtype=np.int64)
    if P:
        n[-1] = seq_len - (P - 1) * page_size
    return n


def page_means(keys: np.ndarray, seq_len: int, page_size: int) -> np.ndarray:
    """Mean key of every page, fp64: kbar_p = (1/n_p) * sum_{t in page p} k_t.

    keys: [>= seq_len, D] token keys of one (request, KV head), any float dtype.
    The sum runs over the page's tokens in token order (one fp64 addition per
    token), then is divided by n_p. Returns [P, D] float64.
    """
    L = int(seq_len)
    P = num_pages(L, page_size)
    D = keys.shape[-1]
    k = np.asarray(keys[:L], dtype=np.float64)
    padded = np.zeros((P * page_size, D), dtype=np.float64)
    padded[:L] = k
    padded = padded.reshape(P, page_size, D)
    counts = page_token_counts(L, page_size)
    acc = np.zeros((P, D), dtype=np.float64)
    for t in range(page_size):
        live = counts > t
        acc[live] = acc[live] + padded[live, t]
    return acc / counts[:, None].astype(np.float64)


def e4m3_round(f32: np.ndarray) -> np.ndarray:
    """Round float32 values to the OCP FP8 E4M3 grid (4 exponent bits, bias
    7, 3 fraction bits; subnormal quantum 2^-9; no infinities; largest
    finite value 448), nearest with ties to even, magnitudes beyond 448
    saturating to 448. A value of exponent e (2^e <= |x| < 2^(e+1), e
    clamped below at -6, the smallest normal exponent) lies on the grid of
    quantum 2^(e-3): |x| / 2^(e-3) is rounded to an integer (rint: ties to
    even), which is exact in fp64 because the division is by a power of
    two. Returned as float32 (every E4M3 value is one)."""
    x = np.asarray(f32, dtype=np.float32).astype(np.float64)
    a = np.abs(x)
    _, ex = np.frexp(a)                  # a = m 2^ex with m in [0.5, 1)
    e = np.maximum(ex.astype(np.int64) - 1, -6)
    q = np.rint(np.ldexp(a, (3 - e).astype(np.int32)))
    v = np.minimum(np.ldexp(q, (e - 3).astype(np.int32)), 448.0)
    return np.copysign(v, x).astype(np.float32)


def stored_summaries(means: np.ndarray, dtype: str = "f32") -> np.ndarray:
    """The page summaries as the kernel stores them: the fp64 mean rounded
    once (round-to-nearest-even) to fp32, returned as float32. With
    dtype="bf16" that fp32 value is rounded once more to bf16: keep the top
    16 bits, rounding to nearest on the 16 dropped bits with ties to even
    (values are finite). The bf16 result is returned widened to float32.
    With dtype="fp8" the fp32 value is rounded once more to OCP FP8 E4M3
    (e4m3_round), returned widened to float32."""
    f32 = np.asarray(means, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return f32
    if dtype == "fp8":
        return e4m3_round(f32)
    if dtype != "bf16":
        raise ValueError(f"unknown summary dtype {dtype!r}")
    bits = f32.view(np.uint32).astype(np.uint64)
    dropped = bits & 0xFFFF
    keep = bits >> 16
    half = 0x8000
    up = (dropped > half) | ((dropped == half) & ((keep & 1) == 1))
    keep = keep + up.astype(np.uint64)
    return (keep << 16).astype(np.uint32).view(np.float32)


# --------------------------------------------------------------------------
# Estimated attention mass and the coverage rule (MOIRA abstract).
# --------------------------------------------------------------------------
def page_logits(q_group: np.ndarray, summaries: np.ndarray, scale: float) -> np.ndarray:
    """l[h, p] = scale * q_h . kbar_p in fp64. q_group: [G, D]; summaries: [P, D]."""
    q = np.asarray(q_group, dtype=np.float64)
    s = np.asarray(summaries, dtype=np.float64)
    return float(scale) * (q @ s.T)


def page_masses(q_group: np.ndarray, summaries: np.ndarray, counts: np.ndarray,
                scale: float) -> np.ndarray:
    """Normalised estimated mass of each page of one (request, KV head).

    w_p = n_p * sum_h exp(l[h, p] - M), M = max over all h, p (a common
    factor that cancels); m_p = w_p / sum_p' w_p'. Returns [P] float64.
    """
    lg = page_logits(q_group, summaries, scale)
    if lg.size == 0:
        return np.zeros(0, dtype=np.float64)
    M = lg.max()
    w = np.asarray(counts, dtype=np.float64) * np.exp(lg - M).sum(axis=0)
    return w / w.sum()


def coverage_select(masses: np.ndarray, gamma: float) -> np.ndarray:
    """Smallest set of pages whose mass reaches gamma, as ascending page ids.

    Pages rank by mass descending, equal masses by page index ascending. With
    C_k the running fp64 sum of the first k ranked masses, k* = min{k : C_k >=
    gamma} and the kept set is the first k* ranked pages. gamma >= 1 keeps all
    pages (rounding never drops one). If rounding leaves C_P < gamma < 1,
    every page is kept.
    """
    m = np.asarray(masses, dtype=np.float64)
    P = m.shape[0]
    if P == 0:
        return np.zeros(0, dtype=np.int64)
    if gamma >= 1.0:
        return np.arange(P, dtype=np.int64)
    order = np.lexsort((np.arange(P), -m))  # last key is primary
    csum = np.cumsum(m[order])
    hit = np.nonzero(csum >= gamma)[0]
    k = int(hit[0]) + 1 if hit.size else P
    return np.sort(order[:k]).astype(np.int64)


def topk_select(masses: np.ndarray, k: int) -> np.ndarray:
    """The k heaviest pages, as ascending page ids: a fixed budget ("Faster
    than Flash", section 1, Figure 1 (a)). Pages rank by mass descending,
    equal masses by page index ascending; k >= P keeps every page."""
    m = np.asarray(masses, dtype=np.float64)
    P = m.shape[0]
    k = max(0, min(int(k), P))
    order = np.lexsort((np.arange(P), -m))  # last key is primary
    return np.sort(order[:k]).astype(np.int64)


def topdelta_select(masses: np.ndarray, delta: float) -> np.ndarray:
    """Pages whose mass is at least delta times the largest one, as ascending
    page ids: a threshold relative to the maximum ("Faster than Flash",
    section 1, Figure 1 (c), and its list of contributions). The maximum is
    the segment's own (the pages take it from a local maximum to avoid a
    global synchronisation; the whole segment's maximum is already at hand
    here). delta <= 0 keeps every page; delta = 1 keeps the pages equal to
    the maximum."""
    m = np.asarray(masses, dtype=np.float64)
    P = m.shape[0]
    if P == 0:
        return np.zeros(0, dtype=np.int64)
    if delta <= 0.0:
        return np.arange(P, dtype=np.int64)
    thr = float(delta) * float(m.max())
    return np.nonzero(m >= thr)[0].astype(np.int64)


def select_pages(q_group: np.ndarray, summaries: np.ndarray, seq_len: int,
                 page_size: int, scale: float, gamma: float) -> np.ndarray:
    """Coverage selection for one (request, KV head) from stored summaries."""
    counts = page_token_counts(seq_len, page_size)
    m = page_masses(q_group, summaries[: counts.shape[0]], counts, scale)
    return coverage_select(m, gamma)


def select_pages_rule(q_group: np.ndarray, summaries: np.ndarray, seq_len: int,
                      page_size: int, scale: float, rule: str, param: float) -> np.ndarray:
    """Selection for one (request, KV head) under a rule: "coverage" (param =
    gamma), "topk" (param = k) or "topdelta" (param = delta), all over the same
    estimated masses."""
    counts = page_token_counts(seq_len, page_size)
    m = page_masses(q_group, summaries[: counts.shape[0]], counts, scale)
    if rule == "coverage":
        return coverage_select(m, param)
    if rule == "topk":
        return topk_select(m, int(param))
    if rule == "topdelta":
        return topdelta_select(m, param)
    raise ValueError(f"unknown rule {rule!r}")


# --------------------------------------------------------------------------
# Attention over the kept pages.
# --------------------------------------------------------------------------
def page_tokens(pages: np.ndarray, seq_len: int, page_size: int) -> np.ndarray:
    """Token indices of the given pages, in page order then token order."""
    out = []
    for p in np.asarray(pages, dtype=np.int64):
        lo = int(p) * page_size
        hi = min(lo + page_size, int(seq_len))
        out.append(np.arange(lo, hi, dtype=np.int64))
    if not out:
        return np.zeros(0, dtype=np.int64)
    return np.concatenate(out)


def sparse_attention(q_group: np.ndarray, keys: np.ndarray, values: np.ndarray,
                     pages: np.ndarray, seq_len: int, page_size: int,
                     scale: float) -> np.ndarray:
    """o_h = sum_{t in T(S)} softmax_t(scale * q_h . k_t) * v_t over the tokens
    T(S) of the kept pages S, in fp64. Returns [G, D] float64 (zeros if S is
    empty)."""
    q = np.asarray(q_group, dtype=np.float64)
    toks = page_tokens(pages, seq_len, page_size)
    if toks.size == 0:
        return np.zeros((q.shape[0], np.asarray(values).shape[-1]), dtype=np.float64)
    K = np.asarray(keys[toks], dtype=np.float64)
    V = np.asarray(values[toks], dtype=np.float64)
    lg = float(scale) * (q @ K.T)
    lg = lg - lg.max(axis=1, keepdims=True)
    p = np.exp(lg)
    return (p @ V) / p.sum(axis=1, keepdims=True)


def attention_partial(q_group: np.ndarray, keys: np.ndarray, values: np.ndarray,
                      pages: np.ndarray, seq_len: int, page_size: int,
                      scale: float):
    """Split-K partial state over a subset of pages: (m [G], l [G], o [G, D]) with
    m the max logit, l = sum exp(logit - m), o = sum exp(logit - m) * v
    (unnormalised). An empty subset gives m = -inf, l = 0, o = 0."""
    q = np.asarray(q_group, dtype=np.float64)
    G = q.shape[0]
    D = np.asarray(values).shape[-1]
    toks = page_tokens(pages, seq_len, page_size)
    if toks.size == 0:
        return (np.full(G, -np.inf), np.zeros(G), np.zeros((G, D)))
    K = np.asarray(keys[toks], dtype=np.float64)
    V = np.asarray(values[toks], dtype=np.float64)
    lg = float(scale) * (q @ K.T)
    m = lg.max(axis=1)
    p = np.exp(lg - m[:, None])
    return (m, p.sum(axis=1), p @ V)


def combine_partials(partials) -> np.ndarray:
    """Log-sum-exp merge of partial states into the normalised output:
    M = max_i m_i, L = sum_i l_i exp(m_i - M), o = sum_i exp(m_i - M) o_i / L.
    Empty partials (m = -inf) contribute nothing; if all are empty the output
    is zero."""
    parts = list(partials)
    ms = np.stack([np.asarray(p[0], dtype=np.float64) for p in parts])   # [n, G]
    ls = np.stack([np.asarray(p[1], dtype=np.float64) for p in parts])   # [n, G]
    os_ = np.stack([np.asarray(p[2], dtype=np.float64) for p in parts])  # [n, G, D]
    M = ms.max(axis=0)
    safeM = np.where(np.isfinite(M), M, 0.0)
    f = np.where(np.isfinite(ms), np.exp(ms - safeM[None, :]), 0.0)       # [n, G]
    L = (ls * f).sum(axis=0)
    O = (os_ * f[:, :, None]).sum(axis=0)
    out = np.zeros_like(O)
    ok = L > 0
    out[ok] = O[ok] / L[ok][:, None]
    return out


# --------------------------------------------------------------------------
# One (request, KV head) carried across decode steps, with page means kept up
# to date on append: the "indexing" that the MOIRA title names.
# --------------------------------------------------------------------------
class OracleHead:
    """Token K/V of one (request, KV head) plus fp64 page means maintained on
    append (only the tail page's mean changes when a token is appended)."""

    def __init__(self, keys: np.ndarray, values: np.ndarray, seq_len: int,
                 page_size: int, capacity: int | None = None, summary_dtype: str = "f32"):
        L = int(seq_len)
        self.summary_dtype = summary_dtype
        D = keys.shape[-1]
        cap = max(int(capacity or 0), L)
        self.page_size = int(page_size)
        self.keys = np.zeros((cap, D), dtype=np.float64)
        self.values = np.zeros((cap, D), dtype=np.float64)
        self.keys[:L] = np.asarray(keys[:L], dtype=np.float64)
        self.values[:L] = np.asarray(values[:L], dtype=np.float64)
        self.seq_len = L
        self.means = page_means(self.keys, L, self.page_size)

    def append(self, k: np.ndarray, v: np.ndarray) -> None:
        L = self.seq_len
        if L >= self.keys.shape[0]:
            grow = max(self.keys.shape[0], 16)
            self.keys = np.concatenate([self.keys, np.zeros((grow, self.keys.shape[1]))])
            self.values = np.concatenate([self.values, np.zeros((grow, self.values.shape[1]))])
        self.keys[L] = np.asarray(k, dtype=np.float64)
        self.values[L] = np.asarray(v, dtype=np.float64)
        self.seq_len = L + 1
        ps = self.page_size
        p = L // ps
        lo = p * ps
        acc = np.zeros(self.keys.shape[1], dtype=np.float64)
        for t in range(lo, L + 1):
            acc = acc + self.keys[t]
        mean = acc / float(L + 1 - lo)
        if p == self.means.shape[0]:
            self.means = np.concatenate([self.means, mean[None, :]])
        else:
            self.means[p] = mean

    def select_rule(self, q_group: np.ndarray, scale: float, rule: str, param: float) -> np.ndarray:
        return select_pages_rule(q_group, stored_summaries(self.means, self.summary_dtype),
                                 self.seq_len, self.page_size, scale, rule, param)

    def select(self, q_group: np.ndarray, scale: float, gamma: float) -> np.ndarray:
        return select_pages(q_group, stored_summaries(self.means, self.summary_dtype), self.seq_len,
                            self.page_size, scale, gamma)

    def attend(self, q_group: np.ndarray, pages: np.ndarray, scale: float) -> np.ndarray:
        return sparse_attention(q_group, self.keys, self.values, pages,
                                self.seq_len, self.page_size, scale)

    def step(self, q_group: np.ndarray, k: np.ndarray, v: np.ndarray,
             scale: float, gamma: float):
        """One decode step: append (k, v), select, attend. Returns (pages, out)."""
        self.append(k, v)
        pages = self.select(q_group, scale, gamma)
        return pages, self.attend(q_group, pages, scale)


def boundary_band_pages(masses: np.ndarray, gamma: float, rel: float = 1e-5) -> np.ndarray:
    """Pages whose inclusion is decided within `rel` (relative to gamma) of the
    gamma boundary: rank positions k with |C_k - gamma| <= rel*gamma or
    |C_{k-1} - gamma| <= rel*gamma. Returned as page ids (any order)."""
    m = np.asarray(masses, dtype=np.float64)
    P = m.shape[0]
    if P == 0 or gamma >= 1.0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((np.arange(P), -m))
    csum = np.cumsum(m[order])
    prev = np.concatenate([[0.0], csum[:-1]])
    tol = rel * gamma
    band = (np.abs(csum - gamma) <= tol) | (np.abs(prev - gamma) <= tol)
    return order[band].astype(np.int64)


def near_tie_pages(masses: np.ndarray, pages: np.ndarray, rel: float = 1e-12) -> np.ndarray:
    """Pages that could swap across the cut by rounding: the kept page(s) of
    least mass and every dropped page whose mass is within `rel` (relative) of
    it, plus every kept page within `rel` of the largest dropped mass. The
    default 1e-12 admits only swaps at fp64 rounding level: a kernel that ranks
    masses computed in fp64 from the same stored summaries differs from this
    oracle by far less."""
    m = np.asarray(masses, dtype=np.float64)
    kept = np.zeros(m.shape[0], dtype=bool)
    kept[np.asarray(pages, dtype=np.int64)] = True
    if kept.all() or not kept.any():
        return np.zeros(0, dtype=np.int64)
    lo_kept = m[kept].min()
    hi_drop = m[~kept].max()
    ids = np.arange(m.shape[0])
    near = (~kept & (np.abs(m - lo_kept) <= rel * max(lo_kept, 1e-300))) | \
           (kept & (np.abs(m - hi_drop) <= rel * max(hi_drop, 1e-300)))
    return ids[near].astype(np.int64)


__all__ += ["boundary_band_pages", "near_tie_pages"]


if __name__ == "__main__":  # pragma: no cover
    rng = np.random.default_rng(0)
    K = rng.standard_normal((40, 8))
    q = rng.standard_normal((2, 8))
    s = stored_summaries(page_means(K, 40, 16))
    print(select_pages(q, s, 40, 16, 1 / math.sqrt(8), 0.9))
