"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each test rests on one of: a hand-derived closed form (tests/golden), a library
routine (torch softmax / scaled_dot_product_attention in fp64 on the CPU),
brute-force enumeration on tiny inputs, or an invariant of the definitions.
The cases are chosen so that a plausible mistake (a dropped token-count
weight, a wrong sign, per-head instead of per-group normalisation, a flipped
tie rule, a strict instead of inclusive comparison, a transposed operand, a
misplaced scale) fails at least one of them.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")))


# ----------------------------------------------------------------- page means
def test_page_mean_progression_closed_form():
    g = GOLD["page_mean_progression"]
    t = np.arange(16, dtype=np.float64)
    keys = np.stack([t, -2 * t, np.ones(16)], axis=1)
    got = O.page_means(keys, g["seq_len"], g["page_size"])
    np.testing.assert_array_equal(got, np.array([g["expected_mean"]]))


def test_page_mean_partial_tail_closed_form():
    g = GOLD["page_mean_tail"]
    keys = np.arange(19, dtype=np.float64)[:, None]
    got = O.page_means(keys, g["seq_len"], g["page_size"])
    np.testing.assert_array_equal(got[:, 0], np.array(g["expected_means"]))


def test_page_mean_is_affine_equivariant():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((77, 8))
    a, b = 0.5, rng.standard_normal(8)      # exact in binary: scale by 1/2
    m1 = O.page_means(K, 77, 16)
    m2 = O.page_means(a * K + b, 77, 16)
    np.testing.assert_allclose(m2, a * m1 + b, rtol=0, atol=1e-14)


def test_incremental_means_equal_batch_bitwise():
    rng = np.random.default_rng(2)
    K = rng.standard_normal((100, 16)).astype(np.float32)
    V = rng.standard_normal((100, 16)).astype(np.float32)
    h = O.OracleHead(K, V, 37, 16)
    for L in range(37, 100):
        h.append(K[L], V[L])
        np.testing.assert_array_equal(h.means, O.page_means(K, L + 1, 16))


def test_stored_summary_is_one_fp32_rounding():
    means = np.array([[1.0 / 3.0, -2.0 / 3.0, 0.1]])
    s = O.stored_summaries(means)
    assert s.dtype == np.float32
    assert float(s[0, 0]) == 0.3333333432674408  # nearest fp32 to 1/3
    assert float(s[0, 1]) == -0.6666666865348816
    assert float(s[0, 2]) == float(np.float32(0.1))


def test_bf16_summary_rounding_matches_torch():
    """bf16 summaries: fp32 first, then nearest bf16 with ties to even. torch's
    own fp32 -> bf16 conversion is an independent implementation of that
    second rounding."""
    import torch
    rng = np.random.default_rng(5)
    means = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-6, 6, 20000),
                            rng.standard_normal(1000) * 1e-30])
    got = O.stored_summaries(means, "bf16")
    ref = torch.from_numpy(means.astype(np.float32)).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_summary_rounding_hand_cases():
    def bits(*u):
        return np.array(u, dtype=np.uint32).view(np.float32).astype(np.float64)
    got = O.stored_summaries(bits(0x3F808000, 0x3F818000, 0x3F808001, 0xBF808000,
                                  0x3F810000, 0x3FFFFFFF, 0x00000000), "bf16").view(np.uint32)
    # halfway -> even (down), halfway -> even (up), above half -> up, sign
    # kept, exact values unchanged, carry into the exponent, zero
    assert got.tolist() == [0x3F800000, 0x3F820000, 0x3F810000, 0xBF800000,
                            0x3F810000, 0x40000000, 0x00000000]
    # the first rounding is to fp32: an fp64 mean just above a bf16 halfway
    # point that rounds to the halfway fp32 value then ties to even
    m = np.array([1.00390625 + 2.0 ** -40])
    assert O.stored_summaries(m, "f32")[0] == np.float32(1.00390625)
    assert O.stored_summaries(m, "bf16")[0] == np.float32(1.0)



# OCP FP8 E4M3 (4 exponent bits, bias 7, 3 fraction bits; largest finite 448,
# smallest subnormal 2^-9). Each expected value is worked out by hand from the
# grid: a value in [2^e, 2^(e+1)) has quantum 2^(e-3), e >= -6.
E4M3_HAND = [
    (1.0, 1.0), (0.1, 0.1015625),            # 0.1 = 12.8 quanta of 2^-7 -> 13
    (0.3, 0.3125),                           # 9.6 quanta of 2^-5 -> 10
    (1.0625, 1.0), (1.1875, 1.25),           # ties: 8.5 -> 8, 9.5 -> 10 (even)
    (-1.1875, -1.25), (1.9375, 2.0),         # sign kept; 15.5 -> 16 carries
    (248.0, 256.0), (240.0, 240.0),          # 15.5 quanta of 16 -> 16; exact
    (448.0, 448.0), (460.0, 448.0), (1000.0, 448.0), (-3.0e5, -448.0),  # saturation
    (2.0 ** -6, 2.0 ** -6), (2.0 ** -9, 2.0 ** -9),   # smallest normal, subnormal
    (2.0 ** -10, 0.0),                       # half a subnormal quantum: tie -> 0
    (3 * 2.0 ** -10, 2.0 ** -8),             # 1.5 quanta -> 2
    (3.5 * 2.0 ** -9, 2.0 ** -7),            # 3.5 quanta -> 4 (even)
    (0.0, 0.0),
]


def test_e4m3_rounding_hand_cases():
    x = np.array([a for a, _ in E4M3_HAND], dtype=np.float32)
    got = O.e4m3_round(x)
    assert got.dtype == np.float32
    assert got.tolist() == [b for _, b in E4M3_HAND]


def test_e4m3_rounding_matches_torch_in_range():
    """torch's float32 -> float8_e4m3fn conversion (nearest, ties to even) is
    an independent implementation of the same rounding for |x| <= 448 (beyond
    it torch does not saturate)."""
    import torch
    rng = np.random.default_rng(9)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-4, 3, 20000),
                        rng.uniform(-448, 448, 5000),
                        (rng.integers(-64, 64, 2000) * 2.0 ** -10)]).astype(np.float32)
    x = x[np.abs(x) <= 448]
    got = O.e4m3_round(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy()
    np.testing.assert_array_equal(got, ref)


def test_e4m3_rounding_idempotent_and_monotone():
    rng = np.random.default_rng(10)
    x = np.sort(rng.standard_normal(50000).astype(np.float32) * 30)
    y = O.e4m3_round(x)
    np.testing.assert_array_equal(O.e4m3_round(y), y)
    assert np.all(np.diff(y.astype(np.float64)) >= 0)
    # at most 256 distinct codes (fewer here: one sign of zero, no NaN)
    assert len(np.unique(y)) <= 255


def test_fp8_summaries_round_through_fp32():
    """fp8 summaries take the fp32 rounding first: an fp64 mean just above the
    E4M3 halfway point 1.0625 rounds to exactly 1.0625 in fp32, which then
    ties to the even neighbour 1.0 (rounding the fp64 value directly would
    give 1.125)."""
    m = np.array([1.0625 + 2.0 ** -40])
    assert O.stored_summaries(m, "f32")[0] == np.float32(1.0625)
    assert O.stored_summaries(m, "fp8")[0] == np.float32(1.0)
    assert O.e4m3_round(np.array([1.0625 + 2.0 ** -20], dtype=np.float32))[0] == np.float32(1.125)


# ---------------------------------------------------------------- page masses
def _summ(rows):
    return np.asarray(rows, dtype=np.float64).astype(np.float32)


def test_masses_ordered_golden():
    g = GOLD["masses_ordered"]
    summ = _summ([[math.log(p + 1), 0.0] for p in range(4)])
    counts = O.page_token_counts(g["seq_len"], g["page_size"])
    m = O.page_masses(np.array(g["q"]), summ, counts, g["scale"])
    np.testing.assert_allclose(m, g["expected_masses"], rtol=0, atol=g["mass_tol"])
    for case in g["selections"]:
        got = O.select_pages(np.array(g["q"]), summ, g["seq_len"], g["page_size"],
                             g["scale"], case["gamma"])
        assert got.tolist() == case["pages"], case


def test_masses_token_weighted_and_tie_rule_golden():
    g = GOLD["masses_token_weighted_ties"]
    summ = _summ(np.zeros((3, 2)))
    counts = O.page_token_counts(g["seq_len"], g["page_size"])
    assert counts.tolist() == [16, 16, 8]
    m = O.page_masses(np.array(g["q"]), summ, counts, g["scale"])
    np.testing.assert_allclose(m, g["expected_masses"], rtol=0, atol=g["mass_tol"])
    for case in g["selections"]:
        got = O.select_pages(np.array(g["q"]), summ, g["seq_len"], g["page_size"],
                             g["scale"], case["gamma"])
        assert got.tolist() == case["pages"], case


def test_masses_group_sum_golden():
    g = GOLD["masses_group_sum"]
    q = np.array([[math.log(3.0), 0.0], [0.0, math.log(2.0)]])
    summ = _summ([[1.0, 0.0], [0.0, 1.0]])
    counts = O.page_token_counts(g["seq_len"], g["page_size"])
    m = O.page_masses(q, summ, counts, g["scale"])
    np.testing.assert_allclose(m, g["expected_masses"], rtol=0, atol=g["mass_tol"])
    for case in g["selections"]:
        got = O.select_pages(q, summ, g["seq_len"], g["page_size"], g["scale"], case["gamma"])
        assert got.tolist() == case["pages"], case


def test_page_size_one_single_head_is_exact_softmax():
    """With one-token pages and G = 1 the page mean is the key itself and the
    estimated mass is exactly the attention probability."""
    rng = np.random.default_rng(3)
    for L, D in [(1, 4), (7, 8), (50, 16)]:
        K = rng.standard_normal((L, D))
        q = rng.standard_normal((1, D))
        scale = 1.0 / math.sqrt(D)
        m = O.page_masses(q, O.page_means(K, L, 1), np.ones(L), scale)
        ref = torch.softmax(scale * (torch.from_numpy(q) @ torch.from_numpy(K).T), dim=-1)
        np.testing.assert_allclose(m, ref.numpy()[0], rtol=1e-13, atol=1e-15)


def test_masses_normalised_and_shift_invariant_single_head():
    rng = np.random.default_rng(4)
    summ = rng.standard_normal((30, 8)).astype(np.float32)
    q = rng.standard_normal((1, 8))
    counts = O.page_token_counts(30 * 16 - 5, 16)
    m = O.page_masses(q, summ, counts, 0.3)
    assert abs(m.sum() - 1.0) < 1e-14
    # a logit offset common to all pages cancels: add c * q/|q|^2 to every summary
    shift = (q[0] / np.dot(q[0], q[0])) * 2.0
    m2 = O.page_masses(q, summ.astype(np.float64) + shift, counts, 0.3)
    np.testing.assert_allclose(m2, m, rtol=1e-6)


def test_top_p_special_case_matches_sorted_cumsum_of_softmax():
    """Page size 1 and G = 1: coverage is nucleus (top-p) selection over exact
    attention probabilities; compare with a sort + cumsum of torch.softmax."""
    rng = np.random.default_rng(5)
    for trial in range(20):
        L = int(rng.integers(1, 200))
        K = rng.standard_normal((L, 8)) * rng.uniform(0.1, 3.0)
        q = rng.standard_normal((1, 8))
        gamma = float(rng.uniform(0.05, 0.999))
        p = torch.softmax(torch.from_numpy(q @ K.T)[0], dim=0)
        vals, idx = torch.sort(p, descending=True, stable=True)
        c = torch.cumsum(vals, 0)
        k = int((c < gamma).sum().item()) + 1
        k = min(k, L)
        expect = sorted(idx[:k].tolist())
        got = O.select_pages(q, O.page_means(K, L, 1), L, 1, 1.0, gamma)
        # the library sums in its own order; only a cut within rounding of
        # gamma may differ
        if got.tolist() != expect:
            assert abs(float(c[k - 1]) - gamma) < 1e-12 or abs(float(c[max(k - 2, 0)]) - gamma) < 1e-12


# -------------------------------------------------------------- coverage rule
def test_inclusive_reach_golden():
    g = GOLD["inclusive_reach"]
    got = O.coverage_select(np.array(g["masses"]), g["gamma"])
    assert got.tolist() == g["pages"]


def _brute_force(m, gamma):
    P = len(m)
    for k in range(1, P + 1):
        best = None
        for sub in itertools.combinations(range(P), k):
            s = sum(m[i] for i in sub)
            if s >= gamma - 1e-12 and (best is None or s > best[0] + 1e-15):
                best = (s, sub)
        if best is not None:
            return k, sorted(best[1])
    return P, list(range(P))


@pytest.mark.parametrize("seed", range(12))
def test_coverage_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    P = int(rng.integers(1, 13))
    w = rng.exponential(1.0, P) ** rng.uniform(0.5, 4.0)
    m = w / w.sum()
    for gamma in [0.1, 0.5, 0.8, 0.9, 0.97, 0.999]:
        got = O.coverage_select(m, gamma)
        k, best = _brute_force(m, gamma)
        assert len(got) == k
        assert got.tolist() == best
        assert m[got].sum() >= gamma - 1e-12
        # minimality: dropping the smallest kept page falls below gamma
        assert m[got].sum() - m[got].min() < gamma


@pytest.mark.parametrize("seed", range(6))
def test_coverage_nested_in_gamma(seed):
    rng = np.random.default_rng(200 + seed)
    m = rng.dirichlet(np.full(300, 0.3))
    prev = set()
    for gamma in np.linspace(0.01, 1.0, 40):
        cur = set(O.coverage_select(m, float(gamma)).tolist())
        assert prev <= cur
        prev = cur
    assert prev == set(range(300))


def test_gamma_one_keeps_underflowing_pages():
    m = np.array([1.0, 0.0, 0.0, 1e-300])
    assert O.coverage_select(m, 1.0).tolist() == [0, 1, 2, 3]
    assert O.coverage_select(m / m.sum(), 0.999).tolist() == [0]


def test_exact_ties_break_by_index():
    m = np.full(10, 0.1)
    assert O.coverage_select(m, 0.25).tolist() == [0, 1, 2]
    m2 = np.array([0.05, 0.3, 0.05, 0.3, 0.3])
    assert O.coverage_select(m2, 0.65).tolist() == [1, 3, 4]
    assert O.coverage_select(m2, 0.92).tolist() == [0, 1, 3, 4]


# ------------------------------------------------------------------ attention
def _sdpa(q, K, V, scale, mask=None):
    tq = torch.from_numpy(q)[None, :, None, :]                 # [1, G, 1, D]
    tk = torch.from_numpy(K)[None, None].expand(1, q.shape[0], -1, -1).contiguous()
    tv = torch.from_numpy(V)[None, None].expand(1, q.shape[0], -1, -1).contiguous()
    am = None if mask is None else torch.from_numpy(mask)[None, None, None, :]
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=am, scale=scale)
    return out[0, :, 0, :].numpy()


def test_dense_attention_equals_sdpa():
    rng = np.random.default_rng(6)
    for L, G, D in [(1, 1, 8), (35, 2, 16), (300, 4, 32)]:
        K = rng.standard_normal((L, D))
        V = rng.standard_normal((L, D))
        q = rng.standard_normal((G, D))
        scale = 1.0 / math.sqrt(D)
        P = O.num_pages(L, 16)
        got = O.sparse_attention(q, K, V, np.arange(P), L, 16, scale)
        np.testing.assert_allclose(got, _sdpa(q, K, V, scale), rtol=1e-12, atol=1e-13)


def test_sparse_attention_equals_masked_sdpa():
    rng = np.random.default_rng(7)
    L, G, D = 200, 4, 16
    K = rng.standard_normal((L, D)) * 2.0
    V = rng.standard_normal((L, D))
    q = rng.standard_normal((G, D))
    P = O.num_pages(L, 16)
    for trial in range(5):
        pages = np.sort(rng.choice(P, size=int(rng.integers(1, P + 1)), replace=False))
        mask = np.zeros(L, dtype=bool)
        mask[O.page_tokens(pages, L, 16)] = True
        got = O.sparse_attention(q, K, V, pages, L, 16, 0.37)
        np.testing.assert_allclose(got, _sdpa(q, K, V, 0.37, mask), rtol=1e-12, atol=1e-13)


def test_attention_uniform_golden():
    g = GOLD["attention_uniform"]
    L = g["seq_len"]
    K = np.ones((L, 2))
    V = np.stack([np.arange(L, dtype=np.float64), np.ones(L)], axis=1)
    got = O.sparse_attention(np.array([[0.3, -0.7]]), K, V, np.array(g["pages"]), L,
                             g["page_size"], 1.0)
    np.testing.assert_allclose(got, g["expected"], rtol=1e-15)


def test_partials_of_any_partition_combine_to_sdpa():
    rng = np.random.default_rng(8)
    L, G, D = 333, 4, 8
    K = rng.standard_normal((L, D)) * 3.0
    V = rng.standard_normal((L, D))
    q = rng.standard_normal((G, D))
    P = O.num_pages(L, 16)
    pages = np.sort(rng.choice(P, size=15, replace=False))
    mask = np.zeros(L, dtype=bool)
    mask[O.page_tokens(pages, L, 16)] = True
    ref = _sdpa(q, K, V, 0.5, mask)
    for trial in range(5):
        cuts = np.sort(rng.choice(np.arange(1, len(pages)), size=3, replace=False))
        parts = [O.attention_partial(q, K, V, chunk, L, 16, 0.5)
                 for chunk in np.split(pages, cuts)]
        parts.append(O.attention_partial(q, K, V, np.array([], dtype=np.int64), L, 16, 0.5))
        np.testing.assert_allclose(O.combine_partials(parts), ref, rtol=1e-12, atol=1e-13)


def test_step_appends_before_select_and_attend():
    """The appended token is part of the context the step attends over."""
    rng = np.random.default_rng(9)
    D = 8
    K = rng.standard_normal((40, D))
    V = rng.standard_normal((40, D))
    h = O.OracleHead(K, V, 32, 16)
    q = rng.standard_normal((2, D))
    pages, out = h.step(q, K[32], V[32], 0.4, 1.0)
    assert pages.tolist() == [0, 1, 2]
    np.testing.assert_allclose(out, _sdpa(q, K[:33], V[:33], 0.4), rtol=1e-12, atol=1e-13)


def test_band_helpers():
    m = np.array([0.5, 0.25, 0.25])
    band = set(O.boundary_band_pages(m, 0.75).tolist())
    assert band == {1, 2}   # ranked 0, 1, 2; C = 0.5, 0.75, 1.0
    assert set(O.near_tie_pages(m, np.array([0, 1])).tolist()) == {1, 2}


# ------------------------------------------------------- top-k and top-delta
def test_topk_is_the_heaviest_subset_brute_force():
    """For distinct masses the k-subset of largest total mass is unique and
    must be topk_select's set (enumerated over all subsets)."""
    import itertools
    rng = np.random.default_rng(12)
    for P in range(1, 8):
        for _ in range(5):
            m = rng.random(P)
            for k in range(0, P + 2):
                kk = min(k, P)
                best = max(itertools.combinations(range(P), kk), key=lambda c: sum(m[list(c)]))
                assert O.topk_select(m, k).tolist() == sorted(best)


def test_topk_ties_and_bounds():
    m = np.array([0.5, 0.2, 0.5, 0.2, 0.2, 0.9])
    assert O.topk_select(m, 1).tolist() == [5]
    assert O.topk_select(m, 2).tolist() == [0, 5]          # of the tied 0.5s, page 0 first
    assert O.topk_select(m, 3).tolist() == [0, 2, 5]
    assert O.topk_select(m, 4).tolist() == [0, 1, 2, 5]    # of the tied 0.2s, page 1 first
    assert O.topk_select(m, 6).tolist() == list(range(6))
    assert O.topk_select(m, 100).tolist() == list(range(6))
    assert O.topk_select(m, 0).tolist() == []


def test_topdelta_special_cases_and_nesting():
    rng = np.random.default_rng(13)
    m = rng.random(50) ** 4
    assert O.topdelta_select(m, 0.0).tolist() == list(range(50))
    assert O.topdelta_select(m, 1.0).tolist() == [int(np.argmax(m))]
    prev = None
    for d in (0.9, 0.5, 0.1, 0.01, 1e-6):                   # smaller delta keeps a superset
        cur = set(O.topdelta_select(m, d).tolist())
        if prev is not None:
            assert prev <= cur
        prev = cur
    # scaling every mass by a power of two changes nothing (exact in fp64)
    for d in (0.3, 0.05):
        assert O.topdelta_select(m * 2.0 ** 37, d).tolist() == O.topdelta_select(m, d).tolist()


def test_topdelta_golden_and_ties_at_the_threshold():
    m = np.array([1.0, 0.5, 0.25, 0.5, 0.125])
    assert O.topdelta_select(m, 0.5).tolist() == [0, 1, 3]   # 0.5 >= 0.5 * 1.0 is kept
    assert O.topdelta_select(m, 0.26).tolist() == [0, 1, 3]
    assert O.topdelta_select(m, 0.25).tolist() == [0, 1, 2, 3]
    assert O.topdelta_select(np.array([2.0, 2.0, 1.0]), 1.0).tolist() == [0, 1]


# ------------------------------------------- the rule dispatcher and OracleHead
def _ordered_summaries(extra_rows=0):
    """Summaries of masses_ordered (kbar_p = (ln(p+1), 0)), optionally with
    extra rows past the request's pages that must be ignored."""
    rows = [[math.log(p + 1), 0.0] for p in range(4)] + [[50.0, 50.0]] * extra_rows
    return _summ(rows)


def test_select_pages_rule_golden():
    """Each rule, reached through the dispatcher, on hand-derived masses. A
    mis-mapped rule or a wrongly cast parameter gives a different list."""
    g = GOLD["masses_ordered"]
    q = np.array(g["q"])
    for case in GOLD["rule_dispatch"]["ordered"]:
        got = O.select_pages_rule(q, _ordered_summaries(), g["seq_len"], g["page_size"],
                                  g["scale"], case["rule"], case["param"])
        assert got.tolist() == case["pages"], case
    gt = GOLD["masses_token_weighted_ties"]
    for case in GOLD["rule_dispatch"]["token_weighted_ties"]:
        got = O.select_pages_rule(np.array(gt["q"]), _summ(np.zeros((3, 2))), gt["seq_len"],
                                  gt["page_size"], gt["scale"], case["rule"], case["param"])
        assert got.tolist() == case["pages"], case
    with pytest.raises(ValueError):
        O.select_pages_rule(q, _ordered_summaries(), 64, 16, 1.0, "nucleus", 0.5)


def test_select_pages_rule_ignores_rows_past_the_request():
    """Summary rows beyond P = ceil(L / page_size) (a pool with capacity for
    later tokens) take no part, exactly as in select_pages."""
    g = GOLD["masses_ordered"]
    q = np.array(g["q"])
    for case in GOLD["rule_dispatch"]["ordered"]:
        got = O.select_pages_rule(q, _ordered_summaries(extra_rows=3), g["seq_len"],
                                  g["page_size"], g["scale"], case["rule"], case["param"])
        assert got.tolist() == case["pages"], case


def test_oracle_head_select_rule_golden():
    """OracleHead.select_rule on tokens whose page means are the
    masses_ordered summaries: every key of page p is (ln(p+1), 0), so the
    maintained means (and, for the coverage rule, OracleHead.select) give the
    hand-derived lists. The head is built from 63 tokens and the 64th is
    appended, so the incremental tail mean takes part too."""
    g = GOLD["masses_ordered"]
    keys = np.repeat(np.array([[math.log(p + 1), 0.0] for p in range(4)]), 16, axis=0)
    vals = np.zeros_like(keys)
    for sdt in ("f32", "bf16"):
        h = O.OracleHead(keys, vals, 63, 16, summary_dtype=sdt)
        h.append(keys[63], vals[63])
        assert h.seq_len == 64
        for case in GOLD["rule_dispatch"]["ordered"]:
            got = h.select_rule(np.array(g["q"]), g["scale"], case["rule"], case["param"])
            assert got.tolist() == case["pages"], (sdt, case)
        cov = h.select(np.array(g["q"]), g["scale"], 0.5)
        assert cov.tolist() == h.select_rule(np.array(g["q"]), g["scale"], "coverage", 0.5).tolist()
