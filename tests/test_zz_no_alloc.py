"""moira_select_pages_noalloc (selection with the library's static scratch in
place of a caller workspace) against moira_select_pages and the oracle.

Two calls in a row on one GPU, the second with a smaller input (fewer
segments and pages, so the scratch holds a larger layout's leftovers): each
must give exactly the lists and lengths of moira_select_pages on the same
inputs (index work: bit-exact), and those lists must match the fp64 oracle.
The larger input runs once more afterwards, on the smaller one's leftovers.
"""

import numpy as np
import pytest
import torch

from gpu_util import (Device, compare_lists, make_problem, note, oracle_heads, oracle_masses,
                      q_group)
from long_context_sparse_summary_amd import moira as M

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    M.load()
    torch.cuda.set_device(0)


def _prepare(pb):
    dv = Device(pb)
    dv.rebuild_summaries()
    q, kn, vn = dv.step_inputs(0)
    M.advance_seq_lens(dv.shape, dv.lens, dv.buf.status)
    M.append_kv(dv.shape, kn, vn, dv.k_pool, dv.v_pool, dv.summ, dv.table, dv.lens, dv.buf.status)
    return dv, q


def _check(dv, q, gamma):
    pb = dv.pb
    # the existing entry point, twice on its own workspace (the second call
    # bins against the first call's reference key)
    for _ in range(2):
        M.select_pages(dv.shape, q, dv.summ, dv.table, dv.lens, gamma, pb.scale, dv.buf.workspace,
                       dv.buf.page_lists, dv.buf.list_lens, dv.buf.status)
    torch.cuda.synchronize()
    ref_lists = dv.buf.page_lists.clone()
    ref_lens = dv.buf.list_lens.clone()
    pl = torch.full_like(dv.buf.page_lists, -7)
    ll = torch.full_like(dv.buf.list_lens, -7)
    M.select_pages_noalloc(dv.shape, q, dv.summ, dv.table, dv.lens, gamma, pb.scale, pl, ll,
                           dv.buf.status)
    torch.cuda.synchronize()
    assert dv.status() == 0
    assert torch.equal(ll, ref_lens)
    for s in range(ll.numel()):
        n = int(ll[s])
        assert torch.equal(pl[s, :n], ref_lists[s, :n]), s
    heads = oracle_heads(pb)
    got = [pl[s, :int(ll[s])].cpu().numpy() for s in range(ll.numel())]
    for r in range(pb.B):
        for j in range(pb.H):
            h = heads[(r, j)]
            h.append(pb.k_tok[r][j, pb.lens[r]].float().numpy(), pb.v_tok[r][j, pb.lens[r]].float().numpy())
            qg = q_group(pb, 0, r, j)
            compare_lists(got[r * pb.H + j], h.select(qg, pb.scale, gamma),
                          oracle_masses(h, qg, pb.scale), gamma, f"noalloc r{r} j{j}")


def test_noalloc_matches_select_pages_on_consecutive_calls():
    big = make_problem(2, 8, 4, 128, [20000, 5000], seed=91, hot=40)
    small = make_problem(1, 4, 4, 128, [3000], seed=92, hot=10)
    dv_big, q_big = _prepare(big)
    dv_small, q_small = _prepare(small)
    for name, dv, q, gamma in [("big", dv_big, q_big, 0.99), ("small", dv_small, q_small, 0.9),
                               ("big again", dv_big, q_big, 0.98)]:
        note(f"[noalloc] {name}: B={dv.pb.B} H={dv.pb.H} lens={dv.pb.lens} gamma={gamma}")
        _check(dv, q, gamma)


def test_noalloc_gamma_one_and_scratch_limit():
    small = make_problem(1, 4, 4, 128, [3000], seed=93, hot=10)
    dv, q = _prepare(small)
    pl = torch.full_like(dv.buf.page_lists, -7)
    ll = torch.full_like(dv.buf.list_lens, -7)
    M.select_pages_noalloc(dv.shape, q, dv.summ, dv.table, dv.lens, 1.0, small.scale, pl, ll,
                           dv.buf.status)
    torch.cuda.synchronize()
    P = (small.lens[0] + 1 + 15) // 16
    assert ll.tolist() == [P] * 4
    assert all(pl[s, :P].tolist() == list(range(P)) for s in range(4))
    # a shape whose workspace exceeds the static scratch is refused before any launch
    huge = M.make_shape(4096, 1, 4, 128, 16384, 1 << 20)
    assert M.select_workspace_bytes(huge) > 32 << 20
    with pytest.raises(M.MoiraError) as e:
        M.select_pages_noalloc(huge, q, dv.summ, dv.table, dv.lens, 0.9, small.scale, pl, ll)
    assert e.value.code == -8


@pytest.mark.parametrize("sdt", [torch.bfloat16, torch.float8_e4m3fn], ids=["bf16", "fp8"])
def test_noalloc_low_precision_summaries(sdt):
    """The same with bf16 and E4M3 page summaries (their own scoring
    kernels), on two calls in a row of different shapes."""
    a = make_problem(1, 8, 4, 128, [9000], seed=94, hot=30, sum_dtype=sdt)
    b = make_problem(2, 2, 8, 128, [700, 4100], seed=95, hot=12, sum_dtype=sdt)
    for name, pb, gamma in [("a", a, 0.99), ("b", b, 0.95)]:
        note(f"[noalloc {sdt}] {name}: B={pb.B} H={pb.H} lens={pb.lens} gamma={gamma}")
        dv, q = _prepare(pb)
        _check(dv, q, gamma)
