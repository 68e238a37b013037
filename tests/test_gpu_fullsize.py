"""Parity at the full workload sizes, in the launch configuration bench.py
times (256 attention workgroups), on sampled (request, KV head) pairs that the
fp64 oracle can afford one at a time.

Each case draws one layer of a workload at its real shape on the GPU, builds
the page summaries, then runs two decode steps (advance, append, select,
attend, combine) through the C ABI. The first step's selection runs the exact
fallback (no reference key yet) and the second uses the band histogram. For
each sampled pair the oracle gets the same prefill tokens, queries and
appended tokens (read from the generator's tensors before the GPU touches
them) and must agree: lists exactly outside the documented boundary bands,
outputs within 2e-3 + 1e-2|ref| on the GPU's own lists.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_close, compare_lists, note
from long_context_sparse_summary_amd import moira as M
from long_context_sparse_summary_amd import workloads as W

pytestmark = pytest.mark.gpu

STEPS = 2
NUM_WORKGROUPS = 256

CASES = [
    # workload, layer, gamma, sampled (request, kv_head) pairs[, summary dtype]
    (3, 0, 0.99, [(0, 0), (0, 5)]),
    (3, 0, 0.99, [(0, 0), (0, 3)], torch.bfloat16),
    (3, 21, 0.98, [(0, 3)]),
    (3, 7, 1.0, [(0, 6)]),
    (2, 0, 0.99, [(0, 1), (0, 7)]),
    (4, 0, 0.99, [(0, 0), (17, 4), (31, 7)]),
    (5, 0, 0.99, [(0, 0), (0, 1), (63, 6)]),
    (5, 0, 1.0, [(9, 2)]),
]


@pytest.mark.parametrize("case", CASES, ids=[f"cfg{c[0]}-l{c[1]}-g{c[2]}" + ("-bf16sum" if len(c) > 4 else "")
                                             for c in CASES])
def test_full_size_sampled(case):
    cfg_id, layer, gamma, sample = case[:4]
    sdt = case[4] if len(case) > 4 else torch.float32
    scode = "bf16" if sdt == torch.bfloat16 else "f32"
    note(f"[fullsize] cfg {cfg_id} layer {layer} gamma {gamma} sample {sample} summaries {scode}")
    cfg = W.shrink(W.get_config(cfg_id), steps=STEPS)
    wl = W.make_workload(cfg, device="cpu", extra_steps=2)
    dev = torch.device("cuda")
    ld = W.make_layer(cfg, wl, layer, device=dev)
    B, H, G, D = cfg.batch, cfg.num_kv_heads, cfg.group, cfg.head_dim
    scale = cfg.scale_f32

    # the oracle's inputs, straight from the generator's tensors
    heads = {}
    for r, j in sample:
        L0 = cfg.context[r] - 1
        K = W.head_tokens(ld.k_pool, wl.block_table, r, j, L0).double().cpu().numpy()
        V = W.head_tokens(ld.v_pool, wl.block_table, r, j, L0).double().cpu().numpy()
        heads[(r, j)] = O.OracleHead(K, V, L0, 16, capacity=L0 + STEPS, summary_dtype=scode)
    qs = ld.q.double().cpu().numpy()
    kn = ld.k_new.double().cpu().numpy()
    vn = ld.v_new.double().cpu().numpy()

    shape = M.make_shape(B, H, G, D, wl.max_pages, wl.num_phys_pages, cfg.torch_kv_dtype(),
                         cfg.torch_q_dtype(), sum_dtype=sdt)
    table = wl.block_table.to(dev)
    lens = wl.prefill_lens.to(dev)
    buf = M.StepBuffers.allocate(shape, NUM_WORKGROUPS, dev)
    buf.out.fill_(float("nan"))
    summ = torch.full((wl.num_phys_pages, H, D), float("nan"), dtype=sdt, device=dev)
    M.page_summaries(shape, ld.k_pool, table, lens, summ, M.SUM_ALL, buf.status)

    exceptions = 0
    for t in range(STEPS):
        note(f"[fullsize] cfg {cfg_id} step {t}")
        M.advance_seq_lens(shape, lens, buf.status)
        M.layer_step(buf, ld.q[t].contiguous(), ld.k_new[t].contiguous(), ld.v_new[t].contiguous(),
                     ld.k_pool, ld.v_pool, summ, table, lens, gamma, scale)
        torch.cuda.synchronize()
        assert int(buf.status.item()) == 0
        lists = buf.page_lists.cpu().numpy()
        ll = buf.list_lens.cpu().numpy()
        out = buf.out.cpu().numpy()
        for r, j in sample:
            h = heads[(r, j)]
            qg = qs[t, r, j * G:(j + 1) * G]
            pages, _ = h.step(qg, kn[t, r, j], vn[t, r, j], scale, gamma)
            got = lists[r * H + j, :ll[r * H + j]].copy()
            masses = O.page_masses(qg, O.stored_summaries(h.means, scode),
                                   O.page_token_counts(h.seq_len, 16), scale)
            exceptions += compare_lists(got, pages, masses, gamma, f"t{t} r{r} j{j}")
            if gamma >= 1.0:
                assert len(got) == h.means.shape[0]
            ref = h.attend(qg, got, scale)
            assert_close(out[r, j * G:(j + 1) * G], ref, f"t{t} r{r} j{j}")
    note(f"[fullsize] cfg {cfg_id}: {exceptions} boundary-band exceptions")
    del ld, summ, buf
    torch.cuda.empty_cache()


def _run_layer(cfg, wl, layer, steps, check_steps, sample, sdt=torch.float32):
    """Run `steps` decode steps of one layer of a full-size workload through
    the C ABI and compare the sampled (request, KV head) pairs with the
    oracle at `check_steps` (the oracle appends at every step)."""
    dev = torch.device("cuda")
    ld = W.make_layer(cfg, wl, layer, device=dev)
    B, H, G, D = cfg.batch, cfg.num_kv_heads, cfg.group, cfg.head_dim
    scale = cfg.scale_f32
    scode = "bf16" if sdt == torch.bfloat16 else "f32"
    heads = {}
    for r, j in sample:
        L0 = cfg.context[r] - 1
        K = W.head_tokens(ld.k_pool, wl.block_table, r, j, L0).double().cpu().numpy()
        V = W.head_tokens(ld.v_pool, wl.block_table, r, j, L0).double().cpu().numpy()
        heads[(r, j)] = O.OracleHead(K, V, L0, 16, capacity=L0 + steps, summary_dtype=scode)
    qs = ld.q.double().cpu().numpy()
    kn = ld.k_new.double().cpu().numpy()
    vn = ld.v_new.double().cpu().numpy()
    shape = M.make_shape(B, H, G, D, wl.max_pages, wl.num_phys_pages, cfg.torch_kv_dtype(),
                         cfg.torch_q_dtype(), sum_dtype=sdt)
    table = wl.block_table.to(dev)
    lens = wl.prefill_lens.to(dev)
    buf = M.StepBuffers.allocate(shape, NUM_WORKGROUPS, dev)
    summ = torch.full((wl.num_phys_pages, H, D), float("nan"), dtype=sdt, device=dev)
    M.page_summaries(shape, ld.k_pool, table, lens, summ, M.SUM_ALL, buf.status)
    exceptions = 0
    for t in range(steps):
        M.advance_seq_lens(shape, lens, buf.status)
        M.layer_step(buf, ld.q[t].contiguous(), ld.k_new[t].contiguous(), ld.v_new[t].contiguous(),
                     ld.k_pool, ld.v_pool, summ, table, lens, 0.99, scale)
        if t not in check_steps:
            for r, j in sample:
                heads[(r, j)].append(kn[t, r, j], vn[t, r, j])
            continue
        torch.cuda.synchronize()
        assert int(buf.status.item()) == 0
        lists = buf.page_lists.cpu().numpy()
        ll = buf.list_lens.cpu().numpy()
        out = buf.out.cpu().numpy()
        for r, j in sample:
            h = heads[(r, j)]
            qg = qs[t, r, j * G:(j + 1) * G]
            pages, _ = h.step(qg, kn[t, r, j], vn[t, r, j], scale, 0.99)
            got = lists[r * H + j, :ll[r * H + j]].copy()
            masses = O.page_masses(qg, O.stored_summaries(h.means, scode),
                                   O.page_token_counts(h.seq_len, 16), scale)
            exceptions += compare_lists(got, pages, masses, 0.99, f"l{layer} t{t} r{r} j{j}")
            assert_close(out[r, j * G:(j + 1) * G], h.attend(qg, got, scale), f"l{layer} t{t} r{r} j{j}")
    del ld, summ, buf
    torch.cuda.empty_cache()
    return exceptions


def test_cfg3_every_layer_first_step():
    """The 128k workload's 32 layers (each its own seeded profile) at the
    first decode step, one sampled KV head per layer."""
    cfg = W.shrink(W.get_config(3), steps=1)
    wl = W.make_workload(cfg, device="cpu", extra_steps=2)
    exceptions = 0
    for layer in range(cfg.layers):
        note(f"[fullsize cfg3 layers] layer {layer}")
        exceptions += _run_layer(cfg, wl, layer, 1, {0}, [(0, layer % cfg.num_kv_heads)])
    note(f"[fullsize cfg3 layers] {exceptions} boundary-band exceptions")


def test_cfg3_later_steps():
    """One layer of the 128k workload over 18 steps (new tail pages open and
    fill), checked at steps 0, 1, 2 and 17."""
    cfg = W.shrink(W.get_config(3), steps=18)
    wl = W.make_workload(cfg, device="cpu", extra_steps=2)
    note("[fullsize cfg3 steps] layer 3, steps 0..17")
    ex = _run_layer(cfg, wl, 3, 18, {0, 1, 2, 17}, [(0, 2), (0, 6)])
    note(f"[fullsize cfg3 steps] {ex} boundary-band exceptions")
