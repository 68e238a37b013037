"""Parity at the full workload sizes, in the launch configuration bench.py
times (256 attention workgroups), for EVERY (request, KV head) pair.

Each case draws a workload at its real shape on the GPU, builds the page
summaries, then runs decode steps (advance, append, select, attend, combine)
through the C ABI. The first step's selection runs the exact fallback (no
reference key yet); later steps use the band histogram. At the checked steps
the GPU's lists and outputs are copied out; afterwards the fp64 oracle replays
every (request, KV head) from the same prefill tokens, queries and appended
tokens (read from the generator's tensors, never from the HIP path) and must
agree: lists exactly outside the documented bands (and a differing list must
itself be a correct answer), outputs within 2e-3 + 1e-2|ref| on the GPU's own
lists.

Coordinate 0 of every value vector is replaced by the token's position
divided by the final length (bf16), so that each output carries one O(1)
coordinate, the weighted mean position, whose error the absolute tolerance
can see even where the weights are nearly uniform over ~65k tokens.

The 128k workload also runs as bench.py runs it: all 32 layers resident, the
whole step (input staging, advance, 32 x (append+select, attend, combine))
captured in one HIP graph and replayed, checked at replays 0, 1, 2, 17, 50
and 99.
"""

import numpy as np
import pytest
import torch

import oracle as O
from gpu_util import assert_close, compare_lists, note
from long_context_sparse_summary_amd import moira as M
from long_context_sparse_summary_amd import workloads as W

pytestmark = pytest.mark.gpu

NUM_WORKGROUPS = 256


def _position_code_values(cfg, wl, ld, steps):
    """Coordinate 0 of every value = position / (final length), in place."""
    dev = ld.v_pool.device
    for r in range(cfg.batch):
        L0 = cfg.context[r] - 1
        Lf = float(L0 + steps)
        P0 = (L0 + 15) // 16
        phys = wl.block_table[r, :P0].to(device=dev, dtype=torch.long)
        pos = torch.arange(P0 * 16, device=dev, dtype=torch.float32).view(P0, 1, 16) / Lf
        ld.v_pool[phys, :, :, 0] = pos.expand(P0, cfg.num_kv_heads, 16).to(ld.v_pool.dtype)
        if L0 < P0 * 16:   # the tail slots past the prefill hold no token yet
            tail = phys[-1]
            ld.v_pool[tail, :, L0 - (P0 - 1) * 16:, 0] = 0
        t = torch.arange(ld.v_new.shape[0], device=dev, dtype=torch.float32)
        ld.v_new[:, r, :, 0] = ((L0 + t) / Lf)[:, None].expand(-1, cfg.num_kv_heads).to(ld.v_new.dtype)


class LayerRun:
    """One layer of a workload on the GPU, stepped eagerly through the ABI."""

    def __init__(self, cfg, wl, layer, sdt=torch.float32, steps=1):
        dev = torch.device("cuda")
        self.cfg, self.wl, self.layer = cfg, wl, layer
        self.ld = W.make_layer(cfg, wl, layer, device=dev)
        _position_code_values(cfg, wl, self.ld, steps)
        B, H, G, D = cfg.batch, cfg.num_kv_heads, cfg.group, cfg.head_dim
        self.shape = M.make_shape(B, H, G, D, wl.max_pages, wl.num_phys_pages, cfg.torch_kv_dtype(),
                                  cfg.torch_q_dtype(), sum_dtype=sdt)
        self.scode = {torch.bfloat16: "bf16", torch.float8_e4m3fn: "fp8"}.get(sdt, "f32")
        self.table = wl.block_table.to(dev)
        self.lens = wl.prefill_lens.to(dev)
        self.buf = M.StepBuffers.allocate(self.shape, NUM_WORKGROUPS, dev)
        self.buf.out.fill_(float("nan"))
        self.summ = torch.full((wl.num_phys_pages, H, D), float("nan"), dtype=sdt, device=dev)
        M.page_summaries(self.shape, self.ld.k_pool, self.table, self.lens, self.summ, M.SUM_ALL,
                         self.buf.status)
        # the oracle's inputs, copied before the GPU appends anything
        self.prefill = {}
        self.qs = self.ld.q.double().cpu().numpy()
        self.kn = self.ld.k_new.double().cpu().numpy()
        self.vn = self.ld.v_new.double().cpu().numpy()

    def oracle_prefill(self, r, j):
        L0 = self.cfg.context[r] - 1
        K = W.head_tokens(self.ld.k_pool, self.wl.block_table, r, j, L0).double().cpu().numpy()
        V = W.head_tokens(self.ld.v_pool, self.wl.block_table, r, j, L0).double().cpu().numpy()
        return K, V, L0

    def step(self, t, gamma):
        ld = self.ld
        M.advance_seq_lens(self.shape, self.lens, self.buf.status)
        M.layer_step(self.buf, ld.q[t].contiguous(), ld.k_new[t].contiguous(),
                     ld.v_new[t].contiguous(), ld.k_pool, ld.v_pool, self.summ, self.table,
                     self.lens, gamma, self.cfg.scale_f32)

    def snapshot(self):
        torch.cuda.synchronize()
        assert int(self.buf.status.item()) == 0
        return (self.buf.page_lists.cpu().numpy().copy(), self.buf.list_lens.cpu().numpy().copy(),
                self.buf.out.cpu().numpy().copy())


def _oracle_check(cfg, prefill_of, qs, kn, vn, snaps, steps, gamma, scode, what, pairs=None):
    """Replay every (request, KV head) in the oracle for `steps` steps and
    compare with the GPU snapshots {step: (lists, lens, out)}."""
    B, H, G = cfg.batch, cfg.num_kv_heads, cfg.group
    scale = cfg.scale_f32
    exceptions = 0
    for r in range(B):
        for j in range(H):
            if pairs is not None and (r, j) not in pairs:
                continue
            K, V, L0 = prefill_of(r, j)
            h = O.OracleHead(K, V, L0, 16, capacity=L0 + steps, summary_dtype=scode)
            del K, V
            for t in range(steps):
                h.append(kn[t, r, j], vn[t, r, j])
                if t not in snaps:
                    continue
                lists, ll, out = snaps[t]
                s = r * H + j
                qg = qs[t, r, j * G:(j + 1) * G]
                got = lists[s, :ll[s]].copy()
                masses = O.page_masses(qg, O.stored_summaries(h.means, scode),
                                       O.page_token_counts(h.seq_len, 16), scale)
                ref_pages = O.coverage_select(masses, gamma)
                exceptions += compare_lists(got, ref_pages, masses, gamma, f"{what} t{t} r{r} j{j}")
                if gamma >= 1.0:
                    assert len(got) == h.means.shape[0]
                assert_close(out[r, j * G:(j + 1) * G], h.attend(qg, got, scale),
                             f"{what} t{t} r{r} j{j}")
    return exceptions


def _run_eager(cfg_id, layer, gamma, steps, checks, sdt=torch.float32, pairs=None):
    cfg = W.shrink(W.get_config(cfg_id), steps=steps)
    wl = W.make_workload(cfg, device="cpu", extra_steps=2)
    what = f"cfg{cfg_id} l{layer} g{gamma}"
    note(f"[fullsize] {what}: {steps} steps, checks {sorted(checks)}, summaries {sdt}")
    run = LayerRun(cfg, wl, layer, sdt, steps)
    snaps = {}
    for t in range(steps):
        run.step(t, gamma)
        if t in checks:
            snaps[t] = run.snapshot()
    note(f"[fullsize] {what}: GPU done, oracle replay")
    ex = _oracle_check(cfg, run.oracle_prefill, run.qs, run.kn, run.vn, snaps, steps, gamma,
                       run.scode, what, pairs)
    note(f"[fullsize] {what}: {ex} differing pages (all in the documented bands)")
    del run
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_cfg3_graph_step_all_layers():
    """The 128k step exactly as bench.py times it: 32 layers in one captured
    graph, replayed 100 times; every layer and KV head checked at replays 0,
    1, 2, 17, 50 and 99."""
    steps, checks = 100, (0, 1, 2, 17, 50, 99)
    cfg = W.shrink(W.get_config(3), steps=steps)
    wl = W.make_workload(cfg, device="cpu", extra_steps=2)
    dev = torch.device("cuda")
    B, H, G, D = cfg.batch, cfg.num_kv_heads, cfg.group, cfg.head_dim
    shape = M.make_shape(B, H, G, D, wl.max_pages, wl.num_phys_pages, cfg.torch_kv_dtype(),
                         cfg.torch_q_dtype())
    table = wl.block_table.to(dev)
    lens = wl.prefill_lens.to(dev)
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    layers = []
    for l in range(cfg.layers):
        ld = W.make_layer(cfg, wl, l, device=dev)
        _position_code_values(cfg, wl, ld, steps)
        summ = torch.empty((wl.num_phys_pages, H, D), dtype=torch.float32, device=dev)
        M.page_summaries(shape, ld.k_pool, table, lens, summ, M.SUM_ALL, status)
        layers.append((ld, summ, M.StepBuffers.allocate(shape, NUM_WORKGROUPS, dev)))
    q_all = torch.stack([ld.q for ld, _, _ in layers], 1).contiguous()      # [steps, layers, B, Hq, D]
    k_all = torch.stack([ld.k_new for ld, _, _ in layers], 1).contiguous()  # [steps, layers, B, H, D]
    v_all = torch.stack([ld.v_new for ld, _, _ in layers], 1).contiguous()
    q_in, k_in, v_in = q_all[0].clone(), k_all[0].clone(), v_all[0].clone()
    t_idx = torch.zeros(1, dtype=torch.long, device=dev)
    torch.cuda.synchronize()
    note(f"[fullsize cfg3 graph] {cfg.layers} layers resident")

    def step():
        torch.index_select(q_all, 0, t_idx, out=q_in.unsqueeze(0))
        torch.index_select(k_all, 0, t_idx, out=k_in.unsqueeze(0))
        torch.index_select(v_all, 0, t_idx, out=v_in.unsqueeze(0))
        M.advance_seq_lens(shape, lens, status)
        for l, (ld, summ, b) in enumerate(layers):
            M.append_select(shape, q_in[l], k_in[l], v_in[l], ld.k_pool, ld.v_pool, summ, table,
                            lens, 0.99, cfg.scale_f32, b.workspace, b.page_lists, b.list_lens, status)
            M.ragged_decode_attn(shape, q_in[l], ld.k_pool, ld.v_pool, table, lens, b.page_lists,
                                 b.list_lens, cfg.scale_f32, NUM_WORKGROUPS, b.partial_o,
                                 b.partial_ml, status)
            M.combine(shape, b.list_lens, NUM_WORKGROUPS, b.partial_o, b.partial_ml, b.out)
        t_idx.add_(1)

    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            step()
    torch.cuda.synchronize()
    assert int(t_idx.item()) == 0 and torch.equal(lens, wl.prefill_lens.to(dev))   # capture ran nothing
    snaps = {l: {} for l in range(cfg.layers)}
    for t in range(steps):
        graph.replay()
        if t in checks:
            torch.cuda.synchronize()
            assert int(status.item()) == 0
            for l, (_, _, b) in enumerate(layers):
                snaps[l][t] = (b.page_lists.cpu().numpy().copy(), b.list_lens.cpu().numpy().copy(),
                               b.out.cpu().numpy().copy())
    torch.cuda.synchronize()
    del graph
    note(f"[fullsize cfg3 graph] {steps} replays done; oracle replay of every layer")
    qs, kn, vn = (x.double().cpu().numpy() for x in (q_all, k_all, v_all))
    total = 0
    for l, (ld, _, _) in enumerate(layers):
        def prefill_of(r, j, ld=ld):
            L0 = cfg.context[r] - 1
            return (W.head_tokens(ld.k_pool, wl.block_table, r, j, L0).double().cpu().numpy(),
                    W.head_tokens(ld.v_pool, wl.block_table, r, j, L0).double().cpu().numpy(), L0)
        total += _oracle_check(cfg, prefill_of, qs[:, l], kn[:, l], vn[:, l], snaps[l], steps, 0.99,
                               "f32", f"cfg3-graph l{l}")
        note(f"[fullsize cfg3 graph] layer {l} ok")
    note(f"[fullsize cfg3 graph] {total} differing pages over 32 layers x 8 heads x 6 steps")
    del layers, q_all, k_all, v_all
    torch.cuda.empty_cache()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("case", [
    (3, 21, 0.98, torch.float32),
    (3, 7, 1.0, torch.float32),
    (3, 0, 0.99, torch.bfloat16),
    (3, 3, 0.99, torch.float8_e4m3fn),
], ids=["cfg3-l21-g0.98", "cfg3-l7-g1.0", "cfg3-l0-g0.99-bf16sum", "cfg3-l3-g0.99-fp8sum"])
def test_cfg3_variants(case):
    """gamma 0.98 and 1 (dense on the same kernels), and bf16 and E4M3 page
    summaries, at the 128k shape: every KV head, steps 0, 1, 2 and 17."""
    cfg_id, layer, gamma, sdt = case
    _run_eager(cfg_id, layer, gamma, 18, {0, 1, 2, 17}, sdt)


@pytest.mark.timeout(600)
def test_cfg2_every_step():
    """The 32k layer: every KV head at every one of its 100 steps."""
    _run_eager(2, 0, 0.99, 100, set(range(100)))


@pytest.mark.timeout(900)
def test_cfg4_serving_batch():
    """32 requests of 4k-128k tokens: all 256 (request, KV head) pairs at
    steps 0, 1 and 49 (the last)."""
    _run_eager(4, 0, 0.99, 50, {0, 1, 49})


@pytest.mark.timeout(900)
@pytest.mark.parametrize("gamma", [0.99, 1.0])
def test_cfg5_load_balance(gamma):
    """64 requests of 64k, group 8, half the heads dominant and half
    near-uniform: all 512 pairs at steps 0, 1 and 19 (the last)."""
    _run_eager(5, 0, gamma, 20, {0, 1, 19})
