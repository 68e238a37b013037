"""Benchmark: one decode step of coverage-rule sparse paged attention on MI355X.

A step = advance the request lengths, then for every layer: append the step's
K/V token (refreshing the tail page summary) and select pages by the coverage
rule (one call), run the self-planning split-K attention over the ragged page
lists, and merge the partial states. The whole step (all layers, plus the staging of the
step's query/K/V inputs) is captured in one HIP graph and replayed; inputs are
resident in HBM before the timed region starts.

Default workload: Llama-3-8B-shaped 32-layer step at 128k context, gamma 0.99
(8 KV heads x group 4, head_dim 128, bf16 K/V in 16-token pages), synthetic
seeded data. Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--config 3] [--gamma 0.99]
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The CPU baseline's BLAS uses the host cores this process may run on, capped
# by OMP_NUM_THREADS where the host sets it (its CPU share); OpenBLAS and MKL
# are told the same count before NumPy loads.
CPU_THREADS = len(os.sched_getaffinity(0))
if os.environ.get("OMP_NUM_THREADS", "").isdigit():
    CPU_THREADS = max(1, min(CPU_THREADS, int(os.environ["OMP_NUM_THREADS"])))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
    os.environ.setdefault(_v, str(CPU_THREADS))

HBM_PEAK_GBPS = 8000.0
CPU_LAYERS = 4          # layers whose inputs the CPU oracle sample draws from
METRIC = "µs per layer decode step at 128k, γ=0.99; effective HBM GB/s (% of roofline)"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=3)
    ap.add_argument("--gamma", type=float, default=None)
    ap.add_argument("--layers", type=int, default=None, help="override the layer count")
    ap.add_argument("--num-workgroups", type=int, default=256,
                    help="attention workgroups: one per CU (each is 8 waves at this shape)")
    ap.add_argument("--summary-dtype", choices=["f32", "bf16", "fp8"], default="f32",
                    help="element type of the page summaries (the mean keys the selection reads)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle time budget (0 = skip)")
    ap.add_argument("--no-dense", dest="dense", action="store_false",
                    help="skip the dense reference: the same kernels with gamma = 1 (context, "
                         "not the metric)")
    ap.add_argument("--profile-eager", type=int, default=0,
                    help="after timing, run N eager steps (for counter collection)")
    ap.add_argument("--rule", choices=["coverage", "topk", "topdelta"], default="coverage",
                    help="selection rule (comparison runs; the metric is the coverage rule)")
    ap.add_argument("--rule-param", type=float, default=None,
                    help="k for topk, delta for topdelta (gamma comes from --gamma)")
    ap.add_argument("--separate-append", action="store_true",
                    help="append and select as two calls instead of moira_append_select")
    ap.add_argument("--fused-combine", action="store_true",
                    help="attention with the merge in one launch "
                         "(moira_ragged_decode_attn_combine) instead of attention + combine")
    ap.add_argument("--padded", action="store_true",
                    help="also time attention over lists padded to each layer's longest "
                         "list (the pad-to-max comparison; context, not the metric)")
    ap.add_argument("--mode", choices=["graph", "eager"], default="graph",
                    help="eager: no graph, launch-by-launch steps (for hardware counters); "
                         "its timing includes host launch overhead and is not the metric")
    return ap.parse_args()


def main():
    args = parse()
    if args.rule != "coverage" and args.rule_param is None:
        print(json.dumps({"error": f"--rule {args.rule} needs --rule-param"}))
        sys.exit(2)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from long_context_sparse_summary_amd import moira as M
    from long_context_sparse_summary_amd import workloads as W

    M.load()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = W.get_config(args.config)
    layers = args.layers or (4 if args.config == 2 else cfg.layers)
    gamma = args.gamma if args.gamma is not None else (0.99 if 0.99 in cfg.gammas else cfg.gammas[0])
    total_steps = args.warmup + args.steps
    in_steps = min(cfg.steps, 100)
    wl = W.make_workload(W.shrink(cfg, steps=in_steps), device="cpu",
                         extra_steps=total_steps * 2 + 8)
    B, H, G, D = cfg.batch, cfg.num_kv_heads, cfg.group, cfg.head_dim
    sum_dt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn}.get(args.summary_dtype,
                                                                    torch.float32)
    sum_bytes = {"bf16": 2, "fp8": 1}.get(args.summary_dtype, 4)
    shape = M.make_shape(B, H, G, D, wl.max_pages, wl.num_phys_pages, cfg.torch_kv_dtype(),
                         cfg.torch_q_dtype(), sum_dtype=sum_dt)
    table = wl.block_table.to(dev)
    lens = wl.prefill_lens.to(dev)
    N = args.num_workgroups
    scale = cfg.scale_f32

    # ---- inputs, resident in HBM -------------------------------------------
    t0 = time.time()
    pools, summs, q_all, kn_all, vn_all, cpu_sample = [], [], [], [], [], []
    status = torch.zeros(1, dtype=torch.int32, device=dev)
    for l in range(layers):
        ld = W.make_layer(W.shrink(cfg, steps=in_steps), wl, l, device=dev)
        if l < CPU_LAYERS and args.cpu_seconds > 0:
            # the oracle's sample: prefill tokens and step inputs straight from the generator
            cpu_sample.append({
                "k": [[W.head_tokens(ld.k_pool, table, r, j, cfg.context[r] - 1).float().cpu().numpy()
                       for j in range(H)] for r in range(B)],
                "v": [[W.head_tokens(ld.v_pool, table, r, j, cfg.context[r] - 1).float().cpu().numpy()
                       for j in range(H)] for r in range(B)],
                "q": ld.q.float().cpu().numpy(), "kn": ld.k_new.float().cpu().numpy(),
                "vn": ld.v_new.float().cpu().numpy()})
        summ = torch.empty((wl.num_phys_pages, H, D), dtype=sum_dt, device=dev)
        M.page_summaries(shape, ld.k_pool, table, lens, summ, M.SUM_ALL, status)
        pools.append((ld.k_pool, ld.v_pool))
        summs.append(summ)
        q_all.append(ld.q)
        kn_all.append(ld.k_new)
        vn_all.append(ld.v_new)
        del ld
    q_all = torch.stack(q_all, 1).contiguous()      # [steps, layers, B, Hq, D]
    kn_all = torch.stack(kn_all, 1).contiguous()    # [steps, layers, B, H, D]
    vn_all = torch.stack(vn_all, 1).contiguous()
    # one byte table per step (q, then k, then v of every layer), so that a
    # single device-indexed copy stages a step's inputs
    n_steps_in = q_all.shape[0]
    parts = [t.view(n_steps_in, -1).view(torch.uint8) for t in (q_all, kn_all, vn_all)]
    cuts = [p_.shape[1] for p_ in parts]
    pad = (-sum(cuts)) % 8                         # rows copied as 8-byte words
    if pad:
        parts.append(torch.zeros((n_steps_in, pad), dtype=torch.uint8, device=parts[0].device))
    # the last word of row i holds the next step's row index, so the staging
    # copy also brings the index the next replay reads
    nxt = ((torch.arange(n_steps_in, dtype=torch.int64) + 1) % n_steps_in).view(-1, 1)
    parts.append(nxt.to(parts[0].device).view(torch.uint8))
    in_all = torch.cat(parts, 1).contiguous().view(torch.int64)   # [steps, words]
    in_shapes = [(t.shape[1:], t.dtype) for t in (q_all, kn_all, vn_all)]
    del q_all, kn_all, vn_all, parts
    torch.cuda.synchronize()
    log(f"workload {cfg.name}: {layers} layers, B={B} H={H} G={G} D={D} ctx={cfg.context[:4]}... "
        f"max_pages={wl.max_pages}, generated in {time.time() - t0:.1f}s, "
        f"{torch.cuda.memory_allocated() / 2**30:.1f} GiB resident")

    bufs = [M.StepBuffers.allocate(shape, N, dev) for _ in range(layers)]
    in_words = torch.empty(in_all.shape[1], dtype=torch.int64, device=dev)
    in_buf = in_words.view(torch.uint8)
    views, o_ = [], 0
    for nb, (shp, dt) in zip(cuts, in_shapes):
        views.append(in_buf[o_:o_ + nb].view(dt).view(shp))
        o_ += nb
    q_in, k_in, v_in = views
    t_idx = torch.zeros(1, dtype=torch.long, device=dev)

    def step(g):
        # stage this step's inputs (indexed on the device), then every layer
        torch.index_select(in_all, 0, t_idx, out=in_words.unsqueeze(0))
        M.advance_seq_lens(shape, lens, status)
        for l in range(layers):
            b = bufs[l]
            kp, vp = pools[l]
            if args.rule != "coverage" and g < 1.0:
                M.append_kv(shape, k_in[l], v_in[l], kp, vp, summs[l], table, lens, status)
                M.select_pages_rule(shape, q_in[l], summs[l], table, lens, args.rule,
                                    args.rule_param, scale, b.workspace, b.page_lists,
                                    b.list_lens, status)
            elif args.separate_append:
                M.append_kv(shape, k_in[l], v_in[l], kp, vp, summs[l], table, lens, status)
                M.select_pages(shape, q_in[l], summs[l], table, lens, g, scale, b.workspace,
                               b.page_lists, b.list_lens, status)
            else:
                M.append_select(shape, q_in[l], k_in[l], v_in[l], kp, vp, summs[l], table, lens,
                                g, scale, b.workspace, b.page_lists, b.list_lens, status)
            if args.fused_combine:
                M.ragged_decode_attn_combine(shape, q_in[l], kp, vp, table, lens, b.page_lists,
                                             b.list_lens, scale, N, b.partial_o, b.partial_ml,
                                             b.counters, b.out, status)
            else:
                M.ragged_decode_attn(shape, q_in[l], kp, vp, table, lens, b.page_lists,
                                     b.list_lens, scale, N, b.partial_o, b.partial_ml, status)
                M.combine(shape, b.list_lens, N, b.partial_o, b.partial_ml, b.out)
        t_idx.copy_(in_words[-1:])   # the next step's row (staged with this one)

    def selected_bytes():
        """Algorithmic bytes of the last step: summaries of every page + K and V
        of the selected pages (token-exact for tail pages)."""
        L = lens.to(torch.long)                                   # [B]
        P = (L + 15) // 16
        tail_n = L - 16 * (P - 1)
        summ_b = float((P * H).sum().item()) * D * sum_bytes
        kv_b, n_sel = 0.0, 0
        for l in range(layers):
            ll = bufs[l].list_lens.to(torch.long).view(B, H)
            last = torch.gather(bufs[l].page_lists.view(B, H, -1).to(torch.long), 2,
                                (ll - 1).clamp(min=0).unsqueeze(2)).squeeze(2)
            has_tail = (ll > 0) & (last == (P - 1).unsqueeze(1))
            toks = ll * 16 - has_tail * (16 - tail_n.unsqueeze(1))
            kv_b += float(toks.sum().item()) * D * 2 * 2
            n_sel += int(ll.sum().item())
        return summ_b * layers, kv_b, n_sel, int((P * H).sum().item()) * layers

    def run_graph(g_gamma, steps, warmup):
        torch.cuda.synchronize()
        stream = torch.cuda.Stream()
        graph = torch.cuda.CUDAGraph()
        lens0 = lens.clone()
        t0_ = t_idx.clone()
        with torch.cuda.stream(stream):
            step(g_gamma)                                          # eager warm-up of every kernel
            torch.cuda.synchronize()
            lens.copy_(lens0)
            t_idx.copy_(t0_)
            torch.cuda.synchronize()
            with torch.cuda.graph(graph, stream=stream):
                step(g_gamma)
        torch.cuda.synchronize()
        for _ in range(warmup):
            graph.replay()
        torch.cuda.synchronize()
        lens_start, t_start = lens.clone(), t_idx.clone()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        # accounting pass: replay the same steps again from the same state,
        # one at a time, each bracketed by events (its spread is reported)
        lens.copy_(lens_start)
        t_idx.copy_(t_start)
        tot = [0.0, 0.0, 0, 0]
        per = []
        for _ in range(steps):
            e0.record()
            graph.replay()
            e1.record()
            torch.cuda.synchronize()
            per.append(e0.elapsed_time(e1))
            sb, kb, ns, npg = selected_bytes()
            tot[0] += sb; tot[1] += kb; tot[2] += ns; tot[3] += npg
        del graph
        return ms, tot, per

    def run_eager(g_gamma, steps, warmup):
        for _ in range(warmup):
            step(g_gamma)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        tot = [0.0, 0.0, 0, 0]
        ms_ = 0.0
        for _ in range(steps):
            e0.record()
            step(g_gamma)
            e1.record()
            torch.cuda.synchronize()
            ms_ += e0.elapsed_time(e1)
            sb, kb, ns, npg = selected_bytes()
            tot[0] += sb; tot[1] += kb; tot[2] += ns; tot[3] += npg
        return ms_, tot, []

    # ---- sparse step (the metric) -------------------------------------------
    runner = run_graph if args.mode == "graph" else run_eager
    ms, (summ_b, kv_b, n_sel, n_pages), per_replay = runner(gamma, args.steps, args.warmup)
    us_layer = ms * 1e3 / (args.steps * layers)
    bytes_step = (summ_b + kv_b) / args.steps
    eff_gbps = bytes_step / (ms * 1e-3 / args.steps) / 1e9
    frac_sel = n_sel / max(n_pages, 1)
    st = int(status.item())
    log(f"sparse gamma={gamma}: {us_layer:.2f} us/layer-step, {eff_gbps:.0f} GB/s effective, "
        f"selected fraction {frac_sel:.4f}, status {st}")

    replay_pct = None
    if per_replay:
        v = sorted(x * 1e3 / layers for x in per_replay)
        pick = lambda f: round(v[min(len(v) - 1, int(f * len(v)))], 3)
        replay_pct = {"p10": pick(0.1), "p50": pick(0.5), "p90": pick(0.9), "n": len(v),
                      "note": "single replays, each bracketed by events (the metric times "
                              "the replays back to back)"}

    # ---- dense reference on the same kernels ----------------------------------------
    dense = None
    if args.dense:
        dms, (dsb, dkb, _, _), _ = runner(1.0, max(args.steps // 4, 5), 3)
        dsteps = max(args.steps // 4, 5)
        dense = {"us_per_layer_step": round(dms * 1e3 / (dsteps * layers), 3),
                 "effective_GBps": round((dkb / dsteps) / (dms * 1e-3 / dsteps) / 1e9, 1),
                 "sparse_speedup": round(dms / dsteps / (ms / args.steps), 3),
                 "note": "gamma = 1 on the same kernels: every page listed, no summary scan"}
        log(f"dense gamma=1: {dense['us_per_layer_step']:.2f} us/layer-step")
        step(gamma)                      # back to the sparse lists for the timing below
        torch.cuda.synchronize()

    # ---- attention kernel timed alone (roofline of the dominant kernel) ----------
    # the 32 layers' launches on the last step's lists, captured in a graph so
    # that host launch gaps stay out; events on the replay stream. The call is
    # the one the step makes (attention alone, or attention with the merge of
    # its partial states with --fused-combine).
    reps = 20

    def attn_all_layers():
        for l in range(layers):
            b = bufs[l]
            kp, vp = pools[l]
            if args.fused_combine:
                M.ragged_decode_attn_combine(shape, q_in[l], kp, vp, table, lens, b.page_lists,
                                             b.list_lens, scale, N, b.partial_o, b.partial_ml,
                                             b.counters, b.out, status)
            else:
                M.ragged_decode_attn(shape, q_in[l], kp, vp, table, lens, b.page_lists,
                                     b.list_lens, scale, N, b.partial_o, b.partial_ml, status)

    astream = torch.cuda.Stream()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    with torch.cuda.stream(astream):
        attn_all_layers()                            # eager warm-up
        torch.cuda.synchronize()
        if args.mode == "graph":
            agraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(agraph, stream=astream):
                attn_all_layers()
            agraph.replay()
            torch.cuda.synchronize()
            a0.record(astream)
            for _ in range(reps):
                agraph.replay()
            a1.record(astream)
        else:                                        # launch by launch (counter runs)
            a0.record(astream)
            for _ in range(reps):
                attn_all_layers()
            a1.record(astream)
    torch.cuda.synchronize()
    if args.mode == "graph":
        del agraph
    _, kv_last, _, _ = selected_bytes()
    attn_bytes = kv_last / layers
    attn_us = 1e3 * a0.elapsed_time(a1) / (reps * layers)
    attn_gbps = attn_bytes / (attn_us * 1e-6) / 1e9
    log(f"attention kernel alone: {attn_us:.2f} us/launch, {attn_bytes / 1e6:.1f} MB/launch, "
        f"{attn_gbps:.0f} GB/s")

    # ---- pad-to-max comparison: every list of a layer padded to its longest ------
    # (the pages 0 .. longest-1 of each (request, KV head): the same number of
    # pages as a padded, masked list reads, on the same self-planning kernel)
    padded = None
    if args.padded:
        P_now = ((lens.to(torch.long) + 15) // 16).repeat_interleave(H)        # [S]
        pad_bufs = []
        for l in range(layers):
            b = bufs[l]
            longest = int(b.list_lens.max().item())
            pl = torch.arange(wl.max_pages, dtype=torch.int32, device=dev).expand(B * H, -1)
            ln = torch.minimum(torch.full((B * H,), longest, dtype=torch.long, device=dev), P_now)
            pad_bufs.append((pl.contiguous(), ln.to(torch.int32).contiguous()))

        def attn_padded():
            for l in range(layers):
                b = bufs[l]
                kp, vp = pools[l]
                pl, ln = pad_bufs[l]
                M.ragged_decode_attn(shape, q_in[l], kp, vp, table, lens, pl, ln, scale, N,
                                     b.partial_o, b.partial_ml, status)

        pstream = torch.cuda.Stream()
        torch.cuda.synchronize()
        with torch.cuda.stream(pstream):
            attn_padded()
            torch.cuda.synchronize()
            pgraph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(pgraph, stream=pstream):
                attn_padded()
            pgraph.replay()
            torch.cuda.synchronize()
            a0.record(pstream)
            for _ in range(reps):
                pgraph.replay()
            a1.record(pstream)
        torch.cuda.synchronize()
        del pgraph
        pad_pages = sum(int(ln.to(torch.long).sum().item()) for _, ln in pad_bufs) / layers
        pad_us = 1e3 * a0.elapsed_time(a1) / (reps * layers)
        padded = {"attention_us_per_launch": round(pad_us, 3),
                  "pages_per_launch": round(pad_pages),
                  "ragged_pages_per_launch": round(
                      sum(int(bufs[l].list_lens.to(torch.long).sum().item()) for l in range(layers)) / layers),
                  "vs_ragged": round(pad_us / attn_us, 3)}
        log(f"attention over lists padded to the longest: {pad_us:.2f} us/launch "
            f"({padded['pages_per_launch']} pages against {padded['ragged_pages_per_launch']})")

    # ---- full summary build (row a1', outside the step) -------------------------
    # moira_page_summaries(ALL) of one layer: reads every token's key, writes
    # one mean per (page, KV head); 8 builds over the layers' pools in turn
    # (no build finds the previous one's keys in cache) captured in a graph,
    # timed with HIP events on the replay stream: the median of 7 replays
    sstream = torch.cuda.Stream()
    summ_scratch = torch.empty_like(summs[0])
    L_now = lens.to(torch.long)
    P_now = (L_now + 15) // 16
    kv_elem = 2 if cfg.kv_dtype == "bf16" else 4
    build_bytes = float(L_now.sum().item()) * H * D * kv_elem + float(P_now.sum().item()) * H * D * sum_bytes
    torch.cuda.synchronize()

    def builds():
        for i in range(8):
            M.page_summaries(shape, pools[i % layers][0], table, lens, summ_scratch, M.SUM_ALL,
                             status)

    with torch.cuda.stream(sstream):
        builds()                                     # eager warm-up
        bgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(bgraph, stream=sstream):
            builds()
        bgraph.replay()
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(8)]
        evs[0].record(sstream)
        for i in range(1, 8):                        # 7 replays of 8 builds, each timed
            bgraph.replay()
            evs[i].record(sstream)
    torch.cuda.synchronize()
    del bgraph
    per_replay = sorted(evs[i - 1].elapsed_time(evs[i]) for i in range(1, 8))
    build_us = 1e3 * per_replay[3] / 8                # median replay, per build
    summary_build = {"us": round(build_us, 2), "bytes": round(build_bytes),
                     "GBps": round(build_bytes / (build_us * 1e-6) / 1e9, 1),
                     "frac_of_peak": round(build_bytes / (build_us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "note": "moira_page_summaries(ALL) of one layer: all keys read once, "
                             "one mean per (page, KV head) written"}
    log(f"full summary build: {build_us:.1f} us, {summary_build['GBps']:.0f} GB/s "
        f"(replays of 8 builds: {1e3 * per_replay[0] / 8:.1f} .. {1e3 * per_replay[-1] / 8:.1f} us each)")
    del summ_scratch

    # ---- streaming ceilings (context) -------------------------------------------------
    x = torch.empty(2**30 // 2, dtype=torch.bfloat16, device=dev)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    for _ in range(10):
        y.copy_(x)
    c1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * x.numel() * 2 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    # read-only: the library's streaming kernel (the 16-byte non-temporal
    # loads the method's kernels use) over the same 1 GiB
    sink = torch.empty(M.stream_read_sink_words(), dtype=torch.int32, device=dev)
    with torch.cuda.stream(sstream):
        M.stream_read(x, sink)
        c0.record(sstream)
        for _ in range(10):
            M.stream_read(x, sink)
        c1.record(sstream)
    torch.cuda.synchronize()
    read_gbps = x.numel() * 2 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    log(f"streaming: copy {copy_gbps:.0f} GB/s (read + write), read-only {read_gbps:.0f} GB/s")
    del sink
    # plain streaming kernel of known size (1 GiB read + 1 GiB written), the
    # calibration of the HBM byte counters (see bench_counters.py)
    for _ in range(3):
        torch.neg(x, out=y)
    torch.cuda.synchronize()
    del x, y

    for _ in range(args.profile_eager):
        step(gamma)
    torch.cuda.synchronize()

    # ---- CPU baseline: the oracle on a bounded sample ----------------------------------
    cpu = None
    if cpu_sample:
        cpu = cpu_baseline(cpu_sample, cfg, gamma, scale, args.cpu_seconds, args.summary_dtype)

    traffic, traffic_src = measured_traffic(args.config)

    out = {
        "metric": METRIC,
        "value": round(us_layer, 3),
        "unit": "us/layer-step",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms / args.steps, 4),
        "replay_us_per_layer": replay_pct,
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: one decode step of {layers} layers in one hipGraph, "
                        f"batch {B}, context {cfg.context[0] if B == 1 else 'mixed'}, "
                        f"{H} KV heads x group {G}, head_dim {D}, 16-token pages, gamma {gamma}",
            "batch": B, "context": cfg.context[0] if B == 1 else cfg.context,
            "layers": layers, "kv_heads": H, "group": G, "head_dim": D, "page_size": 16,
            "gamma": gamma, "num_workgroups": N, "mode": args.mode,
            "summary_dtype": args.summary_dtype,
            "rule": args.rule if args.rule == "coverage" else f"{args.rule}={args.rule_param:g}",
        },
        "effective_GBps": round(eff_gbps, 1),
        "hbm_roofline_frac": round(eff_gbps / HBM_PEAK_GBPS, 4),
        "bytes_per_layer_step": round(bytes_step / layers),
        "selected_fraction": round(frac_sel, 5),
        "roofline": {
            "kernel": ("attn_mfma_kernel with the merge (moira_ragged_decode_attn_combine)"
                       if args.fused_combine else "attn_mfma_kernel (moira_ragged_decode_attn)"),
            "bound": "hbm",
            "achieved": round(attn_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(attn_gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "us_per_launch": round(attn_us, 3),
            "bytes_per_launch": round(attn_bytes),
            "traffic_source": traffic_src,
        },
        "dense": dense,
        "padded": padded,
        "stream_copy_GBps": round(copy_gbps, 1),
        "stream_read_GBps": round(read_gbps, 1),
        "summary_build": summary_build,
        "cpu_baseline": cpu,
        "device_status": st,
    }
    print(json.dumps(out), flush=True)


def measured_traffic(config):
    """HBM bytes per attention launch from the committed counter summary of
    this workload, or None when there is none or the kernel's sources changed
    since the counters were taken."""
    from bench_counters import attn_source_hash
    path = os.path.join(ROOT, "profiles", f"attn_mfma_kernel_traffic_cfg{config}.md")
    rel = os.path.relpath(path, ROOT)
    if not os.path.exists(path):
        return None, f"{rel}: absent"
    rec = None
    with open(path) as f:
        for line in f:
            if line.startswith("traffic-json:"):
                rec = json.loads(line.split(":", 1)[1])
    if rec is None:
        return None, f"{rel}: no traffic record"
    if rec.get("source_hash") != attn_source_hash():
        return None, f"{rel}: stale (kernel sources changed since the counters were taken)"
    return rec["traffic_bytes_per_launch"], rel


def cpu_baseline(sample, cfg, gamma, scale, budget_s, summary_dtype="f32"):
    """Time the fp64 oracle (as it stands) on a bounded sample: whole layer
    steps (append + select + attend for every KV head) of the first layers,
    consecutive steps of each layer, until the time budget is used."""
    import oracle as O
    from threadpoolctl import threadpool_info, threadpool_limits
    limiter = threadpool_limits(limits=CPU_THREADS)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    G = cfg.group
    per_layer = budget_s / len(sample)
    done, secs, steps_run = 0, 0.0, []
    for s in sample:
        nsteps = s["q"].shape[0]
        heads = []
        for r in range(cfg.batch):
            for j in range(cfg.num_kv_heads):
                L0 = cfg.context[r] - 1
                heads.append((r, j, O.OracleHead(s["k"][r][j], s["v"][r][j], L0, 16,
                                                 capacity=L0 + nsteps,
                                                 summary_dtype=summary_dtype)))
        layer_secs, t = 0.0, 0
        while t < nsteps and layer_secs < per_layer:
            t0 = time.perf_counter()
            for r, j, h in heads:
                h.step(s["q"][t, r, j * G:(j + 1) * G], s["kn"][t, r, j], s["vn"][t, r, j], scale, gamma)
            layer_secs += time.perf_counter() - t0
            t += 1
        secs += layer_secs
        done += t
        steps_run.append(t)
        del heads
    us = secs / done * 1e6
    limiter.restore_original_limits()
    return {"value": round(us, 1), "unit": "us/layer-step", "cores": int(threads), "kind": "oracle",
            "host_cores_available": len(os.sched_getaffinity(0)),
            "cores_note": "BLAS threads used by the oracle: the cores this process may run on, "
                          "capped by OMP_NUM_THREADS where the host sets it",
            "sample": f"{done} layer-steps ({secs:.1f} s): layers 0..{len(sample) - 1}, "
                      f"steps 0..{max(steps_run) - 1} of each, all {cfg.batch * cfg.num_kv_heads} "
                      f"(request, KV head) pairs; page means prebuilt and kept incrementally; "
                      f"timed = append + select + attend"}


if __name__ == "__main__":
    main()
