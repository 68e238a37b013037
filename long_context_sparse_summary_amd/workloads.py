"""Seeded synthetic inputs shaped like the long-context decode workloads.

This module only draws inputs and lays them out (KV pool pages, block table,
per-step queries and appended tokens). It holds none of the method's
arithmetic: no page summaries, masses, selection or attention. Both the HIP
path and the fp64 oracle consume what it produces.

The pages measure on RULER at 128k context with a Llama-3-8B-class model
(MOIRA abstract). Neither the benchmark data nor weights exist here, so the
inputs are synthetic stand-ins with the same shapes: 8 KV heads, GQA groups of
4 (8 for the load-balance case), head_dim 128, bf16 K/V in 16-token pages,
contexts up to 128k. Attention concentration is planted by shifting the keys
of a few "hot" pages along the group's query direction, so that the number of
pages needed to reach gamma varies widely across heads and layers, the
property the MOIRA abstract reports.

Recipe (seeds from numpy SeedSequence(20261003, spawn_key=(cfg, layer,
request, kv_head, stream))):
  * keys, values, queries ~ N(0, 1) in fp32, cast once to bf16 (round to
    nearest even) where the workload is bf16;
  * u_j = normalise(sum of the step-0 queries of group j);
  * hot pages of (request, KV head j) get every key shifted by s * u_j, where
    s = 2.0 (tiny case, 3 hot pages) or s = alpha_j * sqrt(D) with
    alpha_j ~ U(1, 4) and a hot-page count 4 + round(596 w_j / max w),
    w ~ Dirichlet(0.5, ..., 0.5) over the KV heads of the request;
  * the load-balance case makes half the KV heads of each request dominant
    (one page shifted by 4 sqrt(D) u_j) and the other half near-uniform
    (keys ~ N(0, 0.1^2));
  * step-t queries are q(0) + 0.1 * eps_t; appended tokens are N(0, 1);
  * physical page ids are a seeded permutation of the pool, so page gathers
    are non-contiguous; the prefill holds L - 1 tokens and step 0 appends
    the L-th.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace
from typing import List, Optional

import numpy as np
import torch

ROOT_SEED = 20261003
S_K, S_V, S_Q, S_HOT, S_STEPNOISE, S_APPEND, S_LEN, S_TABLE = range(8)


def seed_for(cfg: int, layer: int, req: int, head: int, stream: int) -> int:
    ss = np.random.SeedSequence(ROOT_SEED, spawn_key=(cfg, layer, req, head, stream))
    return int(ss.generate_state(1, dtype=np.uint64)[0] & np.uint64((1 << 63) - 1))


def np_rng(cfg, layer, req, head, stream) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(ROOT_SEED, spawn_key=(cfg, layer, req, head, stream)))


def torch_gen(device, cfg, layer, req, head, stream) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed_for(cfg, layer, req, head, stream))
    return g


@dataclass(frozen=True)
class WorkloadConfig:
    cfg_id: int
    name: str
    batch: int
    num_kv_heads: int
    group: int
    head_dim: int
    context: List[int]              # tokens each request attends over at step 0
    layers: int
    gammas: tuple
    steps: int
    kv_dtype: str                   # "bf16" | "f32"
    q_dtype: str
    profile: str                    # "literal3" | "dirichlet" | "bimodal"
    page_size: int = 16
    scale: float = field(default=0.0)

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.group

    @property
    def scale_f32(self) -> float:
        s = self.scale if self.scale else 1.0 / math.sqrt(self.head_dim)
        return float(np.float32(s))

    def torch_kv_dtype(self):
        return torch.bfloat16 if self.kv_dtype == "bf16" else torch.float32

    def torch_q_dtype(self):
        return torch.bfloat16 if self.q_dtype == "bf16" else torch.float32


def _cfg4_contexts(batch: int) -> List[int]:
    rng = np_rng(4, 0, 0, 0, S_LEN)
    u = rng.uniform(math.log(4096), math.log(131072), size=batch)
    return [int(math.floor(math.exp(x))) for x in u]


def get_config(i: int) -> WorkloadConfig:
    """The five workloads: 1 tiny parity case, 2 one 32k layer, 3 the 128k
    32-layer headline step, 4 a ragged 32-request serving batch, 5 a
    64-request load-balance stress with GQA groups of 8."""
    if i == 1:
        return WorkloadConfig(1, "tiny", 1, 2, 2, 64, [1024], 1, (0.9,), 1, "f32", "f32",
                              "literal3", scale=1.0 / 8.0)
    if i == 2:
        return WorkloadConfig(2, "llama3-8b-layer-32k", 1, 8, 4, 128, [32768], 1, (0.99,), 100,
                              "bf16", "bf16", "dirichlet")
    if i == 3:
        return WorkloadConfig(3, "llama3-8b-32layer-128k", 1, 8, 4, 128, [131072], 32,
                              (0.98, 0.99, 1.0), 100, "bf16", "bf16", "dirichlet")
    if i == 4:
        return WorkloadConfig(4, "serving-32req-4k-128k", 32, 8, 4, 128, _cfg4_contexts(32), 1,
                              (0.99,), 50, "bf16", "bf16", "dirichlet")
    if i == 5:
        return WorkloadConfig(5, "balance-64req-64k-g8", 64, 8, 8, 128, [65536] * 64, 1,
                              (0.99, 1.0), 20, "bf16", "bf16", "bimodal")
    raise ValueError(f"no workload {i}")


def shrink(cfg: WorkloadConfig, *, context=None, batch=None, layers=None, steps=None) -> WorkloadConfig:
    """Same structure at a smaller size (for parity cases the oracle finishes
    in seconds)."""
    b = batch if batch is not None else cfg.batch
    ctx = list(cfg.context)
    if context is not None:
        ctx = list(context) if isinstance(context, (list, tuple)) else [int(context)] * b
    if len(ctx) != b:
        ctx = (ctx * ((b + len(ctx) - 1) // len(ctx)))[:b]
    return replace(cfg, batch=b, context=ctx,
                   layers=layers if layers is not None else cfg.layers,
                   steps=steps if steps is not None else cfg.steps)


@dataclass
class Workload:
    cfg: WorkloadConfig
    max_pages: int
    num_phys_pages: int
    block_table: torch.Tensor       # [B, max_pages] int32 physical page ids
    prefill_lens: torch.Tensor      # [B] int32: tokens in the cache before step 0


def make_workload(cfg: WorkloadConfig, device="cpu", extra_steps: int = 0,
                  slack_pages: int = 0) -> Workload:
    """Block table and prefill lengths. Capacity covers cfg.steps + extra_steps
    appended tokens per request."""
    ps = cfg.page_size
    total = cfg.steps + extra_steps
    need = [(L - 1 + total + ps - 1) // ps for L in cfg.context]
    max_pages = max(need) + slack_pages
    num_phys = sum(need) + slack_pages * cfg.batch
    rng = np_rng(cfg.cfg_id, 0, 0, 0, S_TABLE)
    perm = rng.permutation(num_phys).astype(np.int32)
    table = np.full((cfg.batch, max_pages), -1, dtype=np.int32)
    pos = 0
    for r in range(cfg.batch):
        n = need[r] + slack_pages
        table[r, :n] = perm[pos:pos + n]
        pos += n
    lens = np.array([L - 1 for L in cfg.context], dtype=np.int32)
    return Workload(cfg, max_pages, num_phys, torch.from_numpy(table).to(device),
                    torch.from_numpy(lens).to(device))


@dataclass
class LayerData:
    k_pool: torch.Tensor            # [N_phys, H_kv, ps, D]
    v_pool: torch.Tensor
    q: torch.Tensor                 # [steps, B, H_q, D]
    k_new: torch.Tensor             # [steps, B, H_kv, D]
    v_new: torch.Tensor
    hot_pages: dict                 # (r, j) -> list of hot page ids


def _unit(x: torch.Tensor) -> torch.Tensor:
    return x / torch.linalg.vector_norm(x)


def make_layer(cfg: WorkloadConfig, wl: Workload, layer: int, device="cpu",
               poison_unused: bool = False) -> LayerData:
    """Draw one layer's K/V pool, step queries and appended tokens."""
    B, H, G, D, ps = cfg.batch, cfg.num_kv_heads, cfg.group, cfg.head_dim, cfg.page_size
    kvdt, qdt = cfg.torch_kv_dtype(), cfg.torch_q_dtype()
    steps = cfg.steps
    fill = float("nan") if poison_unused else 0.0
    k_pool = torch.full((wl.num_phys_pages, H, ps, D), fill, dtype=kvdt, device=device)
    v_pool = torch.full((wl.num_phys_pages, H, ps, D), fill, dtype=kvdt, device=device)
    q_all = torch.empty((steps, B, H * G, D), dtype=qdt, device=device)
    k_new = torch.empty((steps, B, H, D), dtype=kvdt, device=device)
    v_new = torch.empty((steps, B, H, D), dtype=kvdt, device=device)
    table = wl.block_table.to(device=device, dtype=torch.long)
    hot = {}
    for r in range(B):
        L0 = cfg.context[r] - 1                 # prefill tokens
        P0 = (L0 + ps - 1) // ps
        gq = torch_gen(device, cfg.cfg_id, layer, r, 0, S_Q)
        q0 = torch.randn((H * G, D), generator=gq, device=device, dtype=torch.float32)
        gn = torch_gen(device, cfg.cfg_id, layer, r, 0, S_STEPNOISE)
        eps = torch.randn((steps, H * G, D), generator=gn, device=device, dtype=torch.float32)
        q_all[:, r] = (q0[None] + 0.1 * eps).to(qdt)
        ga = torch_gen(device, cfg.cfg_id, layer, r, 0, S_APPEND)
        k_new[:, r] = torch.randn((steps, H, D), generator=ga, device=device).to(kvdt)
        v_new[:, r] = torch.randn((steps, H, D), generator=ga, device=device).to(kvdt)
        prng = np_rng(cfg.cfg_id, layer, r, 0, S_HOT)
        if cfg.profile == "dirichlet":
            w = prng.dirichlet(np.full(H, 0.5))
            counts = [min(P0, 4 + int(round(596 * w[j] / w.max()))) for j in range(H)]
            alphas = prng.uniform(1.0, 4.0, size=H)
            kinds = ["hot"] * H
        elif cfg.profile == "bimodal":
            dom = set(prng.permutation(H)[: H // 2].tolist())
            counts = [1 if j in dom else 0 for j in range(H)]
            alphas = [4.0] * H
            kinds = ["hot" if j in dom else "uniform" for j in range(H)]
        else:
            counts = [min(P0, 3)] * H
            alphas = [None] * H
            kinds = ["hot"] * H
        for j in range(H):
            u = _unit(q0[j * G:(j + 1) * G].sum(dim=0))
            gk = torch_gen(device, cfg.cfg_id, layer, r, j, S_K)
            gv = torch_gen(device, cfg.cfg_id, layer, r, j, S_V)
            K = torch.randn((P0 * ps, D), generator=gk, device=device, dtype=torch.float32)
            V = torch.randn((P0 * ps, D), generator=gv, device=device, dtype=torch.float32)
            if kinds[j] == "uniform":
                K *= 0.1
            hp = sorted(np_rng(cfg.cfg_id, layer, r, j, S_HOT).choice(P0, size=counts[j], replace=False).tolist()) if counts[j] else []
            hot[(r, j)] = hp
            if hp:
                shift = (2.0 if alphas[j] is None else alphas[j] * math.sqrt(D)) * u
                idx = torch.tensor(hp, device=device, dtype=torch.long)
                Kp = K.view(P0, ps, D)
                Kp[idx] += shift
            K = K.to(kvdt)
            V = V.to(kvdt)
            if L0 < P0 * ps:                       # the tail slots hold no token yet
                K[L0:] = fill
                V[L0:] = fill
            phys = table[r, :P0]
            k_pool[phys, j] = K.view(P0, ps, D)
            v_pool[phys, j] = V.view(P0, ps, D)
    return LayerData(k_pool, v_pool, q_all, k_new, v_new, hot)


def head_tokens(pool: torch.Tensor, block_table: torch.Tensor, r: int, j: int, L: int) -> torch.Tensor:
    """Token-major view [L, D] of (request r, KV head j) gathered from the
    paged pool through the block table (layout only)."""
    ps = pool.shape[2]
    P = (L + ps - 1) // ps
    phys = block_table[r, :P].to(device=pool.device, dtype=torch.long)
    return pool[phys, j].reshape(P * ps, pool.shape[3])[:L]


def pool_from_tokens(tokens: List[torch.Tensor], block_table: torch.Tensor, num_phys: int,
                     page_size: int, fill: float = 0.0) -> torch.Tensor:
    """Scatter per-request token arrays [H_kv, L_r, D] into a paged pool
    [num_phys, H_kv, page_size, D] (layout only)."""
    H, _, D = tokens[0].shape
    pool = torch.full((num_phys, H, page_size, D), fill, dtype=tokens[0].dtype,
                      device=tokens[0].device)
    for r, t in enumerate(tokens):
        L = t.shape[1]
        P = (L + page_size - 1) // page_size
        pad = torch.full((H, P * page_size, D), fill, dtype=t.dtype, device=t.device)
        pad[:, :L] = t
        phys = block_table[r, :P].to(device=t.device, dtype=torch.long)
        pool[phys] = pad.view(H, P, page_size, D).transpose(0, 1)
    return pool
