"""Seeded synthetic inputs for the blockwise Sparse GQA path.

This module only draws random numbers and arranges them into the shapes and structures of the
workloads. It holds none of the method's arithmetic, so both the CPU oracle and the HIP library's
tests and benchmark take their inputs from here.

Value recipes (shared by every workload):
  * q, k, v: N(0, 1) drawn in fp32 and rounded to bf16 (nearest-even).
  * index queries / keys: integers uniform in {-4, ..., 4}, stored exactly in bf16, so block means
    and fp32 score sums are exact (every intermediate is a multiple of 1/B well inside 2^24).
  * indexer weights w[g][h]: 1 (tiny) or uniform in {1, 2}.
  * FP8 K/V caches: N(0, 16^2) drawn in fp32 and converted to E4M3 codes by torch's float8_e4m3fn
    cast (nearest-even; |x| <= 448 always holds in practice), stored as uint8; scales per
    (sequence, group) and K/V uniform in [1/32, 1/16] fp32, so the attended rows have a standard
    deviation of 0.5 .. 1.
  * "adjacent-token correlated" index queries: for every (group, head) an anchor vector per
    segment of 256 queries; every coordinate of a query is redrawn independently with probability
    rho (default 1/8). rho = 1 gives independent queries (stress case).
  * "planted clusters" (long prefill): 16 centre vectors; 16 non-overlapping spans of 2048 index
    keys copy a centre with every coordinate redrawn with probability 1/8. For half of the query
    segments and every group the anchor of all indexer heads is a centre whose span lies wholly
    before the segment, so top-k concentrates on planted spans.

Determinism: every tensor has its own seed derived from (seed0, workload name, tensor name).
A tensor drawn on the CPU is identical on every machine with this torch version. The indexer inputs
of a prefill workload (index queries, index keys, weights) are always drawn on the CPU and then
moved, so stored digests of the oracle's full selections can be recomputed from them anywhere;
q, k, v and the decode caches of large workloads are drawn on the GPU (torch's Philox generator)
and copied to the host where they are checked.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Optional

import torch

SEED0 = 20261202


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_tokens: int          # N (prefill) or L (decode, including the query token)
    n_q_heads: int         # Hq
    n_kv_heads: int        # G
    head_dim: int          # D
    idx_heads: int         # H_I
    idx_dim: int           # d_I
    block: int             # B
    topk_tokens: int       # k
    union_tile: int        # Tq (1 for decode)
    n_seqs: int = 1        # S (decode)
    weights: str = "12"    # "ones" or "12" (uniform in {1, 2})
    qi_mode: str = "corr"  # "iid" or "corr"
    ki_mode: str = "iid"   # "iid" or "clusters"
    rho: float = 0.125
    decode: bool = False

    @property
    def kb(self) -> int:
        return self.topk_tokens // self.block

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads of the measurement plan (shapes and value structures of the pages' setting:
# B = 8, k = 4096 tokens = 512 blocks, GQA 64/8 heads, head_dim 128, 4 indexer heads of dim 64).
TINY = Workload("tiny_prefill_2k", 2048, 8, 1, 128, 4, 64, 8, 256, 16, weights="ones", qi_mode="iid")
PREFILL = Workload("prefill_32k", 32768, 64, 8, 128, 4, 64, 8, 4096, 64)
LONG_PREFILL = Workload("long_prefill_128k", 131072, 64, 8, 128, 4, 64, 8, 4096, 128, ki_mode="clusters")
DECODE = Workload("decode_256k", 262144, 64, 8, 128, 4, 64, 8, 4096, 1, n_seqs=32, decode=True, qi_mode="iid")
ABLATION_B1 = PREFILL.replace(name="ablation_32k_b1_k2048", block=1, topk_tokens=2048)
ABLATION_B8 = PREFILL.replace(name="ablation_32k_b8_k4096")
# rho = 1: neighbouring queries are unrelated, so the tile unions are nearly dense (stress case).
PREFILL_IID = PREFILL.replace(name="prefill_32k_iid", rho=1.0)

WORKLOADS = {w.name: w for w in (TINY, PREFILL, LONG_PREFILL, DECODE, ABLATION_B1, ABLATION_B8, PREFILL_IID)}


def tensor_seed(seed0: int, workload: str, tensor: str) -> int:
    h = hashlib.sha256(f"{seed0}/{workload}/{tensor}".encode()).hexdigest()
    return int(h[:15], 16)


class _Draw:
    """Per-tensor seeded generators on one device."""

    def __init__(self, wl: Workload, device, seed0: int):
        self.wl = wl
        self.device = torch.device(device)
        self.seed0 = seed0

    def gen(self, tensor: str) -> torch.Generator:
        g = torch.Generator(device=self.device)
        g.manual_seed(tensor_seed(self.seed0, self.wl.name, tensor))
        return g

    def normal_bf16(self, tensor: str, shape) -> torch.Tensor:
        x = torch.randn(shape, generator=self.gen(tensor), device=self.device, dtype=torch.float32)
        return x.to(torch.bfloat16)

    def int_bf16(self, tensor: str, shape, gen: Optional[torch.Generator] = None) -> torch.Tensor:
        g = gen if gen is not None else self.gen(tensor)
        return torch.randint(-4, 5, shape, generator=g, device=self.device, dtype=torch.int16).to(torch.bfloat16)

    def weights(self) -> torch.Tensor:
        wl = self.wl
        if wl.weights == "ones":
            return torch.ones((wl.n_kv_heads, wl.idx_heads), device=self.device, dtype=torch.float32)
        g = self.gen("w")
        return torch.randint(1, 3, (wl.n_kv_heads, wl.idx_heads), generator=g, device=self.device,
                             dtype=torch.int32).to(torch.float32)


def _cluster_layout(wl: Workload, draw: _Draw, n_clusters: int = 16, span: int = 2048):
    """Centres [C][dI], span starts [C] (token index), chosen among the N/span aligned slots."""
    g = draw.gen("clusters")
    slots = wl.n_tokens // span
    n_clusters = min(n_clusters, slots)
    perm = torch.randperm(slots, generator=g, device=draw.device)[:n_clusters]
    starts = torch.sort(perm).values * span
    centres = torch.randint(-4, 5, (n_clusters, wl.idx_dim), generator=g, device=draw.device, dtype=torch.int16)
    return centres, starts, span


def index_keys(wl: Workload, draw: _Draw) -> torch.Tensor:
    """Shared index keys ki [N][dI] (bf16 integers)."""
    N, dI = wl.n_tokens, wl.idx_dim
    g = draw.gen("ki")
    ki = torch.randint(-4, 5, (N, dI), generator=g, device=draw.device, dtype=torch.int16)
    if wl.ki_mode == "clusters":
        centres, starts, span = _cluster_layout(wl, draw)
        for c in range(centres.shape[0]):
            s0 = int(starts[c])
            redraw = torch.rand((span, dI), generator=g, device=draw.device) < 0.125
            fresh = torch.randint(-4, 5, (span, dI), generator=g, device=draw.device, dtype=torch.int16)
            ki[s0:s0 + span] = torch.where(redraw, fresh, centres[c].expand(span, dI))
    return ki.to(torch.bfloat16)


def index_queries(wl: Workload, draw: _Draw, n_rows: int, tensor: str = "qi") -> torch.Tensor:
    """Per-group index queries [n_rows][G][H_I][d_I] (bf16 integers)."""
    G, HI, dI = wl.n_kv_heads, wl.idx_heads, wl.idx_dim
    g = draw.gen(tensor)
    fresh = torch.randint(-4, 5, (n_rows, G, HI, dI), generator=g, device=draw.device, dtype=torch.int16)
    if wl.qi_mode == "iid" or wl.rho >= 1.0:
        return fresh.to(torch.bfloat16)
    seg = 256
    n_seg = (n_rows + seg - 1) // seg
    anchors = torch.randint(-4, 5, (n_seg, G, HI, dI), generator=g, device=draw.device, dtype=torch.int16)
    if wl.ki_mode == "clusters":
        centres, starts, span = _cluster_layout(wl, draw)
        use = torch.rand((n_seg, G), generator=g, device=draw.device) < 0.5
        pick = torch.randint(0, 1 << 30, (n_seg, G), generator=g, device=draw.device)
        for m in range(n_seg):
            before = int(((starts + span) <= m * seg).sum())  # clusters wholly before the segment
            if before == 0:
                continue
            for gg in range(G):
                if bool(use[m, gg]):
                    c = int(pick[m, gg]) % before
                    anchors[m, gg, :, :] = centres[c]
    redraw = torch.rand((n_rows, G, HI, dI), generator=g, device=draw.device) < wl.rho
    seg_of = torch.arange(n_rows, device=draw.device) // seg
    base = anchors[seg_of]
    return torch.where(redraw, fresh, base).to(torch.bfloat16)


def index_inputs(wl: Workload, seed0: int = SEED0) -> dict:
    """The indexer inputs of one prefill layer, drawn on the CPU: qi [N][G][HI][dI], ki [N][dI]
    (bf16) and w [G][HI] (fp32)."""
    h = _Draw(wl, "cpu", seed0)
    return {"qi": index_queries(wl, h, wl.n_tokens), "ki": index_keys(wl, h), "w": h.weights()}


def prefill_inputs(wl: Workload, device="cpu", seed0: int = SEED0) -> dict:
    """All inputs of one prefill layer: q [N][Hq][D], k/v [G][N][D], qi [N][G][HI][dI],
    ki [N][dI] (bf16) and w [G][HI] (fp32). The indexer inputs come from index_inputs()."""
    d = _Draw(wl, device, seed0)
    N, Hq, G, D = wl.n_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim
    x = {
        "q": d.normal_bf16("q", (N, Hq, D)),
        "k": d.normal_bf16("k", (G, N, D)),
        "v": d.normal_bf16("v", (G, N, D)),
    }
    for name, t in index_inputs(wl, seed0).items():
        x[name] = t.to(d.device)
    return x


def decode_inputs(wl: Workload, device="cpu", seed0: int = SEED0, n_seqs: Optional[int] = None) -> dict:
    """All inputs of one decode step: q [S][Hq][D], k/v cache [S][G][L][D], ki cache [S][L][dI],
    qi [S][G][HI][dI] (bf16) and w [G][HI] (fp32). Caches are drawn one sequence at a time."""
    d = _Draw(wl, device, seed0)
    S = wl.n_seqs if n_seqs is None else n_seqs
    L, Hq, G, D, dI = wl.n_tokens, wl.n_q_heads, wl.n_kv_heads, wl.head_dim, wl.idx_dim
    kc = torch.empty((S, G, L, D), dtype=torch.bfloat16, device=d.device)
    vc = torch.empty((S, G, L, D), dtype=torch.bfloat16, device=d.device)
    ki = torch.empty((S, L, dI), dtype=torch.bfloat16, device=d.device)
    for s in range(S):
        kc[s] = d.normal_bf16(f"k_cache/{s}", (G, L, D))
        vc[s] = d.normal_bf16(f"v_cache/{s}", (G, L, D))
        ki[s] = d.int_bf16(f"ki_cache/{s}", (L, dI))
    return {
        "q": d.normal_bf16("q", (S, Hq, D)),
        "k_cache": kc,
        "v_cache": vc,
        "ki_cache": ki,
        "qi": index_queries(wl, d, S),
        "w": d.weights(),
    }


def fp8_caches(wl: Workload, device="cpu", seed0: int = SEED0, n_seqs: Optional[int] = None) -> dict:
    """FP8 E4M3 K/V caches for a decode workload: k8, v8 [S][G][L][D] uint8 codes and kv_scale
    [S][G][2] fp32 (key scale, value scale). Drawn one sequence at a time."""
    d = _Draw(wl, device, seed0)
    S = wl.n_seqs if n_seqs is None else n_seqs
    L, G, D = wl.n_tokens, wl.n_kv_heads, wl.head_dim
    k8 = torch.empty((S, G, L, D), dtype=torch.uint8, device=d.device)
    v8 = torch.empty((S, G, L, D), dtype=torch.uint8, device=d.device)
    for s in range(S):
        for name, dst in (("k8", k8), ("v8", v8)):
            x = torch.randn((G, L, D), generator=d.gen(f"{name}/{s}"), device=d.device, dtype=torch.float32)
            dst[s] = (x * 16.0).to(torch.float8_e4m3fn).view(torch.uint8)
            del x
    u = torch.rand((S, G, 2), generator=d.gen("kv_scale"), device=d.device, dtype=torch.float32)
    return {"k8": k8, "v8": v8, "kv_scale": (1.0 + u) / 32.0}


def default_scale(head_dim: int) -> float:
    return 1.0 / math.sqrt(head_dim)
