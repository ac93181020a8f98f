"""Throughput of the blockwise Sparse GQA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload long_prefill_128k|prefill_32k]
                    [--no-decode] [--no-cpu-baseline] [--copy-calibration]

One step = one full-attention layer's prefill over the whole workload: compress -> index + top-k
-> tile union -> gathered-block attention (the four kernels behind sgqa_prefill), on synthetic
inputs already resident in HBM. `value` = prefill tokens per second. The same JSON line carries the
per-stage times (HIP events on the launch stream), the roofline of the dominant kernel (attention
on the matrix cores), the single-token decode step over the 262144-token cache (tokens/s and the
HBM roofline of its gather) and the CPU oracle timed on a bounded sample of the same workload.
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

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E peak (published)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="long_prefill_128k")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ablation", action="store_true")
    ap.add_argument("--no-other-prefill", action="store_true")
    ap.add_argument("--no-1m", action="store_true", help="skip the 1M-token prefill row of the other workloads")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode step of the 32 x 256K workload (no variants): for the decode profiles")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


# The files the prefill attention kernel is built from (the traffic profile is tied to their contents).
ATTEND_SOURCES = ("block_sparse_long_sgqa_amd/csrc/attend.hip", "block_sparse_long_sgqa_amd/csrc/attn_common.hpp")


def profiled_traffic(kernel: str, workload: str, sources):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 summary (FETCH_SIZE + WRITE_SIZE,
    calibrated), or None when there is none or the kernel's sources changed since it was taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_traffic.md")
    if not os.path.exists(path):
        return None
    blob = b"".join(open(os.path.join(ROOT, src), "rb").read() for src in sources)
    cur = hashlib.sha256(blob).hexdigest()[:16]
    for line in open(path):
        if line.startswith(f"traffic {kernel} "):
            kv = dict(t.split("=", 1) for t in line.split()[2:])
            return float(kv["bytes"]) if kv.get("source") == cur else None
    return None


# The files the decode step's kernels are built from.
DECODE_SOURCES = ("block_sparse_long_sgqa_amd/csrc/decode_select.hip", "block_sparse_long_sgqa_amd/csrc/attend.hip",
                  "block_sparse_long_sgqa_amd/csrc/attn_common.hpp")


def profiled_decode_traffic(workload: str):
    """HBM bytes of one decode step (every kernel of sgqa_decode, calibrated FETCH_SIZE + WRITE_SIZE)
    from the committed rocprofv3 summary, or None (none, or the sources changed since)."""
    if workload != "decode_256k":
        return None
    return profiled_traffic("decode_step", workload, DECODE_SOURCES)


def attended_pairs(umask, n_tokens: int, block: int, tile: int) -> int:
    """sum over (i, g) of |J(i,g)|: causally visible tokens of the tile union (exact count)."""
    import torch

    G, T, W = umask.shape
    shifts = torch.arange(32, device=umask.device, dtype=torch.int32)
    total = 0
    for g in range(G):
        bitsel = ((umask[g].unsqueeze(-1) >> shifts) & 1).reshape(T, W * 32).to(torch.int32)
        cum = torch.cumsum(bitsel, dim=1)  # blocks <= b in U
        i = torch.arange(n_tokens, device=umask.device)
        c = i // block
        t = i // tile
        below = torch.where(c > 0, cum[t, (c - 1).clamp(min=0)], torch.zeros_like(c, dtype=torch.int32))
        total += int((below.to(torch.int64) * block + (i - c * block + 1)).sum())
    return total


def flush_caches(torch, scratch):
    """Read a 1 GiB scratch buffer (a sum over it): evicts the 256 MiB last-level cache and every L2
    so that the next kernel reads its inputs from HBM. A read, not a write: after a write the caches
    hold dirty lines whose write-back would be charged to the timed kernel."""
    scratch.sum()


def cold_ms(torch, fn, reps: int, scratch) -> float:
    """Median over reps of one call of fn with the caches flushed before it (HIP events around the
    call alone)."""
    times = []
    for _ in range(reps):
        flush_caches(torch, scratch)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
    times.sort()
    return times[len(times) // 2]


class Timer:
    """HIP events on the stream the library launches on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.marks = []

    def mark(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        self.marks.append(e)

    def spans(self):
        return [a.elapsed_time(b) for a, b in zip(self.marks[:-1], self.marks[1:])]


def bench_prefill(sg, datagen, torch, wl, steps, warmup):
    p = sg.Params(n_tokens=wl.n_tokens, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, block=wl.block,
                  topk_tokens=wl.topk_tokens, union_tile=wl.union_tile)
    t0 = time.time()
    x = datagen.prefill_inputs(wl, device="cuda")
    torch.cuda.synchronize()
    log(f"{wl.name}: inputs drawn on the GPU in {time.time() - t0:.1f}s")
    o = sg.alloc_prefill_outputs(p)
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL)
    out_full = torch.empty_like(o["out"])

    def staged(timer=None):
        if timer:
            timer.mark()
        sg.sgqa_compress(p, x["ki"], o["blk_k"])
        if timer:
            timer.mark()
        sg.sgqa_index_topk(p, x["qi"], x["w"], o["blk_k"], o["topk"])
        if timer:
            timer.mark()
        sg.sgqa_union(p, o["topk"], o["umask"], o["ucount"])
        if timer:
            timer.mark()
        sg.sgqa_attend(p, x["q"], x["k"], x["v"], o["umask"], o["ucount"], o["out"])
        if timer:
            timer.mark()

    def whole():
        sg.sgqa_prefill(p, x["q"], x["k"], x["v"], x["qi"], x["w"], x["ki"], out_full, ws)

    for _ in range(warmup):
        whole()
        staged()
    torch.cuda.synchronize()
    # Timed region 1: the whole layer through sgqa_prefill.
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        whole()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_step = ev0.elapsed_time(ev1) / steps
    # Timed region 2: the same kernels through the single calls, with events between the stages.
    stage_ms = [0.0, 0.0, 0.0, 0.0]
    torch.cuda.synchronize()
    for _ in range(steps):
        tm = Timer(torch)
        staged(tm)
        torch.cuda.synchronize()
        for k, v in enumerate(tm.spans()):
            stage_ms[k] += v / steps
    same = bool(torch.equal(out_full.view(torch.int16), o["out"].view(torch.int16)))
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    union_cold_ms = cold_ms(torch, lambda: sg.sgqa_union(p, o["topk"], o["umask"], o["ucount"]), 10, scratch)
    del scratch
    variants = bench_variants(sg, torch, p, x, o, steps, warmup)
    pairs = attended_pairs(o["umask"], p.n_tokens, p.block, p.union_tile)
    r = p.n_q_heads // p.n_kv_heads
    attn_flops = 4.0 * p.head_dim * pairs * r
    n_blocks = p.n_tokens // p.block
    scored = scored_candidates(p.n_tokens, p.block, p.n_kv_heads)
    index_flops = 2.0 * p.idx_heads * p.idx_dim * scored
    ucount = o["ucount"].double()
    inflation = float((ucount.mean() * p.block / (p.topk_tokens + p.union_tile)).item())
    compress_bytes = p.n_tokens * p.idx_dim * 2 * (1 + 1 / p.block)
    union_bytes = p.n_kv_heads * p.n_tokens * p.kb * 4 + o["umask"].numel() * 4
    res = {
        "p": p,
        "ms_per_step": ms_step,
        "wall_s": wall,
        "stage_ms": dict(zip(["compress", "index_topk", "union", "attend"], stage_ms)),
        "prefill_matches_single_calls": same,
        "attended_pairs": pairs,
        "attn_flops": attn_flops,
        "index_flops": index_flops,
        "union_inflation": inflation,
        "compress_bytes": compress_bytes,
        "union_bytes": union_bytes,
        "union_cold_ms": union_cold_ms,
        "n_blocks": n_blocks,
        "variants": variants,
        "x": x,
    }
    return res


def bench_prefill_light(sg, datagen, torch, wl, steps, warmup):
    """A prefill workload other than the headline one: the whole layer through sgqa_prefill, the
    per-stage times of the single calls, the attention's matrix-core rate and the union inflation."""
    p = sg.Params(n_tokens=wl.n_tokens, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, block=wl.block,
                  topk_tokens=wl.topk_tokens, union_tile=wl.union_tile)
    x = datagen.prefill_inputs(wl, device="cuda")
    o = sg.alloc_prefill_outputs(p)
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL)
    out_full = torch.empty_like(o["out"])
    calls = [lambda: sg.sgqa_compress(p, x["ki"], o["blk_k"]),
             lambda: sg.sgqa_index_topk(p, x["qi"], x["w"], o["blk_k"], o["topk"]),
             lambda: sg.sgqa_union(p, o["topk"], o["umask"], o["ucount"]),
             lambda: sg.sgqa_attend(p, x["q"], x["k"], x["v"], o["umask"], o["ucount"], o["out"])]
    for _ in range(warmup):
        sg.sgqa_prefill(p, x["q"], x["k"], x["v"], x["qi"], x["w"], x["ki"], out_full, ws)
        for c in calls:
            c()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        sg.sgqa_prefill(p, x["q"], x["k"], x["v"], x["qi"], x["w"], x["ki"], out_full, ws)
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    stage = [0.0] * 4
    for _ in range(steps):
        tm = Timer(torch)
        tm.mark()
        for c in calls:
            c()
            tm.mark()
        torch.cuda.synchronize()
        for k, v in enumerate(tm.spans()):
            stage[k] += v / steps
    st = dict(zip(["compress", "index_topk", "union", "attend"], stage))
    pairs = attended_pairs(o["umask"], p.n_tokens, p.block, p.union_tile)
    attn_flops = 4.0 * p.head_dim * pairs * (p.n_q_heads // p.n_kv_heads)
    index_flops = 2.0 * p.idx_heads * p.idx_dim * scored_candidates(p.n_tokens, p.block, p.n_kv_heads)
    inflation = float((o["ucount"].double().mean() * p.block / (p.topk_tokens + p.union_tile)).item())
    res = {"workload": wl.name, "n_tokens": p.n_tokens, "union_tile": p.union_tile, "rho": wl.rho,
           "ms_per_step": ms_step, "tokens_per_s": p.n_tokens / (ms_step / 1e3), "stages_ms": st,
           "attend_TFLOP_per_s": attn_flops / (st["attend"] / 1e3) / 1e12,
           "attend_frac_of_bf16_peak": attn_flops / (st["attend"] / 1e3) / 1e12 / PEAK_BF16_TFLOPS,
           "index_topk_TFLOP_per_s": index_flops / (st["index_topk"] / 1e3) / 1e12,
           "union_inflation": inflation, "attended_pairs": pairs,
           "prefill_matches_single_calls": bool(torch.equal(out_full.view(torch.int16), o["out"].view(torch.int16)))}
    del x, o, ws, out_full
    torch.cuda.empty_cache()
    return res


def bench_variants(sg, torch, p, x, o, steps, warmup):
    """The other prefill calls on the same inputs: the fused selection -> union (what sgqa_prefill
    runs), the masked-union prefill, and the training pair sgqa_attend_fwd + sgqa_attend_bwd."""
    def timed(fn, n_steps):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n_steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n_steps

    N, Hq, G, D = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    res = {}
    m2 = torch.empty_like(o["umask"])
    c2 = torch.empty_like(o["ucount"])
    res["index_union_fused_ms"] = timed(lambda: sg.sgqa_index_union(p, x["qi"], x["w"], o["blk_k"], m2, c2), steps)
    res["index_union_fused_identical"] = bool(torch.equal(m2, o["umask"]) and torch.equal(c2, o["ucount"]))
    del m2, c2
    out = torch.empty((N, Hq, D), dtype=torch.bfloat16, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_PREFILL_MASKED)
    res["prefill_masked_ms"] = timed(
        lambda: sg.sgqa_prefill_masked(p, x["q"], x["k"], x["v"], x["qi"], x["w"], x["ki"], out, ws), max(1, steps // 3))
    del ws
    torch.cuda.empty_cache()
    lse = torch.empty((N, Hq), dtype=torch.float32, device="cuda")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(20261202)
    dout = torch.randn((N, Hq, D), generator=gen, device="cuda").to(torch.bfloat16)
    dq = torch.empty_like(out)
    dk = torch.empty((G, N, D), dtype=torch.bfloat16, device="cuda")
    dv = torch.empty_like(dk)
    ws = sg.workspace(p, sg.SGQA_OP_ATTEND_BWD)
    res["attend_fwd_lse_ms"] = timed(
        lambda: sg.sgqa_attend_fwd(p, x["q"], x["k"], x["v"], o["umask"], o["ucount"], out, lse), steps)
    res["attend_bwd_ms"] = timed(
        lambda: sg.sgqa_attend_bwd(p, x["q"], x["k"], x["v"], o["umask"], o["ucount"], out, lse, dout, dq, dk, dv, ws),
        max(1, steps // 3))
    del out, lse, dout, dq, dk, dv, ws
    torch.cuda.empty_cache()
    return res


def bench_decode(sg, datagen, torch, steps, warmup, wl=None, extras=True):
    """The decode step (and, with extras, the cache build, varlen/paged/FP8 decode). The roofline is
    taken on the cold step (caches flushed before every rep: the step's 134 MB of block keys would
    otherwise stay in the 256 MiB last-level cache between steps); the warm mean is reported too."""
    wl = wl or datagen.DECODE
    p = sg.Params(n_tokens=wl.n_tokens, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, block=wl.block,
                  topk_tokens=wl.topk_tokens, union_tile=1, n_seqs=wl.n_seqs)
    t0 = time.time()
    y = datagen.decode_inputs(wl, device="cuda")
    torch.cuda.synchronize()
    log(f"{wl.name}: caches drawn on the GPU in {time.time() - t0:.1f}s")
    blk = torch.empty((p.n_seqs, p.n_tokens // p.block, p.idx_dim), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((p.n_seqs, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device="cuda")
    ws = sg.workspace(p, sg.SGQA_OP_DECODE)
    for _ in range(warmup):
        sg.sgqa_compress(p, y["ki_cache"], blk)
        sg.sgqa_decode(p, y["q"], y["k_cache"], y["v_cache"], blk, y["qi"], y["w"], out, ws)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    ev[0].record()
    for _ in range(steps):
        sg.sgqa_compress(p, y["ki_cache"], blk)
    ev[1].record()
    for _ in range(steps):
        sg.sgqa_decode(p, y["q"], y["k_cache"], y["v_cache"], blk, y["qi"], y["w"], out, ws)
    ev[2].record()
    torch.cuda.synchronize()
    compress_ms = ev[0].elapsed_time(ev[1]) / steps
    warm_ms = ev[1].elapsed_time(ev[2]) / steps
    scratch = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    step_ms = cold_ms(torch, lambda: sg.sgqa_decode(p, y["q"], y["k_cache"], y["v_cache"], blk, y["qi"], y["w"], out,
                                                    ws), max(steps, 10), scratch)
    compress_cold_ms = cold_ms(torch, lambda: sg.sgqa_compress(p, y["ki_cache"], blk), max(steps, 10), scratch)
    del scratch
    c = (p.n_tokens - 1) // p.block
    gather_bytes = p.n_seqs * p.n_kv_heads * (p.kb + 1) * p.block * p.head_dim * 2 * 2
    index_bytes = p.n_seqs * c * p.idx_dim * 2
    qo_bytes = 2 * p.n_seqs * p.n_q_heads * p.head_dim * 2
    step_bytes = gather_bytes + index_bytes + qo_bytes
    cache_build_bytes = p.n_seqs * p.n_tokens * p.idx_dim * 2 * (1 + 1 / p.block)
    res = {
        "metric": "decode tok/s",
        "value": p.n_seqs / (step_ms / 1e3),
        "unit": "tokens/s",
        "ms_per_step": step_ms,
        "timing": "cold: median of single steps, a 1 GiB read before each flushes the caches",
        "warm_ms_per_step": warm_ms,
        "config": {"workload": wl.name, "n_seqs": p.n_seqs, "ctx": p.n_tokens, "n_q_heads": p.n_q_heads,
                   "n_kv_heads": p.n_kv_heads, "block": p.block, "topk_tokens": p.topk_tokens},
        "roofline": {"bound": "hbm", "achieved": step_bytes / (step_ms / 1e3) / 1e9, "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": step_bytes / (step_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
                     "traffic": profiled_decode_traffic(wl.name), "algorithmic_bytes_per_step": step_bytes},
        "warm_roofline_frac": step_bytes / (warm_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "cache_compress": {"ms": compress_ms, "bytes": cache_build_bytes,
                           "GB_per_s": cache_build_bytes / (compress_ms / 1e3) / 1e9,
                           "cold_ms": compress_cold_ms,
                           "cold_GB_per_s": cache_build_bytes / (compress_cold_ms / 1e3) / 1e9},
    }
    if extras:
        res["varlen"] = bench_decode_varlen(sg, torch, p, y, blk, out, ws, steps, warmup)
        res["fp8"] = bench_decode_fp8(sg, datagen, torch, wl, p, y, blk, out, ws, steps, warmup,
                                      gather_bytes // 2 + index_bytes + qo_bytes)
    del y
    torch.cuda.empty_cache()
    return res


def scored_candidates(n_tokens: int, block: int, n_groups: int) -> int:
    """Sum over queries i < N of c(i) = floor(i/B), times the groups: the (row, block) pairs scored."""
    q_, r_ = divmod(n_tokens, block)
    return n_groups * (block * q_ * (q_ - 1) // 2 + r_ * q_)


def token_coverage(torch, sel1, selb, block: int, i_min: int = 0, rows_per_chunk: int = 4096) -> float:
    """Mean over rows (g, i >= i_min) of |T1 & TB| / |T1|: T1 = the token-level selection plus token i,
    TB = the tokens of the block-level selection plus the own block's visible tokens (every token of
    T1 is <= i, so a T1 token is covered iff its block is selected or is i's own block).
    sel1 [G, N, K1] token ids, selb [G, N, KB] block ids, both -1 padded (GPU tensors)."""
    G, N, _ = sel1.shape
    nbc = (N + block - 1) // block
    total = 0.0
    rows = 0
    for g in range(G):
        for i0 in range(i_min, N, rows_per_chunk):
            i1 = min(N, i0 + rows_per_chunk)
            s1 = sel1[g, i0:i1].long()
            sb = selb[g, i0:i1].long()
            R = i1 - i0
            inb = torch.zeros((R, nbc + 1), dtype=torch.bool, device=sel1.device)
            inb.scatter_(1, torch.where(sb >= 0, sb, torch.full_like(sb, nbc)), True)
            own = (torch.arange(i0, i1, device=sel1.device) // block).unsqueeze(1)
            inb.scatter_(1, own, True)
            valid = s1 >= 0
            hit = torch.gather(inb, 1, torch.where(valid, s1 // block, torch.full_like(s1, nbc))) & valid
            cov = (hit.sum(1).double() + 1.0) / (valid.sum(1).double() + 1.0)  # + token i itself
            total += float(cov.sum().item())
            rows += R
    return total / rows


def bench_ablation(sg, datagen, torch, steps, warmup):
    """Granularity ablation on the 32K prefill inputs: index + top-k at (B = 1, k = 2048) against
    compress + index + top-k at (B = 8, k = 4096), on the same indexer queries and keys."""
    wl = datagen.PREFILL
    x = datagen.prefill_inputs(wl, device="cuda")
    N, G = wl.n_tokens, wl.n_kv_heads
    out = {}
    sels = {}
    for B, k in ((1, 2048), (8, 4096)):
        p = sg.Params(n_tokens=N, n_q_heads=wl.n_q_heads, n_kv_heads=G, block=B, topk_tokens=k,
                      union_tile=wl.union_tile)
        blk = torch.empty((N // B, p.idx_dim), dtype=torch.bfloat16, device="cuda")
        topk = torch.empty((G, N, p.kb), dtype=torch.int32, device="cuda")

        def run():
            if B > 1:
                sg.sgqa_compress(p, x["ki"], blk)
                sg.sgqa_index_topk(p, x["qi"], x["w"], blk, topk)
            else:  # B = 1: the block keys are the index keys themselves
                sg.sgqa_index_topk(p, x["qi"], x["w"], x["ki"], topk)

        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            run()
        e1.record()
        torch.cuda.synchronize()
        out[f"B{B}_k{k}_ms"] = e0.elapsed_time(e1) / steps
        out[f"B{B}_k{k}_scored_pairs"] = scored_candidates(N, B, G)
        sels[B] = topk
    out["time_ratio_B1_over_B8"] = out["B1_k2048_ms"] / out["B8_k4096_ms"]
    out["count_ratio_B1_over_B8"] = out["B1_k2048_scored_pairs"] / out["B8_k4096_scored_pairs"]
    out["token_coverage_B8_vs_B1"] = token_coverage(torch, sels[1], sels[8], 8)
    out["token_coverage_B8_vs_B1_rows_past_k"] = token_coverage(torch, sels[1], sels[8], 8, i_min=4096)
    out["workload"] = "prefill_32k inputs (C1), B=1 k=2048 vs B=8 k=4096"
    del x, sels
    torch.cuda.empty_cache()
    return out


def achieved_peaks(torch):
    """Reference rates measured on this GPU next to the published peaks: a 2 GiB device copy (bytes
    read + written) and a large bf16 GEMM (the vendor library)."""
    a = torch.empty(1 << 30, dtype=torch.int16, device="cuda").fill_(1)
    b = torch.empty_like(a)
    m = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    n = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    for _ in range(3):
        b.copy_(a)
        torch.matmul(m, n)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    for _ in range(10):
        b.copy_(a)
    e[1].record()
    for _ in range(10):
        torch.matmul(m, n)
    e[2].record()
    torch.cuda.synchronize()
    copy_s = e[0].elapsed_time(e[1]) / 10 / 1e3
    gemm_s = e[1].elapsed_time(e[2]) / 10 / 1e3
    res = {"copy_GB_per_s": 2 * a.numel() * 2 / copy_s / 1e9, "spec_hbm_GB_per_s": PEAK_HBM_GBS,
           "gemm_bf16_TFLOP_per_s": 2.0 * 8192 ** 3 / gemm_s / 1e12, "spec_bf16_TFLOP_per_s": PEAK_BF16_TFLOPS}
    del a, b, m, n
    torch.cuda.empty_cache()
    return res


def decode_step_bytes(p, lens) -> int:
    """Algorithmic bytes of one decode step at per-sequence lengths: the block keys of every candidate,
    the K/V rows of Sel + own block, q in and out."""
    total = 0
    for L in lens:
        c = (L - 1) // p.block
        kb = min(p.kb, c)
        own = L - (L - 1) // p.block * p.block
        total += c * p.idx_dim * 2 + p.n_kv_heads * (kb * p.block + own) * p.head_dim * 2 * 2
    return total + 2 * len(lens) * p.n_q_heads * p.head_dim * 2


def bench_decode_varlen(sg, torch, p, y, blk, out, ws, steps, warmup):
    """Incremental-decode calls on the decode workload's shapes: varlen decode with sequence lengths
    drawn uniformly from [L/2, L] (seeded), on the dense caches and on a paged pool (64-token pages,
    shuffled page table), and one sgqa_append of a token per sequence."""
    S, C = p.n_seqs, p.n_tokens
    g = torch.Generator(device="cuda")
    g.manual_seed(20261202)
    lens = torch.randint(C // 2, C + 1, (S,), generator=g, device="cuda", dtype=torch.int32)
    lens_l = [int(v) for v in lens.cpu()]
    bytes_step = decode_step_bytes(p, lens_l)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / steps

    res = {"lens": "uniform in [L/2, L], seeded", "mean_len": sum(lens_l) / S}
    ms = timed(lambda: sg.sgqa_decode_varlen(p, y["q"], y["k_cache"], y["v_cache"], blk, y["qi"], y["w"], lens, out, ws))
    res["dense"] = {"ms_per_step": ms, "tokens_per_s": S / (ms / 1e3),
                    "GB_per_s": bytes_step / (ms / 1e3) / 1e9, "hbm_frac": bytes_step / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}
    # Paged pool: its own data (the throughput does not depend on the values).
    pt = 64
    per = C // pt
    n_pages = S * per
    pool_shape = (n_pages, p.n_kv_heads, pt, p.head_dim)
    kpool = torch.empty(pool_shape, dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    vpool = torch.empty(pool_shape, dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    table = torch.randperm(n_pages, generator=g, device="cuda").to(torch.int32).view(S, per)
    pages = sg.Pages(table, pt, n_pages)
    ms = timed(lambda: sg.sgqa_decode_varlen(p, y["q"], kpool, vpool, blk, y["qi"], y["w"], lens, out, ws,
                                             pages=pages))
    res["paged_64"] = {"ms_per_step": ms, "tokens_per_s": S / (ms / 1e3),
                       "GB_per_s": bytes_step / (ms / 1e3) / 1e9,
                       "hbm_frac": bytes_step / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}
    # Append of one token per sequence into the paged pool (positions = lens - 1, in place).
    idx_cache = y["ki_cache"]
    k_new = torch.empty((S, p.n_kv_heads, p.head_dim), dtype=torch.bfloat16, device="cuda").normal_(generator=g)
    i_new = y["ki_cache"][:, 0].contiguous()
    pos = lens - 1
    ms = timed(lambda: sg.sgqa_append(p, k_new, k_new, i_new, pos, kpool, vpool, idx_cache, blk, pages=pages))
    res["append_ms"] = ms
    res["step_bytes"] = bytes_step
    del kpool, vpool
    torch.cuda.empty_cache()
    return res


def bench_decode_fp8(sg, datagen, torch, wl, p, y, blk, out, ws, steps, warmup, step_bytes):
    """The decode step of the same workload over FP8 E4M3 K/V caches (sgqa_decode_fp8, dense, every
    sequence at full length): the K/V gather reads half the bytes of the bf16 step."""
    del y["k_cache"], y["v_cache"]
    torch.cuda.empty_cache()
    f = datagen.fp8_caches(wl, device="cuda")

    def step():
        sg.sgqa_decode_fp8(p, y["q"], f["k8"], f["v8"], f["kv_scale"], blk, y["qi"], y["w"], out, ws)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del f
    torch.cuda.empty_cache()
    return {"ms_per_step": ms, "tokens_per_s": p.n_seqs / (ms / 1e3), "step_bytes": step_bytes,
            "GB_per_s": step_bytes / (ms / 1e3) / 1e9,
            "hbm_frac": step_bytes / (ms / 1e3) / 1e9 / PEAK_HBM_GBS}


def host_cpu() -> dict:
    """Model, sockets, cores and hardware threads of the host (lscpu, else /proc/cpuinfo)."""
    import subprocess

    info = {}
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            k, _, v = line.partition(":")
            info[k.strip()] = v.strip()
    except (OSError, subprocess.SubprocessError):
        pass
    model = info.get("Model name")
    if not model and os.path.exists("/proc/cpuinfo"):
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    res = {"model": model, "sockets": info.get("Socket(s)"), "cores_per_socket": info.get("Core(s) per socket"),
           "threads_per_core": info.get("Thread(s) per core"), "cpus_online": info.get("CPU(s)") or os.cpu_count()}
    try:
        res["cpus_usable"] = len(os.sched_getaffinity(0))
    except AttributeError:
        pass
    return res


def cpu_baseline(oracle, datagen, torch, np, res, wl, decode_res):
    """The oracle as it is, on a bounded sample of the same prefill: whole union tiles spread over
    the sequence (mean position ~ N/2), every group; each stage wall-clocked on its own (block
    compression of the whole sequence, index + top-k of every query of the sampled tiles, the union
    (a pass over the whole [G][N][K_B] selection array), attention of the sampled queries), with the
    GPU's time for the same work (stage time scaled to the sampled rows) and the speed-up. Plus the
    oracle's decode of one sequence of the decode workload against the GPU step per sequence."""
    import numpy as np  # noqa: F811

    p = res["p"]
    x = res["x"]

    def bits(t):
        return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)

    host = {k: bits(x[k]) for k in ("q", "k", "v", "qi", "ki")}
    w = x["w"].cpu().numpy()
    T = p.n_tiles
    n_sample_tiles = 4 if p.n_tokens >= 65536 else 8
    tiles = [int((2 * s + 1) * T // (2 * n_sample_tiles)) for s in range(n_sample_tiles)]
    rows = np.concatenate([np.arange(t * p.union_tile, min(p.n_tokens, (t + 1) * p.union_tile)) for t in tiles])
    rows = rows.astype(np.int32)
    threads = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or os.cpu_count()
    wall = {}
    t0 = time.perf_counter()
    kbar = oracle.compress(host["ki"], p.block)
    wall["compress"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    sel = oracle.index_topk(host["qi"], w, kbar, p.block, p.kb, rows=rows)
    wall["index_topk"] = time.perf_counter() - t0
    full = np.full((p.n_kv_heads, p.n_tokens, p.kb), -1, dtype=np.int32)
    full[:, rows] = sel
    t0 = time.perf_counter()
    umask, _ = oracle.union(full, p.n_tokens, p.block, p.union_tile)
    wall["union"] = time.perf_counter() - t0
    del full
    t0 = time.perf_counter()
    oracle.attend(host["q"], host["k"], host["v"], umask, p.block, p.union_tile, rows=rows)
    wall["attend"] = time.perf_counter() - t0
    dt = sum(wall.values())
    frac = len(rows) / p.n_tokens  # the GPU's share of a stage for the sampled rows
    st = res["stage_ms"]
    gpu = {"compress": st["compress"] / 1e3, "index_topk": st["index_topk"] / 1e3 * frac, "union": st["union"] / 1e3,
           "attend": st["attend"] / 1e3 * frac}
    stages = {k: {"oracle_s": wall[k], "gpu_s": gpu[k], "speedup": wall[k] / gpu[k] if gpu[k] > 0 else None}
              for k in wall}
    out = {"value": len(rows) / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
           "sample": f"{len(rows)} queries = {n_sample_tiles} whole union tiles of {p.union_tile} spread over "
                     f"the {p.n_tokens}-token sequence (tiles {tiles}), all {p.n_kv_heads} groups and "
                     f"{p.n_q_heads} heads; compress of all keys + index/top-k + union + attention; "
                     f"{dt:.1f} s wall",
           "stages": stages, "host": host_cpu()}
    if decode_res is not None:
        wl_d = datagen.DECODE
        y = datagen.decode_inputs(wl_d, device="cuda", n_seqs=1)
        t0 = time.perf_counter()
        kbar_d = oracle.compress(bits(y["ki_cache"]), wl_d.block)
        oracle.decode(bits(y["q"]), bits(y["k_cache"]), bits(y["v_cache"]), kbar_d, bits(y["qi"]), y["w"],
                      wl_d.block, wl_d.kb)
        dd = time.perf_counter() - t0
        gpu_seq = decode_res["ms_per_step"] / 1e3 / decode_res["config"]["n_seqs"]
        out["decode"] = {"oracle_s_per_sequence": dd, "gpu_s_per_sequence": gpu_seq, "speedup": dd / gpu_seq,
                         "sample": f"1 sequence of the {wl_d.name} workload (L={wl_d.n_tokens}): block keys of the "
                                   f"whole cache, selection and attention"}
        del y
        torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import block_sparse_long_sgqa_amd as sg
    import datagen

    if not os.path.exists(sg.LIB_PATH):
        from block_sparse_long_sgqa_amd import build as hip_build

        hip_build.build()
    sg.lib()
    wl = datagen.WORKLOADS[args.workload]
    log(f"workload {wl.name}: N={wl.n_tokens} Hq={wl.n_q_heads} G={wl.n_kv_heads} B={wl.block} "
        f"k={wl.topk_tokens} Tq={wl.union_tile}")

    if args.copy_calibration:
        # A plain streaming kernel of known size for the HBM byte counters: read 1 GiB, write 1 GiB
        # (in-place multiply), after a 2 GiB write that evicts the source from the caches.
        a = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
        evict = torch.zeros(1 << 29, dtype=torch.float32, device="cuda")
        torch.cuda.synchronize()
        a.mul_(2.0)
        torch.cuda.synchronize()
        del a, evict

    if args.decode_only:
        d = bench_decode(sg, datagen, torch, args.steps, args.warmup, extras=False)
        print(json.dumps(dict(d, n_gpus=1, steps=args.steps, warmup=args.warmup, higher_is_better=True,
                              scaling="weak", vs_baseline=None, dtype="bf16",
                              data="synthetic (seeded; shapes and value structure of the pages' setting)")),
              flush=True)
        return
    res = bench_prefill(sg, datagen, torch, wl, args.steps, args.warmup)
    p = res["p"]
    st = res["stage_ms"]
    attn_tflops = res["attn_flops"] / (st["attend"] / 1e3) / 1e12
    line = {
        "metric": "prefill tokens/s (one full-attention layer, B=8 k=4096)",
        "value": p.n_tokens / (res["ms_per_step"] / 1e3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; shapes and value structure of the pages' setting)",
        "config": {"workload": wl.name, "n_tokens": p.n_tokens, "n_q_heads": p.n_q_heads,
                   "n_kv_heads": p.n_kv_heads, "head_dim": p.head_dim, "block": p.block,
                   "topk_tokens": p.topk_tokens, "union_tile": p.union_tile, "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "attend", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": attn_tflops / PEAK_BF16_TFLOPS,
                     "traffic": profiled_traffic("attend", "long_prefill_128k", ATTEND_SOURCES)
                     if wl.name == "long_prefill_128k" else None,
                     "algorithmic_flops_per_launch": res["attn_flops"]},
        "stages_ms": st,
        "stage_rooflines": {
            "compress": {"bound": "hbm", "GB_per_s": res["compress_bytes"] / (st["compress"] / 1e3) / 1e9},
            "index_topk": {"bound": "mfma", "TFLOP_per_s": res["index_flops"] / (st["index_topk"] / 1e3) / 1e12},
            "union": {"bound": "hbm", "GB_per_s": res["union_bytes"] / (st["union"] / 1e3) / 1e9},
            "attend": {"bound": "mfma", "TFLOP_per_s": attn_tflops},
        },
        "variants": dict(res["variants"], **{
            # the four gradient products dV = P^T dO, dP = dO V^T, dQ = dS K, dK = dS^T Q over the
            # attended pairs (the score recompute is not counted)
            "attend_bwd_TFLOP_per_s": 2.0 * res["attn_flops"] / (res["variants"]["attend_bwd_ms"] / 1e3) / 1e12}),
        "union_inflation": res["union_inflation"],
        "attended_pairs": res["attended_pairs"],
        "union_cold": {"ms": res["union_cold_ms"],
                       "GB_per_s": res["union_bytes"] / (res["union_cold_ms"] / 1e3) / 1e9},
        "prefill_matches_single_calls": res["prefill_matches_single_calls"],
    }
    decode_res = None
    if not args.no_decode:
        keep = {k: res[k] for k in ("p", "x", "stage_ms")}
        del res
        torch.cuda.empty_cache()
        decode_res = bench_decode(sg, datagen, torch, args.steps, args.warmup)
        line["decode"] = decode_res
        log("decode at L=131072 (the metric's 128K context)")
        line["decode"]["ctx_131072"] = bench_decode(sg, datagen, torch, args.steps, args.warmup,
                                                     wl=datagen.DECODE.replace(name="decode_128k", n_tokens=131072),
                                                     extras=False)
        res = keep
    if not args.no_cpu_baseline:
        import oracle

        log("timing the CPU oracle on a bounded sample")
        line["cpu_baseline"] = cpu_baseline(oracle, datagen, torch, np, res, wl, decode_res)
    del res
    torch.cuda.empty_cache()
    if not args.no_other_prefill and wl.name == "long_prefill_128k":
        log("other prefill workloads: 32K and the 32K i.i.d.-query stress row")
        line["other_prefill"] = {w.name: bench_prefill_light(sg, datagen, torch, w, args.steps, args.warmup)
                                 for w in (datagen.PREFILL, datagen.PREFILL_IID)}
        if not args.no_1m:
            # The context length the pages' architecture aims at: one pass (about 2.5 s of GPU work).
            w1m = datagen.LONG_PREFILL.replace(name="long_prefill_1m", n_tokens=1 << 20)
            log("1M-token prefill (one timed pass)")
            line["other_prefill"][w1m.name] = bench_prefill_light(sg, datagen, torch, w1m, 1, 1)
            torch.cuda.empty_cache()
    if not args.no_ablation:
        log("granularity ablation on the 32K inputs")
        line["ablation"] = bench_ablation(sg, datagen, torch, 3, 1)
        line["achieved_peaks"] = achieved_peaks(torch)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
