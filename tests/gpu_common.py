"""Shared helpers of the GPU parity tests: device inputs, oracle chains and comparisons.

Inputs come from ``datagen`` only; expected values come from ``oracle`` only (never from the HIP
path). The HIP path is reached exclusively through the C ABI binding.
"""
from __future__ import annotations

import numpy as np
import torch

import block_sparse_long_sgqa_amd as sg
import datagen
import oracle

# Attention tolerance on unit-scale outputs (max-abs and mean-abs error against the fp64 oracle).
# The max-abs bar scales with the output where an output exceeds unit scale (queries attending a
# handful of keys return nearly single V rows, up to ~4.5 for N(0,1) values): per element
# |got - want| <= MAX_ABS * max(1, |want|). Rounding the exact output to the bf16 result alone costs
# up to 2^-9 |want|, 0.0078 at |want| = 4, most of an absolute 1e-2.
MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def say(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)


def params_of(wl: datagen.Workload, **kw) -> sg.Params:
    d = dict(n_tokens=wl.n_tokens, n_q_heads=wl.n_q_heads, n_kv_heads=wl.n_kv_heads, block=wl.block,
             topk_tokens=wl.topk_tokens, union_tile=wl.union_tile, n_seqs=wl.n_seqs, head_dim=wl.head_dim,
             idx_heads=wl.idx_heads, idx_dim=wl.idx_dim)
    d.update(kw)
    return sg.Params(**d)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_dev(x: dict, device="cuda") -> dict:
    return {k: v.to(device).contiguous() for k, v in x.items()}


def assert_close_attention(got_bf16: torch.Tensor, want_f64: np.ndarray, what: str) -> None:
    got = bf16_to_f64(bits(got_bf16)).reshape(want_f64.shape)
    err = np.abs(got - want_f64)
    assert np.isfinite(got).all(), f"{what}: non-finite outputs"
    mx, mean = float(err.max()), float(err.mean())
    rel = float((err / np.maximum(1.0, np.abs(want_f64))).max())
    say(f"{what}: max_abs={mx:.3e} mean_abs={mean:.3e} max_abs/max(1,|want|)={rel:.3e}")
    assert rel <= MAX_ABS, f"{what}: max error {rel} of max(1, |want|) (max abs {mx})"
    assert mean <= MEAN_ABS, f"{what}: mean abs error {mean}"


class OracleChain:
    """The oracle's own compress -> top-k -> union, computed on host copies of the inputs."""

    def __init__(self, x_host: dict, p: sg.Params):
        self.p = p
        self.ki = bits(x_host["ki"])
        self.qi = bits(x_host["qi"])
        self.w = x_host["w"].cpu().numpy().astype(np.float32)
        self.kbar = oracle.compress(self.ki, p.block)

    def topk(self, rows=None) -> np.ndarray:
        return oracle.index_topk(self.qi, self.w, self.kbar, self.p.block, self.p.kb, rows=rows)

    def tile_rows(self, t: int) -> np.ndarray:
        i0 = t * self.p.union_tile
        return np.arange(i0, min(self.p.n_tokens, i0 + self.p.union_tile), dtype=np.int32)

    def union_of_tiles(self, tiles) -> tuple:
        """Oracle U(t,g) masks/counts for the listed tiles (topk computed for their rows only)."""
        p = self.p
        rows = np.concatenate([self.tile_rows(t) for t in tiles])
        sel = self.topk(rows)                                 # [G][len(rows)][kb]
        full = np.full((p.n_kv_heads, p.n_tokens, p.kb), -1, dtype=np.int32)
        full[:, rows] = sel
        umask, ucount = oracle.union(full, p.n_tokens, p.block, p.union_tile)
        return umask, ucount, sel, rows
