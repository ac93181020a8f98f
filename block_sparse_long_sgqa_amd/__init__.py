"""Python binding of libsgqa, the blockwise Sparse GQA hot path for AMD MI355X (gfx950).

The names mirror the C ABI in ``include/sgqa.h``. This module only marshals arguments: it checks
dtypes, devices, shapes and contiguity of torch tensors, passes their device pointers and the
current HIP stream to the library, and turns a nonzero status into an exception. Every step of the
path runs in the library's HIP kernels; there is no fallback. PyTorch provides device memory and
streams only.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsgqa.so")

SGQA_OK = 0
SGQA_ERR_NULL = 1
SGQA_ERR_SHAPE = 2
SGQA_ERR_ALIGN = 3
SGQA_ERR_WORKSPACE = 4
SGQA_ERR_DEVICE = 5
SGQA_ERR_HIP = 6
SGQA_ERR_SCRATCH = 7

# Scratch the library holds per GPU for sgqa_decode_noalloc.
NOALLOC_SCRATCH_BYTES = 64 << 20

SGQA_OP_COMPRESS = 0
SGQA_OP_INDEX_TOPK = 1
SGQA_OP_UNION = 2
SGQA_OP_ATTEND = 3
SGQA_OP_PREFILL = 4
SGQA_OP_DECODE = 5
SGQA_OP_ATTEND_MASKED = 6
SGQA_OP_PREFILL_MASKED = 7
SGQA_OP_ATTEND_BWD = 8

# Every symbol include/sgqa.h declares.
EXPORTED = ("sgqa_abi_version", "sgqa_status_string", "sgqa_workspace_size", "sgqa_compress", "sgqa_index_topk",
            "sgqa_union", "sgqa_attend", "sgqa_prefill", "sgqa_decode", "sgqa_decode_varlen", "sgqa_append",
            "sgqa_decode_fp8", "sgqa_index_union", "sgqa_attend_masked", "sgqa_prefill_masked",
            "sgqa_attend_fwd", "sgqa_attend_bwd", "sgqa_decode_noalloc")


class sgqa_pages(ctypes.Structure):
    """Mirror of `sgqa_pages` in include/sgqa.h (paged K/V cache descriptor)."""

    _fields_ = [("table", ctypes.c_void_p), ("max_pages", ctypes.c_int32), ("page_tokens", ctypes.c_int32),
                ("n_pages", ctypes.c_int32)]


class SgqaError(RuntimeError):
    def __init__(self, status: int, call: str, text: str):
        super().__init__(f"{call}: status {status} ({text})")
        self.status = status


class sgqa_params(ctypes.Structure):
    _fields_ = [
        ("n_tokens", ctypes.c_int32),
        ("n_seqs", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_heads", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("block", ctypes.c_int32),
        ("topk_tokens", ctypes.c_int32),
        ("union_tile", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
    ]


@dataclasses.dataclass
class Params:
    """Sizes of one call (see ``sgqa_params`` in include/sgqa.h)."""

    n_tokens: int
    n_q_heads: int
    n_kv_heads: int
    block: int = 8
    topk_tokens: int = 4096
    union_tile: int = 64
    n_seqs: int = 1
    head_dim: int = 128
    idx_heads: int = 4
    idx_dim: int = 64
    softmax_scale: float = 0.0

    @property
    def kb(self) -> int:
        return self.topk_tokens // self.block

    @property
    def n_tiles(self) -> int:
        return (self.n_tokens + self.union_tile - 1) // self.union_tile

    @property
    def n_words(self) -> int:
        return ((self.n_tokens + self.block - 1) // self.block + 31) // 32

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def c(self) -> sgqa_params:
        return sgqa_params(self.n_tokens, self.n_seqs, self.n_q_heads, self.n_kv_heads, self.head_dim,
                           self.idx_heads, self.idx_dim, self.block, self.topk_tokens, self.union_tile,
                           float(self.softmax_scale))


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libsgqa.so. Raises if it has not been built (no fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m block_sparse_long_sgqa_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P = ctypes.c_void_p
        PP = ctypes.POINTER(sgqa_params)
        L.sgqa_abi_version.argtypes = []
        L.sgqa_abi_version.restype = ctypes.c_int
        L.sgqa_status_string.argtypes = [ctypes.c_int]
        L.sgqa_status_string.restype = ctypes.c_char_p
        L.sgqa_workspace_size.argtypes = [PP, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]
        L.sgqa_workspace_size.restype = ctypes.c_int
        L.sgqa_compress.argtypes = [PP, P, P, P]
        L.sgqa_index_topk.argtypes = [PP, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_union.argtypes = [PP, P, P, P, P]
        L.sgqa_attend.argtypes = [PP, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_prefill.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_decode.argtypes = [PP, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_decode_noalloc.argtypes = [PP, P, P, P, P, P, P, P, P, P]
        PG = ctypes.POINTER(sgqa_pages)
        L.sgqa_decode_varlen.argtypes = [PP, P, P, P, PG, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_append.argtypes = [PP, P, P, P, P, P, P, PG, P, P, P]
        L.sgqa_decode_fp8.argtypes = [PP, P, P, P, P, PG, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_index_union.argtypes = [PP, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_attend_masked.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_prefill_masked.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_attend_fwd.argtypes = [PP, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        L.sgqa_attend_bwd.argtypes = [PP, P, P, P, P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
        for name in ("sgqa_compress", "sgqa_index_topk", "sgqa_union", "sgqa_attend", "sgqa_prefill", "sgqa_decode",
                     "sgqa_decode_varlen", "sgqa_append", "sgqa_decode_fp8", "sgqa_index_union",
                     "sgqa_attend_masked", "sgqa_prefill_masked", "sgqa_attend_fwd", "sgqa_attend_bwd",
                     "sgqa_decode_noalloc"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().sgqa_status_string(int(status)).decode()


def _check(status: int, call: str) -> None:
    if status != SGQA_OK:
        raise SgqaError(status, call, status_string(status))


def _ptr(t: Optional[torch.Tensor], name: str, dtype: torch.dtype, shape=None):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: expected a GPU tensor, got {t.device}")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (the library never copies)")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def workspace_size(p: Params, op: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().sgqa_workspace_size(ctypes.byref(p.c()), op, ctypes.byref(out)), "sgqa_workspace_size")
    return int(out.value)


def workspace(p: Params, op: int, device="cuda") -> torch.Tensor:
    """A device byte buffer of the size op needs (at least 16 bytes so the pointer is valid)."""
    return torch.empty(max(16, workspace_size(p, op)), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------------ calls

def sgqa_compress(p: Params, idx_k: torch.Tensor, blk_k: torch.Tensor, stream=None) -> None:
    S, N, B, dI = p.n_seqs, p.n_tokens, p.block, p.idx_dim
    a = _ptr(idx_k, "idx_k", torch.bfloat16, (S, N, dI) if S > 1 else None)
    b = _ptr(blk_k, "blk_k", torch.bfloat16, (S, N // B, dI) if S > 1 else None)
    if S == 1:
        if idx_k.numel() != N * dI or blk_k.numel() != (N // B) * dI:
            raise ValueError("idx_k must hold N*d_I and blk_k floor(N/B)*d_I elements")
    _check(lib().sgqa_compress(ctypes.byref(p.c()), a, b, _stream(stream)), "sgqa_compress")


def sgqa_index_topk(p: Params, idx_q, idx_w, blk_k, topk, ws=None, stream=None) -> None:
    N, G = p.n_tokens, p.n_kv_heads
    args = (_ptr(idx_q, "idx_q", torch.bfloat16, (N, G, p.idx_heads, p.idx_dim)),
            _ptr(idx_w, "idx_w", torch.float32, (G, p.idx_heads)),
            _ptr(blk_k, "blk_k", torch.bfloat16, (N // p.block, p.idx_dim)),
            _ptr(topk, "topk", torch.int32, (G, N, p.kb)))
    wsp = _ptr(ws, "ws", torch.uint8)
    _check(lib().sgqa_index_topk(ctypes.byref(p.c()), *args, wsp, ws.numel() if ws is not None else 0,
                                 _stream(stream)), "sgqa_index_topk")


def sgqa_union(p: Params, topk, umask, ucount, stream=None) -> None:
    G = p.n_kv_heads
    args = (_ptr(topk, "topk", torch.int32, (G, p.n_tokens, p.kb)),
            _ptr(umask, "umask", torch.int32, (G, p.n_tiles, p.n_words)),
            _ptr(ucount, "ucount", torch.int32, (G, p.n_tiles)))
    _check(lib().sgqa_union(ctypes.byref(p.c()), *args, _stream(stream)), "sgqa_union")


def sgqa_index_union(p: Params, idx_q, idx_w, blk_k, umask, ucount, ws=None, stream=None) -> None:
    N, G = p.n_tokens, p.n_kv_heads
    args = (_ptr(idx_q, "idx_q", torch.bfloat16, (N, G, p.idx_heads, p.idx_dim)),
            _ptr(idx_w, "idx_w", torch.float32, (G, p.idx_heads)),
            _ptr(blk_k, "blk_k", torch.bfloat16, (N // p.block, p.idx_dim)),
            _ptr(umask, "umask", torch.int32, (G, p.n_tiles, p.n_words)),
            _ptr(ucount, "ucount", torch.int32, (G, p.n_tiles)))
    wsp = _ptr(ws, "ws", torch.uint8)
    _check(lib().sgqa_index_union(ctypes.byref(p.c()), *args, wsp, ws.numel() if ws is not None else 0,
                                  _stream(stream)), "sgqa_index_union")


def sgqa_attend(p: Params, q, k, v, umask, ucount, out, ws=None, stream=None) -> None:
    N, Hq, G, D = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    args = (_ptr(q, "q", torch.bfloat16, (N, Hq, D)), _ptr(k, "k", torch.bfloat16, (G, N, D)),
            _ptr(v, "v", torch.bfloat16, (G, N, D)),
            _ptr(umask, "umask", torch.int32, (G, p.n_tiles, p.n_words)),
            _ptr(ucount, "ucount", torch.int32, (G, p.n_tiles)), _ptr(out, "out", torch.bfloat16, (N, Hq, D)))
    wsp = _ptr(ws, "ws", torch.uint8)
    _check(lib().sgqa_attend(ctypes.byref(p.c()), *args, wsp, ws.numel() if ws is not None else 0,
                             _stream(stream)), "sgqa_attend")


def sgqa_prefill(p: Params, q, k, v, idx_q, idx_w, idx_k, out, ws, stream=None) -> None:
    N, Hq, G, D = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    args = (_ptr(q, "q", torch.bfloat16, (N, Hq, D)), _ptr(k, "k", torch.bfloat16, (G, N, D)),
            _ptr(v, "v", torch.bfloat16, (G, N, D)),
            _ptr(idx_q, "idx_q", torch.bfloat16, (N, G, p.idx_heads, p.idx_dim)),
            _ptr(idx_w, "idx_w", torch.float32, (G, p.idx_heads)),
            _ptr(idx_k, "idx_k", torch.bfloat16, (N, p.idx_dim)),
            _ptr(out, "out", torch.bfloat16, (N, Hq, D)))
    _check(lib().sgqa_prefill(ctypes.byref(p.c()), *args, _ptr(ws, "ws", torch.uint8), ws.numel(),
                              _stream(stream)), "sgqa_prefill")


def sgqa_attend_fwd(p: Params, q, k, v, umask, ucount, out, lse, stream=None) -> None:
    N, Hq, G, D = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    args = (_ptr(q, "q", torch.bfloat16, (N, Hq, D)), _ptr(k, "k", torch.bfloat16, (G, N, D)),
            _ptr(v, "v", torch.bfloat16, (G, N, D)),
            _ptr(umask, "umask", torch.int32, (G, p.n_tiles, p.n_words)),
            _ptr(ucount, "ucount", torch.int32, (G, p.n_tiles)), _ptr(out, "out", torch.bfloat16, (N, Hq, D)),
            _ptr(lse, "lse", torch.float32, (N, Hq)))
    _check(lib().sgqa_attend_fwd(ctypes.byref(p.c()), *args, None, 0, _stream(stream)), "sgqa_attend_fwd")


def sgqa_attend_bwd(p: Params, q, k, v, umask, ucount, out, lse, dout, dq, dk, dv, ws, stream=None) -> None:
    N, Hq, G, D = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    args = (_ptr(q, "q", torch.bfloat16, (N, Hq, D)), _ptr(k, "k", torch.bfloat16, (G, N, D)),
            _ptr(v, "v", torch.bfloat16, (G, N, D)),
            _ptr(umask, "umask", torch.int32, (G, p.n_tiles, p.n_words)),
            _ptr(ucount, "ucount", torch.int32, (G, p.n_tiles)), _ptr(out, "out", torch.bfloat16, (N, Hq, D)),
            _ptr(lse, "lse", torch.float32, (N, Hq)), _ptr(dout, "dout", torch.bfloat16, (N, Hq, D)),
            _ptr(dq, "dq", torch.bfloat16, (N, Hq, D)), _ptr(dk, "dk", torch.bfloat16, (G, N, D)),
            _ptr(dv, "dv", torch.bfloat16, (G, N, D)))
    _check(lib().sgqa_attend_bwd(ctypes.byref(p.c()), *args, _ptr(ws, "ws", torch.uint8), ws.numel(),
                                 _stream(stream)), "sgqa_attend_bwd")


def sgqa_attend_masked(p: Params, q, k, v, topk, umask, ucount, out, ws, stream=None) -> None:
    N, Hq, G, D = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    args = (_ptr(q, "q", torch.bfloat16, (N, Hq, D)), _ptr(k, "k", torch.bfloat16, (G, N, D)),
            _ptr(v, "v", torch.bfloat16, (G, N, D)), _ptr(topk, "topk", torch.int32, (G, N, p.kb)),
            _ptr(umask, "umask", torch.int32, (G, p.n_tiles, p.n_words)),
            _ptr(ucount, "ucount", torch.int32, (G, p.n_tiles)), _ptr(out, "out", torch.bfloat16, (N, Hq, D)))
    _check(lib().sgqa_attend_masked(ctypes.byref(p.c()), *args, _ptr(ws, "ws", torch.uint8), ws.numel(),
                                    _stream(stream)), "sgqa_attend_masked")


def sgqa_prefill_masked(p: Params, q, k, v, idx_q, idx_w, idx_k, out, ws, stream=None) -> None:
    N, Hq, G, D = p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    args = (_ptr(q, "q", torch.bfloat16, (N, Hq, D)), _ptr(k, "k", torch.bfloat16, (G, N, D)),
            _ptr(v, "v", torch.bfloat16, (G, N, D)),
            _ptr(idx_q, "idx_q", torch.bfloat16, (N, G, p.idx_heads, p.idx_dim)),
            _ptr(idx_w, "idx_w", torch.float32, (G, p.idx_heads)),
            _ptr(idx_k, "idx_k", torch.bfloat16, (N, p.idx_dim)),
            _ptr(out, "out", torch.bfloat16, (N, Hq, D)))
    _check(lib().sgqa_prefill_masked(ctypes.byref(p.c()), *args, _ptr(ws, "ws", torch.uint8), ws.numel(),
                                     _stream(stream)), "sgqa_prefill_masked")


def sgqa_decode(p: Params, q, k_cache, v_cache, blk_k, idx_q, idx_w, out, ws, topk_out=None, stream=None) -> None:
    S, L, Hq, G, D = p.n_seqs, p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    args = (_ptr(q, "q", torch.bfloat16, (S, Hq, D)), _ptr(k_cache, "k_cache", torch.bfloat16, (S, G, L, D)),
            _ptr(v_cache, "v_cache", torch.bfloat16, (S, G, L, D)),
            _ptr(blk_k, "blk_k", torch.bfloat16, (S, L // p.block, p.idx_dim)),
            _ptr(idx_q, "idx_q", torch.bfloat16, (S, G, p.idx_heads, p.idx_dim)),
            _ptr(idx_w, "idx_w", torch.float32, (G, p.idx_heads)),
            _ptr(topk_out, "topk_out", torch.int32, (S, G, p.kb)),
            _ptr(out, "out", torch.bfloat16, (S, Hq, D)))
    _check(lib().sgqa_decode(ctypes.byref(p.c()), *args, _ptr(ws, "ws", torch.uint8), ws.numel(),
                             _stream(stream)), "sgqa_decode")


def sgqa_decode_noalloc(p: Params, q, k_cache, v_cache, blk_k, idx_q, idx_w, out, topk_out=None,
                        stream=None) -> None:
    """sgqa_decode with the library's own per-GPU scratch instead of a workspace (allocates nothing)."""
    S, L, Hq, G, D = p.n_seqs, p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    args = (_ptr(q, "q", torch.bfloat16, (S, Hq, D)), _ptr(k_cache, "k_cache", torch.bfloat16, (S, G, L, D)),
            _ptr(v_cache, "v_cache", torch.bfloat16, (S, G, L, D)),
            _ptr(blk_k, "blk_k", torch.bfloat16, (S, L // p.block, p.idx_dim)),
            _ptr(idx_q, "idx_q", torch.bfloat16, (S, G, p.idx_heads, p.idx_dim)),
            _ptr(idx_w, "idx_w", torch.float32, (G, p.idx_heads)),
            _ptr(topk_out, "topk_out", torch.int32, (S, G, p.kb)),
            _ptr(out, "out", torch.bfloat16, (S, Hq, D)))
    _check(lib().sgqa_decode_noalloc(ctypes.byref(p.c()), *args, _stream(stream)), "sgqa_decode_noalloc")


class Pages:
    """A paged K/V cache: `table` [S][max_pages] int32 on the GPU, pools [n_pages][G][page_tokens][D]."""

    def __init__(self, table, page_tokens: int, n_pages: int):
        self.table = table
        self.page_tokens = page_tokens
        self.n_pages = n_pages

    def c(self, n_seqs: int) -> sgqa_pages:
        t = _ptr(self.table, "page table", torch.int32)
        if self.table.dim() != 2 or self.table.shape[0] != n_seqs:
            raise ValueError(f"page table: expected [{n_seqs}][max_pages], got {tuple(self.table.shape)}")
        return sgqa_pages(t.value, self.table.shape[1], self.page_tokens, self.n_pages)


def _cache_shape(p: Params, pages: Optional[Pages]):
    if pages is None:
        return (p.n_seqs, p.n_kv_heads, p.n_tokens, p.head_dim)
    return (pages.n_pages, p.n_kv_heads, pages.page_tokens, p.head_dim)


def sgqa_decode_varlen(p: Params, q, k_cache, v_cache, blk_k, idx_q, idx_w, seq_lens, out, ws, pages=None,
                       topk_out=None, stream=None) -> None:
    S, C, Hq, G, D = p.n_seqs, p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    shp = _cache_shape(p, pages)
    pg = pages.c(S) if pages is not None else None
    args = (_ptr(q, "q", torch.bfloat16, (S, Hq, D)), _ptr(k_cache, "k_cache", torch.bfloat16, shp),
            _ptr(v_cache, "v_cache", torch.bfloat16, shp), ctypes.byref(pg) if pg is not None else None,
            _ptr(blk_k, "blk_k", torch.bfloat16, (S, C // p.block, p.idx_dim)),
            _ptr(idx_q, "idx_q", torch.bfloat16, (S, G, p.idx_heads, p.idx_dim)),
            _ptr(idx_w, "idx_w", torch.float32, (G, p.idx_heads)),
            _ptr(seq_lens, "seq_lens", torch.int32, (S,)),
            _ptr(topk_out, "topk_out", torch.int32, (S, G, p.kb)),
            _ptr(out, "out", torch.bfloat16, (S, Hq, D)))
    _check(lib().sgqa_decode_varlen(ctypes.byref(p.c()), *args, _ptr(ws, "ws", torch.uint8), ws.numel(),
                                    _stream(stream)), "sgqa_decode_varlen")


def sgqa_append(p: Params, k_new, v_new, idx_k_new, positions, k_cache, v_cache, idx_k_cache, blk_k, pages=None,
                stream=None) -> None:
    S, C, G, D = p.n_seqs, p.n_tokens, p.n_kv_heads, p.head_dim
    shp = _cache_shape(p, pages)
    pg = pages.c(S) if pages is not None else None
    args = (_ptr(k_new, "k_new", torch.bfloat16, (S, G, D)), _ptr(v_new, "v_new", torch.bfloat16, (S, G, D)),
            _ptr(idx_k_new, "idx_k_new", torch.bfloat16, (S, p.idx_dim)),
            _ptr(positions, "positions", torch.int32, (S,)),
            _ptr(k_cache, "k_cache", torch.bfloat16, shp), _ptr(v_cache, "v_cache", torch.bfloat16, shp),
            ctypes.byref(pg) if pg is not None else None,
            _ptr(idx_k_cache, "idx_k_cache", torch.bfloat16, (S, C, p.idx_dim)),
            _ptr(blk_k, "blk_k", torch.bfloat16, (S, C // p.block, p.idx_dim)))
    _check(lib().sgqa_append(ctypes.byref(p.c()), *args, _stream(stream)), "sgqa_append")


def _codes(t, name: str, shape):
    """FP8 E4M3 cache as its uint8 codes (a float8_e4m3fn tensor is reinterpreted, never converted)."""
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return _ptr(t, name, torch.uint8, shape)


def sgqa_decode_fp8(p: Params, q, k_cache, v_cache, kv_scale, blk_k, idx_q, idx_w, out, ws, seq_lens=None,
                    pages=None, topk_out=None, stream=None) -> None:
    """Decode over FP8 E4M3 K/V caches (uint8 codes or float8_e4m3fn) with kv_scale [S][G][2] fp32."""
    S, C, Hq, G, D = p.n_seqs, p.n_tokens, p.n_q_heads, p.n_kv_heads, p.head_dim
    shp = _cache_shape(p, pages)
    pg = pages.c(S) if pages is not None else None
    args = (_ptr(q, "q", torch.bfloat16, (S, Hq, D)), _codes(k_cache, "k_cache", shp),
            _codes(v_cache, "v_cache", shp), _ptr(kv_scale, "kv_scale", torch.float32, (S, G, 2)),
            ctypes.byref(pg) if pg is not None else None,
            _ptr(blk_k, "blk_k", torch.bfloat16, (S, C // p.block, p.idx_dim)),
            _ptr(idx_q, "idx_q", torch.bfloat16, (S, G, p.idx_heads, p.idx_dim)),
            _ptr(idx_w, "idx_w", torch.float32, (G, p.idx_heads)),
            _ptr(seq_lens, "seq_lens", torch.int32, (S,)),
            _ptr(topk_out, "topk_out", torch.int32, (S, G, p.kb)),
            _ptr(out, "out", torch.bfloat16, (S, Hq, D)))
    _check(lib().sgqa_decode_fp8(ctypes.byref(p.c()), *args, _ptr(ws, "ws", torch.uint8), ws.numel(),
                                 _stream(stream)), "sgqa_decode_fp8")


# ------------------------------------------------------------------------------------ helpers

def alloc_prefill_outputs(p: Params, device="cuda") -> dict:
    """Output/intermediate tensors of the single calls, shaped as the ABI documents."""
    G = p.n_kv_heads
    return {
        "blk_k": torch.empty((max(p.n_tokens // p.block, 1), p.idx_dim), dtype=torch.bfloat16, device=device),
        "topk": torch.empty((G, p.n_tokens, p.kb), dtype=torch.int32, device=device),
        "umask": torch.empty((G, p.n_tiles, p.n_words), dtype=torch.int32, device=device),
        "ucount": torch.empty((G, p.n_tiles), dtype=torch.int32, device=device),
        "out": torch.empty((p.n_tokens, p.n_q_heads, p.head_dim), dtype=torch.bfloat16, device=device),
    }
